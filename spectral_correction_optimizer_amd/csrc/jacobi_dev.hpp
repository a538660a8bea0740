// Device helpers of the blocked Jacobi kernels shared by jacobi.hip (pair
// rounds) and quad.hip (rounds of four-block groups): the pair solve's
// moving-frame sweep, the rotation formula and the apply's operand order.
#pragma once

#include "common.hpp"
#include "internal.hpp"

namespace scopt {
namespace {

constexpr int PW = kPw;  // 64 rows per pair block

// ---------------------------------------------------------------------------------
// Pair solve: one cyclic sweep of 2x2 Jacobi rotations on the 64x64 pair Gram.
//
// The sweep runs in a moving frame ("slots"): at every step pair j rotates slots
// (2j, 2j+1), and afterwards every column moves to slot sigma(s) -- slot 0 stays,
// the others advance one place along the cycle 1, 3, 5, ..., 63, 62, 60, ..., 2.
// This is the circle (round-robin tournament) ordering: in 63 steps every two
// columns share a pair exactly once, and the cycle closes, so the final frame is
// the original one.  Reads of a step are then at fixed, conflict-free LDS
// addresses, and the move is folded into the step's writes.
constexpr int SG = 66;  // LDS row stride of G (upper triangle + diagonal, slot frame)
constexpr int SR = 68;  // LDS row stride of R^T (row = slot, column = original row of R)
// A lower-triangle entry of G, never read: it takes the writes of lanes without a block.
constexpr int kSink = (PW - 1) * SG;

__device__ __forceinline__ int slot_next(int s) {
    return s == 0 ? 0 : s == 2 ? 1 : (s & 1) ? (s == 63 ? 62 : s + 2) : s - 2;
}
// Position of slot s (> 0) on the cycle, and the slot at position k.
__device__ __forceinline__ int cycle_pos(int s) { return (s & 1) ? (s - 1) >> 1 : 32 + ((62 - s) >> 1); }
__device__ __forceinline__ int cycle_slot(int k) { return k < 32 ? 2 * k + 1 : 126 - 2 * k; }

// Pair-blocks (i < j) of each bank class t = (2 i + j) mod 16, in order of i then
// j (30 or 32 per class): bit 15 marks an entry, bits 0-7 hold i, bits 8-15 j.
struct BlockTable {
    unsigned short v[16][32];
};
constexpr BlockTable make_block_table() {
    BlockTable t{};
    for (int c = 0; c < 16; ++c) {
        int n = 0;
        for (int i = 0; i < 32; ++i)
            for (int e = 0; e < 2; ++e) {
                const int j = ((c - 2 * i) & 15) + 16 * e;
                if (j > i) t.v[c][n++] = (unsigned short)(0x8000 | i | (j << 8));
            }
    }
    return t;
}
__constant__ BlockTable kBlocks = make_block_table();

// Rotation of a pair with Gram entries g_pp, g_pq, g_qq: the angle that zeroes
// g_pq, as c, s and c - 1; the identity when either column is at or below the
// zero floor or the pair is orthogonal to the threshold tol.
__device__ __forceinline__ void pair_rotation(float gpp, float gpq, float gqq, float floor2,
                                              float tol, float& c, float& sn, float& cm1) {
    c = 1.0f;
    sn = 0.0f;
    cm1 = 0.0f;
    if (gpp > floor2 && gqq > floor2 && fabsf(gpq) > tol * __builtin_amdgcn_sqrtf(gpp * gqq)) {
        const float zeta = (gqq - gpp) * 0.5f * __builtin_amdgcn_rcpf(gpq);
        const float az = fabsf(zeta);
        // t = sign(zeta) / (|zeta| + sqrt(1 + zeta^2)), without overflow
        const float den = az < 1e18f ? az + __builtin_amdgcn_sqrtf(fmaf(az, az, 1.0f)) : 2.0f * az;
        const float t = copysignf(__builtin_amdgcn_rcpf(den), zeta);
        const float hq = __builtin_amdgcn_sqrtf(fmaf(t, t, 1.0f));
        c = __builtin_amdgcn_rcpf(hq);
        sn = t * c;
        cm1 = -t * sn * __builtin_amdgcn_rcpf(1.0f + hq);
    }
}

// Row of the pair block fed by lane half hl at contraction step s of the apply.
// The order is chosen so that a lane's 32 B operands are exactly the 32 rows of
// its 32x32 MFMA outputs (row 8 (r / 4) + 4 hl + r % 4 of acc0, 32 more of acc1).
__device__ __forceinline__ int apply_row(int s, int hl) {
    return 32 * (s >> 4) + 8 * ((s & 15) >> 2) + 4 * hl + (s & 3);
}
// a b over 32x32x16 bfloat16 products of the three-way splits of a and b: the six
// largest part products, smallest first (float32-equivalent)
__device__ __forceinline__ v16f mfma_split6(const Split8& a, const Split8& b, v16f acc) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.l, b.h, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.m, b.m, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.h, b.l, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.m, b.h, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.h, b.m, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.h, b.h, acc, 0, 0, 0);
    return acc;
}

__device__ __forceinline__ int insert_zero_bit(int v, int b) {
    return ((v >> b) << (b + 1)) | (v & ((1 << b) - 1));
}
__device__ __forceinline__ int remove_bit(int v, int b) {
    return ((v >> (b + 1)) << b) | (v & ((1 << b) - 1));
}

// One cyclic sweep of the pair solve on NW wavefronts (wave w of the pair, lane l):
// G (upper triangle, slot frame, stride SG) and R^T = 0 (stride SR) in copy 0 on
// entry; cc / ss hold a step's 32 rotations.  Wave w takes its share of each bank
// class's pair-blocks and the R^T columns [64 w / NW, 64 (w + 1) / NW); every wave
// computes all 32 rotations of a step (redundant but identical, no exchange).
// NB = 2: two copies, a step reads one and writes the other (one barrier per
// step); NB = 1: one copy, two barriers per step.  The barriers are workgroup
// barriers: every wave of the workgroup runs the 63 steps.  Returns the copy that
// holds the result (G rotated, R^T = (Q - I)^T).
// QF: R^T holds Q^T itself (I on entry, Q^T on exit): the rows of a rotated pair
// need no correction of the identity's entries, whose columns move with the frame
// (their bookkeeping is a fifth of a step's arithmetic).  The caller takes Q - I
// from it with diag_to_delta.
template <int NW, int NB, bool QF = false>
__device__ __forceinline__ int pair_sweep(float (*G)[PW * SG], float (*RT)[PW * SR], float* cc,
                                          float* ss, int l, int w, float floor2, float tol) {
    constexpr int NU = 8 / NW;   // pair-blocks of G per lane
    constexpr int NK = 8 / NW;   // 8-column groups of R^T per lane
    constexpr int CW = PW / NW;  // columns of R^T per wave
    // 3. per-lane addresses (the one-wavefront kernel's, restricted to the wave's
    //    share).  A correction of R's identity entries in a column of another
    //    wave goes to the row's padding column PW, which is never read.
    const int jr = l >> 1, hh = l & 1, cls = l & 15, odd = (l >> 4) & 1;
    int blk_ij[NU], blk_rd[NU], blk_wr[NU][4];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        const int v = kBlocks.v[cls][NU * ((l >> 4) + 4 * w) + u];
        const bool ok = v & 0x8000;
        const int i = ok ? v & 255 : 0, j = ok ? (v >> 8) & 127 : 1;
        blk_ij[u] = i | (j << 8);
        blk_rd[u] = 2 * i * SG + 2 * j;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int ee = odd ? (e ^ 1) : e;
            const int r = slot_next(2 * i + (ee >> 1)), c = slot_next(2 * j + (ee & 1));
            blk_wr[u][e] = ok ? min(r, c) * SG + max(r, c) : kSink;
        }
    }
    const int sp_ = slot_next(2 * jr), sq_ = slot_next(2 * jr + 1);
    const int dg_pp = sp_ * SG + sp_, dg_qq = sq_ * SG + sq_, dg_pq = min(sp_, sq_) * SG + max(sp_, sq_);
    const int cb = CW * w;
    const int rt_rd = 2 * jr * SR + cb + 4 * hh, rt_wp = sp_ * SR + cb + 4 * hh, rt_wq = sq_ * SR + cb + 4 * hh;
    int kp = QF ? 0 : (jr == 0 ? -1 : cycle_pos(2 * jr)), kq = QF ? 0 : cycle_pos(2 * jr + 1);
    __syncthreads();
    v2f dpq = *(const v2f*)&G[0][2 * jr * SG + 2 * jr];
    float gqq = G[0][(2 * jr + 1) * SG + 2 * jr + 1];
    int cur = 0;
#pragma unroll 1
    for (int ir = 0; ir < PW - 1; ++ir) {
        const float* Gr = G[cur];
        float* Gw = G[NB == 2 ? cur ^ 1 : cur];
        const float* Rr = RT[cur];
        float* Rw = RT[NB == 2 ? cur ^ 1 : cur];
        __asm__ volatile("" ::"v"(dpq), "v"(gqq));
        v2f x0[NU], x1[NU];
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            x0[u] = *(const v2f*)&Gr[blk_rd[u]];
            x1[u] = *(const v2f*)&Gr[blk_rd[u] + SG];
        }
        v4f xr[NK], yr[NK];
#pragma unroll
        for (int k = 0; k < NK; ++k) {
            xr[k] = *(const v4f*)&Rr[rt_rd + 8 * k];
            yr[k] = *(const v4f*)&Rr[rt_rd + SR + 8 * k];
        }
        const int op = QF ? 0 : (kp < 0 ? 0 : cycle_slot(kp)), oq = QF ? 0 : cycle_slot(kq);
        float xop = 0.0f, yop = 0.0f, xoq = 0.0f, yoq = 0.0f;
        if constexpr (!QF) {
            xop = Rr[2 * jr * SR + op];
            yop = Rr[(2 * jr + 1) * SR + op];
            xoq = Rr[2 * jr * SR + oq];
            yoq = Rr[(2 * jr + 1) * SR + oq];
        }
        const float gpp = dpq[0], gpq = dpq[1];
        float c, sn, cm1;
        pair_rotation(gpp, gpq, gqq, floor2, tol, c, sn, cm1);
        cc[jr] = c;
        ss[jr] = sn;
        __asm__ volatile("" ::: "memory");
        float wv[NU][4];
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int i = blk_ij[u] & 255, j = (blk_ij[u] >> 8) & 255;
            const float ci = cc[i], si = ss[i], cj = cc[j], sj = ss[j];
            const float y00 = cj * x0[u][0] - sj * x0[u][1], y01 = sj * x0[u][0] + cj * x0[u][1];
            const float y10 = cj * x1[u][0] - sj * x1[u][1], y11 = sj * x1[u][0] + cj * x1[u][1];
            const float z00 = ci * y00 - si * y10, z01 = ci * y01 - si * y11;
            const float z10 = si * y00 + ci * y10, z11 = si * y01 + ci * y11;
            wv[u][0] = odd ? z01 : z00;
            wv[u][1] = odd ? z00 : z01;
            wv[u][2] = odd ? z11 : z10;
            wv[u][3] = odd ? z10 : z11;
        }
        if (NB == 1) __syncthreads();  // every wave has read this step's G and R^T
#pragma unroll
        for (int u = 0; u < NU; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e) Gw[blk_wr[u][e]] = wv[u][e];
        if (w == 0) {
            const float y00 = c * gpp - sn * gpq, y01 = sn * gpp + c * gpq;
            const float y10 = c * gpq - sn * gqq, y11 = sn * gpq + c * gqq;
            Gw[dg_pp] = c * y00 - sn * y10;
            Gw[dg_pq] = c * y01 - sn * y11;
            Gw[dg_qq] = sn * y01 + c * y11;
        }
#pragma unroll
        for (int k = 0; k < NK; ++k) {
            v4f np, nq;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                np[e] = fmaf(cm1, xr[k][e], xr[k][e]) - sn * yr[k][e];
                nq[e] = fmaf(cm1, yr[k][e], yr[k][e]) + sn * xr[k][e];
            }
            *(v4f*)&Rw[rt_wp + 8 * k] = np;
            *(v4f*)&Rw[rt_wq + 8 * k] = nq;
        }
        if constexpr (!QF) {
            const int cop = op / CW == w ? op : PW, coq = oq / CW == w ? oq : PW;
            Rw[sp_ * SR + cop] = fmaf(cm1, xop, xop) - sn * yop + cm1;
            Rw[sq_ * SR + cop] = fmaf(cm1, yop, yop) + sn * xop + sn;
            Rw[sp_ * SR + coq] = fmaf(cm1, xoq, xoq) - sn * yoq - sn;
            Rw[sq_ * SR + coq] = fmaf(cm1, yoq, yoq) + sn * xoq + cm1;
            kp = kp < 0 ? -1 : (kp == 0 ? 62 : kp - 1);
            kq = kq == 0 ? 62 : kq - 1;
        }
        __syncthreads();
        dpq = *(const v2f*)&Gw[2 * jr * SG + 2 * jr];
        gqq = Gw[(2 * jr + 1) * SG + 2 * jr + 1];
        if (NB == 2) cur ^= 1;
    }
    return cur;
}

// The QF sweep of the group solve with the 32 rotations of a step computed once,
// by wave 0 of the pair, and published as (c, s, c - 1) in rot[] before the step's
// first barrier; the other waves read them after it (the step already has two
// barriers: reads | writes).  The same rotations and arithmetic as pair_sweep<NW, 1,
// true>, so the same results, with the rotation's vector work (about a quarter of a
// step, square roots and reciprocals included) done by one wave instead of four.
// On entry G holds the pair Gram and R^T = I (copy 0, as pair_sweep).  A lane
// writes its blocks' four entries in the same order in every quarter-wave (the
// pair rounds' sweep alternates it to spread the writes over the banks): the
// swap's four selects a block cost more than the conflicts they avoid here
// (group solve 0.65-0.68 -> 0.63-0.64 ms for 768 groups).
template <int NW>
__device__ __forceinline__ void pair_sweep_q(float* G, float* RT, v4f* rot, int l, int w, float floor2,
                                             float tol) {
    constexpr int NU = 8 / NW;   // pair-blocks of G per lane
    constexpr int NK = 8 / NW;   // 8-column groups of R^T per lane
    constexpr int CW = PW / NW;  // columns of R^T per wave
    const int jr = l >> 1, hh = l & 1, cls = l & 15;
    int blk_ij[NU], blk_rd[NU], blk_wr[NU][4];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        const int v = kBlocks.v[cls][NU * ((l >> 4) + 4 * w) + u];
        const bool ok = v & 0x8000;
        const int i = ok ? v & 255 : 0, j = ok ? (v >> 8) & 127 : 1;
        blk_ij[u] = i | (j << 8);
        blk_rd[u] = 2 * i * SG + 2 * j;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int ee = e;
            const int r = slot_next(2 * i + (ee >> 1)), c = slot_next(2 * j + (ee & 1));
            blk_wr[u][e] = ok ? min(r, c) * SG + max(r, c) : kSink;
        }
    }
    const int sp_ = slot_next(2 * jr), sq_ = slot_next(2 * jr + 1);
    const int dg_pp = sp_ * SG + sp_, dg_qq = sq_ * SG + sq_, dg_pq = min(sp_, sq_) * SG + max(sp_, sq_);
    const int cb = CW * w;
    const int rt_rd = 2 * jr * SR + cb + 4 * hh, rt_wp = sp_ * SR + cb + 4 * hh, rt_wq = sq_ * SR + cb + 4 * hh;
    __syncthreads();
    v2f dpq = {0.0f, 0.0f};
    float gqq = 0.0f;
    if (w == 0) {
        dpq = *(const v2f*)&G[2 * jr * SG + 2 * jr];
        gqq = G[(2 * jr + 1) * SG + 2 * jr + 1];
    }
#pragma unroll 1
    for (int ir = 0; ir < PW - 1; ++ir) {
        __asm__ volatile("" ::"v"(dpq), "v"(gqq));
        v2f x0[NU], x1[NU];
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            x0[u] = *(const v2f*)&G[blk_rd[u]];
            x1[u] = *(const v2f*)&G[blk_rd[u] + SG];
        }
        v4f xr[NK], yr[NK];
#pragma unroll
        for (int k = 0; k < NK; ++k) {
            xr[k] = *(const v4f*)&RT[rt_rd + 8 * k];
            yr[k] = *(const v4f*)&RT[rt_rd + SR + 8 * k];
        }
        const float gpp = dpq[0], gpq = dpq[1];
        float c = 1.0f, sn = 0.0f, cm1 = 0.0f;
        if (w == 0) {
            pair_rotation(gpp, gpq, gqq, floor2, tol, c, sn, cm1);
            if (hh == 0) rot[jr] = v4f{c, sn, cm1, 0.0f};
        }
        __syncthreads();  // the rotations are published; every wave has read this step's G and R^T
        if (w != 0) {
            const v4f r = rot[jr];
            c = r[0];
            sn = r[1];
            cm1 = r[2];
        }
        float wv[NU][4];
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int i = blk_ij[u] & 255, j = (blk_ij[u] >> 8) & 255;
            const v2f csi = *(const v2f*)&rot[i], csj = *(const v2f*)&rot[j];
            const float ci = csi[0], si = csi[1], cj = csj[0], sj = csj[1];
            const float y00 = cj * x0[u][0] - sj * x0[u][1], y01 = sj * x0[u][0] + cj * x0[u][1];
            const float y10 = cj * x1[u][0] - sj * x1[u][1], y11 = sj * x1[u][0] + cj * x1[u][1];
            const float z00 = ci * y00 - si * y10, z01 = ci * y01 - si * y11;
            const float z10 = si * y00 + ci * y10, z11 = si * y01 + ci * y11;
            wv[u][0] = z00;
            wv[u][1] = z01;
            wv[u][2] = z10;
            wv[u][3] = z11;
        }
#pragma unroll
        for (int u = 0; u < NU; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e) G[blk_wr[u][e]] = wv[u][e];
        if (w == 0) {
            const float y00 = c * gpp - sn * gpq, y01 = sn * gpp + c * gpq;
            const float y10 = c * gpq - sn * gqq, y11 = sn * gpq + c * gqq;
            G[dg_pp] = c * y00 - sn * y10;
            G[dg_pq] = c * y01 - sn * y11;
            G[dg_qq] = sn * y01 + c * y11;
        }
#pragma unroll
        for (int k = 0; k < NK; ++k) {
            v4f np, nq;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                np[e] = fmaf(cm1, xr[k][e], xr[k][e]) - sn * yr[k][e];
                nq[e] = fmaf(cm1, yr[k][e], yr[k][e]) + sn * xr[k][e];
            }
            *(v4f*)&RT[rt_wp + 8 * k] = np;
            *(v4f*)&RT[rt_wq + 8 * k] = nq;
        }
        __syncthreads();
        if (w == 0) {
            dpq = *(const v2f*)&G[2 * jr * SG + 2 * jr];
            gqq = G[(2 * jr + 1) * SG + 2 * jr + 1];
        }
    }
}

// Q^T (stride SR, 64 x 64, as a QF sweep leaves it) to (Q - I)^T, by NT threads
// (t < NT, four per row).  The off-diagonal entries are those of Q - I already.
// A diagonal entry near 1 has lost its small distance to 1 in float32, so that
// distance is taken from the column's other entries (Q orthogonal): with S the
// sum of their squares, q_cc - 1 = -S / (1 + sqrt(1 - S)), exact to float32
// rounding relative to S; when q_cc is not near 1 (at or below 1/2) q_cc - 1
// itself is that accurate.  Row c of Q^T is column c of Q.
template <int NT>
__device__ __forceinline__ void diag_to_delta(float* RT, int t) {
    static_assert(NT == 4 * PW, "four threads per row");
    const int c = t >> 2, qq = t & 3;
    float sq = 0.0f;
#pragma unroll
    for (int e = 0; e < PW / 4; ++e) {
        const int r = 16 * qq + e;
        const float v = RT[c * SR + r];
        sq = r == c ? sq : fmaf(v, v, sq);
    }
    sq += __shfl_xor(sq, 1);
    sq += __shfl_xor(sq, 2);
    if ((c >> 4) == qq) {
        const float d = RT[c * SR + c];
        RT[c * SR + c] = d > 0.5f ? -sq / (1.0f + __builtin_amdgcn_sqrtf(fmaxf(1.0f - sq, 0.0f))) : d - 1.0f;
    }
}

}  // namespace
}  // namespace scopt
