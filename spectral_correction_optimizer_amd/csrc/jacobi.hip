// Blocked one-sided Jacobi (Hestenes) SVD sweeps on gfx950.
//
// The spectral-correction optimizer takes a thin SVD of each matrix's anchor
// momentum ("Key design 3" of the papernotes.org notes on "Communication-
// Efficient LLM Adaptation over Decentralized GPU Meshes").  The operand A
// (K x k, K >= k; A = M or M^T) is kept as rows = columns of A.  Its k columns
// are cut into blocks of b = 32; a sweep visits every block pair once in nb - 1
// rounds of nb/2 disjoint pairs (XOR order for power-of-two nb, round-robin
// otherwise: block_pair).  One round is three launches over all pairs of all
// matrices:
//
//   gram   per (pair, K split): G_part = X X^T, X = the pair's 64 rows of A,
//          fp32 MFMA accumulation restarted every 256 columns and summed in
//          fp64 registers (bounds the rounding of long dot products).
//   solve  per pair: sum the split partials in fixed order (fp64), measure the
//          largest relative off-diagonal |g_pq| / sqrt(g_pp g_qq); if above the
//          tolerance run one cyclic sweep of 2x2 Jacobi rotations on the 64x64
//          Gram in LDS (circle order in a moving frame, 32 disjoint rotations
//          per step), accumulating Q; store R = Q - I.
//   apply  per (pair, run of 128-column chunks, A or V): X <- X + R^T X on fp32
//          MFMA.  The correction form keeps the rounding of near-identity
//          rotations at the level of one addition.
//
// Every row of A and V belongs to exactly one pair per round, so the kernels
// of a round never write the same memory from two workgroups.  Reductions run
// in a fixed order: results are bitwise reproducible.
#include "common.hpp"
#include "internal.hpp"
#include "jacobi_dev.hpp"

namespace scopt {

namespace {

constexpr int KC = 32;           // K columns per LDS stage
constexpr int CHUNK = 256;       // fp32 accumulation length before folding into fp64

// Physical row of A / V holding local column rho (0..63) of block pair (I, J).
__device__ __forceinline__ int pair_row(const MatDev& md, int blkI, int blkJ, int rho) {
    return gld(md.perm + (rho < kJb ? blkI * kJb + rho : blkJ * kJb + (rho - kJb)));
}

// R = Q - I and the rotate flag of each pair slot, in two buffers by the parity
// of the round, so that a round's rotations stay readable through the next round
// (the V rows take two rounds' rotations in one pass: jac_apply_v2_kernel).
__device__ __forceinline__ float* rot_of(const MatDev& md, int round, int slot) {
    return md.rot + ((int64_t)(round & 1) * (md.nb / 2) + slot) * (PW * PW);
}
__device__ __forceinline__ int* rflag_of(const MatDev& md, int round, int slot) {
    return md.rot_flag + (round & 1) * (md.nb / 2) + slot;
}

// Selective polishing (sel set after a failed certificate): only pairs with a
// block above the convergence threshold in the certificate's normalized Gram
// (the cross block or either diagonal block, from bmax) are worked on; the
// others were certified and keep their orthogonality up to second-order terms
// of the rotations elsewhere (the re-certification checks it).
__device__ __forceinline__ bool pair_selected(const MatDev& md, const MatFlags& fl, int bI, int bJ) {
    if (!fl.sel) return true;
    const float t = md.tol_conv;
    const float* b = md.bmax;
    const int nb = md.nb;
    return gld(b + bI * nb + bJ) > t || gld(b + bI * nb + bI) > t || gld(b + bJ * nb + bJ) > t;
}

}  // namespace

// ---------------------------------------------------------------------------------
// Pair Gram G = X X^T (64 x 64, X = the pair's 64 rows of A over one K split).
// Only the 10 upper-triangle 16x16 tiles are computed (v_mfma_f32_16x16x4_f32),
// 3/3/2/2 per wave, and mirrored on output.  For X X^T the A and B operands of
// a tile are strips of the same rows, so a wave reads each of its strips once
// per k-step.  LDS holds X k-major with the row index XOR-swizzled by
// 8 * ((k >> 2) & 7): the transposing stores and the fragment reads are then
// both free of bank conflicts (row stride 80 floats).
namespace {
constexpr int GXS = 80;

template <int NT>
struct GramTiles {
    v4f acc[NT];
    double acc64[NT][4];
};

__device__ __forceinline__ float gram_frag(const float (*Xs)[GXS], int k, int t, int lane, int sw) {
    return Xs[k][(16 * t + (lane & 15)) ^ sw];
}
}  // namespace

__global__ __launch_bounds__(256) void jac_gram_kernel(const MatDev* __restrict__ mats,
                                                       const MatFlags* __restrict__ flags,
                                                       const GramItem* __restrict__ items,
                                                       int round, int skip_fused) {
    __shared__ float Xs[2][KC][GXS];
    const GramItem it = items[blockIdx.x];
    if (flags[it.mat].done) return;
    const MatDev& md = mats[it.mat];
    const int nb = md.nb;
    // after a sweep's first round the fused apply of the previous round wrote it
    if (skip_fused && it.fused && round % (nb - 1) != 0) return;
    int bI, bJ;
    block_pair(nb, round % (nb - 1), it.slot, &bI, &bJ);
    if (!pair_selected(md, flags[it.mat], bI, bJ)) return;
    const int x_begin = it.x0, x_end = it.x1;

    // loader: 64 rows x 32 columns = 512 float4 slots, 2 per thread
    // slot s: row = s >> 3, q = s & 7 (columns 4q..4q+3 of the stage)
    const float* rowp[2];
    int lrow[2], lq[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        int s = threadIdx.x + 256 * e;
        lrow[e] = s >> 3;
        lq[e] = s & 7;
        rowp[e] = md.A + (int64_t)pair_row(md, bI, bJ, lrow[e]) * md.K_ld;
    }
    // two register sets: the loads of a stage are issued two stages before its
    // LDS store, so about two stages of compute cover the memory latency
    float4 regA[2], regB[2];
    auto gload = [&](float4 (&reg)[2], int x0) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const v4f v = __builtin_nontemporal_load((const SC_GLOBAL v4f*)(rowp[e] + x0 + 4 * lq[e]));
            reg[e] = make_float4(v.x, v.y, v.z, v.w);
        }
    };
    auto lstore = [&](const float4 (&reg)[2], int b) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int col = lrow[e] ^ (8 * lq[e]);
            Xs[b][4 * lq[e] + 0][col] = reg[e].x;
            Xs[b][4 * lq[e] + 1][col] = reg[e].y;
            Xs[b][4 * lq[e] + 2][col] = reg[e].z;
            Xs[b][4 * lq[e] + 3][col] = reg[e].w;
        }
    };

    const int lane = threadIdx.x & 63;
    // wave index made visibly uniform so that the tile switch is a scalar branch
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // tiles (row strip, column strip) per wave
    int ti[3], tj[3], nt;
    if (wave == 0) { ti[0] = 0; tj[0] = 0; ti[1] = 0; tj[1] = 1; ti[2] = 0; tj[2] = 2; nt = 3; }
    else if (wave == 1) { ti[0] = 0; tj[0] = 3; ti[1] = 1; tj[1] = 1; ti[2] = 1; tj[2] = 2; nt = 3; }
    else if (wave == 2) { ti[0] = 1; tj[0] = 3; ti[1] = 2; tj[1] = 2; ti[2] = 0; tj[2] = 0; nt = 2; }
    else { ti[0] = 2; tj[0] = 3; ti[1] = 3; tj[1] = 3; ti[2] = 0; tj[2] = 0; nt = 2; }
    v4f acc[3];
    double acc64[3][4];
#pragma unroll
    for (int t = 0; t < 3; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            acc[t][r] = 0.0f;
            acc64[t][r] = 0.0;
        }
    const int nst = (x_end - x_begin) / KC;  // split bounds are multiples of KC
    auto compute = [&](int b) {
#pragma unroll
        for (int kk = 0; kk < KC; kk += 4) {
            const int k = kk + (lane >> 4);
            const int sw = 8 * ((kk >> 2) & 7);
#define SC_MF(t, a, b) acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[t], 0, 0, 0)
            switch (wave) {  // wave-uniform: a scalar branch, fragments chosen at compile time
                case 0: {
                    const float f0 = gram_frag(Xs[b], k, 0, lane, sw), f1 = gram_frag(Xs[b], k, 1, lane, sw),
                                f2 = gram_frag(Xs[b], k, 2, lane, sw);
                    SC_MF(0, f0, f0); SC_MF(1, f0, f1); SC_MF(2, f0, f2);
                    break;
                }
                case 1: {
                    const float f0 = gram_frag(Xs[b], k, 0, lane, sw), f1 = gram_frag(Xs[b], k, 1, lane, sw),
                                f2 = gram_frag(Xs[b], k, 2, lane, sw), f3 = gram_frag(Xs[b], k, 3, lane, sw);
                    SC_MF(0, f0, f3); SC_MF(1, f1, f1); SC_MF(2, f1, f2);
                    break;
                }
                case 2: {
                    const float f1 = gram_frag(Xs[b], k, 1, lane, sw), f2 = gram_frag(Xs[b], k, 2, lane, sw),
                                f3 = gram_frag(Xs[b], k, 3, lane, sw);
                    SC_MF(0, f1, f3); SC_MF(1, f2, f2);
                    break;
                }
                default: {
                    const float f2 = gram_frag(Xs[b], k, 2, lane, sw), f3 = gram_frag(Xs[b], k, 3, lane, sw);
                    SC_MF(0, f2, f3); SC_MF(1, f3, f3);
                    break;
                }
            }
#undef SC_MF
        }
    };
    auto fold = [&](int st) {
        if (((st + 1) * KC) % CHUNK == 0 || st + 1 == nst) {
#pragma unroll
            for (int t = 0; t < 3; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    acc64[t][r] += (double)acc[t][r];
                    acc[t][r] = 0.0f;
                }
        }
    };
    if (nst > 0) {
        gload(regA, x_begin);
        lstore(regA, 0);
    }
    if (nst > 1) gload(regA, x_begin + KC);
    if (nst > 2) gload(regB, x_begin + 2 * KC);
    __syncthreads();
    // stage st lives in Xs[st & 1]; at the top of an even stage regA holds stage
    // st + 1 and regB stage st + 2 (both possibly still in flight)
    for (int st = 0; st < nst; st += 2) {
        compute(0);
        fold(st);
        if (st + 1 < nst) lstore(regA, 1);
        if (st + 3 < nst) gload(regA, x_begin + (st + 3) * KC);
        __syncthreads();
        if (st + 1 >= nst) break;
        compute(1);
        fold(st + 1);
        if (st + 2 < nst) lstore(regB, 0);
        if (st + 4 < nst) gload(regB, x_begin + (st + 4) * KC);
        __syncthreads();
    }
    // 16x16 output layout: lane l, register r -> row 4 (l / 16) + r, column l % 16.
    // Only the upper tiles are stored; the solve mirrors them.
    double* out = md.gram + ((int64_t)it.slot * md.nsplit + it.split) * (PW * PW);
#pragma unroll
    for (int t = 0; t < 3; ++t) {
        if (t >= nt) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * ti[t] + 4 * (lane >> 4) + r, col = 16 * tj[t] + (lane & 15);
            gst(out + row * PW + col, acc64[t][r]);
        }
    }
}


__global__ __launch_bounds__(64) void jac_solve_kernel(const MatDev* __restrict__ mats,
                                                       MatFlags* __restrict__ flags,
                                                       const SolveItem* __restrict__ items,
                                                       int round) {
    // One wavefront per pair: LDS accesses of a wavefront are carried out in
    // issue order, so the steps need no barriers, only compiler fences that keep
    // the accesses in program order; all reads of a step precede its writes.
    // G: float32 working copy of the pair Gram (upper triangle), scaled by
    // 1 / max diagonal so that the solve does not depend on the magnitude.
    // R: the accumulated rotation minus the identity, Q = I + R, kept directly
    // in float32 (stored transposed, one slot per row).  Each 2x2 rotation enters
    // R through (c - 1) = -t s / (1 + h), h = sqrt(1 + t^2), and s, so a tiny
    // rotation is carried exactly (storing Q itself in float32 would round c to 1
    // while s != 0, a biased growth of the column norms over thousands of
    // rotations).  c = 1 / h and s = t c satisfy c^2 + s^2 = 1 to float32
    // rounding, so float32 parameters suffice.
    __shared__ __align__(16) float G[PW * SG];
    __shared__ __align__(16) float RT[PW * SR];
    __shared__ float cc[PW / 2], ss[PW / 2];  // rotation of each pair of the step
    __shared__ double rs[PW];                 // 1 / sqrt(g_aa) above the zero floor, else 0

    const SolveItem it = items[blockIdx.x];
    MatFlags& fl = flags[it.mat];
    if (fl.done) return;
    const MatDev& md = mats[it.mat];
    const float tol = md.tol;
    const int l = threadIdx.x;
    int bI, bJ;
    block_pair(md.nb, round % (md.nb - 1), it.slot, &bI, &bJ);
    if (!pair_selected(md, fl, bI, bJ)) {
        if (l == 0) *rflag_of(md, round, it.slot) = 0;
        return;
    }
    if (fl.sel && l == 0) atomicAdd(&fl.sel_pairs, 1);

    // 1. the pair Gram: split partials summed in fixed order (fp64).  Lane l
    //    takes the diagonal entry of column l and 4 entries of each stored upper
    //    16x16 tile (10 of 16); all loads of a split are in flight together.
    const double* gp = md.gram + (int64_t)it.slot * md.nsplit * (PW * PW);
    double dl = 0.0, acc[40];
#pragma unroll
    for (int e = 0; e < 40; ++e) acc[e] = 0.0;
    auto tile_row = [&](int e) {
        const int t = e >> 2, ti = t < 4 ? 0 : t < 7 ? 1 : t < 9 ? 2 : 3;
        return 16 * ti + (l >> 4) + 4 * (e & 3);
    };
    auto tile_col = [&](int e) {
        const int t = e >> 2, ti = t < 4 ? 0 : t < 7 ? 1 : t < 9 ? 2 : 3;
        const int tj = ti + t - (ti == 0 ? 0 : ti == 1 ? 4 : ti == 2 ? 7 : 9);
        return 16 * tj + (l & 15);
    };
#pragma unroll 2
    for (int sp = 0; sp < it.nsplit; ++sp) {
        const double* g = gp + (int64_t)sp * PW * PW;
        dl += gld(g + l * (PW + 1));
#pragma unroll
        for (int e = 0; e < 40; ++e) acc[e] += gld(g + tile_row(e) * PW + tile_col(e));
    }
    double dmax = dl;
    for (int o = 32; o > 0; o >>= 1) dmax = fmax(dmax, __shfl_xor(dmax, o));
    const double scale = dmax > 0.0 ? 1.0 / dmax : 1.0;
    const double floor2d = (double)fl.floor2;
    const float floor2 = (float)(floor2d * scale);
    rs[l] = dl > floor2d ? 1.0 / sqrt(dl) : 0.0;
    __syncthreads();

    // 2. G keeps the upper triangle.  The largest relative off-diagonal
    //    |g_ab| / sqrt(g_aa g_bb) over columns above the zero floor (rs = 0 below it).
    float mo = 0.0f;
#pragma unroll
    for (int e = 0; e < 40; ++e) {
        const int a = tile_row(e), b = tile_col(e);
        if (a <= b) G[a * SG + b] = (float)(acc[e] * scale);
        if (a < b) mo = max_nan_inf(mo, (float)(fabs(acc[e]) * rs[a] * rs[b]));
    }
    for (int o = 32; o > 0; o >>= 1) mo = fmaxf(mo, __shfl_xor(mo, o));
    if (l == 0) atomicMax(&fl.sweep_max, __float_as_uint(mo));
    int* rflag = rflag_of(md, round, it.slot);
    if (!(mo > tol)) {
        // columns unchanged: their norms for the next sweep's ordering
        gst(md.cnorm + pair_row(md, bI, bJ, l), (float)dl);
        if (l == 0) *rflag = 0;
        return;
    }
    for (int e = l; e < PW * SR / 4; e += 64) *(v4f*)&RT[4 * e] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    // 3. per-lane addresses, fixed for the whole sweep.
    //    Rotation: lanes 2j, 2j+1 both compute pair j's.
    //    G: lane l takes the pair-blocks (i < j) of bank class t = l % 16, numbers
    //    8 (l / 16) .. + 7 within the class: the 16 lanes of a quarter read 16
    //    distinct bank pairs.  Its 4 entries go to their moved slots (upper
    //    triangle); odd lane quarters write them in the order (0,1), (0,0), (1,1),
    //    (1,0), which puts the two quarters of a half-wave on opposite banks.
    //    Pair j's own 2x2 block: lanes 2j and 2j+1 (the same values).
    //    R^T: lane l updates rows (slots) 2j, 2j+1 of pair j = l / 2, columns
    //    8 k + 4 (l % 2) .. + 3, k = 0..7.
    const int jr = l >> 1, hh = l & 1, cls = l & 15, odd = (l >> 4) & 1;
    int blk_ij[8], blk_rd[8], blk_wr[8][4];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        // past the end of a class: computes on block (0, 1), writes nothing
        const int v = kBlocks.v[cls][8 * (l >> 4) + u];
        const bool ok = v & 0x8000;
        const int i = ok ? v & 255 : 0, j = ok ? (v >> 8) & 127 : 1;
        blk_ij[u] = i | (j << 8);
        blk_rd[u] = 2 * i * SG + 2 * j;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int ee = odd ? (e ^ 1) : e;  // entry (ee >> 1, ee & 1) of the block
            const int r = slot_next(2 * i + (ee >> 1)), c = slot_next(2 * j + (ee & 1));
            blk_wr[u][e] = ok ? min(r, c) * SG + max(r, c) : kSink;
        }
    }
    const int sp_ = slot_next(2 * jr), sq_ = slot_next(2 * jr + 1);
    const int dg_pp = sp_ * SG + sp_, dg_qq = sq_ * SG + sq_, dg_pq = min(sp_, sq_) * SG + max(sp_, sq_);
    const int rt_rd = 2 * jr * SR + 4 * hh, rt_wp = sp_ * SR + 4 * hh, rt_wq = sq_ * SR + 4 * hh;
    // original columns held by slots 2 jr, 2 jr + 1: positions on the cycle
    int kp = jr == 0 ? -1 : cycle_pos(2 * jr), kq = cycle_pos(2 * jr + 1);
    __syncthreads();
    // rotation inputs of the step: g_pp, g_pq, g_qq of the lane's pair
    v2f dpq = *(const v2f*)&G[2 * jr * SG + 2 * jr];
    float gqq = G[(2 * jr + 1) * SG + 2 * jr + 1];

#pragma unroll 1
    for (int ir = 0; ir < PW - 1; ++ir) {
        // ---- reads (the rotation inputs were read at the end of the last step)
        __asm__ volatile("" ::"v"(dpq), "v"(gqq));
        v2f x0[8], x1[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            x0[u] = *(const v2f*)&G[blk_rd[u]];
            x1[u] = *(const v2f*)&G[blk_rd[u] + SG];
        }
        v4f xr[8], yr[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            xr[k] = *(const v4f*)&RT[rt_rd + 8 * k];
            yr[k] = *(const v4f*)&RT[rt_rd + SR + 8 * k];
        }
        // the elements of rows 2 jr, 2 jr + 1 at the original columns op, oq held by
        // the pair's slots: R's identity entries sit there (both lanes read them)
        const int op = kp < 0 ? 0 : cycle_slot(kp), oq = cycle_slot(kq);
        const float xop = RT[2 * jr * SR + op], yop = RT[(2 * jr + 1) * SR + op];
        const float xoq = RT[2 * jr * SR + oq], yoq = RT[(2 * jr + 1) * SR + oq];
        // ---- rotation of pair jr (both lanes of the pair compute and publish it)
        const float gpp = dpq[0], gpq = dpq[1];
        float c, sn, cm1;
        pair_rotation(gpp, gpq, gqq, floor2, tol, c, sn, cm1);
        cc[jr] = c;
        ss[jr] = sn;
        __asm__ volatile("" ::: "memory");
        // ---- G: off-diagonal pair-blocks; columns first ([x_p, x_q] <-
        //      [c x_p - s x_q, s x_p + c x_q]), then rows with pair i's rotation
        float wv[8][4];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
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
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e) G[blk_wr[u][e]] = wv[u][e];
        // ---- G: the pair's own block (both lanes write the same values)
        {
            const float y00 = c * gpp - sn * gpq, y01 = sn * gpp + c * gpq;
            const float y10 = c * gpq - sn * gqq, y11 = sn * gpq + c * gqq;
            G[dg_pp] = c * y00 - sn * y10;
            G[dg_pq] = c * y01 - sn * y11;
            G[dg_qq] = sn * y01 + c * y11;
        }
        // ---- R <- R J: rows 2 jr, 2 jr + 1 of R^T, written to their moved slots
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            v4f np, nq;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                np[e] = fmaf(cm1, xr[k][e], xr[k][e]) - sn * yr[k][e];
                nq[e] = fmaf(cm1, yr[k][e], yr[k][e]) + sn * xr[k][e];
            }
            *(v4f*)&RT[rt_wp + 8 * k] = np;
            *(v4f*)&RT[rt_wq + 8 * k] = nq;
        }
        // plus J - I on those four elements: both lanes of the pair overwrite them
        // with the same corrected values
        RT[sp_ * SR + op] = fmaf(cm1, xop, xop) - sn * yop + cm1;
        RT[sq_ * SR + op] = fmaf(cm1, yop, yop) + sn * xop + sn;
        RT[sp_ * SR + oq] = fmaf(cm1, xoq, xoq) - sn * yoq - sn;
        RT[sq_ * SR + oq] = fmaf(cm1, yoq, yoq) + sn * xoq + cm1;
        kp = kp < 0 ? -1 : (kp == 0 ? 62 : kp - 1);
        kq = kq == 0 ? 62 : kq - 1;
        __asm__ volatile("" ::: "memory");
        // rotation inputs of the next step
        dpq = *(const v2f*)&G[2 * jr * SG + 2 * jr];
        gqq = G[(2 * jr + 1) * SG + 2 * jr + 1];
    }
    __syncthreads();
    // 4. R row-major [b][a] (X_new[a] = X[a] + sum_b R[b][a] X[b]); the frame is the
    //    original one again, so R[b][a] = R^T[a][b]
    float* Rg = rot_of(md, round, it.slot);
#pragma unroll 4
    for (int b0 = 0; b0 < PW; b0 += 4) {
        const v4f v = *(const v4f*)&RT[l * SR + b0];
#pragma unroll
        for (int e = 0; e < 4; ++e) gst(Rg + (b0 + e) * PW + l, v[e]);
    }
    // rotated squared column norms (diagonal of Q^T G Q) for the next sweep's ordering
    gst(md.cnorm + pair_row(md, bI, bJ, l), (float)(G[l * SG + l] * dmax));
    if (l == 0) {
        *rflag = 1;
        atomicAdd(&fl.pairs_applied, 1);
        if (fl.sel) atomicAdd(&fl.sel_rot, 1);
    }
}

// ---------------------------------------------------------------------------------
// The same sweep on NW wavefronts per pair.  Wave w updates, within every bank
// class, the pair-blocks of G numbered NU (4 w + l / 16) .. + NU - 1, and the
// columns [64 w / NW, 64 (w + 1) / NW) of R^T; every wave computes all 32
// rotations of a step (from the same entries of G, so identically).  Every entry
// goes through the arithmetic of the one-wavefront kernel in the same order: the
// results are identical.  The one-wavefront solve spends most of a step waiting
// on LDS round trips (rotation parameters, then the next step's inputs) with
// nothing else to issue on its SIMD; more waves per pair split the arithmetic
// and give each SIMD other waves to run meanwhile.
//  NB = 2: G and R^T are held twice; a step reads one copy and writes the other,
//    so one barrier per step puts all writes of a step before the reads of the
//    next and all reads of a step before the writes of the step after (69 KB of
//    LDS, two pairs per CU: for launches of few pairs).
//  NB = 1: one copy and two barriers per step, reads | writes (35 KB): four pairs
//    per CU as with one wavefront (for launches that fill the chip).
template <int NW, int NB>
__global__ __launch_bounds__(64 * NW) void jac_solve_waves_kernel(const MatDev* __restrict__ mats,
                                                                MatFlags* __restrict__ flags,
                                                                const SolveItem* __restrict__ items,
                                                                int round) {
    static_assert(NW == 2 || NW == 4 || NW == 8, "two, four or eight wavefronts per pair");
    static_assert(NB == 1 || NB == 2, "one or two copies of G and R^T");
    constexpr int NE = 40 / NW;  // stored Gram entries per lane in the load
    constexpr int CW = PW / NW;  // columns of R^T per wave
    __shared__ __align__(16) float G[NB][PW * SG];
    __shared__ __align__(16) float RT[NB][PW * SR];
    __shared__ float cc[PW / 2], ss[PW / 2];
    __shared__ double rs[PW];
    __shared__ float mos[NW];

    const SolveItem it = items[blockIdx.x];
    MatFlags& fl = flags[it.mat];
    if (fl.done) return;
    const MatDev& md = mats[it.mat];
    const float tol = md.tol;
    const int l = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int bI, bJ;
    block_pair(md.nb, round % (md.nb - 1), it.slot, &bI, &bJ);
    if (!pair_selected(md, fl, bI, bJ)) {
        if (threadIdx.x == 0) *rflag_of(md, round, it.slot) = 0;
        return;
    }
    if (fl.sel && threadIdx.x == 0) atomicAdd(&fl.sel_pairs, 1);

    // 1. the pair Gram as in the one-wavefront kernel; every wave sums the
    //    diagonal, the stored upper tiles are shared out (entries NE w .. + NE - 1)
    const double* gp = md.gram + (int64_t)it.slot * md.nsplit * (PW * PW);
    const int e0 = NE * w;
    double dl = 0.0, acc[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e) acc[e] = 0.0;
    auto tile_row = [&](int e) {
        const int t = e >> 2, ti = t < 4 ? 0 : t < 7 ? 1 : t < 9 ? 2 : 3;
        return 16 * ti + (l >> 4) + 4 * (e & 3);
    };
    auto tile_col = [&](int e) {
        const int t = e >> 2, ti = t < 4 ? 0 : t < 7 ? 1 : t < 9 ? 2 : 3;
        const int tj = ti + t - (ti == 0 ? 0 : ti == 1 ? 4 : ti == 2 ? 7 : 9);
        return 16 * tj + (l & 15);
    };
#pragma unroll 2
    for (int sp = 0; sp < it.nsplit; ++sp) {
        const double* g = gp + (int64_t)sp * PW * PW;
        dl += gld(g + l * (PW + 1));
#pragma unroll
        for (int e = 0; e < NE; ++e) acc[e] += gld(g + tile_row(e0 + e) * PW + tile_col(e0 + e));
    }
    double dmax = dl;
    for (int o = 32; o > 0; o >>= 1) dmax = fmax(dmax, __shfl_xor(dmax, o));
    const double scale = dmax > 0.0 ? 1.0 / dmax : 1.0;
    const double floor2d = (double)fl.floor2;
    const float floor2 = (float)(floor2d * scale);
    if (w == 0) rs[l] = dl > floor2d ? 1.0 / sqrt(dl) : 0.0;
    __syncthreads();

    // 2. the upper triangle into the first copy of G; the largest relative
    //    off-diagonal over the waves
    float mo = 0.0f;
#pragma unroll
    for (int e = 0; e < NE; ++e) {
        const int a = tile_row(e0 + e), b = tile_col(e0 + e);
        if (a <= b) G[0][a * SG + b] = (float)(acc[e] * scale);
        if (a < b) mo = max_nan_inf(mo, (float)(fabs(acc[e]) * rs[a] * rs[b]));
    }
    for (int o = 32; o > 0; o >>= 1) mo = fmaxf(mo, __shfl_xor(mo, o));
    if (l == 0) mos[w] = mo;
    __syncthreads();
    mo = mos[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) mo = fmaxf(mo, mos[i]);
    if (threadIdx.x == 0) atomicMax(&fl.sweep_max, __float_as_uint(mo));
    int* rflag = rflag_of(md, round, it.slot);
    if (!(mo > tol)) {
        if (w == 0) {
            gst(md.cnorm + pair_row(md, bI, bJ, l), (float)dl);
            if (l == 0) *rflag = 0;
        }
        return;
    }
    for (int e = threadIdx.x; e < PW * SR / 4; e += 64 * NW) *(v4f*)&RT[0][4 * e] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    const int cur = pair_sweep<NW, NB>(G, RT, cc, ss, l, w, floor2, tol);
    const int cb = CW * w;
    // 4. R and the rotated column norms from the copy the last step wrote
    const float* Rf = RT[cur];
    float* Rg = rot_of(md, round, it.slot);
#pragma unroll 4
    for (int b0 = cb; b0 < cb + CW; b0 += 4) {
        const v4f v = *(const v4f*)&Rf[l * SR + b0];
#pragma unroll
        for (int e = 0; e < 4; ++e) gst(Rg + (b0 + e) * PW + l, v[e]);
    }
    if (w == 0) gst(md.cnorm + pair_row(md, bI, bJ, l), (float)(G[cur][l * SG + l] * dmax));
    if (threadIdx.x == 0) {
        *rflag = 1;
        atomicAdd(&fl.pairs_applied, 1);
        if (fl.sel) atomicAdd(&fl.sel_rot, 1);
    }
}

// ---------------------------------------------------------------------------------

__global__ __launch_bounds__(kApplyThreads) void jac_apply_kernel(const MatDev* __restrict__ mats,
                                                        const MatFlags* __restrict__ flags,
                                                        const ApplyItem* __restrict__ items,
                                                        int round) {
    // A workgroup updates 64 rows over a run of consecutive chunks of
    // kApplyCols columns; in a chunk, wave w owns columns [x0 + 32 w, x0 + 32 w + 32).
    // Only R goes through LDS (staged once for the run, split into three bfloat16
    // planes in MFMA operand order): each lane loads 32 rows of its column straight
    // into registers; split, they are its B operands of the four 16-row k-steps of
    // v_mfma_f32_32x32x16_bf16 (k-step t: rows 16 t .. + 15, the lane's half being
    // apply_row(8 t .. 8 t + 7, hl)), and unsplit the old values of its output
    // elements, so X_new = X + R^T X needs no re-read.  Six part products per
    // product (float32-equivalent) take 2.7x fewer matrix-core cycles than
    // v_mfma_f32_32x32x2_f32.  The loads of chunk c + 1 are issued before the
    // MFMAs of chunk c (two register sets).
    // R^T as planes: [plane][32-row output tile][k-step][lane]
    __shared__ v8bf Rp[3][2][4][64];
    const ApplyItem it = items[blockIdx.x];
    if (flags[it.mat].done) return;
    const MatDev& md = mats[it.mat];
    if (*rflag_of(md, round, it.slot) == 0) return;
    int bI, bJ;
    block_pair(md.nb, round % (md.nb - 1), it.slot, &bI, &bJ);
    float* base = it.which == 0 ? md.A : md.V;
    const int ld = it.which == 0 ? md.K_ld : md.kpad;  // multiple of 64
    // the operand (kpad rows of ld floats) as a buffer; byte offsets: the lane's
    // row and column in VGPRs, the chunk's first column (wave-uniform) in an SGPR
    const __amdgpu_buffer_rsrc_t buf = buf_rsrc(base, (uint32_t)md.kpad * ld * 4u);

    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int hl = lane >> 5, ll = lane & 31;
    int voff[PW / 2];
#pragma unroll
    for (int s = 0; s < PW / 2; ++s) voff[s] = (pair_row(md, bI, bJ, apply_row(s, hl)) * ld + ll) * 4;
    // first column of the wave in chunk c, and whether the wave's 32 columns are
    // in (they are all in or all out: ld is a multiple of 64)
    auto col0 = [&](int c) { return (it.chunk + c) * kApplyCols + wave * 32; };
    auto load = [&](float (&x)[PW / 2], int c) {
        if (col0(c) >= ld) return;
        const int so = col0(c) * 4;
#pragma unroll
        for (int s = 0; s < PW / 2; ++s) x[s] = buf_load_f32<kBufNT>(buf, voff[s], so);
    };
    auto update = [&](const float (&x)[PW / 2], int c) {
        if (col0(c) >= ld) return;
        v16f acc0, acc1;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            acc0[r] = 0.0f;
            acc1[r] = 0.0f;
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            float f[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) f[e] = x[8 * t + e];
            const Split8 xs = split8(f);
            const Split8 r0{Rp[0][0][t][lane], Rp[1][0][t][lane], Rp[2][0][t][lane]};
            const Split8 r1{Rp[0][1][t][lane], Rp[1][1][t][lane], Rp[2][1][t][lane]};
            acc0 = mfma_split6(r0, xs, acc0);
            acc1 = mfma_split6(r1, xs, acc1);
        }
        // acc0 register r is row apply_row(r, hl), acc1 register r is row apply_row(16 + r, hl)
        const int so = col0(c) * 4;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            buf_store_f32<kBufNT>(x[r] + acc0[r], buf, voff[r], so);
            buf_store_f32<kBufNT>(x[16 + r] + acc1[r], buf, voff[16 + r], so);
        }
    };
    float xa[PW / 2], xb[PW / 2];
    load(xa, 0);
    const float* R = rot_of(md, round, it.slot);
    // operand A of tile tl, k-step t for lane l: R^T[32 tl + l % 32][b] = R[b][32 tl + l % 32]
    // at the 8 rows b = apply_row(8 t + e, l / 32)
    for (int idx = threadIdx.x; idx < 2 * 4 * 64; idx += kApplyThreads) {
        const int tl = idx >> 8, t = (idx >> 6) & 3, l = idx & 63;
        float f[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = gld(R + apply_row(8 * t + e, l >> 5) * PW + 32 * tl + (l & 31));
        const Split8 sp = split8(f);
        Rp[0][tl][t][l] = sp.h;
        Rp[1][tl][t][l] = sp.m;
        Rp[2][tl][t][l] = sp.l;
    }
    __syncthreads();
    const int n = it.nchunk;
    for (int c = 0; c < n; c += 2) {
        if (c + 1 < n) load(xb, c + 1);
        update(xa, c);
        if (c + 1 >= n) break;
        if (c + 2 < n) load(xa, c + 2);
        update(xb, c + 1);
    }
}

// ---------------------------------------------------------------------------------
// Rotation apply of a round fused with the next round's pair Grams.  For a
// power-of-two block count, round r pairs block p with p ^ m (m = nb - 1 - r) and
// round r + 1 with p ^ m', m' = m - 1: the four blocks {p, p^m, p^m', p^m^m'} form
// two pairs in each round.  A workgroup takes such a group over one column split,
// in 128-column chunks: waves 0-3 apply pair A's rotation and waves 4-7 pair B's,
// 32 columns each (as jac_apply_kernel, the next chunk's loads in flight), and
// store the rotated rows; the chunk's 128 new rows then go through LDS into the
// next round's six 32 x 32 Gram tiles (two pairs: lower-lower, lower-upper,
// upper-upper): wave w forms the three tiles of pair w / 4 over columns
// 32 (w % 4) .. + 31 of each chunk, splitting its two row fragments once per
// k-step, on the bfloat16 matrix cores with each float split exactly into three
// bfloat16 parts and the six largest part products (v_mfma_f32_32x32x16_bf16,
// float32 accumulation over the wave's <= 256 columns of the split).  At the end
// of the split the four quarters of each tile are summed in float64 in a fixed order
// into the split partial the solve of round r + 1 reads, so the operand is not
// read again for that round's Gram.  In the last round of a sweep (the next one
// starts with the sort) only the rotations are applied.
namespace {
constexpr int TLD = 2 * PW + 4;  // LDS row stride of a chunk's 128 new rows (128 columns)

}  // namespace

__global__ __launch_bounds__(512) void jac_apply_gram_kernel(const MatDev* __restrict__ mats,
                                                          const MatFlags* __restrict__ flags,
                                                          const FusedItem* __restrict__ items,
                                                          int round) {
    // the two rotations as bfloat16 planes (hi, mid, lo) in MFMA operand order:
    // [pair][plane][32-row output tile][16-row k-step][lane]
    __shared__ v8bf Rp[2][3][2][4][64];
    __shared__ __align__(16) float Ts[2 * PW][TLD];
    const FusedItem it = items[blockIdx.x];
    if (flags[it.mat].done) return;
    const MatDev& md = mats[it.mat];
    const int nb = md.nb, rr = round % (nb - 1);
    const bool gram = rr < nb - 2;  // the next round belongs to this sweep
    // the group's pairs: A = (a0, a1), B = (b0, b1) (lower block first) in this
    // round, A' = (n0, n1), B' = (n2, n3) in the next
    int a0, a1, b0, b1, slotA, slotB, n0 = 0, n1 = 0, n2 = 0, n3 = 0, slotA2 = 0, slotB2 = 0;
    if (gram) {
        const int m = nb - 1 - rr, h = 31 - __builtin_clz(m), m2 = m - 1;
        const int h2 = 31 - __builtin_clz(m2);
        // two pivot bits on which m and m2 are independent: p has zeros there
        const int lo = (m & (m - 1)) == 0 ? h - 1 : __builtin_ctz(m);
        const int p = insert_zero_bit(insert_zero_bit(it.group, lo), h);
        a0 = p;
        a1 = p ^ m;
        b0 = ((p ^ m2) >> h) & 1 ? p ^ m2 ^ m : p ^ m2;
        b1 = b0 ^ m;
        slotA = remove_bit(a0, h);
        slotB = remove_bit(b0, h);
        n0 = p;
        n1 = p ^ m2;
        n2 = ((p ^ m) >> h2) & 1 ? p ^ m ^ m2 : p ^ m;
        n3 = n2 ^ m2;
        slotA2 = remove_bit(n0, h2);
        slotB2 = remove_bit(n2, h2);
    } else {
        slotA = 2 * it.group;
        slotB = slotA + 1;
        block_pair(nb, rr, slotA, &a0, &a1);
        block_pair(nb, rr, slotB, &b0, &b1);
    }
    const bool rotA = *rflag_of(md, round, slotA) != 0, rotB = *rflag_of(md, round, slotB) != 0;
    if (!gram && !rotA && !rotB) return;
    const int ld = md.K_ld;
    const __amdgpu_buffer_rsrc_t buf = buf_rsrc(md.A, (uint32_t)md.kpad * ld * 4u);
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int q = wave >> 2, wq = wave & 3;  // the wave's pair and column quarter
    const bool rot = q == 0 ? rotA : rotB;
    const int hl = lane >> 5, ll = lane & 31;
    int voff[PW / 2];
#pragma unroll
    for (int s = 0; s < PW / 2; ++s)
        voff[s] = (pair_row(md, q == 0 ? a0 : b0, q == 0 ? a1 : b1, apply_row(s, hl)) * ld + ll) * 4;
    auto col0 = [&](int c) { return it.x0 + c * kApplyCols + wq * 32; };
    auto load = [&](float (&x)[PW / 2], int c) {
        const int so = col0(c) * 4;
#pragma unroll
        for (int s = 0; s < PW / 2; ++s) x[s] = buf_load_f32<kBufNT>(buf, voff[s], so);
    };
    // the wave's Gram work: the next round's pair wave / 4 (A' or B'; its lower
    // block U and upper block V as rows of the chunk block), tiles U U^T, U V^T,
    // V V^T over the chunk's columns 32 (wave % 4) .. + 31
    auto tblk = [&](int blk) { return blk == a0 ? 0 : blk == a1 ? 1 : blk == b0 ? 2 : 3; };
    const int urow = 32 * tblk(wave < 4 ? n0 : n2) + ll, vrow = 32 * tblk(wave < 4 ? n1 : n3) + ll;
    const int ucol = 32 * (wave & 3) + 8 * hl;
    v16f gacc[3];
#pragma unroll
    for (int j = 0; j < 3; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) gacc[j][r] = 0.0f;
    auto frag = [&](int row, int col) {
        float f[8];
        const v4f lo4 = *(const v4f*)&Ts[row][col], hi4 = *(const v4f*)&Ts[row][col + 4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            f[e] = lo4[e];
            f[4 + e] = hi4[e];
        }
        return split8(f);
    };
    auto update = [&](float (&x)[PW / 2], int c) {
        if (rot) {
            // R^T X on the bfloat16 matrix cores: k-step t covers rows 16 t .. + 15,
            // of which the lane's x[8 t .. 8 t + 7] are the half hl (apply_row), so
            // its B operand is its own registers
            Split8 xs[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                float f[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) f[e] = x[8 * t + e];
                xs[t] = split8(f);
            }
            v16f acc0, acc1;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                acc0[r] = 0.0f;
                acc1[r] = 0.0f;
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const Split8 r0{Rp[q][0][0][t][lane], Rp[q][1][0][t][lane], Rp[q][2][0][t][lane]};
                const Split8 r1{Rp[q][0][1][t][lane], Rp[q][1][1][t][lane], Rp[q][2][1][t][lane]};
                acc0 = mfma_split6(r0, xs[t], acc0);
                acc1 = mfma_split6(r1, xs[t], acc1);
            }
            const int so = col0(c) * 4;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                x[r] += acc0[r];
                x[16 + r] += acc1[r];
                buf_store_f32<kBufNT>(x[r], buf, voff[r], so);
                buf_store_f32<kBufNT>(x[16 + r], buf, voff[16 + r], so);
            }
        }
        if (!gram) return;
        // the chunk's new rows (row = 64 pair + pair row, column = chunk column)
#pragma unroll
        for (int s = 0; s < PW / 2; ++s) Ts[PW * q + apply_row(s, hl)][32 * wq + ll] = x[s];
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const Split8 fu = frag(urow, ucol + 16 * ks);
            const Split8 fv = frag(vrow, ucol + 16 * ks);
            gacc[0] = mfma_split6(fu, fu, gacc[0]);
            gacc[1] = mfma_split6(fu, fv, gacc[1]);
            gacc[2] = mfma_split6(fv, fv, gacc[2]);
        }
        __syncthreads();  // before the next chunk's rows
    };
    float xa[PW / 2], xb[PW / 2];
    load(xa, 0);
    // operand A of tile tl, k-step t for lane l: R^T[32 tl + l % 32][b] = R[b][32 tl + l % 32]
    // at the 8 rows b = apply_row(8 t + e, l / 32) of the lane's half of the k-step
    for (int idx = threadIdx.x; idx < 2 * 2 * 4 * 64; idx += 512) {
        const int pq = idx >> 9, tl = (idx >> 8) & 1, t = (idx >> 6) & 3, l = idx & 63;
        const float* R = rot_of(md, round, pq == 0 ? slotA : slotB);
        float f[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = gld(R + apply_row(8 * t + e, l >> 5) * PW + 32 * tl + (l & 31));
        const Split8 sp = split8(f);
        Rp[pq][0][tl][t][l] = sp.h;
        Rp[pq][1][tl][t][l] = sp.m;
        Rp[pq][2][tl][t][l] = sp.l;
    }
    __syncthreads();
    if (!gram && !rot) return;  // no barrier follows without the Gram
    const int n = (it.x1 - it.x0) / kApplyCols;
    for (int c = 0; c < n; c += 2) {
        if (c + 1 < n) load(xb, c + 1);
        update(xa, c);
        if (c + 1 >= n) break;
        if (c + 2 < n) load(xa, c + 2);
        update(xb, c + 1);
    }
    if (!gram) return;
    // 4. per tile the four column quarters summed in float64 (quarter order) into
    //    the split partials of the next round's pairs: A' from waves 0-3, B' from
    //    waves 4-7; the upper tiles of the 64 x 64 Gram (its lower triangle is not
    //    read)
    float* red = &Ts[0][0];
#pragma unroll
    for (int ps = 0; ps < 2; ++ps) {
        if ((wave >> 2) == ps)
#pragma unroll
            for (int j = 0; j < 3; ++j)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4)
                    *(v4f*)&red[((3 * (wave - 4 * ps) + j) * 64 + lane) * 16 + 4 * r4] =
                        v4f{gacc[j][4 * r4], gacc[j][4 * r4 + 1], gacc[j][4 * r4 + 2], gacc[j][4 * r4 + 3]};
        __syncthreads();
        double* out = md.gram + ((int64_t)(ps == 0 ? slotA2 : slotB2) * md.nsplit + it.split) * (PW * PW);
        for (int e = threadIdx.x; e < 3 * 1024; e += 512) {
            const int t = e >> 10, l = (e >> 4) & 63, r = e & 15;
            double sum = 0.0;
#pragma unroll
            for (int k4 = 0; k4 < 4; ++k4) sum += (double)red[(3 * k4 + t) * 1024 + (e & 1023)];
            const int i = 8 * (r >> 2) + 4 * (l >> 5) + (r & 3), jj = l & 31;
            const int row = (t == 2 ? 32 : 0) + i, col = (t == 0 ? 0 : 32) + jj;
            gst(out + row * PW + col, sum);
        }
        __syncthreads();
    }
}


// ---------------------------------------------------------------------------------
// V rows: the rotations of two consecutive rounds in one pass.  V does not feed the
// sweeps (every round's rotations come from A's Gram), so the update of V for round
// r (even within the sweep) waits and is applied together with round r + 1's.  For
// r even, m = nb - 1 - r is odd, and the group {p, p^m, p^1, p^m^1} (p with zeros
// at bit 0 and at the top bit h of m) holds two pairs of each round:
//   round r:      (p, p^m), (p^1, p^m^1)
//   round r + 1:  (p, p^m^1), (p^1, p^m)          (m' = m - 1 = m ^ 1)
// With the blocks in register slots 0 = p, 1 = p^m, 2 = p^1, 3 = p^m^1 the pairs are
// (0, 1), (2, 3) and then (0, 3), (2, 1) for every group and round.  A wave keeps 32
// columns of the group's 128 rows in registers (16 rows of each block per lane, in
// the row order of jac_apply_kernel) through both rounds' products and moves them
// once; the next chunk's loads are in flight meanwhile.  In the last round of a
// sweep (r = nb - 2) it applies that round's two pairs of group g, slots 2g, 2g + 1.
// Each product is formed exactly as in jac_apply_kernel (same split, same part
// products in the same order, float32 sums) and the rows between the two rounds
// are the same float32 values: V is bitwise the same as with one pass per round.
__global__ __launch_bounds__(kV2Threads) void jac_apply_v2_kernel(const MatDev* __restrict__ mats,
                                                                const MatFlags* __restrict__ flags,
                                                                const FusedItem* __restrict__ items,
                                                                int round) {
    // the four rotations as bfloat16 planes in MFMA operand order:
    // [pair][plane][32-row output tile][16-row k-step][lane]
    __shared__ v8bf Rp[4][3][2][4][64];
    const FusedItem it = items[blockIdx.x];
    if (flags[it.mat].done) return;
    const MatDev& md = mats[it.mat];
    const int nb = md.nb, rr = round % (nb - 1);
    const bool two = (rr & 1) != 0;  // rounds r = rr - 1 and rr
    if (!two && rr < nb - 2) return;  // this round's V update waits for the next round
    int blk[4], slot[4], rnd[4];      // pairs 0, 1: first round; 2, 3: second round
    if (two) {
        const int m = nb - rr, h = 31 - __builtin_clz(m);
        const int p = insert_zero_bit(insert_zero_bit(it.group, 0), h);
        blk[0] = p;
        blk[1] = p ^ m;
        blk[2] = p ^ 1;
        blk[3] = p ^ m ^ 1;
        slot[0] = remove_bit(blk[0], h);
        slot[1] = remove_bit(blk[2], h);
        slot[2] = remove_bit(blk[0], h);  // (p, p^m^1): the top bit of m - 1 is h
        slot[3] = remove_bit(blk[2], h);  // (p^1, p^m)
        rnd[0] = rnd[1] = round - 1;
        rnd[2] = rnd[3] = round;
    } else {
        slot[0] = 2 * it.group;
        slot[1] = slot[0] + 1;
        block_pair(nb, rr, slot[0], &blk[0], &blk[1]);
        block_pair(nb, rr, slot[1], &blk[2], &blk[3]);
        slot[2] = slot[3] = 0;
        rnd[0] = rnd[1] = rnd[2] = rnd[3] = round;
    }
    bool rot[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) rot[q] = (q < 2 || two) && *rflag_of(md, rnd[q], slot[q]) != 0;
    // a block is moved when a rotated pair holds it
    const bool need[4] = {rot[0] || rot[2], rot[0] || rot[3], rot[1] || rot[3], rot[1] || rot[2]};
    if (!(need[0] || need[1] || need[2] || need[3])) return;
    const int ld = md.kpad;  // multiple of 64
    const __amdgpu_buffer_rsrc_t buf = buf_rsrc(md.V, (uint32_t)md.kpad * ld * 4u);
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int hl = lane >> 5, ll = lane & 31;
    // lane's rows: 16 of each block (apply_row(e, hl), e < 16, of the block's 32),
    // two physical row numbers (< 2^16) per register; byte offset row * 4 ld + 4 ll
    unsigned int rows2[4][8];
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            rows2[b][e] = (unsigned int)gld(md.perm + blk[b] * kJb + apply_row(2 * e, hl)) |
                          ((unsigned int)gld(md.perm + blk[b] * kJb + apply_row(2 * e + 1, hl)) << 16);
    const unsigned int ld4 = 4u * ld, ll4 = 4u * ll;
    auto voff = [&](int b, int e) {
        const unsigned int r = (e & 1) ? rows2[b][e >> 1] >> 16 : rows2[b][e >> 1] & 0xffffu;
        return (int)(__umul24(r, ld4) + ll4);
    };
    auto col0 = [&](int c) { return it.x0 + c * kV2Cols + wave * 32; };
    auto load = [&](float (&x)[4][16], int c) {
        if (col0(c) >= ld) return;
        const int so = col0(c) * 4;
#pragma unroll
        for (int b = 0; b < 4; ++b)
            if (need[b])
#pragma unroll
                for (int e = 0; e < 16; ++e) x[b][e] = buf_load_f32<kBufNT>(buf, voff(b, e), so);
    };
    // X <- X + R^T X for the pair (U, W) of register slots, rotation q
    auto apply = [&](float (&x)[4][16], int q, int U, int W) {
        v16f acc0, acc1;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            acc0[r] = 0.0f;
            acc1[r] = 0.0f;
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            float f[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) f[e] = t < 2 ? x[U][8 * t + e] : x[W][8 * (t - 2) + e];
            const Split8 xs = split8(f);
            const Split8 r0{Rp[q][0][0][t][lane], Rp[q][1][0][t][lane], Rp[q][2][0][t][lane]};
            const Split8 r1{Rp[q][0][1][t][lane], Rp[q][1][1][t][lane], Rp[q][2][1][t][lane]};
            acc0 = mfma_split6(r0, xs, acc0);
            acc1 = mfma_split6(r1, xs, acc1);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            x[U][r] += acc0[r];
            x[W][r] += acc1[r];
        }
    };
    auto update = [&](float (&x)[4][16], int c) {
        if (col0(c) >= ld) return;
        if (rot[0]) apply(x, 0, 0, 1);
        if (rot[1]) apply(x, 1, 2, 3);
        if (rot[2]) apply(x, 2, 0, 3);
        if (rot[3]) apply(x, 3, 2, 1);
        const int so = col0(c) * 4;
#pragma unroll
        for (int b = 0; b < 4; ++b)
            if (need[b])
#pragma unroll
                for (int e = 0; e < 16; ++e) buf_store_f32<kBufNT>(x[b][e], buf, voff(b, e), so);
    };
    float xa[4][16], xb[4][16];
    load(xa, 0);
    // operand A of tile tl, k-step t for lane l: R^T[32 tl + l % 32][b] = R[b][32 tl + l % 32]
    // at the 8 rows b = apply_row(8 t + e, l / 32) (as jac_apply_kernel)
    for (int idx = threadIdx.x; idx < 4 * 2 * 4 * 64; idx += kV2Threads) {
        const int q = idx >> 9, tl = (idx >> 8) & 1, t = (idx >> 6) & 3, l = idx & 63;
        if (!rot[q]) continue;
        const float* R = rot_of(md, rnd[q], slot[q]);
        float f[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = gld(R + apply_row(8 * t + e, l >> 5) * PW + 32 * tl + (l & 31));
        const Split8 sp = split8(f);
        Rp[q][0][tl][t][l] = sp.h;
        Rp[q][1][tl][t][l] = sp.m;
        Rp[q][2][tl][t][l] = sp.l;
    }
    __syncthreads();
    const int n = (it.x1 - it.x0 + kV2Cols - 1) / kV2Cols;
    for (int c = 0; c < n; c += 2) {
        if (c + 1 < n) load(xb, c + 1);
        update(xa, c);
        if (c + 1 >= n) break;
        if (c + 2 < n) load(xa, c + 2);
        update(xb, c + 1);
    }
}

// ---------------------------------------------------------------------------------
// Sweep-start ordering (de Rijk): at the first round of each of a matrix's
// sweeps, sort its physical rows by decreasing squared norm (ties by row
// index) into perm, so that blocks hold columns of similar size; this cuts
// the number of sweeps by about a quarter on the workloads' matrices.
// Bitonic sort of up to kSortMax (norm, row) keys in LDS, one workgroup per matrix.
namespace {
constexpr int kSortMax = 4096;  // 32 KB of LDS
}
__global__ __launch_bounds__(256) void jac_sort_kernel(const MatDev* __restrict__ mats,
                                                       const MatFlags* __restrict__ flags,
                                                       const int* __restrict__ mat_idx,
                                                       int round, int quad) {
    __shared__ float key[kSortMax];
    __shared__ int idx[kSortMax];
    const int i = mat_idx[blockIdx.x];
    if (flags[i].done || flags[i].sel) return;  // selective sweeps keep bmax's column order
    const MatDev& md = mats[i];
    if (round % (quad ? quad_passes(md.nb) : md.nb - 1) != 0) return;
    if (md.kpad > kSortMax) return;  // beyond the LDS sort size the order stays as it is
    int n2 = 1;
    while (n2 < md.kpad) n2 <<= 1;
    for (int j = threadIdx.x; j < n2; j += blockDim.x) {
        key[j] = j < md.kpad ? md.cnorm[j] : -1.0f;
        idx[j] = j;
    }
    __syncthreads();
    for (int size = 2; size <= n2; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int t = threadIdx.x; t < n2 / 2; t += blockDim.x) {
                const int lo = 2 * t - (t & (stride - 1));
                const int hi = lo + stride;
                const bool desc = (lo & size) == 0;  // final order: descending
                const float ka = key[lo], kb = key[hi];
                const int ia = idx[lo], ib = idx[hi];
                // "a before b" in the final order: larger norm first, then smaller row
                const bool a_first = ka > kb || (ka == kb && ia < ib);
                if (a_first != desc) {
                    key[lo] = kb;
                    key[hi] = ka;
                    idx[lo] = ib;
                    idx[hi] = ia;
                }
            }
            __syncthreads();
        }
    }
    for (int j = threadIdx.x; j < md.kpad; j += blockDim.x) md.perm[j] = idx[j];
}

hipError_t launch_jacobi_sort(const MatDev* mats, const MatFlags* flags, const int* mat_idx,
                              int nmat, int round, int quad, hipStream_t st) {
    hipLaunchKernelGGL(jac_sort_kernel, dim3(nmat), dim3(256), 0, st, mats, flags, mat_idx, round,
                       quad);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------
// End-of-round bookkeeping: a matrix whose sweep ended this round is
// converged when nothing above tolerance was seen during the sweep, or when the
// sweep saw at most the sweep-stop value (stop_factor in the Cholesky factor
// phase, stop_plain in plain sweeps; 0 = off).  By then the convergence is
// quadratic (on the 16-block workload, sweeps that saw at most 1e-4 were
// followed by ones that saw about 1e-6, the rotation threshold), so the sweep
// that would only confirm it rotates almost nothing; a certificate checks the
// result instead: after the factor phase the one of A = M V (failing pairs are
// polished), after plain sweeps the final Gram's (early = 1; a failing matrix
// sweeps on).
__global__ void jac_sweep_end_kernel(const MatDev* __restrict__ mats, MatFlags* __restrict__ flags,
                                     const int* __restrict__ mat_idx, int nmat, int round,
                                     int quad, int max_sweeps, float stop_factor, float stop_plain) {
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= nmat) return;
    const int i = mat_idx[t];
    MatFlags& f = flags[i];
    if (f.done) return;
    // rounds (or quad passes) per sweep
    const int per = quad ? quad_passes(mats[i].nb) : mats[i].nb - 1;
    if (round % per != per - 1) return;
    f.sweeps += 1;
    if (f.sel) f.sel_sweeps += 1;
    const float mo = __uint_as_float(f.sweep_max);
    f.sweep_max = 0u;
    const float stop = f.precond ? stop_factor : stop_plain;
    if (!(mo <= 3.402823466e38f)) {
        f.done = 1;  // a non-finite operand: stop, reported as not converged
    } else if (!(mo > mats[i].tol_conv)) {
        f.converged = 1;
        f.done = 1;
    } else if (!(mo > stop)) {
        f.converged = 1;
        f.done = 1;
        if (!f.precond) f.early = 1;
    } else if (f.sel ? f.sel_sweeps >= kSelSweeps
                     : f.sweeps - f.sweep_base - f.sel_sweeps >= max_sweeps) {
        f.done = 1;
    }
}

hipError_t launch_jacobi_gram(const MatDev* mats, const MatFlags* flags, const GramItem* gi,
                              int ngi, int round, int skip_fused, hipStream_t st) {
    hipLaunchKernelGGL(jac_gram_kernel, dim3(ngi), dim3(256), 0, st, mats, flags, gi, round, skip_fused);
    return hipGetLastError();
}

int solve_waves_for(int nsi) {
    return nsi <= kSolveSmallMax ? 8 : 4;
}

hipError_t launch_jacobi_solve(const MatDev* mats, MatFlags* flags, const SolveItem* si, int nsi,
                               int round, int waves, int copies, hipStream_t st) {
    if (waves == 0) waves = solve_waves_for(nsi);
    if (copies == 0) copies = nsi <= kSolveSmallMax ? 2 : 1;
    const bool two = copies == 2;
    if (waves == 8 && two)
        hipLaunchKernelGGL((jac_solve_waves_kernel<8, 2>), dim3(nsi), dim3(512), 0, st, mats, flags, si, round);
    else if (waves == 8)
        hipLaunchKernelGGL((jac_solve_waves_kernel<8, 1>), dim3(nsi), dim3(512), 0, st, mats, flags, si, round);
    else if (waves == 4 && two)
        hipLaunchKernelGGL((jac_solve_waves_kernel<4, 2>), dim3(nsi), dim3(256), 0, st, mats, flags, si, round);
    else if (waves == 4)
        hipLaunchKernelGGL((jac_solve_waves_kernel<4, 1>), dim3(nsi), dim3(256), 0, st, mats, flags, si, round);
    else if (waves == 2 && two)
        hipLaunchKernelGGL((jac_solve_waves_kernel<2, 2>), dim3(nsi), dim3(128), 0, st, mats, flags, si, round);
    else if (waves == 2)
        hipLaunchKernelGGL((jac_solve_waves_kernel<2, 1>), dim3(nsi), dim3(128), 0, st, mats, flags, si, round);
    else
        hipLaunchKernelGGL(jac_solve_kernel, dim3(nsi), dim3(64), 0, st, mats, flags, si, round);
    return hipGetLastError();
}

hipError_t launch_jacobi_apply(const MatDev* mats, const MatFlags* flags, const ApplyItem* ai,
                               int nai, int round, hipStream_t st) {
    if (nai == 0) return hipSuccess;
    hipLaunchKernelGGL(jac_apply_kernel, dim3(nai), dim3(kApplyThreads), 0, st, mats, flags, ai, round);
    return hipGetLastError();
}

hipError_t launch_jacobi_apply_gram(const MatDev* mats, const MatFlags* flags, const FusedItem* fi,
                                   int nfi, int round, hipStream_t st) {
    if (nfi == 0) return hipSuccess;
    hipLaunchKernelGGL(jac_apply_gram_kernel, dim3(nfi), dim3(512), 0, st, mats, flags, fi, round);
    return hipGetLastError();
}

hipError_t launch_jacobi_apply_v2(const MatDev* mats, const MatFlags* flags, const FusedItem* vi,
                                  int nvi, int round, hipStream_t st) {
    if (nvi <= 0) return hipSuccess;
    hipLaunchKernelGGL(jac_apply_v2_kernel, dim3(nvi), dim3(kV2Threads), 0, st, mats, flags, vi,
                       round);
    return hipGetLastError();
}

hipError_t launch_jacobi_sweep_end(const MatDev* mats, MatFlags* flags, const int* mat_idx,
                                   int nmat, int round, int quad, int max_sweeps, float stop_factor,
                                   float stop_plain, hipStream_t st) {
    hipLaunchKernelGGL(jac_sweep_end_kernel, dim3((nmat + 63) / 64), dim3(64), 0, st, mats, flags,
                       mat_idx, nmat, round, quad, max_sweeps, stop_factor, stop_plain);
    return hipGetLastError();
}

}  // namespace scopt
