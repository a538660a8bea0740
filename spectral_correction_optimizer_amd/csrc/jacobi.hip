// Blocked one-sided Jacobi (Hestenes) SVD sweeps on gfx950.
//
// The spectral-correction optimizer takes a thin SVD of each matrix's anchor
// momentum ("Key design 3" of the papernotes.org notes on "Communication-
// Efficient LLM Adaptation over Decentralized GPU Meshes").  The operand A
// (K x k, K >= k; A = M or M^T) is kept as rows = columns of A.  Its k columns
// are cut into blocks of b = 32; a sweep visits every block pair once in
// round-robin order (nb - 1 rounds of nb/2 disjoint pairs).  One round is three
// launches over all pairs of all matrices:
//
//   gram   per (pair, K split): G_part = X X^T, X = the pair's 64 rows of A,
//          fp32 MFMA accumulation restarted every 256 columns and summed in
//          fp64 registers (bounds the rounding of long dot products).
//   solve  per pair: sum the split partials in fixed order (fp64), measure the
//          largest relative off-diagonal |g_pq| / sqrt(g_pp g_qq); if above the
//          tolerance run one cyclic sweep of 2x2 Jacobi rotations on the 64x64
//          Gram in LDS (round-robin order, 32 disjoint rotations per step),
//          accumulating Q; store R = Q - I.
//   apply  per (pair, 128-column chunk, A or V): X <- X + R^T X on fp32 MFMA.
//          The correction form keeps the rounding of near-identity rotations
//          at the level of one addition.
//
// Every row of A and V belongs to exactly one pair per round, so the kernels
// of a round never write the same memory from two workgroups.  Reductions run
// in a fixed order: results are bitwise reproducible.
#include "common.hpp"
#include "internal.hpp"

namespace scopt {

namespace {

constexpr int PW = kPw;          // 64 rows per pair block
constexpr int KC = 32;           // K columns per LDS stage
constexpr int CHUNK = 256;       // fp32 accumulation length before folding into fp64

// Physical row of A / V holding local column rho (0..63) of block pair (I, J).
__device__ __forceinline__ int pair_row(const MatDev& md, int blkI, int blkJ, int rho) {
    return gld(md.perm + (rho < kJb ? blkI * kJb + rho : blkJ * kJb + (rho - kJb)));
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
                                                       int round) {
    __shared__ float Xs[2][KC][GXS];
    const GramItem it = items[blockIdx.x];
    if (flags[it.mat].done) return;
    const MatDev& md = mats[it.mat];
    const int nb = md.nb;
    int bI, bJ;
    rr_pair(nb, round % (nb - 1), it.slot, &bI, &bJ);
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

// ---------------------------------------------------------------------------------
__global__ __launch_bounds__(64) void jac_solve_kernel(const MatDev* __restrict__ mats,
                                                       MatFlags* __restrict__ flags,
                                                       const SolveItem* __restrict__ items,
                                                       int round) {
    // One wavefront per pair: LDS accesses of a wavefront are carried out in
    // issue order, so the steps of the inner sweep need no barriers, only
    // compiler fences that keep the accesses in program order.
    // G: float32 working copy of the pair Gram, scaled by 1 / max diagonal so
    // that the solve does not depend on the matrix's magnitude.
    // R: the accumulated rotation minus the identity, Q = I + R, kept directly
    // in float32.  Each 2x2 rotation enters R through (c - 1) = -t s / (1 + h),
    // h = sqrt(1 + t^2), and s, so a tiny rotation is carried exactly (storing
    // Q itself in float32 would round c to 1 while s != 0, a biased growth of
    // the column norms over thousands of rotations).  c = 1 / h and s = t c
    // satisfy c^2 + s^2 = 1 to float32 rounding, so float32 parameters suffice.
    __shared__ float G[PW][PW + 1];
    __shared__ float R[PW][PW + 1];
    __shared__ float4 cs[PW / 2];  // per pair of the step: c, s, c - 1, p | q << 8
    __shared__ double rs[PW];      // 1 / sqrt(g_aa) above the zero floor, else 0

    const SolveItem it = items[blockIdx.x];
    MatFlags& fl = flags[it.mat];
    if (fl.done) return;
    const MatDev& md = mats[it.mat];
    const float tol = md.tol;
    const int l = threadIdx.x;
    int bI, bJ;
    rr_pair(md.nb, round % (md.nb - 1), it.slot, &bI, &bJ);

    // 1. diagonal of the pair Gram: split partials summed in fixed order (fp64)
    const double* gp = md.gram + (int64_t)it.slot * md.nsplit * (PW * PW);
    double dl = 0.0;
    for (int sp = 0; sp < it.nsplit; ++sp) dl += gld(gp + (int64_t)sp * PW * PW + l * (PW + 1));
    double dmax = dl;
    for (int o = 32; o > 0; o >>= 1) dmax = fmax(dmax, __shfl_xor(dmax, o));
    const double scale = dmax > 0.0 ? 1.0 / dmax : 1.0;
    const double floor2d = (double)fl.floor2;
    const float floor2 = (float)(floor2d * scale);
    const double rsl = dl > floor2d ? 1.0 / sqrt(dl) : 0.0;
    rs[l] = rsl;
    __syncthreads();

    // 2. the stored upper 16x16 tiles (10 of 16), each read once and mirrored in
    //    LDS; the largest relative off-diagonal |g_ab| / sqrt(g_aa g_bb) over
    //    columns above the zero floor (rs = 0 below it)
    float mo = 0.0f;
#pragma unroll 1
    for (int t = 0; t < 10; ++t) {
        const int ti = t < 4 ? 0 : t < 7 ? 1 : t < 9 ? 2 : 3;
        const int tj = ti + t - (ti == 0 ? 0 : ti == 1 ? 4 : ti == 2 ? 7 : 9);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int a = 16 * ti + (l >> 4) + 4 * k, b = 16 * tj + (l & 15);
            double s = 0.0;
            for (int sp = 0; sp < it.nsplit; ++sp) s += gld(gp + (int64_t)sp * PW * PW + a * PW + b);
            const float g = (float)(s * scale);
            G[a][b] = g;
            if (ti != tj) G[b][a] = g;  // a diagonal tile is stored whole
            if (a < b) mo = fmaxf(mo, (float)(fabs(s) * rs[a] * rs[b]));
        }
    }
#pragma unroll 8
    for (int e = 0; e < PW; ++e) R[e][l] = 0.0f;
    for (int o = 32; o > 0; o >>= 1) mo = fmaxf(mo, __shfl_xor(mo, o));
    if (l == 0) atomicMax(&fl.sweep_max, __float_as_uint(mo));
    int* rflag = md.rot_flag + it.slot;
    if (!(mo > tol)) {
        // columns unchanged: their norms for the next sweep's ordering
        gst(md.cnorm + pair_row(md, bI, bJ, l), (float)dl);
        if (l == 0) *rflag = 0;
        return;
    }
    __syncthreads();

    // 3. one cyclic sweep of 2x2 rotations on G (G <- J^T G J), accumulating R.
    //    Lane l: pair j = l % 32 of the step, half h = l / 32.  Both halves
    //    compute pair j's rotation from G; the lower half publishes it in cs.
    //    G: lane l updates the 2x2 blocks (i, j), i = 16 h + m, rows p_i, q_i x
    //    columns p_j, q_j -- every entry of G belongs to one lane per step.
    //    R: columns p_j, q_j of rows a = h + 2 m.  A lane issues all its reads
    //    of a step before its first write, so the LDS latency is paid once.
    const int j = l & 31, h = l >> 5;
#pragma unroll 1
    for (int ir = 0; ir < PW - 1; ++ir) {
        int pj, qj;
        rr_pair(PW, ir, j, &pj, &qj);
        float c = 1.0f, sn = 0.0f, cm1 = 0.0f;
        {
            const float gpp = G[pj][pj], gqq = G[qj][qj], gpq = G[pj][qj];
            if (gpp > floor2 && gqq > floor2 &&
                fabsf(gpq) > tol * __builtin_amdgcn_sqrtf(gpp * gqq)) {
                const float zeta = (gqq - gpp) * 0.5f * __builtin_amdgcn_rcpf(gpq);
                const float az = fabsf(zeta);
                // t = sign(zeta) / (|zeta| + sqrt(1 + zeta^2)), without overflow
                const float den =
                    az < 1e18f ? az + __builtin_amdgcn_sqrtf(fmaf(az, az, 1.0f)) : 2.0f * az;
                const float t = copysignf(__builtin_amdgcn_rcpf(den), zeta);
                const float hh = __builtin_amdgcn_sqrtf(fmaf(t, t, 1.0f));
                c = __builtin_amdgcn_rcpf(hh);
                sn = t * c;
                cm1 = -t * sn * __builtin_amdgcn_rcpf(1.0f + hh);
            }
        }
        if (h == 0) cs[j] = make_float4(c, sn, cm1, __int_as_float(pj | (qj << 8)));
        __asm__ volatile("" ::: "memory");
        float4 ri[16];
#pragma unroll
        for (int m = 0; m < 16; ++m) ri[m] = cs[16 * h + m];
        float x[16][4];
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            const int pq = __float_as_int(ri[m].w), pi = pq & 255, qi = pq >> 8;
            x[m][0] = G[pi][pj];
            x[m][1] = G[pi][qj];
            x[m][2] = G[qi][pj];
            x[m][3] = G[qi][qj];
        }
        const bool rot = sn != 0.0f;
        float xr[32], yr[32];
        if (rot) {
#pragma unroll
            for (int m = 0; m < 32; ++m) {
                xr[m] = R[h + 2 * m][pj];
                yr[m] = R[h + 2 * m][qj];
            }
        }
        // G: columns first ([x_p, x_q] <- [c x_p - s x_q, s x_p + c x_q]), then
        // rows with pair i's rotation
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            const int pq = __float_as_int(ri[m].w), pi = pq & 255, qi = pq >> 8;
            const float ci = ri[m].x, si = ri[m].y;
            const float y00 = c * x[m][0] - sn * x[m][1], y01 = sn * x[m][0] + c * x[m][1];
            const float y10 = c * x[m][2] - sn * x[m][3], y11 = sn * x[m][2] + c * x[m][3];
            G[pi][pj] = ci * y00 - si * y10;
            G[qi][pj] = si * y00 + ci * y10;
            G[pi][qj] = ci * y01 - si * y11;
            G[qi][qj] = si * y01 + ci * y11;
        }
        // R <- R J (plus J - I on rows p_j, q_j)
        if (rot) {
#pragma unroll
            for (int m = 0; m < 32; ++m) {
                R[h + 2 * m][pj] = fmaf(cm1, xr[m], xr[m]) - sn * yr[m];
                R[h + 2 * m][qj] = fmaf(cm1, yr[m], yr[m]) + sn * xr[m];
            }
            if ((pj & 1) == h) {
                R[pj][pj] += cm1;
                R[pj][qj] += sn;
            }
            if ((qj & 1) == h) {
                R[qj][pj] -= sn;
                R[qj][qj] += cm1;
            }
        }
        __asm__ volatile("" ::: "memory");
    }
    __syncthreads();
    // 4. R row-major [b][a] (X_new[a] = X[a] + sum_b R[b][a] X[b])
    float* Rg = md.rot + (int64_t)it.slot * PW * PW;
#pragma unroll 8
    for (int e = 0; e < PW; ++e) gst(Rg + e * PW + l, R[e][l]);
    // rotated squared column norms (diagonal of Q^T G Q) for the next sweep's ordering
    gst(md.cnorm + pair_row(md, bI, bJ, l), (float)(G[l][l] * dmax));
    if (l == 0) {
        *rflag = 1;
        atomicAdd(&fl.pairs_applied, 1);
    }
}

// ---------------------------------------------------------------------------------
namespace {
// Row of the pair block fed by lane half hl at contraction step s of the apply.
// The order is chosen so that a lane's 32 B operands are exactly the 32 rows of
// its 32x32 MFMA outputs (row 8 (r / 4) + 4 hl + r % 4 of acc0, 32 more of acc1).
__device__ __forceinline__ int apply_row(int s, int hl) {
    return 32 * (s >> 4) + 8 * ((s & 15) >> 2) + 4 * hl + (s & 3);
}
constexpr int RLD = 72;  // LDS row stride of R: rows 4 apart fall 32 banks apart
}  // namespace

__global__ __launch_bounds__(kApplyThreads) void jac_apply_kernel(const MatDev* __restrict__ mats,
                                                        const MatFlags* __restrict__ flags,
                                                        const ApplyItem* __restrict__ items,
                                                        int round) {
    // A workgroup updates 64 rows x kApplyCols columns; wave w owns columns
    // [x0 + 32 w, x0 + 32 w + 32).  Only R goes through LDS: each lane loads
    // 32 rows of its column straight into registers; they are both its MFMA B
    // operands (B[k][j] = X[b][n] over the contraction order apply_row) and the
    // old values of its output elements, so X_new = X + R^T X needs no re-read.
    __shared__ float Rs[PW][RLD];
    const ApplyItem it = items[blockIdx.x];
    if (flags[it.mat].done) return;
    const MatDev& md = mats[it.mat];
    if (md.rot_flag[it.slot] == 0) return;
    int bI, bJ;
    rr_pair(md.nb, round % (md.nb - 1), it.slot, &bI, &bJ);
    float* base = it.which == 0 ? md.A : md.V;
    const int ld = it.which == 0 ? md.K_ld : md.kpad;  // multiple of 64
    const int x0 = it.chunk * kApplyCols;

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int hl = lane >> 5, ll = lane & 31;
    const int n = x0 + wave * 32 + ll;
    const bool active = x0 + wave * 32 < ld;  // a wave's 32 columns are all in or all out
    float xb[PW / 2];
    int prow[PW / 2];  // physical rows (kept as indices: fewer registers than pointers)
#pragma unroll
    for (int s = 0; s < PW / 2; ++s) prow[s] = pair_row(md, bI, bJ, apply_row(s, hl));
    float* const col = base + n;
    if (active) {
#pragma unroll
        for (int s = 0; s < PW / 2; ++s)
            xb[s] = __builtin_nontemporal_load(gptr(col + (int64_t)prow[s] * ld));
    }
    const float* R = md.rot + (int64_t)it.slot * PW * PW;
    for (int idx = threadIdx.x; idx < PW * PW / 4; idx += kApplyThreads) {
        const int b = idx >> 4, a4 = (idx & 15) * 4;
        *(v4f*)&Rs[b][a4] = gld4(R + b * PW + a4);
    }
    __syncthreads();
    if (!active) return;

    v16f acc0, acc1;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        acc0[r] = 0.0f;
        acc1[r] = 0.0f;
    }
#pragma unroll
    for (int s = 0; s < PW / 2; ++s) {
        const int b = apply_row(s, hl);
        acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(Rs[b][ll], xb[s], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(Rs[b][32 + ll], xb[s], acc1, 0, 0, 0);
    }
    // acc0 register r is row apply_row(r, hl), acc1 register r is row apply_row(16 + r, hl)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        __builtin_nontemporal_store(xb[r] + acc0[r], gptr(col + (int64_t)prow[r] * ld));
        __builtin_nontemporal_store(xb[16 + r] + acc1[r], gptr(col + (int64_t)prow[16 + r] * ld));
    }
}

// ---------------------------------------------------------------------------------
// Sweep-start ordering (de Rijk): at the first round of each of a matrix's
// sweeps, sort its physical rows by decreasing squared norm (ties by row
// index) into perm, so that blocks hold columns of similar size; this cuts
// the number of sweeps by about a quarter on the workloads' matrices.
// Bitonic sort of up to 2048 (norm, row) keys in LDS, one workgroup per matrix.
__global__ __launch_bounds__(256) void jac_sort_kernel(const MatDev* __restrict__ mats,
                                                       const MatFlags* __restrict__ flags,
                                                       const int* __restrict__ mat_idx,
                                                       int round) {
    __shared__ float key[2048];
    __shared__ int idx[2048];
    const int i = mat_idx[blockIdx.x];
    if (flags[i].done) return;
    const MatDev& md = mats[i];
    if (round % (md.nb - 1) != 0) return;
    if (md.kpad > 2048) return;  // beyond the LDS sort size the order stays as it is
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
                              int nmat, int round, hipStream_t st) {
    hipLaunchKernelGGL(jac_sort_kernel, dim3(nmat), dim3(256), 0, st, mats, flags, mat_idx, round);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------
// End-of-round bookkeeping: a matrix whose sweep ended this round is
// converged when nothing above tolerance was seen during the sweep.
__global__ void jac_sweep_end_kernel(const MatDev* __restrict__ mats, MatFlags* __restrict__ flags,
                                     const int* __restrict__ mat_idx, int nmat, int round,
                                     int max_sweeps) {
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= nmat) return;
    const int i = mat_idx[t];
    MatFlags& f = flags[i];
    if (f.done) return;
    f.rounds_active += 1;
    const int nbm1 = mats[i].nb - 1;
    if (round % nbm1 != nbm1 - 1) return;
    f.sweeps += 1;
    const float mo = __uint_as_float(f.sweep_max);
    f.sweep_max = 0u;
    if (!(mo > mats[i].tol_conv)) {
        f.converged = 1;
        f.done = 1;
    } else if (f.sweeps - f.sweep_base >= max_sweeps) {
        f.done = 1;
    }
}

hipError_t launch_jacobi_gram(const MatDev* mats, const MatFlags* flags, const GramItem* gi,
                              int ngi, int round, hipStream_t st) {
    hipLaunchKernelGGL(jac_gram_kernel, dim3(ngi), dim3(256), 0, st, mats, flags, gi, round);
    return hipGetLastError();
}

hipError_t launch_jacobi_solve(const MatDev* mats, MatFlags* flags, const SolveItem* si, int nsi,
                               int round, hipStream_t st) {
    hipLaunchKernelGGL(jac_solve_kernel, dim3(nsi), dim3(64), 0, st, mats, flags, si, round);
    return hipGetLastError();
}

hipError_t launch_jacobi_apply(const MatDev* mats, const MatFlags* flags, const ApplyItem* ai,
                               int nai, int round, hipStream_t st) {
    hipLaunchKernelGGL(jac_apply_kernel, dim3(nai), dim3(kApplyThreads), 0, st, mats, flags, ai, round);
    return hipGetLastError();
}

hipError_t launch_jacobi_sweep_end(const MatDev* mats, MatFlags* flags, const int* mat_idx,
                                   int nmat, int round, int max_sweeps,
                                   hipStream_t st) {
    hipLaunchKernelGGL(jac_sweep_end_kernel, dim3((nmat + 63) / 64), dim3(64), 0, st, mats, flags,
                       mat_idx, nmat, round, max_sweeps);
    return hipGetLastError();
}

}  // namespace scopt
