// Cholesky preconditioning of the Jacobi SVD for operands at least twice as long
// as wide, in refreshes that start from the previous factors (A = M V_prev with
// nearly orthogonal columns).
//
// With C = A^T A = L L^T, i.e. A = Q R with R = L^T, the SVD of A follows from
// the SVD of the k x k lower-triangular X = R^T = L:  X = U_x S V_x^T gives
// R = V_x S U_x^T and A = (Q V_x) S U_x^T, so the right singular vectors of A
// are U_x, the normalized columns of X after its one-sided Jacobi sweeps (the
// factor phase).  The rotations of X need not be accumulated at all; the
// sweeps move rows k long instead of K and touch no V, and the columns of X
// (rows of R, graded like the singular values) converge in fewer sweeps than
// those of A.  Afterwards V <- U_x^T-combination of V_prev (one k x k GEMM),
// A = M V is formed once and ordinary sweeps polish it until converged.  This
// only pays if X^T X matches A^T A to about the sweep tolerance; hence:
//
//   chol_syrk    C = A^T A (lower 128 x 128 tiles), float32 MFMA products whose
//                running sums are folded into float64 every 256 columns, the
//                same scheme as the pair Gram of the sweeps;
//   chol_diag    factor a 64 x 64 diagonal tile in float64 (LDS);
//   chol_panel   L_ib,jb = C_ib,jb L_jb,jb^-T below it (float64);
//   chol_update  C_ib,kb -= L_ib,jb L_kb,jb^T for the trailing lower tiles
//                (float64 FMA, register-blocked);
//   chol_commit  rows of the operand <- float32(columns of L) (tiled transpose).
//
// Rounding L to float32 perturbs each entry by 2^-24 of itself, well inside the
// sweep tolerance.
//
// A pivot that keeps less than a tenth of its column's squared norm (the
// column nearly lies in the span of the previous ones), or a column at or
// below the zero floor (U_x would be undefined there), rejects the matrix: it
// sits the factor phase out and runs plain sweeps in the polishing phase.
#include "common.hpp"
#include "internal.hpp"

namespace scopt {

namespace {
constexpr int CT = 64;   // Cholesky tile
constexpr double kKeep = 0.1;

__device__ __forceinline__ bool chol_active(const MatDev& md, const MatFlags& f, int jb) {
    return !f.chol_fail && jb * CT < md.k;
}
}  // namespace

// ---------------------------------------------------------------------------------
// C = A^T A over the rows of the Jacobi operand (row j = column j of A, length
// K_ld, zero padded).  One workgroup per lower 128 x 128 tile (ti >= tj); eight
// waves of 64 x 32 (2 x 1 blocks of v_mfma_f32_32x32x16_bf16) over the exact
// three-way bfloat16 split of the operand (six part products, float32
// accumulation, the dropped ones below 2^-23 of each product).  K advances by 32
// columns (two 16-column halves) through double-buffered LDS holding the split
// rows of both strips (the diagonal tiles read one strip); the float32
// accumulators are folded into float64 every 256 columns.  Eight waves of 64 x 32
// keep the float64 sums at 64 registers a lane, so two waves share each SIMD.
// Within a fold span the loop body is one block (the next step's loads and split
// are issued unconditionally, the last step's into the idle buffer) so the next
// step's split is scheduled between the products.  FULL: k is a multiple of the
// tile, every strip row exists (no masking).
namespace {
constexpr int SB = 128, SKB = 32, SFOLD = 256;
}

template <bool FULL>
__global__ __launch_bounds__(512) void chol_syrk_kernel(const MatDev* __restrict__ mats,
                                                        const MatFlags* __restrict__ flags,
                                                        const SyrkItem* __restrict__ items,
                                                        int only_regram) {
    __shared__ __align__(16) __bf16 Xs[2][2][3][2][SB * 16];  // [buffer][strip][plane][half of the step]
    const SyrkItem it = items[blockIdx.x];
    if (only_regram && !flags[it.mat].regram) return;
    const MatDev& md = mats[it.mat];
    const bool diag = it.ti == it.tj;
    const int k = md.k, ld = md.K_ld;
    const int r0[2] = {it.ti * SB, it.tj * SB};

    // loader: thread t holds 8 consecutive columns 16 s + 8 h (s = (t >> 1) & 1,
    // h = t & 1) of the step's 32, of strip row t >> 2; rows at or beyond k read as zero
    const int nstrip = diag ? 1 : 2;
    const int lrow = threadIdx.x >> 2, lsub = (threadIdx.x >> 1) & 1, lhalf = threadIdx.x & 1;
    float4 reg[2][2];
    auto gload = [&](int x0) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            if (t >= nstrip) break;
            const int row = r0[t] + lrow;
            const float* q = md.A + (int64_t)(FULL ? row : min(row, k - 1)) * ld + x0 + 16 * lsub + 8 * lhalf;
            reg[t][0] = load4(q);
            reg[t][1] = load4(q + 4);
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            if (t >= nstrip) break;
            const bool in = FULL || r0[t] + lrow < k;
            const float f[8] = {in ? reg[t][0].x : 0.f, in ? reg[t][0].y : 0.f, in ? reg[t][0].z : 0.f,
                                in ? reg[t][0].w : 0.f, in ? reg[t][1].x : 0.f, in ? reg[t][1].y : 0.f,
                                in ? reg[t][1].z : 0.f, in ? reg[t][1].w : 0.f};
            const Split8 sp = split8(f);
            const int o = split_chunk16(lrow, lhalf);
            *(v8bf*)&Xs[buf][t][0][lsub][o] = sp.h;
            *(v8bf*)&Xs[buf][t][1][lsub][o] = sp.m;
            *(v8bf*)&Xs[buf][t][2][lsub][o] = sp.l;
        }
    };

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int hl = lane >> 5, ll = lane & 31;
    const int wr = (wave >> 2) * 64, wc = (wave & 3) * 32;
    const int sj = diag ? 0 : 1;
    const int fa0 = split_chunk16(wr + ll, hl), fa1 = split_chunk16(wr + 32 + ll, hl);
    const int fb = split_chunk16(wc + ll, hl);
    v16f acc[2];
    double acc64[2][16];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            acc[a][r] = 0.0f;
            acc64[a][r] = 0.0;
        }
    const int nst = ld / SKB;  // K_ld is a multiple of 128
    gload(0);
    lstore(0);
    __syncthreads();
    for (int st0 = 0; st0 < nst; st0 += SFOLD / SKB) {
        const int st1 = min(st0 + SFOLD / SKB, nst);
        for (int st = st0; st < st1; ++st) {
            const int buf = st & 1;
            const int sn = st + 1 < nst ? st + 1 : st;
            gload(sn * SKB);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                v8bf a[2][3], b[3];
#pragma unroll
                for (int p = 0; p < 3; ++p) {
                    a[0][p] = *(const v8bf*)&Xs[buf][0][p][h][fa0];
                    a[1][p] = *(const v8bf*)&Xs[buf][0][p][h][fa1];
                    b[p] = *(const v8bf*)&Xs[buf][sj][p][h][fb];
                }
#define SC_TERM(PA, PB)                                         \
    _Pragma("unroll") for (int i = 0; i < 2; ++i)                \
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i][PA], b[PB], acc[i], 0, 0, 0);
                SC_TERM(2, 0) SC_TERM(1, 1) SC_TERM(0, 2) SC_TERM(1, 0) SC_TERM(0, 1) SC_TERM(0, 0)
#undef SC_TERM
            }
            lstore(buf ^ 1);  // the idle buffer: no wave reads it before the barrier
            __builtin_amdgcn_sched_group_barrier(0x100, 9, 0);
#pragma unroll
            for (int i = 0; i < 24; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x200, 6, 0);
            __syncthreads();
        }
#pragma unroll
        for (int a2 = 0; a2 < 2; ++a2)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                acc64[a2][r] += (double)acc[a2][r];
                acc[a2][r] = 0.0f;
            }
    }
    // 32x32 output layout: lane l, register r -> row 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32
#pragma unroll
    for (int a2 = 0; a2 < 2; ++a2)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = r0[0] + wr + 32 * a2 + 8 * (r >> 2) + 4 * hl + (r & 3);
            const int col = r0[1] + wc + ll;
            if (row < k && col < k) gst(md.chol + (int64_t)row * k + col, acc64[a2][r]);
        }
}

// ---------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void chol_diag_kernel(const MatDev* __restrict__ mats,
                                                        MatFlags* __restrict__ flags,
                                                        const int* __restrict__ mat_idx, int jb) {
    __shared__ double T[CT][CT + 1];
    __shared__ double piv[CT];
    __shared__ int fail;
    const int i = mat_idx[blockIdx.x];
    MatFlags& f = flags[i];
    const MatDev& md = mats[i];
    if (!chol_active(md, f, jb)) return;
    const int k = md.k, r0 = jb * CT;
    double* C = md.chol;  // [k][k], lower triangle
    for (int idx = threadIdx.x; idx < CT * CT; idx += blockDim.x) {
        const int r = idx >> 6, c = idx & 63;
        const int gr = r0 + r, gc = r0 + c;
        T[r][c] = (gr < k && gc < k) ? (c <= r ? C[(int64_t)gr * k + gc] : 0.0) : (r == c ? 1.0 : 0.0);
    }
    if (threadIdx.x == 0) fail = 0;
    __syncthreads();
    for (int c = 0; c < CT; ++c) {
        if (threadIdx.x == 0) {
            const int gc = r0 + c;
            double l = 1.0;  // padding: identity
            if (gc < k) {
                const double orig = md.norm2[gc];
                const double p = T[c][c];
                if (!(orig > (double)f.floor2) || !(p > kKeep * orig)) fail = 1;
                else l = sqrt(p);
            }
            piv[c] = l;
        }
        __syncthreads();
        if (fail) break;
        const double l = piv[c];
        for (int r = c + 1 + threadIdx.x; r < CT; r += blockDim.x)
            T[r][c] = l > 0.0 ? T[r][c] / l : 0.0;
        __syncthreads();
        // trailing lower triangle: thread (tid / 16, tid % 16) strides rows and columns by 16
        for (int r = c + 1 + (threadIdx.x >> 4); r < CT; r += 16)
            for (int s = c + 1 + (threadIdx.x & 15); s <= r; s += 16) T[r][s] -= T[r][c] * T[s][c];
        __syncthreads();
    }
    if (fail) {
        if (threadIdx.x == 0) f.chol_fail = 1;
        return;
    }
    for (int idx = threadIdx.x; idx < CT * CT; idx += blockDim.x) {
        const int r = idx >> 6, c = idx & 63;
        const int gr = r0 + r, gc = r0 + c;
        if (gr < k && gc <= gr) C[(int64_t)gr * k + gc] = c < r ? T[r][c] : piv[r];
    }
}

// X L^T = B for the tile rows below the diagonal tile:
//   x_c = (b_c - sum_{s<c} x_s L[c][s]) / L[c][c], one thread per row.
__global__ __launch_bounds__(256) void chol_panel_kernel(const MatDev* __restrict__ mats,
                                                         const MatFlags* __restrict__ flags,
                                                         const int* __restrict__ mat_idx, int jb) {
    __shared__ double Lp[CT * (CT + 1) / 2];  // diagonal tile, packed lower triangle
    __shared__ double B[CT][CT + 1];
    const int i = mat_idx[blockIdx.y];
    const MatFlags& f = flags[i];
    const MatDev& md = mats[i];
    if (!chol_active(md, f, jb)) return;
    const int k = md.k, nbk = (k + CT - 1) / CT;
    const int ib = jb + 1 + blockIdx.x;
    if (ib >= nbk) return;
    double* C = md.chol;
    const int r0 = ib * CT, c0 = jb * CT;
    for (int idx = threadIdx.x; idx < CT * CT; idx += blockDim.x) {
        const int r = idx >> 6, c = idx & 63;
        if (c <= r)
            Lp[r * (r + 1) / 2 + c] =
                (c0 + r < k) ? C[(int64_t)(c0 + r) * k + c0 + c] : (r == c ? 1.0 : 0.0);
        B[r][c] = (r0 + r < k && c0 + c < k) ? C[(int64_t)(r0 + r) * k + c0 + c] : 0.0;
    }
    __syncthreads();
    // X L^T = B column by column (right-looking): column c is final once the
    // terms of columns s < c are subtracted (in that order) and it is divided by
    // L_cc; then every thread subtracts its share of column c's terms from the
    // columns after it
    for (int c = 0; c < CT; ++c) {
        if (threadIdx.x < CT) {
            const double d = Lp[c * (c + 1) / 2 + c];
            B[threadIdx.x][c] = d > 0.0 ? B[threadIdx.x][c] / d : 0.0;
        }
        __syncthreads();
        for (int idx = threadIdx.x; idx < CT * (CT - 1 - c); idx += blockDim.x) {
            const int r = idx & (CT - 1), sc = c + 1 + (idx >> 6);
            B[r][sc] -= B[r][c] * Lp[sc * (sc + 1) / 2 + c];
        }
        __syncthreads();
    }
    for (int idx = threadIdx.x; idx < CT * CT; idx += blockDim.x) {
        const int r = idx >> 6, c = idx & 63;
        if (r0 + r < k && c0 + c < k) C[(int64_t)(r0 + r) * k + c0 + c] = B[r][c];
    }
}

// C -= sum over the npan panels jb .. jb + npan - 1 of L_:,p L_:,p^T, on the lower
// part of the output columns [cfirst * 64, cend) (cend = (cfirst + cnt) * 64, or k
// when cnt = 0) and the rows from cfirst * 64 on: one 64-wide column of tiles
// (cnt = 1) or the whole trailing triangle.  128 x 128 blocks; 16 x 16 threads,
// each an 8 x 8 block of outputs (rows ty + 16 a, columns tx + 16 b), each sum over
// the panels' 64 npan columns in order; the panels pass through LDS 16 columns at
// a time, transposed (rows padded by one element), the next chunk prefetched into
// registers.  Entries above the diagonal or beyond k are not written.
__global__ __launch_bounds__(256) void chol_update_kernel(const MatDev* __restrict__ mats,
                                                          const MatFlags* __restrict__ flags,
                                                          const int* __restrict__ mat_idx, int jb, int npan,
                                                          int cfirst, int cnt) {
    constexpr int UB = 2 * CT, US = 16;
    __shared__ double P[US][UB + 1];  // the block's rows of the panels, k-major: P[s][r]
    __shared__ double Q[US][UB + 1];  // the block's columns' rows of the panels: Q[s][c]
    const int i = mat_idx[blockIdx.y];
    const MatFlags& f = flags[i];
    const MatDev& md = mats[i];
    if (!chol_active(md, f, jb)) return;
    const int k = md.k, nbk = (k + CT - 1) / CT;
    if (cfirst >= nbk) return;
    const int r0 = cfirst * CT;
    const int cend = cnt ? min(nbk, cfirst + cnt) * CT : nbk * CT;
    const int nrb = (k - r0 + UB - 1) / UB, ncb = (cend - r0 + UB - 1) / UB;
    const int t = blockIdx.x;
    if (t >= nrb * ncb) return;
    const int a = t / ncb, b = t % ncb;
    if (b > a) return;  // above the diagonal
    const int ri = r0 + a * UB, rk = r0 + b * UB, c0 = jb * CT, ns = npan * CT;
    double* C = md.chol;
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    double acc[8][8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int v = 0; v < 8; ++v) acc[u][v] = 0.0;
    // element j of a thread in a chunk: idx = tid + 256 j, row idx / 16, column idx % 16
    constexpr int NE = US * UB / 256;
    double pr[NE], qr[NE];
    // global-address-space loads at clamped addresses (generic loads would also
    // count on the LDS wait counter, so every fragment read below would wait for
    // this prefetch); out-of-range entries are zeroed when the values go to LDS,
    // one chunk later, so that nothing waits for the loads before then
    auto gl = [&](int s0) {
#pragma unroll
        for (int j = 0; j < NE; ++j) {
            const int idx = threadIdx.x + 256 * j, r = idx >> 4, gsc = min(c0 + s0 + (idx & (US - 1)), k - 1);
            pr[j] = gld(C + (int64_t)min(ri + r, k - 1) * k + gsc);
            qr[j] = gld(C + (int64_t)min(rk + r, k - 1) * k + gsc);
        }
    };
    gl(0);
    for (int s0 = 0; s0 < ns; s0 += US) {
#pragma unroll
        for (int j = 0; j < NE; ++j) {
            const int idx = threadIdx.x + 256 * j, r = idx >> 4, s = idx & (US - 1);
            const bool sok = c0 + s0 + s < k;
            P[s][r] = (ri + r < k && sok) ? pr[j] : 0.0;
            Q[s][r] = (rk + r < k && sok) ? qr[j] : 0.0;
        }
        __syncthreads();
        if (s0 + US < ns) gl(s0 + US);
#pragma unroll 4
        for (int s = 0; s < US; ++s) {
            double pv[8], qv[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                pv[u] = P[s][ty + 16 * u];
                qv[u] = Q[s][tx + 16 * u];
            }
#pragma unroll
            for (int u = 0; u < 8; ++u)
#pragma unroll
                for (int v = 0; v < 8; ++v) acc[u][v] = fma(pv[u], qv[v], acc[u][v]);
        }
        __syncthreads();
    }
    // C -= acc in batches of two rows: the batch's 16 old values are loaded
    // together (global address space; clamped addresses inside the k x k matrix,
    // values outside the block's lower triangle read but not written), all 16 new
    // values formed, then the masked stores.  Per-element branches made each
    // load, and with generic addresses each store, its own memory round trip.
#pragma unroll
    for (int u0 = 0; u0 < 8; u0 += 2) {
        double nv[2][8];
#pragma unroll
        for (int du = 0; du < 2; ++du)
#pragma unroll
            for (int v = 0; v < 8; ++v) {
                const int row = min(ri + ty + 16 * (u0 + du), k - 1), col = min(rk + tx + 16 * v, k - 1);
                nv[du][v] = gld(C + (int64_t)row * k + col);
            }
#pragma unroll
        for (int du = 0; du < 2; ++du)
#pragma unroll
            for (int v = 0; v < 8; ++v) nv[du][v] -= acc[u0 + du][v];
#pragma unroll
        for (int du = 0; du < 2; ++du)
#pragma unroll
            for (int v = 0; v < 8; ++v) {
                const int row = ri + ty + 16 * (u0 + du), col = rk + tx + 16 * v;
                if (row < k && col < cend && col <= row) gst(C + (int64_t)row * k + col, nv[du][v]);
            }
    }
}

// Accepted factorizations: the rows of the Jacobi operand become the float32
// columns of L (row j = X[:, j], X = L), klen long, zero above the diagonal of
// L and beyond k.  64 x 64 tiles transposed through LDS.  A rejected matrix
// keeps its operand and sits the factor phase out (done = 1).
__global__ __launch_bounds__(256) void chol_commit_kernel(const MatDev* __restrict__ mats,
                                                          MatFlags* __restrict__ flags,
                                                          const int* __restrict__ mat_idx) {
    __shared__ float T[CT][CT + 1];
    const int i = mat_idx[blockIdx.z];
    MatFlags& f = flags[i];
    const MatDev& md = mats[i];
    if (f.chol_fail) {
        if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) f.done = 1;
        return;
    }
    const int k = md.k, klen = md.klen;
    const int j0 = blockIdx.y * CT;  // operand rows (columns of L)
    const int c0 = blockIdx.x * CT;  // operand columns (rows of L)
    if (j0 >= k || c0 >= klen) return;
    for (int idx = threadIdx.x; idx < CT * CT; idx += blockDim.x) {
        const int r = idx >> 6, c = idx & 63;  // T[r][c] = L[c0 + r][j0 + c]
        const int lr = c0 + r, lc = j0 + c;
        T[r][c] = (lr < k && lc < k && lc <= lr) ? (float)md.chol[(int64_t)lr * k + lc] : 0.0f;
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < CT * CT; idx += blockDim.x) {
        const int r = idx >> 6, c = idx & 63;  // operand[j0 + r][c0 + c] = L[c0 + c][j0 + r]
        if (j0 + r < k) md.A[(int64_t)(j0 + r) * md.K_ld + c0 + c] = T[c][r];
    }
    if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) f.precond = 1;
}

// inv[j] = 1 / ||operand row j|| over its klen entries (float64 sum), j < k, into
// md.invn, for the matrices whose factor phase ran: the row scales of V = U_x^T V_prev.
__global__ __launch_bounds__(256) void factor_invnorm_kernel(const MatDev* __restrict__ mats,
                                                             const MatFlags* __restrict__ flags,
                                                             const int* __restrict__ mat_idx) {
    __shared__ double red[4];
    const int i = mat_idx[blockIdx.y];
    const MatDev& md = mats[i];
    const int j = blockIdx.x;
    if (!flags[i].precond || j >= md.k) return;
    const float* x = md.A + (int64_t)j * md.K_ld;
    double acc = 0.0;
    for (int c = threadIdx.x; c < md.klen; c += blockDim.x) acc += (double)x[c] * (double)x[c];
    acc = block_sum_f64(acc, red);
    if (threadIdx.x == 0) md.invn[j] = acc > 0.0 ? (float)(1.0 / sqrt(acc)) : 0.0f;
}

hipError_t launch_factor_invnorm(const MatDev* mats, const MatFlags* flags, const int* mat_idx,
                                 int nmat, int max_k, hipStream_t st) {
    hipLaunchKernelGGL(factor_invnorm_kernel, dim3(max_k, nmat), dim3(256), 0, st, mats, flags,
                       mat_idx);
    return hipGetLastError();
}

hipError_t launch_chol_syrk(const MatDev* mats, const MatFlags* flags, const SyrkItem* items,
                            int nitems, int only_regram, bool full, hipStream_t st) {
    if (full)
        hipLaunchKernelGGL(chol_syrk_kernel<true>, dim3(nitems), dim3(512), 0, st, mats, flags, items,
                           only_regram);
    else
        hipLaunchKernelGGL(chol_syrk_kernel<false>, dim3(nitems), dim3(512), 0, st, mats, flags, items,
                           only_regram);
    return hipGetLastError();
}

hipError_t launch_cholesky(const MatDev* mats, MatFlags* flags, const int* mat_idx, int nmat,
                           int max_nbk, int max_klen, hipStream_t st) {
    // Two panels per pass over the trailing triangle (look-ahead): factor panel jb,
    // update only tile column jb + 1 with it, factor panel jb + 1, then update the rest
    // of the trailing triangle with both.  Grids are sized for the largest matrix;
    // the kernels skip what a smaller one does not have.
    auto upd = [&](int jb, int npan, int cfirst, int cnt) {
        const int rows = max_nbk * CT - cfirst * CT;
        const int cols = cnt ? std::min(max_nbk - cfirst, cnt) * CT : rows;
        const int nrb = (rows + 2 * CT - 1) / (2 * CT), ncb = (cols + 2 * CT - 1) / (2 * CT);
        if (nrb > 0 && ncb > 0)
            hipLaunchKernelGGL(chol_update_kernel, dim3(nrb * ncb, nmat), dim3(256), 0, st, mats, flags,
                               mat_idx, jb, npan, cfirst, cnt);
    };
    auto panel = [&](int jb) {
        const int nt = max_nbk - jb - 1;
        if (nt > 0)
            hipLaunchKernelGGL(chol_panel_kernel, dim3(nt, nmat), dim3(256), 0, st, mats, flags,
                               mat_idx, jb);
    };
    for (int jb = 0; jb < max_nbk; jb += 2) {
        hipLaunchKernelGGL(chol_diag_kernel, dim3(nmat), dim3(256), 0, st, mats, flags, mat_idx, jb);
        if (jb + 1 >= max_nbk) break;
        panel(jb);
        upd(jb, 1, jb + 1, 1);
        hipLaunchKernelGGL(chol_diag_kernel, dim3(nmat), dim3(256), 0, st, mats, flags, mat_idx, jb + 1);
        if (jb + 2 >= max_nbk) break;
        panel(jb + 1);
        upd(jb, 2, jb + 2, 0);
    }
    hipLaunchKernelGGL(chol_commit_kernel, dim3((max_klen + CT - 1) / CT, max_nbk, nmat), dim3(256),
                       0, st, mats, flags, mat_idx);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------
// Normalized Gram of the final operand for the Loewdin step and the convergence
// certificate: one workgroup per lower 64 x 64 tile (a >= b) of md.chol.  The
// upper tile of E is written through an LDS transpose.
__global__ __launch_bounds__(256) void gram_to_e_kernel(const MatDev* __restrict__ mats,
                                                        MatFlags* __restrict__ flags,
                                                        const int* __restrict__ mat_idx,
                                                        int only_regram) {
    __shared__ float T[CT][CT + 1];
    __shared__ double rdi[CT], cdi[CT];
    __shared__ float red[4];
    const int i = mat_idx[blockIdx.y];
    MatFlags& f = flags[i];
    if (only_regram && !f.regram) return;
    const MatDev& md = mats[i];
    const int k = md.k, nt = (k + CT - 1) / CT;
    const int t = blockIdx.x;
    if (t >= nt * (nt + 1) / 2) return;
    int a = (int)((sqrtf(8.0f * t + 1.0f) - 1.0f) * 0.5f);
    while ((a + 1) * (a + 2) / 2 <= t) ++a;
    while (a * (a + 1) / 2 > t) --a;
    const int b = t - a * (a + 1) / 2;
    const int r0 = a * CT, c0 = b * CT;
    const double* C = md.chol;
    const double fl2 = (double)f.floor2;
    if (threadIdx.x < CT) {
        const int r = r0 + threadIdx.x, c = c0 + threadIdx.x;
        const double dr = r < k ? C[(int64_t)r * k + r] : 0.0, dc = c < k ? C[(int64_t)c * k + c] : 0.0;
        rdi[threadIdx.x] = dr > fl2 ? 1.0 / sqrt(dr) : 0.0;
        cdi[threadIdx.x] = dc > fl2 ? 1.0 / sqrt(dc) : 0.0;
    }
    __syncthreads();
    float mo = 0.0f;
    for (int idx = threadIdx.x; idx < CT * CT; idx += blockDim.x) {
        const int r = idx >> 6, c = idx & 63;
        const int gr = r0 + r, gc = c0 + c;
        float e = 0.0f;
        if (gr < k && gc < k && gc < gr) {
            e = (float)(gld(C + (int64_t)gr * k + gc) * rdi[r] * cdi[c]);
            mo = max_nan_inf(mo, fabsf(e));
        }
        T[r][c] = e;
        if (gr < k && gc < k && (a != b || gc <= gr)) gst(md.E + (int64_t)gr * k + gc, e);
    }
    for (int o = 32; o > 0; o >>= 1) mo = fmaxf(mo, __shfl_xor(mo, o));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mo;
    __syncthreads();
    if (threadIdx.x == 0)
        atomicMax(&f.check_off, __float_as_uint(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]))));
    // mirror: E[c0 + c][r0 + r] = T[r][c]
    for (int idx = threadIdx.x; idx < CT * CT; idx += blockDim.x) {
        const int c = idx >> 6, r = idx & 63;
        const int gr = r0 + r, gc = c0 + c;
        if (gr < k && gc < k && gc < gr) gst(md.E + (int64_t)gc * k + gr, T[r][c]);
    }
}

hipError_t launch_gram_to_e(const MatDev* mats, MatFlags* flags, const int* mat_idx, int nmat,
                            int max_t64, int only_regram, hipStream_t st) {
    hipLaunchKernelGGL(gram_to_e_kernel, dim3(max_t64 * (max_t64 + 1) / 2, nmat), dim3(256), 0, st,
                       mats, flags, mat_idx, only_regram);
    return hipGetLastError();
}

__global__ void certify_kernel(const MatDev* __restrict__ mats, MatFlags* __restrict__ flags,
                               const int* __restrict__ mat_idx, int nmat) {
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= nmat) return;
    const int i = mat_idx[t];
    MatFlags& f = flags[i];
    if (!(__uint_as_float(f.check_off) > mats[i].tol_conv)) {
        f.converged = 1;
        f.done = 1;
        f.regram = 0;
    } else {
        f.converged = 0;
        f.done = 0;
        f.check_off = 0u;
        f.regram = 1;
    }
}

__global__ void certify_early_kernel(const MatDev* __restrict__ mats, MatFlags* __restrict__ flags,
                                     const int* __restrict__ mat_idx, int nmat) {
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= nmat) return;
    const int i = mat_idx[t];
    MatFlags& f = flags[i];
    if (!f.early) return;
    f.early = 0;
    if (!(__uint_as_float(f.check_off) > mats[i].tol_conv)) return;
    f.converged = 0;
    f.done = 0;
    f.check_off = 0u;
    f.regram = 1;
}

hipError_t launch_certify_early(const MatDev* mats, MatFlags* flags, const int* mat_idx, int nmat,
                                hipStream_t st) {
    hipLaunchKernelGGL(certify_early_kernel, dim3((nmat + 63) / 64), dim3(64), 0, st, mats, flags,
                       mat_idx, nmat);
    return hipGetLastError();
}

hipError_t launch_certify(const MatDev* mats, MatFlags* flags, const int* mat_idx, int nmat,
                          hipStream_t st) {
    hipLaunchKernelGGL(certify_kernel, dim3((nmat + 63) / 64), dim3(64), 0, st, mats, flags, mat_idx,
                       nmat);
    return hipGetLastError();
}

// Start of the polishing phase (A = M V already recomputed by a GEMM): clear
// the convergence state, count the sweep cap from here, keep the work counters
// of the factor phase apart.  The column order (perm) and the norms it was
// sorted by (cnorm) carry over: the factor's Gram equals A's up to rounding.
__global__ void phase2_reset_kernel(MatFlags* __restrict__ flags, const int* __restrict__ mat_idx,
                                    int nmat) {
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= nmat) return;
    MatFlags& f = flags[mat_idx[t]];
    f.precond = 0;
    f.done = 0;
    f.converged = 0;
    f.sweep_max = 0u;
    f.sweep_base = f.sweeps;
    f.pairs_pre = f.pairs_applied;
    f.quads_pre = f.quads_applied;
    f.check_off = 0u;
    f.sel = 0;
}

hipError_t launch_phase2_reset(const MatDev* mats, MatFlags* flags, const int* mat_idx, int nmat,
                               hipStream_t st) {
    (void)mats;
    hipLaunchKernelGGL(phase2_reset_kernel, dim3((nmat + 63) / 64), dim3(64), 0, st, flags, mat_idx,
                       nmat);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------
// Selective polishing.  A matrix fails the certificate when a few of its column
// pairs are not orthogonal enough; at the workload's spectra these are the
// pairs of a large and a small singular value (an error of the factor phase's
// right vectors is amplified by their ratio in A = M V), all in the blocks of
// the largest columns.  One workgroup per (block I of the column order,
// matrix) reduces the certificate's E over the columns of block I against
// every block J: bmax[I][J] = max |E_ij| (NaN counted as infinity).  The first
// workgroup of a matrix then sets sel, which limits the polishing sweeps to
// the pairs marked above the convergence threshold (pair_selected).
__global__ __launch_bounds__(256) void polish_mark_kernel(const MatDev* __restrict__ mats,
                                                          MatFlags* __restrict__ flags,
                                                          const int* __restrict__ mat_idx) {
    __shared__ int inv[kSelMaxK];
    __shared__ unsigned int bm[kSelMaxK / kJb];
    const int i = mat_idx[blockIdx.y];
    const MatDev& md = mats[i];
    MatFlags& f = flags[i];
    if (f.done || !md.bmax) return;
    const int bI = blockIdx.x, nb = md.nb, k = md.k;
    if (bI >= nb) return;
    for (int j = threadIdx.x; j < md.kpad; j += blockDim.x) inv[gld(md.perm + j)] = j;
    for (int j = threadIdx.x; j < nb; j += blockDim.x) bm[j] = 0u;
    __syncthreads();
    for (int a = 0; a < kJb; ++a) {
        const int pa = gld(md.perm + bI * kJb + a);  // physical row; padding rows are zero
        if (pa >= k) continue;
        const float* e = md.E + (int64_t)pa * k;
        for (int c = threadIdx.x; c < k; c += blockDim.x) {
            const float v = fabsf(gld(e + c));
            const unsigned int u = v == v ? __float_as_uint(v) : 0x7f800000u;
            if (u) atomicMax(&bm[inv[c] / kJb], u);
        }
    }
    __syncthreads();
    for (int j = threadIdx.x; j < nb; j += blockDim.x)
        gst(md.bmax + (int64_t)bI * nb + j, __uint_as_float(bm[j]));
    if (bI == 0 && threadIdx.x == 0) f.sel = 1;
}

hipError_t launch_polish_mark(const MatDev* mats, MatFlags* flags, const int* mat_idx, int nmat,
                              int max_nb, hipStream_t st) {
    hipLaunchKernelGGL(polish_mark_kernel, dim3(max_nb, nmat), dim3(256), 0, st, mats, flags, mat_idx);
    return hipGetLastError();
}

__global__ void polish_full_kernel(MatFlags* __restrict__ flags, const int* __restrict__ mat_idx,
                                   int nmat) {
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= nmat) return;
    MatFlags& f = flags[mat_idx[t]];
    f.sel = 0;
    f.sweep_max = 0u;
}

hipError_t launch_polish_full(MatFlags* flags, const int* mat_idx, int nmat, hipStream_t st) {
    hipLaunchKernelGGL(polish_full_kernel, dim3((nmat + 63) / 64), dim3(64), 0, st, flags, mat_idx,
                       nmat);
    return hipGetLastError();
}

}  // namespace scopt
