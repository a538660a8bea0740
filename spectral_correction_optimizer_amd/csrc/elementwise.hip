// Streaming kernels of libscopt: anchor EMA, fused convex combination + AdamW,
// and the small per-row passes of the SVD refresh (operand load, row norms,
// normalization, Tikhonov response).
//
// Method references (papernotes.org notes on "Communication-Efficient LLM
// Adaptation over Decentralized GPU Meshes"): the anchor-momentum EMA of
// "Key design 2"; the Tikhonov response d_i = s_i/(s_i + tau_p) and the convex
// combination G_proj = alpha G_mask + (1 - alpha) G_filt of "Key design 3";
// AdamW from "Overall framework" / "Training strategy".
#include "common.hpp"
#include "internal.hpp"

namespace scopt {

// Workgroup shapes of the two streaming passes.  Both run over 1024-element
// chunks, so a workgroup issues all its loads at once and ends: measured on the
// 112-matrix workload, one float4 per thread and 256 threads moved the EMA at
// 6.5 TB/s and two float4 per thread and 128 threads the AdamW pass at 5.8 TB/s,
// against 5.5 and 5.2 TB/s with 16384-element chunks looped by each workgroup.
constexpr int kEmaThreads = 256;
constexpr int kAdamThreads = 128;

// Matrix of a per-matrix workgroup: entry b of the index list, or b itself.
__device__ __forceinline__ int mat_of(const int* mat_idx, int b) { return mat_idx ? mat_idx[b] : b; }

// ---------------------------------------------------------------------------------
// Anchor EMA:  M <- beta * M + (1 - beta) * G_anc
// One workgroup per chunk; 4 consecutive elements per thread and iteration.
// 12 B/element (10 B with bf16 G_anc).
template <typename GT>
__global__ __launch_bounds__(kEmaThreads) void ema_kernel(const MatDev* __restrict__ mats,
                                                          const Chunk* __restrict__ chunks,
                                                          PtrTable g, float beta,
                                                          int* __restrict__ nonfinite) {
    const Chunk c = chunks[blockIdx.x];
    float* __restrict__ M = mats[c.mat].Manc + c.off;
    const GT* __restrict__ G = (const GT*)g.p[c.mat] + c.off;
    const float omb = 1.0f - beta;
    bool bad = false;
    const int len = c.len;
    const int nvec = len >> 2;
    for (int v = threadIdx.x; v < nvec; v += kEmaThreads) {
        const float4 mv = load4_nt(M + 4 * v);
        const float4 gv = load4_nt(G + 4 * v);
        float4 r;
        r.x = fmaf(beta, mv.x, omb * gv.x);
        r.y = fmaf(beta, mv.y, omb * gv.y);
        r.z = fmaf(beta, mv.z, omb * gv.z);
        r.w = fmaf(beta, mv.w, omb * gv.w);
        bad |= !(isfinite(gv.x) && isfinite(gv.y) && isfinite(gv.z) && isfinite(gv.w));
        store4_nt(M + 4 * v, r);
    }
    for (int i = 4 * nvec + threadIdx.x; i < len; i += kEmaThreads) {
        float gv = Elem<GT>::load(G, i);
        bad |= !isfinite(gv);
        M[i] = fmaf(beta, M[i], omb * gv);
    }
    if (__any(bad) && (threadIdx.x & 63) == 0) atomicOr(nonfinite, 1);
}

hipError_t launch_ema(const MatDev* mats, const Chunk* chunks, int nchunks, const PtrTable& g,
                      bool g_bf16, float beta, int* nonfinite, hipStream_t st) {
    if (nchunks <= 0) return hipSuccess;
    if (g_bf16)
        hipLaunchKernelGGL(ema_kernel<uint16_t>, dim3(nchunks), dim3(kEmaThreads), 0, st, mats,
                           chunks, g, beta, nonfinite);
    else
        hipLaunchKernelGGL(ema_kernel<float>, dim3(nchunks), dim3(kEmaThreads), 0, st, mats,
                           chunks, g, beta, nonfinite);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------
// Convex combination + AdamW, one pass:
//   g = alpha G + (1 - alpha) G_filt
//   m = b1 m + (1 - b1) g;  v = b2 v + (1 - b2) g^2
//   W = W - (lr wd) W - (lr / bc1) m / (sqrt(v) / sqrt(bc2) + eps)
// Host passes step_size = lr / bc1, inv_sqrt_bc2 = 1 / sqrt(bc2), lr_wd = lr * wd
// (computed in double).  Reads G, G_filt, W, m, v; writes W, m, v (and G_proj
// when kept): 32 B/element for float32 W and G.
struct AdamScalars {
    float alpha, oma, b1, omb1, b2, omb2, eps, step_size, inv_sqrt_bc2, lr_wd;
};

__device__ __forceinline__ float adam_elem(float G, float Gf, float& m, float& v, float w,
                                           const AdamScalars& a, float& gp) {
    float g = fmaf(a.alpha, G, a.oma * Gf);
    gp = g;
    m = fmaf(a.b1, m, a.omb1 * g);
    v = fmaf(a.b2, v, a.omb2 * (g * g));
    float denom = fmaf(sqrtf(v), a.inv_sqrt_bc2, a.eps);
    // Form the whole update first (|u| << ulp(w), so its own rounding is
    // negligible) and round at w's scale once: W - (lr wd W + step m / denom).
    // Rounding w - lr wd w separately would add a second w-scale rounding per
    // step and let the stored weights drift from the exactly rounded values.
    float u = fmaf(a.lr_wd, w, a.step_size * (m / denom));
    return w - u;
}

template <typename WT>
__device__ __forceinline__ void store_w4(WT* p, float4 w);
template <>
__device__ __forceinline__ void store_w4<float>(float* p, float4 w) {
    gst4(p, v4f{w.x, w.y, w.z, w.w});
}
template <>
__device__ __forceinline__ void store_w4<uint16_t>(uint16_t* p, float4 w) {
    uint2 u;
    u.x = (uint32_t)f32_to_bf16(w.x) | ((uint32_t)f32_to_bf16(w.y) << 16);
    u.y = (uint32_t)f32_to_bf16(w.z) | ((uint32_t)f32_to_bf16(w.w) << 16);
    *(uint2*)p = u;
}
template <typename WT>
__device__ __forceinline__ void store_w1(WT* p, float w);
template <>
__device__ __forceinline__ void store_w1<float>(float* p, float w) {
    *p = w;
}
template <>
__device__ __forceinline__ void store_w1<uint16_t>(uint16_t* p, float w) {
    *p = f32_to_bf16(w);
}

template <typename WT, typename GT>
__global__ __launch_bounds__(kAdamThreads) void combine_adamw_kernel(
    const MatDev* __restrict__ mats, const Chunk* __restrict__ chunks, PtrTable wt, PtrTable gt,
    AdamScalars a, int keep_proj, int* __restrict__ nonfinite) {
    const Chunk c = chunks[blockIdx.x];
    const MatDev& md = mats[c.mat];
    WT* __restrict__ W = (WT*)wt.p[c.mat] + c.off;
    const GT* __restrict__ G = (const GT*)gt.p[c.mat] + c.off;
    const float* __restrict__ Gf = md.Gfilt + c.off;
    float* __restrict__ Mm = md.madam + c.off;
    float* __restrict__ Vv = md.vadam + c.off;
    float* __restrict__ Gp = keep_proj ? md.Gproj + c.off : nullptr;
    bool bad = false;
    const int len = c.len;
    const int nvec = len >> 2;
    for (int v0 = threadIdx.x; v0 < nvec; v0 += 2 * kAdamThreads) {
        float4 gv[2], fv[2], wv[2], mv[2], vv[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            int v = v0 + u * kAdamThreads;
            if (v < nvec) {
                gv[u] = load4_nt(G + 4 * v);
                fv[u] = load4_nt(Gf + 4 * v);
                wv[u] = load4_nt(W + 4 * v);
                mv[u] = load4_nt(Mm + 4 * v);
                vv[u] = load4_nt(Vv + 4 * v);
            }
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            int v = v0 + u * kAdamThreads;
            if (v < nvec) {
                float4 w, p;
                w.x = adam_elem(gv[u].x, fv[u].x, mv[u].x, vv[u].x, wv[u].x, a, p.x);
                w.y = adam_elem(gv[u].y, fv[u].y, mv[u].y, vv[u].y, wv[u].y, a, p.y);
                w.z = adam_elem(gv[u].z, fv[u].z, mv[u].z, vv[u].z, wv[u].z, a, p.z);
                w.w = adam_elem(gv[u].w, fv[u].w, mv[u].w, vv[u].w, wv[u].w, a, p.w);
                bad |= !(isfinite(gv[u].x) && isfinite(gv[u].y) && isfinite(gv[u].z) &&
                         isfinite(gv[u].w));
                store4_nt(W + 4 * v, w);
                store4_nt(Mm + 4 * v, mv[u]);
                store4_nt(Vv + 4 * v, vv[u]);
                if (Gp) store4_nt(Gp + 4 * v, p);
            }
        }
    }
    for (int i = 4 * nvec + threadIdx.x; i < len; i += kAdamThreads) {
        float G1 = Elem<GT>::load(G, i);
        float m = Mm[i], v = Vv[i], p;
        float w = adam_elem(G1, Gf[i], m, v, Elem<WT>::load(W, i), a, p);
        bad |= !isfinite(G1);
        store_w1<WT>(W + i, w);
        Mm[i] = m;
        Vv[i] = v;
        if (Gp) Gp[i] = p;
    }
    if (__any(bad) && (threadIdx.x & 63) == 0) atomicOr(nonfinite, 1);
}

hipError_t launch_combine_adamw(const MatDev* mats, const Chunk* chunks, int nchunks,
                                const PtrTable& w, const PtrTable& g, bool w_bf16, bool g_bf16,
                                float alpha, float beta1, float beta2, float eps, float step_size,
                                float inv_sqrt_bc2, float lr_wd, int keep_proj, int* nonfinite,
                                hipStream_t st) {
    if (nchunks <= 0) return hipSuccess;
    AdamScalars a{alpha, 1.0f - alpha, beta1, 1.0f - beta1, beta2, 1.0f - beta2,
                  eps,   step_size,    inv_sqrt_bc2, lr_wd};
    dim3 grid(nchunks), blk(kAdamThreads);
    if (!w_bf16 && !g_bf16)
        hipLaunchKernelGGL((combine_adamw_kernel<float, float>), grid, blk, 0, st, mats, chunks, w,
                           g, a, keep_proj, nonfinite);
    else if (w_bf16 && g_bf16)
        hipLaunchKernelGGL((combine_adamw_kernel<uint16_t, uint16_t>), grid, blk, 0, st, mats,
                           chunks, w, g, a, keep_proj, nonfinite);
    else if (w_bf16)
        hipLaunchKernelGGL((combine_adamw_kernel<uint16_t, float>), grid, blk, 0, st, mats, chunks,
                           w, g, a, keep_proj, nonfinite);
    else
        hipLaunchKernelGGL((combine_adamw_kernel<float, uint16_t>), grid, blk, 0, st, mats,
                           chunks, w, g, a, keep_proj, nonfinite);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------
// Jacobi operand load.  A holds the columns of the Jacobi operand as rows:
//   m >= n:  A = M,   A_rows[j][x] = M[x][j]   (transpose, 32x32 LDS tiles)
//   m <  n:  A = M^T, A_rows[j][x] = M[j][x]   (copy)
// zero beyond k rows / K columns; V <- identity (kpad x kpad).
__global__ __launch_bounds__(256) void jacobi_load_kernel(const MatDev* __restrict__ mats,
                                                          const int* __restrict__ mat_idx) {
    __shared__ float tile[32][33];
    const MatDev& md = mats[mat_of(mat_idx, blockIdx.y)];
    const int tj = md.kpad / 32, tx = md.K_ld / 32;
    const int ntA = tj * tx;
    const int ntV = (md.kpad / 32) * (md.kpad / 32);
    const int lx = threadIdx.x & 31, ly = threadIdx.x >> 5;  // 32 x 8
    for (int t = blockIdx.x; t < ntA + ntV; t += gridDim.x) {
        if (t < ntA) {
            const int j0 = (t / tx) * 32, x0 = (t % tx) * 32;
            if (md.tall) {
                // read M[x0 + r][j0 + lx] (coalesced in j), write A[j0 + r][x0 + lx]
#pragma unroll
                for (int r = ly; r < 32; r += 8) {
                    int x = x0 + r, j = j0 + lx;
                    tile[r][lx] = (x < md.m && j < md.n) ? md.Manc[(int64_t)x * md.n + j] : 0.0f;
                }
                __syncthreads();
#pragma unroll
                for (int r = ly; r < 32; r += 8)
                    md.A[(int64_t)(j0 + r) * md.K_ld + x0 + lx] = tile[lx][r];
                __syncthreads();
            } else {
#pragma unroll
                for (int r = ly; r < 32; r += 8) {
                    int j = j0 + r, x = x0 + lx;
                    md.A[(int64_t)j * md.K_ld + x] =
                        (j < md.m && x < md.n) ? md.Manc[(int64_t)j * md.n + x] : 0.0f;
                }
            }
        } else {
            const int tv = t - ntA, nv = md.kpad / 32;
            const int j0 = (tv / nv) * 32, x0 = (tv % nv) * 32;
#pragma unroll
            for (int r = ly; r < 32; r += 8)
                md.V[(int64_t)(j0 + r) * md.kpad + x0 + lx] = (j0 + r == x0 + lx) ? 1.0f : 0.0f;
        }
    }
}

hipError_t launch_jacobi_load(const MatDev* mats, const int* mat_idx, int nmat, int max_kpad,
                              int max_K, hipStream_t st) {
    int tiles = (max_kpad / 32) * ((max_K + 31) / 32) + (max_kpad / 32) * (max_kpad / 32);
    int gx = tiles < 2048 ? tiles : 2048;
    if (gx < 1) gx = 1;
    hipLaunchKernelGGL(jacobi_load_kernel, dim3(gx, nmat), dim3(256), 0, st, mats, mat_idx);
    return hipGetLastError();
}

// Warm start of a refresh from the previous factors: V <- [W 0; 0 I] (rows of
// the previous accumulated-side singular vectors) and zero padding rows of A
// (the rows j < k of A are then written by the GEMM A_rows = W op(M)).
__global__ __launch_bounds__(256) void jacobi_warm_kernel(const MatDev* __restrict__ mats,
                                                          const int* __restrict__ mat_idx) {
    const MatDev& md = mats[mat_of(mat_idx, blockIdx.y)];
    const int64_t nv = (int64_t)md.kpad * md.kpad;
    const int64_t na = (int64_t)(md.kpad - md.k) * md.K_ld;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nv + na;
         i += (int64_t)gridDim.x * blockDim.x) {
        if (i < nv) {
            const int j = (int)(i / md.kpad), x = (int)(i % md.kpad);
            md.V[i] = (j < md.k && x < md.k) ? md.W[(int64_t)j * md.k + x] : (j == x ? 1.0f : 0.0f);
        } else {
            md.A[(int64_t)md.k * md.K_ld + (i - nv)] = 0.0f;
        }
    }
}

hipError_t launch_jacobi_warm(const MatDev* mats, const int* mat_idx, int nmat, hipStream_t st) {
    hipLaunchKernelGGL(jacobi_warm_kernel, dim3(512, nmat), dim3(256), 0, st, mats, mat_idx);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------
// Row norms in float64 with a fixed reduction order (deterministic).
// which = 0: rows j < kpad of A (length K_ld); 1: rows j < k of V (length k).
__global__ __launch_bounds__(256) void rownorm_kernel(const MatDev* __restrict__ mats,
                                                      const int* __restrict__ mat_idx, int which) {
    __shared__ double red[4];
    const MatDev& md = mats[mat_of(mat_idx, blockIdx.y)];
    const int j = blockIdx.x;
    const int rows = which == 0 ? md.kpad : md.k;
    if (j >= rows) return;
    const float* x = which == 0 ? md.A + (int64_t)j * md.K_ld : md.V + (int64_t)j * md.kpad;
    const int len = which == 0 ? md.K_ld : md.k;
    double acc = 0.0;
    for (int i = threadIdx.x; i < len; i += blockDim.x) {
        double v = x[i];
        acc += v * v;
    }
    acc = block_sum_f64(acc, red);
    if (threadIdx.x == 0) md.norm2[j] = acc;
}

hipError_t launch_rownorm(const MatDev* mats, const int* mat_idx, int nmat, int which, int max_kpad,
                          hipStream_t st) {
    hipLaunchKernelGGL(rownorm_kernel, dim3(max_kpad, nmat), dim3(256), 0, st, mats, mat_idx, which);
    return hipGetLastError();
}

// floor2 = (2^-24 ||M||_F)^2: a column of A whose squared norm stays below it
// is indistinguishable from float32 rounding noise of M and is treated as zero.
__global__ __launch_bounds__(256) void init_flags_kernel(const MatDev* __restrict__ mats,
                                                         const int* __restrict__ mat_idx,
                                                         MatFlags* __restrict__ flags) {
    __shared__ double red[4];
    const int mi = mat_of(mat_idx, blockIdx.x);
    const MatDev& md = mats[mi];
    double acc = 0.0;
    for (int j = threadIdx.x; j < md.kpad; j += blockDim.x) acc += md.norm2[j];
    acc = block_sum_f64(acc, red);
    if (threadIdx.x == 0) {
        MatFlags& f = flags[mi];
        const double e = 5.9604644775390625e-08;  // 2^-24
        f.floor2 = (float)(acc * e * e);
        f.sweep_max = 0u;
        f.converged = 0;
        f.sweeps = 0;
        f.done = 0;
        f.pairs_applied = 0;
        f.sweep_base = 0;
        f.precond = 0;
        f.chol_fail = 0;
        f.pairs_pre = 0;
        f.check_off = 0u;
        f.regram = 0;
        f.sel = 0;
        f.sel_pairs = 0;
        f.sel_rot = 0;
        f.sel_sweeps = 0;
        f.early = 0;
        f.quads_applied = 0;
        f.quads_pre = 0;
    }
    // identity column order; column norms for the first sweep's ordering
    for (int j = threadIdx.x; j < md.kpad; j += blockDim.x) {
        md.perm[j] = j;
        md.cnorm[j] = (float)md.norm2[j];
    }
}

hipError_t launch_jacobi_init_flags(const MatDev* mats, const int* mat_idx, MatFlags* flags,
                                    int nmat, hipStream_t st) {
    hipLaunchKernelGGL(init_flags_kernel, dim3(nmat), dim3(256), 0, st, mats, mat_idx, flags);
    return hipGetLastError();
}

// which = 0: rows of A -> unit rows in place, s_j = ||row||; rows at or below
// the floor (and padding rows) become zero with s_j = 0.
// which = 1: rows j < k of V -> unit rows in place (first k entries).
__global__ __launch_bounds__(256) void normalize_kernel(const MatDev* __restrict__ mats,
                                                        const int* __restrict__ mat_idx,
                                                        const MatFlags* __restrict__ flags,
                                                        int which) {
    const int mi = mat_of(mat_idx, blockIdx.y);
    const MatDev& md = mats[mi];
    const int j = blockIdx.x;
    if (which == 0) {
        if (j >= md.kpad) return;
        const double n2 = md.norm2[j];
        const bool keep = j < md.k && n2 > (double)flags[mi].floor2;
        const float sv = keep ? (float)sqrt(n2) : 0.0f;
        float* x = md.A + (int64_t)j * md.K_ld;
        for (int i = threadIdx.x; i < md.K_ld; i += blockDim.x) x[i] = keep ? x[i] / sv : 0.0f;
        if (threadIdx.x == 0) md.s[j] = sv;
    } else {
        // Rows of V drift from unit norm by rounding; A = M V holds for the
        // unnormalized V, so s_j = ||a_j|| / ||v_j|| is the value for unit v_j.
        if (j >= md.k) return;
        const double n2 = md.norm2[j];
        const float nv = (float)sqrt(n2);
        float* x = md.V + (int64_t)j * md.kpad;
        for (int i = threadIdx.x; i < md.k; i += blockDim.x) x[i] = nv > 0.0f ? x[i] / nv : 0.0f;
        if (threadIdx.x == 0 && n2 > 0.0) md.s[j] = (float)((double)md.s[j] / sqrt(n2));
    }
}

hipError_t launch_normalize(const MatDev* mats, const int* mat_idx, const MatFlags* flags,
                            int nmat, int which, int max_kpad, hipStream_t st) {
    hipLaunchKernelGGL(normalize_kernel, dim3(max_kpad, nmat), dim3(256), 0, st, mats, mat_idx,
                       flags, which);
    return hipGetLastError();
}

// d_j = s_j / (s_j + tau), and 0 where s_j + tau = 0.
__global__ __launch_bounds__(256) void filter_kernel(const MatDev* __restrict__ mats,
                                                     const int* __restrict__ mat_idx, float tau) {
    const MatDev& md = mats[mat_of(mat_idx, blockIdx.x)];
    for (int j = threadIdx.x; j < md.kpad; j += blockDim.x) {
        float s = md.s[j];
        float den = s + tau;
        md.d[j] = den != 0.0f ? s / den : 0.0f;
    }
}

hipError_t launch_filter(const MatDev* mats, const int* mat_idx, int nmat, float tau,
                         hipStream_t st) {
    hipLaunchKernelGGL(filter_kernel, dim3(nmat), dim3(256), 0, st, mats, mat_idx, tau);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------
// Plain 2-D transpose through a 32x32 LDS tile (factor import / export).
__global__ __launch_bounds__(256) void transpose_kernel(const float* __restrict__ src, int rows,
                                                        int cols, int ld_src,
                                                        float* __restrict__ dst, int ld_dst) {
    __shared__ float tile[32][33];
    const int r0 = blockIdx.y * 32, c0 = blockIdx.x * 32;
    const int lx = threadIdx.x & 31, ly = threadIdx.x >> 5;
    for (int r = ly; r < 32; r += 8) {
        const int rr = r0 + r, cc = c0 + lx;
        tile[r][lx] = (rr < rows && cc < cols) ? src[(int64_t)rr * ld_src + cc] : 0.0f;
    }
    __syncthreads();
    for (int r = ly; r < 32; r += 8) {
        const int cc = c0 + r, rr = r0 + lx;
        if (cc < cols && rr < rows) dst[(int64_t)cc * ld_dst + rr] = tile[lx][r];
    }
}

hipError_t launch_transpose(const float* src, int rows, int cols, int ld_src, float* dst,
                            int ld_dst, hipStream_t st) {
    dim3 grid((cols + 31) / 32, (rows + 31) / 32);
    hipLaunchKernelGGL(transpose_kernel, grid, dim3(256), 0, st, src, rows, cols, ld_src, dst,
                       ld_dst);
    return hipGetLastError();
}

}  // namespace scopt
