// Grouped GEMM on the gfx950 float32 matrix cores (v_mfma_f32_32x32x2_f32).
//
// Used for the two-sided projection X = U^T G V and the reconstruction
// G_filt = U X_filt V^T ("Key design 3" of the papernotes.org notes on
// "Communication-Efficient LLM Adaptation over Decentralized GPU Meshes"),
// with diag(d) applied as an output-row / output-column scale or a scale of
// the reduction index, and for the refresh's projector and re-orthogonalization
// products.  C = alpha * op(A) op(B) [* scales] + beta * Cin, float32 accumulate.
//
// Tiling: a 256-thread workgroup computes a 128 x 128 tile; its four waves
// each own 64 x 64 (2 x 2 MFMA blocks of 32 x 32, 64 accumulator registers).
// K advances in steps of 16 through double-buffered LDS; operand tiles are
// stored k-major in LDS so each MFMA operand is one conflict-free 32-float
// row segment per half-wave.  Workgroup ids are remapped so that each XCD
// (own L2) works on a contiguous range of tiles; tiles are row-major within a
// problem so consecutive tiles share the A panel.
#include <type_traits>

#include "common.hpp"
#include "internal.hpp"

namespace scopt {

namespace {

constexpr int BM = 128, BN = 128, BK = 16;
constexpr int LDS_STRIDE = 128 + 32;  // rows k and k+1 land on disjoint bank halves

template <bool TRANS, typename T>
struct TileLoader;

// A operand, not transposed: A[M][K] row-major, tile 128(m) x 16(k).
// Slot s in [0, 512): row = s >> 2, k4 = s & 3.
// B operand, transposed: B[N][K]; identical pattern with n in place of m.
template <typename T>
struct TileLoader<false, T> {
    float4 r[2];
    __device__ void load(const T* __restrict__ p, int ld, int rows, int kdim, int r0, int k0,
                         bool vec_ok, const float* kscale) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            int s = threadIdx.x + e * 256;
            int row = r0 + (s >> 2), kk = k0 + 4 * (s & 3);
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (row < rows) {
                const T* q = p + (int64_t)row * ld + kk;
                if (vec_ok && kk + 3 < kdim) {
                    v = load4(q);
                } else {
                    if (kk + 0 < kdim) v.x = Elem<T>::load(q, 0);
                    if (kk + 1 < kdim) v.y = Elem<T>::load(q, 1);
                    if (kk + 2 < kdim) v.z = Elem<T>::load(q, 2);
                    if (kk + 3 < kdim) v.w = Elem<T>::load(q, 3);
                }
            }
            (void)kscale;
            r[e] = v;
        }
    }
    __device__ void store(float (*S)[LDS_STRIDE]) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            int s = threadIdx.x + e * 256;
            int row = s >> 2, kq = 4 * (s & 3);
            S[kq + 0][row] = r[e].x;
            S[kq + 1][row] = r[e].y;
            S[kq + 2][row] = r[e].z;
            S[kq + 3][row] = r[e].w;
        }
    }
};

// A operand transposed (stored [K][M]) or B not transposed (B[K][N]):
// tile 16(k) x 128(m or n). Slot s: k = s >> 5, c4 = s & 31.
template <typename T>
struct TileLoader<true, T> {
    float4 r[2];
    __device__ void load(const T* __restrict__ p, int ld, int cols, int kdim, int c0, int k0,
                         bool vec_ok, const float* kscale) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            int s = threadIdx.x + e * 256;
            int kk = k0 + (s >> 5), c = c0 + 4 * (s & 31);
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (kk < kdim) {
                const T* q = p + (int64_t)kk * ld + c;
                if (vec_ok && c + 3 < cols) {
                    v = load4(q);
                } else {
                    if (c + 0 < cols) v.x = Elem<T>::load(q, 0);
                    if (c + 1 < cols) v.y = Elem<T>::load(q, 1);
                    if (c + 2 < cols) v.z = Elem<T>::load(q, 2);
                    if (c + 3 < cols) v.w = Elem<T>::load(q, 3);
                }
                if (kscale) {
                    float f = gld(kscale + kk);
                    v.x *= f;
                    v.y *= f;
                    v.z *= f;
                    v.w *= f;
                }
            }
            r[e] = v;
        }
    }
    __device__ void store(float (*S)[LDS_STRIDE]) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            int s = threadIdx.x + e * 256;
            *(float4*)&S[s >> 5][4 * (s & 31)] = r[e];
        }
    }
};

// Transposed-B loader with a k-scale: the non-transposed-A pattern (rows = n)
// but each of the 4 k values gets its own factor.
template <typename T>
struct TileLoaderRowsK : TileLoader<false, T> {
    __device__ void load(const T* __restrict__ p, int ld, int rows, int kdim, int r0, int k0,
                         bool vec_ok, const float* kscale) {
        TileLoader<false, T>::load(p, ld, rows, kdim, r0, k0, vec_ok, nullptr);
        if (kscale) {
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                int s = threadIdx.x + e * 256;
                int kk = k0 + 4 * (s & 3);
                float4& v = this->r[e];
                if (kk + 0 < kdim) v.x *= gld(kscale + kk + 0);
                if (kk + 1 < kdim) v.y *= gld(kscale + kk + 1);
                if (kk + 2 < kdim) v.z *= gld(kscale + kk + 2);
                if (kk + 3 < kdim) v.w *= gld(kscale + kk + 3);
            }
        }
    }
};

__device__ __forceinline__ bool aligned16(const void* p, int elem_bytes) {
    return ((uintptr_t)p & (uintptr_t)(4 * elem_bytes - 1)) == 0;
}

}  // namespace

template <bool TA, bool TB, typename TEA, typename TEB>
__global__ __launch_bounds__(256, 2) void gemm_grouped_kernel(const GemmProb* __restrict__ probs,
                                                              int nprob, PtrTable ptrs) {
    __shared__ float As[2][BK][LDS_STRIDE];
    __shared__ float Bs[2][BK][LDS_STRIDE];

    const int wg = xcd_remap(blockIdx.x, gridDim.x);
    int lo = 0, hi = nprob - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (probs[mid].tile_start <= wg) lo = mid;
        else hi = mid - 1;
    }
    const GemmProb& P = probs[lo];
    if (P.gate && *P.gate == 0) return;
    const int local = wg - P.tile_start;
    const int m0 = (local / P.tiles_n) * BM, n0 = (local % P.tiles_n) * BN;
    const int M = P.M, N = P.N, K = P.K;
    const TEA* __restrict__ Ap = (const TEA*)(P.a_ptr >= 0 ? ptrs.p[P.a_ptr] : P.A);
    const TEB* __restrict__ Bp = (const TEB*)(P.b_ptr >= 0 ? ptrs.p[P.b_ptr] : P.B);
    const float* kscale = P.k_scale;
    const bool va = (P.lda % 4 == 0) && aligned16(Ap, sizeof(TEA));
    const bool vb = (P.ldb % 4 == 0) && aligned16(Bp, sizeof(TEB));

    TileLoader<TA, TEA> la;
    // B: not transposed -> [K][N] k-rows (the "true" pattern); transposed -> [N][K].
    typename std::conditional<TB, TileLoaderRowsK<TEB>, TileLoader<true, TEB> >::type lb;

    auto load_tiles = [&](int k0) {
        la.load(Ap, P.lda, M, K, m0, k0, va, nullptr);
        lb.load(Bp, P.ldb, N, K, n0, k0, vb, kscale);
    };

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
    v16f acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int nk = (K + BK - 1) / BK;
    load_tiles(0);
    la.store(As[0]);
    lb.store(Bs[0]);
    __syncthreads();
    const int hl = lane >> 5, ll = lane & 31;
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) load_tiles((kt + 1) * BK);
#pragma unroll
        for (int kk = 0; kk < BK; kk += 2) {
            float a0 = As[buf][kk + hl][wm + ll];
            float a1 = As[buf][kk + hl][wm + 32 + ll];
            float b0 = Bs[buf][kk + hl][wn + ll];
            float b1 = Bs[buf][kk + hl][wn + 32 + ll];
            acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b0, acc[0][0], 0, 0, 0);
            acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b1, acc[0][1], 0, 0, 0);
            acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b0, acc[1][0], 0, 0, 0);
            acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b1, acc[1][1], 0, 0, 0);
        }
        if (kt + 1 < nk) {
            la.store(As[buf ^ 1]);
            lb.store(Bs[buf ^ 1]);
        }
        __syncthreads();
    }

    // Epilogue.  MFMA 32x32 output layout: lane l, register r ->
    // row 8*(r/4) + 4*(l/32) + r%4, column l%32.
    const float alpha = P.alpha, beta = P.beta;
    const bool zdiag = (P.flags & GF_ZERO_DIAG) != 0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int col = n0 + wn + 32 * j + ll;
            if (col >= N) continue;
            const float cs = P.col_scale ? gld(P.col_scale + col) : 1.0f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm + 32 * i + 8 * (r >> 2) + 4 * hl + (r & 3);
                if (row >= M) continue;
                float v = alpha * acc[i][j][r] * cs;
                if (P.row_scale) v *= gld(P.row_scale + row);
                if (zdiag && row == col) v = 0.0f;
                if (P.Cin) v += beta * gld(P.Cin + (int64_t)row * P.ldcin + col);
                gst(P.C + (int64_t)row * P.ldc + col, v);
            }
        }
    }
}

hipError_t launch_gemm(const GemmProb* probs_dev, int nprob, int total_tiles, bool ta, bool tb,
                       bool a_bf16, bool b_bf16, const PtrTable& ptrs, hipStream_t st) {
    if (nprob <= 0 || total_tiles <= 0) return hipSuccess;
    dim3 grid(total_tiles), blk(256);
#define SC_GEMM_CASE(TA_, TB_, EA, EB)                                                         \
    if (ta == TA_ && tb == TB_ && a_bf16 == (sizeof(EA) == 2) && b_bf16 == (sizeof(EB) == 2)) { \
        hipLaunchKernelGGL((gemm_grouped_kernel<TA_, TB_, EA, EB>), grid, blk, 0, st, probs_dev, \
                           nprob, ptrs);                                                       \
        return hipGetLastError();                                                              \
    }
    SC_GEMM_CASE(false, false, float, float)
    SC_GEMM_CASE(false, false, uint16_t, float)
    SC_GEMM_CASE(false, false, float, uint16_t)
    SC_GEMM_CASE(false, true, float, float)
    SC_GEMM_CASE(false, true, uint16_t, float)
    SC_GEMM_CASE(true, false, float, float)
#undef SC_GEMM_CASE
    return hipErrorInvalidValue;
}

}  // namespace scopt
