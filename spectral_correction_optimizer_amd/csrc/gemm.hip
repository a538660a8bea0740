// Grouped GEMM on the gfx950 bfloat16 matrix cores with float32-level accuracy
// (three-way bfloat16 split of each operand, v_mfma_f32_32x32x16_bf16).
//
// Used for the two-sided projection X = U^T G V and the reconstruction
// G_filt = U X_filt V^T ("Key design 3" of the papernotes.org notes on
// "Communication-Efficient LLM Adaptation over Decentralized GPU Meshes"),
// with diag(d) applied as an output-row / output-column scale or a scale of
// the reduction index, and for the refresh's projector and re-orthogonalization
// products.  C = alpha * op(A) op(B) [* scales] + beta * Cin, float32 accumulate.
//
// Tiling: a 256-thread workgroup computes a 256 x 128 tile; its four waves
// each own 128 x 64 (4 x 2 MFMA blocks of 32 x 32, 128 accumulator registers).
// K advances in steps of 16 through double-buffered LDS holding the split
// operand tiles row-major (k contiguous), so each MFMA operand is one 16-byte
// read per lane.  Workgroup ids are remapped so that each XCD (own L2) works
// on a contiguous range of tiles; tiles are row-major within a problem so
// consecutive tiles share the A panel.
#include <type_traits>

#include "common.hpp"
#include "internal.hpp"

namespace scopt {

namespace {

constexpr int BM = kGemmBM, BN = kGemmBN, BK = 16;
static_assert(BK == 16, "split_chunk16 lays out 16 k per row");

// Loader of an operand tile into registers: thread t holds 8 consecutive k
// values of one tile row (row = m of A or n of B).
//   KMAJOR = false: the operand is stored [rows][K] (A not transposed, B
//     transposed): row = t >> 1, k half = t & 1; two 16-byte loads when VEC
//     (rows 16-byte aligned and K a multiple of 8), else eight element loads.
//   KMAJOR = true: stored [K][rows] (A transposed, B not transposed): row =
//     t & 127, k half = t >> 7, eight element loads, each coalesced over 64
//     consecutive rows.
// Every load is issued (addresses clamped into the operand; rows, kdim >= 1)
// and elements outside it are zeroed when the tile is stored, so loading is
// free of per-lane branches.  FULL: every tile lies inside its operand (rows
// and K multiples of the tile), so nothing is clamped or zeroed.  KS: the
// loader also fetches the k scales of its 8 values when the problem has them.
// the stand-in source of an absent epilogue term (read, never applied)
__device__ const float kEpiOne[1] = {1.0f};

template <bool KMAJOR, bool VEC, bool KS, bool FULL, typename T>
struct TileLoader {
    float v[8], ks[KS ? 8 : 1];
    int row, half, rr, kk;
    __device__ void load(const T* __restrict__ p, int ld, int rows, int kdim, int r0, int k0,
                         const float* kscale, int roff = 0) {
        row = roff + (KMAJOR ? (threadIdx.x & 127) : (threadIdx.x >> 1));
        half = KMAJOR ? (threadIdx.x >> 7) : (threadIdx.x & 1);
        rr = r0 + row;
        kk = k0 + 8 * half;
        const int rc = FULL ? rr : min(rr, rows - 1);
        auto kc = [&](int k) { return FULL ? k : min(k, kdim - 1); };
        if (!KMAJOR && VEC) {
            const T* q = p + (int64_t)rc * ld + (FULL ? kk : min(kk, kdim - 8));
            const float4 a = load4(q), b = load4(q + 4);
            v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
            v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
        } else if (!KMAJOR) {
            const T* q = p + (int64_t)rc * ld;
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = Elem<T>::load(q, kc(kk + j));
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = Elem<T>::load(p, (int64_t)kc(kk + j) * ld + rc);
        }
        if (KS && kscale) {
#pragma unroll
            for (int j = 0; j < 8; ++j) ks[j] = gld(kscale + kc(kk + j));
        }
    }
    // NP = 3: the exact three-way split; NP = 2: hi and mid parts only
    // (|x - hi - mid| <= 2^-16 |x|), for products that are small corrections.
    template <int NR, int NP>
    __device__ void store(__bf16 (*S)[NR * BK], int rows, int kdim, bool scaled) const {
        float f[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float x = (FULL || (rr < rows && kk + j < kdim)) ? v[j] : 0.0f;
            if (KS && scaled) x *= ks[KS ? j : 0];
            f[j] = x;
        }
        const int o = split_chunk16(row, half);
        if constexpr (NP == 3) {
            const Split8 s = split8(f);
            *(v8bf*)&S[0][o] = s.h;
            *(v8bf*)&S[1][o] = s.m;
            *(v8bf*)&S[2][o] = s.l;
        } else {
            v8bf h, m;
            split8_hm(f, h, m);
            *(v8bf*)&S[0][o] = h;
            *(v8bf*)&S[1][o] = m;
        }
    }
};


}  // namespace

// C = alpha op(A) op(B) [scales] + beta Cin with float32 operands and outputs.
// Each operand element is split exactly into three bfloat16 parts and the
// product is formed from the six largest of the nine part products on the
// bfloat16 matrix cores (v_mfma_f32_32x32x16_bf16, float32 accumulation); the
// three dropped ones (mid*lo, lo*mid, lo*lo) are below 2^-23 of |a b|, the
// order of float32 rounding.  This is the bfloat16 splitting of Henry, Tang and
// Heinecke ("Leveraging the bfloat16 artificial intelligence datatype for
// higher-precision computations", 2019); the bfloat16 cores run it 2.7x faster
// than float32 MFMA for the same float32-level result.
// NP = 2 (two parts per operand, the products hi*hi, hi*mid, mid*hi) leaves out
// at most about 3 * 2^-16 |a b| per term: used only for the Loewdin step's E X,
// a correction added to X whose entries |E_ij| are at or below the convergence
// threshold (~1e-6), so the error relative to X stays at or below float32
// rounding.
template <int NP, bool TA, bool TB, bool VEC, bool FULL, typename TEA, typename TEB>
__global__ __launch_bounds__(256, 2) void gemm_grouped_kernel(const GemmProb* __restrict__ probs,
                                                              int nprob, PtrTable ptrs) {
    static_assert(NP == 2 || NP == 3, "two or three bfloat16 parts per operand");
    __shared__ __align__(16) __bf16 As[2][NP][BM * BK];
    __shared__ __align__(16) __bf16 Bs[2][NP][BN * BK];
    static_assert(BM == 256 && BN == 128, "tile shape of the wave layout below");

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

    // A: [M][K] unless transposed; B: [K][N] unless transposed ([N][K]).
    // A's 256 tile rows take two loaders (rows 0-127 and 128-255).
    TileLoader<TA, VEC, false, FULL, TEA> la0, la1;
    TileLoader<!TB, VEC, true, FULL, TEB> lb;
    auto load_tiles = [&](int k0) {
        la0.load(Ap, P.lda, M, K, m0, k0, nullptr, 0);
        la1.load(Ap, P.lda, M, K, m0, k0, nullptr, 128);
        lb.load(Bp, P.ldb, N, K, n0, k0, kscale);
    };
    auto store_tiles = [&](int buf) {
        la0.template store<BM, NP>(As[buf], M, K, false);
        la1.template store<BM, NP>(As[buf], M, K, false);
        lb.template store<BN, NP>(Bs[buf], N, K, kscale != nullptr);
    };

    // waves 2 x 2, each 128 (m) x 64 (n): 4 x 2 MFMA blocks of 32 x 32
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = (wave >> 1) * 128, wn = (wave & 1) * 64;
    const int hl = lane >> 5, ll = lane & 31;
    v16f acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    // fragment of lane (ll, hl): row ll of a 32-row block, k = 8 hl .. 8 hl + 7
    int fa[4], fb[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[i] = split_chunk16(wm + 32 * i + ll, hl);
#pragma unroll
    for (int j = 0; j < 2; ++j) fb[j] = split_chunk16(wn + 32 * j + ll, hl);

    const int nk = (K + BK - 1) / BK;
    if (nk > 0) {
        load_tiles(0);
        store_tiles(0);
        __syncthreads();
    }
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        // the next tile (the last one again in the last step: the loop body stays one
        // block, so the next tile's split can be scheduled between the products)
        const int kn = (kt + 1 < nk ? kt + 1 : kt) * BK;
        load_tiles(kn);
        v8bf a[4][NP], b[2][NP];
#pragma unroll
        for (int p = 0; p < NP; ++p) {
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i][p] = *(const v8bf*)&As[buf][p][fa[i]];
#pragma unroll
            for (int j = 0; j < 2; ++j) b[j][p] = *(const v8bf*)&Bs[buf][p][fb[j]];
        }
        // smallest terms first; consecutive products go to different accumulators
#define SC_TERM(PA, PB)                                                                        \
    _Pragma("unroll") for (int i = 0; i < 4; ++i)                                               \
        _Pragma("unroll") for (int j = 0; j < 2; ++j)                                           \
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i][PA], b[j][PB], acc[i][j], 0, 0, 0);
        if constexpr (NP == 3) {
            SC_TERM(2, 0) SC_TERM(1, 1) SC_TERM(0, 2) SC_TERM(1, 0) SC_TERM(0, 1) SC_TERM(0, 0)
        } else {
            SC_TERM(1, 0) SC_TERM(0, 1) SC_TERM(0, 0)
        }
#undef SC_TERM
        // written to the other buffer, which no wave reads before the barrier
        store_tiles(buf ^ 1);
        // the fragment reads first, then the products interleaved with the next
        // tile's split and stores
        __builtin_amdgcn_sched_group_barrier(0x100, 4 * NP + 2 * NP, 0);
#pragma unroll
        for (int i = 0; i < 8 * NP; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x200, 16, 0);
        __syncthreads();
    }

    // Epilogue.  MFMA 32x32 output layout: lane l, register r ->
    // row 8*(r/4) + 4*(l/32) + r%4, column l%32.  Per 32-row block, every load
    // (row scales, column scales, Cin) is issued before any is used, at clamped
    // (always valid) addresses and without branches: absent terms read one element
    // of kEpiOne and are not applied.  (Per-element branches made each load a
    // separate memory round trip.)
    const float alpha = P.alpha, beta = P.beta;
    const bool zdiag = (P.flags & GF_ZERO_DIAG) != 0;
    const bool has_rs = P.row_scale != nullptr, has_cs = P.col_scale != nullptr, has_cin = P.Cin != nullptr;
    const float* rsp = has_rs ? P.row_scale : kEpiOne;
    const float* csp = has_cs ? P.col_scale : kEpiOne;
    const float* cinp = has_cin ? P.Cin : kEpiOne;
    const int rsm = has_rs ? 1 : 0, csm = has_cs ? 1 : 0, cinm = has_cin ? 1 : 0;
    float cs[2];
    int colc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int col = n0 + wn + 32 * j + ll;
        colc[j] = min(col, N - 1);
        cs[j] = gld(csp + csm * colc[j]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float rs[16];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int col = n0 + wn + 32 * j + ll;
            float cin[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int rowc = min(m0 + wm + 32 * i + 8 * (r >> 2) + 4 * hl + (r & 3), M - 1);
                if (j == 0) rs[r] = gld(rsp + rsm * rowc);
                cin[r] = gld(cinp + cinm * ((int64_t)rowc * P.ldcin + colc[j]));
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm + 32 * i + 8 * (r >> 2) + 4 * hl + (r & 3);
                float v = alpha * acc[i][j][r] * cs[j];
                if (has_rs) v *= rs[r];
                if (zdiag && row == col) v = 0.0f;
                if (has_cin) v += beta * cin[r];
                if (FULL || (row < M && col < N)) gst(P.C + (int64_t)row * P.ldc + col, v);
            }
        }
    }
}

hipError_t launch_gemm(const GemmProb* probs_dev, int nprob, int total_tiles, bool ta, bool tb,
                       bool a_bf16, bool b_bf16, bool vec, bool full, int parts, const PtrTable& ptrs,
                       hipStream_t st) {
    if (nprob <= 0 || total_tiles <= 0) return hipSuccess;
    dim3 grid(total_tiles), blk(256);
    if (ta) vec = false;  // a k-major A has no row loads to vectorize
#define SC_GEMM_CASE_F(NP_, TA_, TB_, V_, F_, EA, EB)                                           \
    if (parts == NP_ && ta == TA_ && tb == TB_ && vec == V_ && full == F_ &&                   \
        a_bf16 == (sizeof(EA) == 2) && b_bf16 == (sizeof(EB) == 2)) {                           \
        hipLaunchKernelGGL((gemm_grouped_kernel<NP_, TA_, TB_, V_, F_, EA, EB>), grid, blk, 0, st, \
                           probs_dev, nprob, ptrs);                                             \
        return hipGetLastError();                                                               \
    }
#define SC_GEMM_CASE_NP(NP_, TA_, TB_, V_, EA, EB) \
    SC_GEMM_CASE_F(NP_, TA_, TB_, V_, false, EA, EB) SC_GEMM_CASE_F(NP_, TA_, TB_, V_, true, EA, EB)
#define SC_GEMM_CASE(TA_, TB_, V_, EA, EB) SC_GEMM_CASE_NP(3, TA_, TB_, V_, EA, EB)
    SC_GEMM_CASE_NP(2, false, false, true, float, float)
    SC_GEMM_CASE_NP(2, false, false, false, float, float)
    SC_GEMM_CASE(false, false, true, float, float)
    SC_GEMM_CASE(false, false, false, float, float)
    SC_GEMM_CASE(false, false, true, uint16_t, float)
    SC_GEMM_CASE(false, false, false, uint16_t, float)
    SC_GEMM_CASE(false, false, true, float, uint16_t)
    SC_GEMM_CASE(false, false, false, float, uint16_t)
    SC_GEMM_CASE(false, true, true, float, float)
    SC_GEMM_CASE(false, true, false, float, float)
    SC_GEMM_CASE(false, true, true, uint16_t, float)
    SC_GEMM_CASE(false, true, false, uint16_t, float)
    SC_GEMM_CASE(true, false, false, float, float)
#undef SC_GEMM_CASE
#undef SC_GEMM_CASE_NP
#undef SC_GEMM_CASE_F
    return hipErrorInvalidValue;
}

}  // namespace scopt
