// In-graph activation mask on gfx950 ("Key design 1" of the papernotes.org
// notes on "Communication-Efficient LLM Adaptation over Decentralized GPU
// Meshes"): at a pipeline boundary every token keeps K of its H hidden
// dimensions, chosen by a pseudo-random function of (layer, step, batch) that
// sender and receiver evaluate locally, so only the K kept values travel; the
// gradient goes back through the same index set.
//
// The kept set of token i is the K dimensions j with the smallest 64-bit hash
// u = mix64(seed + (i H + j + 1) gamma) (ties to the smaller j), listed in
// ascending order; mix64 is the SplitMix64 output function (Steele, Lea and
// Flood, OOPSLA 2014), gamma its golden-ratio increment.
//
//   mask_indices  one wavefront per token (mask_indices_wave_kernel): the
//                 hashes below a threshold that admits between K and `cap` of
//                 them, collected in dimension order; a register bitonic sort
//                 of their hashes gives the K-th smallest, and the candidates up
//                 to it are the kept set, already in ascending order.  For
//                 parameters where `cap` would be large or K not well below H,
//                 one workgroup per token sorts all H (mask_indices_kernel).
//                 Integer work, ALU bound.
//   mask_pack     kept values of each token, in index order (a gather; bound by
//                 HBM sectors touched)
//   mask_unpack   dense rows with zeros elsewhere (an LDS row per token, then
//                 16-byte streaming row writes; HBM bound)
#include <cmath>

#include "common.hpp"
#include "internal.hpp"

namespace scopt {

namespace {
constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

// ascending bitonic sort of n (a power of two, <= 2 * blockDim.x * iterations)
// entries of (key, val) in LDS, by key then val
template <typename K, typename V>
__device__ void bitonic_sort(K* key, V* val, int n) {
    for (int size = 2; size <= n; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int t = threadIdx.x; t < n / 2; t += blockDim.x) {
                const int lo = 2 * t - (t & (stride - 1));
                const int hi = lo + stride;
                const bool up = (lo & size) == 0;  // this run ascends
                const K ka = key[lo], kb = key[hi];
                const V va = val[lo], vb = val[hi];
                const bool a_first = ka < kb || (ka == kb && va < vb);
                if (a_first != up) {
                    key[lo] = kb;
                    key[hi] = ka;
                    val[lo] = vb;
                    val[hi] = va;
                }
            }
            __syncthreads();
        }
    }
}
}  // namespace

// The K smallest of H uniform 64-bit hashes lie, almost surely, below a
// threshold t0 at which w = K + 5 sqrt(K) + 16 of the H values are expected
// (the count below t0 is binomial, standard deviation under sqrt(w)): the
// workgroup collects the hashes below t0 (order of collection immaterial),
// sorts those candidates instead of all H, and keeps the first K.  Exact
// whenever at least K and at most `cap` values fall below t0 (every value left
// out is then larger than every kept one), cap the power of two at or above
// w + 6 sqrt(w); otherwise (about once in 10^7 tokens), or when cap would
// exceed kCand or w is not well below H, all H are sorted.
namespace {
constexpr int kCand = 512;
}

__global__ __launch_bounds__(256) void mask_indices_kernel(uint64_t seed, int64_t T, int H, int K,
                                                           int32_t* __restrict__ idx) {
    __shared__ uint64_t key[kMaskMaxH];
    __shared__ int32_t dim[kMaskMaxH];
    __shared__ int ncand;
    int hp = 1;
    while (hp < H) hp <<= 1;
    const double want = K + 5.0 * sqrt((double)K) + 16.0;  // expected candidates below t0
    int cap = 1;
    while (cap < want + 6.0 * sqrt(want)) cap <<= 1;
    const bool fast = cap <= kCand && want < 0.5 * H;
    const uint64_t t0 = fast ? (uint64_t)(want / H * 18446744073709551616.0) : ~0ull;
    for (int64_t row = blockIdx.x; row < T; row += gridDim.x) {
        const uint64_t base = (uint64_t)row * (uint64_t)H + 1ull;
        int n = hp;
        bool done = false;
        if (fast) {
            if (threadIdx.x == 0) ncand = 0;
            __syncthreads();
            for (int j = threadIdx.x; j < H; j += blockDim.x) {
                const uint64_t u = mix64(seed + (base + (uint64_t)j) * kGamma);
                if (u < t0) {
                    const int slot = atomicAdd(&ncand, 1);
                    if (slot < cap) {
                        key[slot] = u;
                        dim[slot] = j;
                    }
                }
            }
            __syncthreads();
            const int c = ncand;
            if (c >= K && c <= cap) {
                for (int j = c + threadIdx.x; j < cap; j += blockDim.x) {
                    key[j] = ~0ull;
                    dim[j] = 0x7fffffff;
                }
                __syncthreads();
                n = cap;
                done = true;
            }
            __syncthreads();  // every thread has read ncand before it is reset
        }
        if (!done) {
            for (int j = threadIdx.x; j < hp; j += blockDim.x) {
                key[j] = j < H ? mix64(seed + (base + (uint64_t)j) * kGamma) : ~0ull;
                dim[j] = j < H ? j : 0x7fffffff;
            }
            __syncthreads();
            n = hp;
        }
        bitonic_sort(key, dim, n);
        // the first K dimensions, sorted ascending (keys reused as 64-bit values)
        int kp = 1;
        while (kp < K) kp <<= 1;
        for (int j = threadIdx.x; j < kp; j += blockDim.x) key[j] = j < K ? (uint64_t)dim[j] : ~0ull;
        __syncthreads();
        if (K > 1) bitonic_sort(key, dim, kp);
        int32_t* out = idx + row * K;
        for (int j = threadIdx.x; j < K; j += blockDim.x) gst(out + j, (int32_t)key[j]);
        __syncthreads();
    }
}

// One wavefront per token (64-thread workgroups, so __syncthreads orders the
// wave's LDS accesses).  The hashes of a token are distinct (mix64 is a
// bijection and the inputs seed + (i H + j + 1) gamma differ for distinct j,
// gamma odd), so the number of them below t grows by one at each hash: starting
// from t0, bisection on t finds a threshold with K <= count <= CAP (almost
// always t0 itself).  Those candidates are collected in dimension order (ballot
// compaction), their hashes sorted in registers (R = CAP / 64 per lane, bitonic;
// lanes exchange through shuffles), and every candidate whose hash is at most
// the K-th smallest is kept: exactly K, in ascending dimension order.
template <int R>
__global__ __launch_bounds__(64) void mask_indices_wave_kernel(uint64_t seed, int64_t T, int H, int K,
                                                              uint64_t t0, int32_t* __restrict__ idx) {
    constexpr int CAP = 64 * R;
    __shared__ uint64_t ck[CAP];
    __shared__ int32_t cj[CAP];
    const int lane = threadIdx.x;
    const uint64_t below = (1ull << lane) - 1ull;
    for (int64_t row = blockIdx.x; row < T; row += gridDim.x) {
        // hash input of dimension j: seed + (row H + j + 1) gamma, stepped by 64 gamma
        const uint64_t z0 = seed + ((uint64_t)row * (uint64_t)H + 1ull + (uint64_t)lane) * kGamma;
        uint64_t t = t0, lo = 0, hi = 0;
        bool have_hi = false;
        int n;
        for (;;) {
            n = 0;
            uint64_t z = z0;
            for (int j0 = 0; j0 < H; j0 += 64, z += 64ull * kGamma) {
                const int j = j0 + lane;
                const uint64_t u = j < H ? mix64(z) : ~0ull;
                const bool c = j < H && u < t;
                const uint64_t m = __ballot(c);
                const int pos = n + __popcll(m & below);
                if (c && pos < CAP) {
                    ck[pos] = u;
                    cj[pos] = j;
                }
                n += __popcll(m);
            }
            if (n >= K && n <= CAP) break;
            if (n < K) {
                lo = t;
                t = have_hi ? lo + (hi - lo) / 2 : (t > (~0ull >> 1) ? ~0ull : 2 * t + 1);
            } else {
                hi = t;
                have_hi = true;
                t = lo + (hi - lo) / 2;
            }
        }
        __syncthreads();
        // the K-th smallest candidate hash: ascending bitonic sort of CAP entries,
        // entry e = R lane + r (padding ~0 is above every candidate, all < t)
        uint64_t v[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int e = R * lane + r;
            v[r] = e < n ? ck[e] : ~0ull;
        }
        for (int size = 2; size <= CAP; size <<= 1) {
            for (int stride = size >> 1; stride >= R; stride >>= 1) {
                const int d = stride / R;  // partner lane distance
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const int e = R * lane + r;
                    const uint64_t y = __shfl_xor(v[r], d);
                    const bool keep_min = ((e & stride) == 0) == ((e & size) == 0);
                    v[r] = keep_min ? (v[r] < y ? v[r] : y) : (v[r] < y ? y : v[r]);
                }
            }
#pragma unroll
            for (int stride = R / 2; stride > 0; stride >>= 1) {
                if (stride >= size) continue;
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    if (r & stride) continue;
                    const int e = R * lane + r;
                    const bool up = (e & size) == 0;
                    const uint64_t a = v[r], b = v[r + stride];
                    if ((a > b) == up) {
                        v[r] = b;
                        v[r + stride] = a;
                    }
                }
            }
        }
        uint64_t mine = v[0];
#pragma unroll
        for (int r = 1; r < R; ++r)
            if ((K - 1) % R == r) mine = v[r];
        const uint64_t uk = __shfl(mine, (K - 1) / R);
        // the kept dimensions, in candidate (ascending dimension) order
        int32_t* out = idx + row * K;
        int cnt = 0;
        for (int i0 = 0; i0 < n; i0 += 64) {
            const int i = i0 + lane;
            const bool sel = i < n && ck[i] <= uk;
            const uint64_t m = __ballot(sel);
            if (sel) gst(out + cnt + __popcll(m & below), cj[i]);
            cnt += __popcll(m);
        }
        __syncthreads();  // the candidate lists are rewritten for the next token
    }
}

template <typename E>
__global__ __launch_bounds__(256) void mask_pack_kernel(const E* __restrict__ x, const int32_t* __restrict__ idx,
                                                        int64_t T, int H, int K, E* __restrict__ packed) {
    const int64_t n = T * (int64_t)K;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n;
         e += (int64_t)gridDim.x * blockDim.x) {
        const int64_t row = e / K;
        const int j = min(max(gld(idx + e), 0), H - 1);  // entries outside [0, H) are clamped
        gst(packed + e, gld(x + row * H + j));
    }
}

// Four tokens per workgroup, one per wavefront: each wave's LDS row of H
// elements, zeroed once, takes the K kept values of its token; the row then
// goes out as 16-byte streaming stores (VEC: H e a multiple of 16 bytes and x
// 16-byte aligned; else element stores), and each chunk is cleared again as it
// is read, ready for the wave's next token.  Streaming stores keep the dense
// rows out of L2 (0.058 -> 0.042 ms for 65536 bf16 rows of 2048).
template <typename E, bool VEC>
__global__ __launch_bounds__(256) void mask_unpack_kernel(const E* __restrict__ packed,
                                                          const int32_t* __restrict__ idx, int64_t T, int H,
                                                          int K, E* __restrict__ x) {
    extern __shared__ __align__(16) unsigned char mask_rows[];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nchunk = (H * (int)sizeof(E) + 15) / 16;
    v4f* const cells = reinterpret_cast<v4f*>(mask_rows) + wave * nchunk;
    E* const rowbuf = reinterpret_cast<E*>(cells);
    for (int c = threadIdx.x; c < 4 * nchunk; c += 256) reinterpret_cast<v4f*>(mask_rows)[c] = v4f{0.f, 0.f, 0.f, 0.f};
    __syncthreads();
    for (int64_t r0 = 4 * (int64_t)blockIdx.x; r0 < T; r0 += 4 * (int64_t)gridDim.x) {
        const int64_t row = r0 + wave;
        if (row < T)
            for (int k = lane; k < K; k += 64)
                rowbuf[min(max(gld(idx + row * K + k), 0), H - 1)] = gld(packed + row * K + k);
        __syncthreads();
        if (row < T) {
            if (VEC) {
                SC_GLOBAL v4f* out = (SC_GLOBAL v4f*)(x + row * H);
                for (int c = lane; c < nchunk; c += 64) {
                    __builtin_nontemporal_store(cells[c], out + c);
                    cells[c] = v4f{0.f, 0.f, 0.f, 0.f};
                }
            } else {
                for (int j = lane; j < H; j += 64) {
                    gst(x + row * H + j, rowbuf[j]);
                    rowbuf[j] = E(0);
                }
            }
        }
        __syncthreads();
    }
}

namespace {
int grid_rows(int64_t T) { return (int)(T < 65536 ? T : 65536); }
}  // namespace

hipError_t launch_mask_indices(uint64_t seed, int64_t T, int H, int K, int32_t* idx, hipStream_t st) {
    if (T <= 0 || K <= 0) return hipSuccess;
    // the candidate threshold of the one-wavefront kernel: w = K + 5 sqrt(K) + 16 hashes
    // expected below t0, room for w + 6 sqrt(w) candidates
    const double want = K + 5.0 * std::sqrt((double)K) + 16.0;
    int cap = 64;
    while (cap < want + 6.0 * std::sqrt(want)) cap <<= 1;
    if (cap <= 512 && want < 0.5 * H) {
        const uint64_t t0 = (uint64_t)(want / H * 18446744073709551616.0);
        const dim3 grid(grid_rows(T) * 4 < T ? grid_rows(T) * 4 : (unsigned)T);
#define SC_MASK_WAVE(R_)                                                                        \
    if (cap == 64 * R_) {                                                                     \
        hipLaunchKernelGGL(mask_indices_wave_kernel<R_>, grid, dim3(64), 0, st, seed, T, H, K, \
                           t0, idx);                                                          \
        return hipGetLastError();                                                             \
    }
        SC_MASK_WAVE(1) SC_MASK_WAVE(2) SC_MASK_WAVE(4) SC_MASK_WAVE(8)
#undef SC_MASK_WAVE
    }
    hipLaunchKernelGGL(mask_indices_kernel, dim3(grid_rows(T)), dim3(256), 0, st, seed, T, H, K, idx);
    return hipGetLastError();
}

hipError_t launch_mask_pack(bool bf16, const void* x, const int32_t* idx, int64_t T, int H, int K,
                            void* packed, hipStream_t st) {
    const int64_t n = T * (int64_t)K;
    if (n <= 0) return hipSuccess;
    const int64_t blocks = (n + 255) / 256;
    const dim3 grid((unsigned)(blocks < 65536 ? blocks : 65536));
    if (bf16)
        hipLaunchKernelGGL(mask_pack_kernel<uint16_t>, grid, dim3(256), 0, st, (const uint16_t*)x, idx, T, H,
                           K, (uint16_t*)packed);
    else
        hipLaunchKernelGGL(mask_pack_kernel<float>, grid, dim3(256), 0, st, (const float*)x, idx, T, H, K,
                           (float*)packed);
    return hipGetLastError();
}

hipError_t launch_mask_unpack(bool bf16, const void* packed, const int32_t* idx, int64_t T, int H, int K,
                              void* x, hipStream_t st) {
    if (T <= 0) return hipSuccess;
    const int esz = bf16 ? 2 : 4;
    const size_t lds = 4 * (((size_t)H * esz + 15) / 16 * 16);  // four rows
    const bool vec = ((size_t)H * esz) % 16 == 0 && ((uintptr_t)x & 15) == 0;
    const int64_t groups = (T + 3) / 4;
    const dim3 grid((unsigned)(groups < 262144 ? groups : 262144));
#define SC_UNPACK(E_, V_)                                                                          \
    hipLaunchKernelGGL((mask_unpack_kernel<E_, V_>), grid, dim3(256), lds, st, (const E_*)packed, idx, T, H, K, \
                       (E_*)x)
    if (bf16) {
        if (vec) SC_UNPACK(uint16_t, true); else SC_UNPACK(uint16_t, false);
    } else {
        if (vec) SC_UNPACK(float, true); else SC_UNPACK(float, false);
    }
#undef SC_UNPACK
    return hipGetLastError();
}

}  // namespace scopt
