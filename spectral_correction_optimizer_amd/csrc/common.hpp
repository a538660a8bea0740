// Device helpers shared by the HIP kernels of libscopt (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace scopt {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));

// Raw buffer access (gfx9 buffer resource: 48-bit base, no stride, num_records
// bytes, the gfx9 default format word): 32-bit byte offsets in VGPRs plus a
// wave-uniform offset in an SGPR; accesses beyond num_records read zero and
// write nothing.  kBufNT selects the nontemporal (streaming) cache policy.
constexpr int kBufNT = 2;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}
template <int AUX>
__device__ __forceinline__ float buf_load_f32(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, AUX));
}
template <int AUX>
__device__ __forceinline__ void buf_store_f32(float v, __amdgpu_buffer_rsrc_t r, int voff, int soff) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned int, v), r, voff, soff, AUX);
}

// bfloat16 <-> float32.  bf16 is the upper half of an IEEE float32;
// narrowing rounds to nearest, ties to even (NaN stays NaN).
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(((uint32_t)b) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)0x7fc0;
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Running maximum of non-negative convergence measures in which a NaN counts as
// +infinity (fmaxf would drop it): a non-finite operand then reads as far from
// converged instead of as converged.
__device__ __forceinline__ float max_nan_inf(float m, float x) {
    return x <= m ? m : (x == x ? x : __builtin_huge_valf());
}

// Device-memory accessors that compile to global_load / global_store.  A
// pointer read from a struct in memory is generic, and generic (flat) accesses
// are counted by the LDS wait counter as well: an s_waitcnt for an LDS read
// would then also wait for every outstanding global prefetch.  All buffers of
// the library and the caller's tensors are device (global) memory.
#define SC_GLOBAL __attribute__((address_space(1)))
typedef unsigned int v2u __attribute__((ext_vector_type(2)));
template <typename T>
__device__ __forceinline__ SC_GLOBAL T* gptr(T* p) {
    return (SC_GLOBAL T*)p;
}
template <typename T>
__device__ __forceinline__ const SC_GLOBAL T* gptr(const T* p) {
    return (const SC_GLOBAL T*)p;
}
template <typename T>
__device__ __forceinline__ T gld(const T* p) {
    return *gptr(p);
}
template <typename T>
__device__ __forceinline__ void gst(T* p, T v) {
    *gptr(p) = v;
}
__device__ __forceinline__ v4f gld4(const float* p) { return *(const SC_GLOBAL v4f*)p; }
__device__ __forceinline__ void gst4(float* p, v4f v) { *(SC_GLOBAL v4f*)p = v; }

template <typename T> struct Elem;
template <> struct Elem<float> {
    __device__ __forceinline__ static float load(const float* p, int64_t i) { return gld(p + i); }
};
template <> struct Elem<uint16_t> {
    __device__ __forceinline__ static float load(const uint16_t* p, int64_t i) {
        return bf16_to_f32(gld(p + i));
    }
};

// Streaming (nontemporal) variants for data touched once per pass: they keep
// the stream from displacing other lines in the caches.  4-element aligned.
__device__ __forceinline__ float4 load4_nt(const float* p) {
    const v4f v = __builtin_nontemporal_load((const SC_GLOBAL v4f*)p);
    return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float4 load4_nt(const uint16_t* p) {
    const v2u u = __builtin_nontemporal_load((const SC_GLOBAL v2u*)p);
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                       __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
}
__device__ __forceinline__ void store4_nt(float* p, float4 w) {
    __builtin_nontemporal_store(v4f{w.x, w.y, w.z, w.w}, (SC_GLOBAL v4f*)p);
}
__device__ __forceinline__ void store4_nt(uint16_t* p, float4 w) {
    const v2u u = {(uint32_t)f32_to_bf16(w.x) | ((uint32_t)f32_to_bf16(w.y) << 16),
                   (uint32_t)f32_to_bf16(w.z) | ((uint32_t)f32_to_bf16(w.w) << 16)};
    __builtin_nontemporal_store(u, (SC_GLOBAL v2u*)p);
}

// Load 4 consecutive elements (the address must be 4-element aligned).
__device__ __forceinline__ float4 load4(const float* p) {
    const v4f v = gld4(p);
    return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float4 load4(const uint16_t* p) {
    const v2u u = *(const SC_GLOBAL v2u*)p;
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                       __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
}

// The compute units of an MI355X are spread over 8 dies (XCDs), each with
// its own L2; consecutive workgroup ids are dealt round robin to the XCDs.
// Remap so that every XCD receives a contiguous range of logical ids: tiles
// that share operand panels then share an L2.
__device__ __forceinline__ int xcd_remap(int wg, int nwg) {
    const int nx = 8;
    int per = nwg / nx, rem = nwg % nx;
    int x = wg % nx, slot = wg / nx;
    // XCDs with index < rem get per + 1 ids.
    int base = x * per + (x < rem ? x : rem);
    int cnt = per + (x < rem ? 1 : 0);
    if (slot >= cnt) return wg;  // cannot happen when nwg ids are launched
    return base + slot;
}

// Sum of v over the workgroup (wave shuffles, then the per-wave partials in a
// fixed order); red holds blockDim.x / 64 doubles.  Every thread gets the sum.
__device__ __forceinline__ double block_sum_f64(double v, double* red) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    double s = 0.0;
    const int nw = blockDim.x >> 6;
    for (int i = 0; i < nw; ++i) s += red[i];
    __syncthreads();
    return s;
}

// Round-robin ("circle") pairing of nb items: round r in [0, nb-1),
// slot i in [0, nb/2); returns p < q.
__device__ __host__ __forceinline__ void rr_pair(int nb, int r, int i, int* p, int* q) {
    int n = nb - 1, a, b;
    if (i == 0) {
        a = nb - 1;
        b = r;
    } else {
        a = (r + i) % n;
        b = (r - i + n) % n;
    }
    *p = a < b ? a : b;
    *q = a < b ? b : a;
}

// Block pair of slot i in round r of a sweep over nb blocks.  For nb a power of
// two: the XOR ordering, round r pairs block p with p ^ m, m = nb - 1 - r (slot i
// is p with a zero bit inserted at the top bit of m): the first round pairs the
// most distant blocks of the norm order, the last one neighbours.  It needs one
// or two sweeps fewer than the round-robin ordering, which serves the other
// block counts, and than the ascending XOR order.
__device__ __host__ __forceinline__ void block_pair(int nb, int r, int i, int* p, int* q) {
    if ((nb & (nb - 1)) == 0) {
        const int m = nb - 1 - r, h = 31 - __builtin_clz(m);
        const int lo = i & ((1 << h) - 1);
        *p = ((i >> h) << (h + 1)) | lo;
        *q = *p ^ m;
    } else {
        rr_pair(nb, r, i, p, q);
    }
}

// ---- float32 products on the bfloat16 matrix cores -------------------------------
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// Exact three-way split of float32 values into bfloat16 parts, x = hi + mid + lo:
// hi = RNE(x), mid = RNE(x - hi), lo = x - hi - mid (|x - hi| <= 2^-8 |x|; mid
// and lo carry the next 8 and the last <= 8 significant bits; both differences
// are exact in float32).  Of the nine part products of a * b the six largest
// (hh, hm, mh, hl, lh, mm) leave out less than 2^-23 |a b|.
struct Split8 {
    v8bf h, m, l;
};
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
// Two floats rounded to bfloat16 (nearest even) in one instruction
// (v_cvt_pk_bf16_f32), packed low / high; the parts read back as floats by a
// shift and a mask.
__device__ __forceinline__ unsigned int pack_bf16x2(float a, float b) {
    return __builtin_bit_cast(unsigned int, __builtin_convertvector((v2f){a, b}, v2bf));
}
__device__ __forceinline__ float bf16_lo(unsigned int p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float bf16_hi(unsigned int p) { return __uint_as_float(p & 0xffff0000u); }
// f = h + m + l exactly: h = bf16(f), m = bf16(f - h), l = bf16(f - h - m), each
// rounded to nearest even, two elements per conversion
__device__ __forceinline__ Split8 split8(const float (&f)[8]) {
    v4u h, m, l;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const unsigned int hp = pack_bf16x2(f[2 * i], f[2 * i + 1]);
        const float r0 = f[2 * i] - bf16_lo(hp), r1 = f[2 * i + 1] - bf16_hi(hp);
        const unsigned int mp = pack_bf16x2(r0, r1);
        h[i] = hp;
        m[i] = mp;
        l[i] = pack_bf16x2(r0 - bf16_lo(mp), r1 - bf16_hi(mp));
    }
    return Split8{__builtin_bit_cast(v8bf, h), __builtin_bit_cast(v8bf, m), __builtin_bit_cast(v8bf, l)};
}
// the first two parts only (|f - h - m| <= 2^-16 |f|)
__device__ __forceinline__ void split8_hm(const float (&f)[8], v8bf& hv, v8bf& mv) {
    v4u h, m;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const unsigned int hp = pack_bf16x2(f[2 * i], f[2 * i + 1]);
        h[i] = hp;
        m[i] = pack_bf16x2(f[2 * i] - bf16_lo(hp), f[2 * i + 1] - bf16_hi(hp));
    }
    hv = __builtin_bit_cast(v8bf, h);
    mv = __builtin_bit_cast(v8bf, m);
}

// LDS layout of a split operand tile: per plane, rows of 16 k (k contiguous) as
// two 8-element chunks whose order flips with bit 2 of the row, so the 16-byte
// MFMA fragment reads of 8 consecutive lanes (8 rows) and the loaders' 16-byte
// writes cover all banks once.  Element offset of chunk `half` of `row`.
__device__ __forceinline__ int split_chunk16(int row, int half) {
    return row * 16 + ((half ^ ((row >> 2) & 1)) << 3);
}

}  // namespace scopt
