// Blocked one-sided Jacobi sweeps in rounds of four-block groups ("quad passes").
//
// The spectral-correction optimizer takes a thin SVD of each matrix's anchor
// momentum ("Key design 3" of the papernotes.org notes on "Communication-
// Efficient LLM Adaptation over Decentralized GPU Meshes") by one-sided Jacobi
// sweeps.  A sweep must solve every pair of the nb column blocks once.  For a
// power-of-two nb the pair rounds are the masks m = 1 .. nb - 1 (round m pairs
// block p with p ^ m).  When log2 nb is even the nonzero masks split into lines
// {m0, m1, m2 = m0 ^ m1} (2-dimensional subspaces of GF(2)^log2 nb): the three
// rounds of one line pair the blocks inside groups of four, the cosets
// {p, p ^ m0, p ^ m1, p ^ m2}, so one pass over a group's 128 operand rows can
// carry all three rounds.  A sweep becomes (nb - 1) / 3 passes of three launches:
//
//   gram   per (group, column split): the 128 x 128 Gram of the group's rows
//          (ten 32 x 32 tiles, bfloat16 three-way split products with float32
//          sums over at most 256 columns, folded in float64);
//   solve  per group: the three rounds in LDS: each round solves its two block
//          pairs by one cyclic sweep of 2x2 rotations (the pair solve of the
//          pair rounds, unchanged), then takes the Gram of the next round's pairs
//          from the rotated one (G' = Q^T G Q; the cross block between the two
//          pairs as (I + R_P)^T C (I + R_Q)), and folds the round into the
//          group's rotation R = Q_1 Q_2 Q_3 - I;
//   apply  per (group, column run, A or V rows): X <- X + R^T X over the group's
//          128 rows (bfloat16 three-way split, six part products), one read and
//          one write of every row per three rounds.
//
// The same rotations as three pair rounds, in another order: every block pair
// is solved once per sweep.  The lines are taken level by level, mimicking the
// descending XOR order of the pair rounds (first the masks with the top bit set,
// each with one with the next bit as its top bit, then the same on two fewer
// bits, ...); a numpy model of the method on the workload's spectrum needed the
// same sweeps as that order (7 on the Cholesky factor, 7 - 8 on plain operands,
// 512 columns in 64 blocks).
#include "common.hpp"
#include "internal.hpp"
#include "jacobi_dev.hpp"

namespace scopt {

namespace {

// ---- the lines of every supported block count -------------------------------------
// Level with n bits (n even, from log2 nb down to 2): q = n - 2, x < 2^q, f = alpha x
// in GF(2^q): masks a = 2^(n-1) + x, a' = 2^(n-1) + (x ^ 2^q ^ f), c = 2^q + f with
// a ^ a' = c.  f and x ^ f = (1 + alpha) x are bijections, so the level covers every
// mask with top bit n - 1 or n - 2 once.  Within a level the lines go by c
// descending.  Stored per line: the three masks, largest first.
constexpr int kQuadLines = 1 + 5 + 21 + 85;  // nb = 4, 16, 64, 256

constexpr int gf_mul_alpha(int x, int q) {
    // x * alpha in GF(2^q) (alpha = the class of the polynomial t), q = 2, 4, 6
    const int poly = q == 2 ? 0x7 : q == 4 ? 0x13 : 0x43;
    x <<= 1;
    return (x >> q) ? x ^ poly : x;
}

struct QuadTable {
    unsigned char m[kQuadLines][3];
};
constexpr QuadTable make_quad_table() {
    QuadTable t{};
    int o = 0;
    for (int n0 = 2; n0 <= 8; n0 += 2)
        for (int n = n0; n >= 2; n -= 2) {
            const int q = n - 2, cnt = 1 << q;
            // lines of this level by c descending: f runs from 2^q - 1 down to 0
            for (int fi = cnt - 1; fi >= 0; --fi) {
                int x = 0;
                for (int y = 0; y < cnt; ++y)
                    if ((q > 0 ? gf_mul_alpha(y, q) : 0) == fi) x = y;
                const int a = (1 << (n - 1)) + x;
                const int a2 = (1 << (n - 1)) + (x ^ (1 << q) ^ fi);
                const int c = (1 << q) + fi;
                const int hi = a > a2 ? a : a2, lo = a > a2 ? a2 : a;
                t.m[o][0] = (unsigned char)hi;
                t.m[o][1] = (unsigned char)lo;
                t.m[o][2] = (unsigned char)c;
                ++o;
            }
        }
    return t;
}
__constant__ QuadTable kQuad = make_quad_table();

__device__ __forceinline__ int quad_base(int nb) {
    return nb == 4 ? 0 : nb == 16 ? 1 : nb == 64 ? 6 : 27;
}

// Blocks of group g in pass `pass` (of the sweep): slots 0 = p, 1 = p ^ m0,
// 2 = p ^ m2, 3 = p ^ m1, p with zeros at the top bits h of m0 and h2 of m2
// (m0 and m1 share the top bit, m2 lacks it; the coset has one such element).
__device__ __forceinline__ void quad_blocks(int nb, int pass, int g, int blk[4]) {
    const int li = quad_base(nb) + pass % quad_passes(nb);
    const int m0 = kQuad.m[li][0], m2 = kQuad.m[li][2];
    const int h = 31 - __builtin_clz(m0), h2 = 31 - __builtin_clz(m2);
    const int p = insert_zero_bit(insert_zero_bit(g, h2), h);
    blk[0] = p;
    blk[1] = p ^ m0;
    blk[2] = p ^ m2;
    blk[3] = p ^ m0 ^ m2;
}

// Slot pairs of the three rounds of a pass, masks m0, m1, m2: (P0, P1), (Q0, Q1).
__constant__ int kQuadPairs[3][4] = {{0, 1, 2, 3}, {0, 3, 1, 2}, {0, 2, 1, 3}};

constexpr int QN = 4 * kJb;           // 128 rows per group
constexpr int QTILES = 10;            // upper 32 x 32 tiles of the group Gram
constexpr int QPART = QTILES * 1024;  // doubles per (group, split) partial
// Gram tile t: blocks (kTi[t], kTj[t]), kTi <= kTj; tiles 0-4 by waves 0-3, 5-9 by 4-7.
__constant__ int kTi[QTILES] = {0, 0, 0, 0, 1, 1, 1, 2, 2, 3};
__constant__ int kTj[QTILES] = {0, 1, 2, 3, 1, 2, 3, 2, 3, 3};

// Per group: nsplit partials of the group Gram.
__device__ __forceinline__ double* quad_part(const MatDev& md, int g) {
    return md.gram + (int64_t)g * md.nsplit * QPART;
}

}  // namespace

// ---------------------------------------------------------------------------------
// Group Gram over operand columns [x0, x1) (a multiple of 128):
// chunks of 128 columns; each thread loads 8 consecutive columns of a row (16
// threads per row: 512 contiguous bytes), splits them once into bfloat16 hi / mid
// / lo and stores the three planes in LDS (row-major, MFMA fragment order), so the
// product phase only reads fragments.  The next chunk's loads are issued as soon
// as the current one is in LDS.  Wave w forms the five tiles of its set (w / 4)
// over the chunk's columns 32 (w % 4) .. + 31 (two 16-column k-steps); after every
// 8 chunks (so each wave sums at most 256 columns in float32) the four column
// quarters of each tile are added in float64 in a fixed order to the split's
// sums, written at the end as its partial (tile-major, row-major).
namespace {
constexpr int QGW = 128;        // columns per chunk of the group Gram
constexpr int QGRS = QGW + 8;   // bfloat16 row stride of a plane (16-byte aligned rows)
}  // namespace

__global__ __launch_bounds__(512) void jac_quad_gram_kernel(const MatDev* __restrict__ mats,
                                                        const MatFlags* __restrict__ flags,
                                                        const FusedItem* __restrict__ items,
                                                        int pass) {
    __shared__ __align__(16) __bf16 Ps[3][QN * QGRS];
    const FusedItem it = items[blockIdx.x];
    if (flags[it.mat].done) return;
    const MatDev& md = mats[it.mat];
    int blk[4];
    quad_blocks(md.nb, pass, it.group, blk);
    const int ld = md.K_ld;
    const __amdgpu_buffer_rsrc_t buf = buf_rsrc(md.A, (uint32_t)md.kpad * ld * 4u);
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int hl = lane >> 5, ll = lane & 31;
    // loader: rows 32 u + tid / 16 (u < 4), columns 8 (tid % 16) .. + 7
    const int lrow = threadIdx.x >> 4, lcol = 8 * (threadIdx.x & 15);
    int roff[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) roff[u] = (gld(md.perm + blk[u] * kJb + lrow) * ld + lcol) * 4;
    v4u x[8];
    // the loader's row of block u of chunk c
    auto load_part = [&](int c, int u) {
        // wave-uniform: the buffer offset must be a scalar (else every load loops)
        const int so = __builtin_amdgcn_readfirstlane((it.x0 + c * QGW) * 4);
        x[2 * u] = __builtin_amdgcn_raw_buffer_load_b128(buf, roff[u], so, kBufNT);
        x[2 * u + 1] = __builtin_amdgcn_raw_buffer_load_b128(buf, roff[u] + 16, so, kBufNT);
    };
    const int set = wave >> 2, cq = wave & 3;
    v16f acc[5];
#pragma unroll
    for (int t = 0; t < 5; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[t][r] = 0.0f;
    auto frag = [&](int b, int col) {
        const int o = (32 * b + ll) * QGRS + col;
        return Split8{*(const v8bf*)&Ps[0][o], *(const v8bf*)&Ps[1][o], *(const v8bf*)&Ps[2][o]};
    };
    const int n = (it.x1 - it.x0) / QGW;
    // float64 sums of the four column quarters, folded in after every 8 chunks (each
    // wave then has summed at most 256 columns in float32); thread owns entries
    // e = tid + 512 k of the partial (tile e / 1024, MFMA output order within it)
    float* red = (float*)&Ps[0][0];
    double sum[QPART / 512];
#pragma unroll
    for (int k = 0; k < QPART / 512; ++k) sum[k] = 0.0;
    auto fold = [&]() {
#pragma unroll 1
        for (int qq = 0; qq < 4; ++qq) {
            if (cq == qq)
#pragma unroll
                for (int t = 0; t < 5; ++t)
#pragma unroll
                    for (int r4 = 0; r4 < 4; ++r4)
                        *(v4f*)&red[((5 * set + t) * 64 + lane) * 16 + 4 * r4] =
                            v4f{acc[t][4 * r4], acc[t][4 * r4 + 1], acc[t][4 * r4 + 2], acc[t][4 * r4 + 3]};
            __syncthreads();
#pragma unroll
            for (int k = 0; k < QPART / 512; ++k) sum[k] += (double)red[threadIdx.x + 512 * k];
            __syncthreads();
        }
#pragma unroll
        for (int t = 0; t < 5; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[t][r] = 0.0f;
    };
    // Each block's row of the next chunk is requested as soon as this chunk's is
    // split (its registers are then free), so the loads stay in flight through the
    // split, both barriers and the products, not only through the products.  The
    // last chunk is peeled: a branch around the loads would make the wait counts
    // conservative (the last block's split would wait for the next chunk's loads).
    auto chunk = [&](int c, auto more_t) {
        constexpr bool more = decltype(more_t)::value;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            float f[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                f[e] = __uint_as_float(x[2 * u][e]);
                f[4 + e] = __uint_as_float(x[2 * u + 1][e]);
            }
            const Split8 sp = split8(f);
            const int o = (32 * u + lrow) * QGRS + lcol;
            *(v8bf*)&Ps[0][o] = sp.h;
            *(v8bf*)&Ps[1][o] = sp.m;
            *(v8bf*)&Ps[2][o] = sp.l;
            if constexpr (more) load_part(c + 1, u);
        }
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int col = 32 * cq + 16 * ks + 8 * hl;
            // the five tiles' part products interleaved (independent accumulators
            // back to back); each tile's six products in mfma_split6's order
            Split8 fa[5], fb[5];
            if (set == 0) {
                const Split8 f0 = frag(0, col), f1 = frag(1, col), f2 = frag(2, col), f3 = frag(3, col);
                fa[0] = f0; fb[0] = f0;
                fa[1] = f0; fb[1] = f1;
                fa[2] = f0; fb[2] = f2;
                fa[3] = f0; fb[3] = f3;
                fa[4] = f1; fb[4] = f1;
            } else {
                const Split8 f1 = frag(1, col), f2 = frag(2, col), f3 = frag(3, col);
                fa[0] = f1; fb[0] = f2;
                fa[1] = f1; fb[1] = f3;
                fa[2] = f2; fb[2] = f2;
                fa[3] = f2; fb[3] = f3;
                fa[4] = f3; fb[4] = f3;
            }
#pragma unroll
            for (int t = 0; t < 5; ++t) acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[t].l, fb[t].h, acc[t], 0, 0, 0);
#pragma unroll
            for (int t = 0; t < 5; ++t) acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[t].m, fb[t].m, acc[t], 0, 0, 0);
#pragma unroll
            for (int t = 0; t < 5; ++t) acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[t].h, fb[t].l, acc[t], 0, 0, 0);
#pragma unroll
            for (int t = 0; t < 5; ++t) acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[t].m, fb[t].h, acc[t], 0, 0, 0);
#pragma unroll
            for (int t = 0; t < 5; ++t) acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[t].h, fb[t].m, acc[t], 0, 0, 0);
#pragma unroll
            for (int t = 0; t < 5; ++t) acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[t].h, fb[t].h, acc[t], 0, 0, 0);
        }
        __syncthreads();  // before the next chunk's rows
        if ((c & 7) == 7 || c + 1 == n) fold();
    };
#pragma unroll
    for (int u = 0; u < 4; ++u) load_part(0, u);
#pragma unroll 1
    for (int c = 0; c + 1 < n; ++c) chunk(c, std::true_type{});
    if (n > 0) chunk(n - 1, std::false_type{});
    double* out = quad_part(md, it.group) + (int64_t)it.split * QPART;
#pragma unroll
    for (int k = 0; k < QPART / 512; ++k) {
        const int e = threadIdx.x + 512 * k;
        const int t = e >> 10, l = (e >> 4) & 63, r = e & 15;
        const int i = 8 * (r >> 2) + 4 * (l >> 5) + (r & 3), j = l & 31;
        gst(out + t * 1024 + i * 32 + j, sum[k]);
    }
}

// ---------------------------------------------------------------------------------
// Group solve: the three rounds of a pass on one group (waves 0-3: pair P of the
// round, 4-7: pair Q), entirely on chip: the two pair Grams (upper triangles,
// float32, the group Gram scaled by its largest diagonal) in LDS, the cross block
// C = G[P][Q] (64 x 64) in registers (thread t: row t / 8, columns 8 (t % 8) ..
// + 7) while the pairs are swept.  After a round's sweeps, C' = (I + R_P)^T C
// (I + R_Q) on the float32 matrix cores, and the next round's pair Grams and
// cross block are the same group Gram entries in the next round's pairing (a
// permutation through LDS).  The composed rotation R (128 x 128, row-major:
// x_new = x + R^T x over the group's rows in slot order) goes to the rotation
// buffer.
namespace {
// group row of pair-local index a (< 64) of the pair of slots (u0, u1)
__device__ __forceinline__ int qrow(int u0, int u1, int a) {
    return a < kJb ? kJb * u0 + a : kJb * u1 + (a - kJb);
}
// pair-local index of group row x in the pair of slots (u0, u1), -1 if not in it
__device__ __forceinline__ int qloc(int u0, int u1, int x) {
    const int sx = x >> 5;
    return sx == u0 ? (x & 31) : sx == u1 ? kJb + (x & 31) : -1;
}
// LDS of the group solve, one array: the two pair Grams (upper triangles, stride
// SG), then the two R^T (stride SR); the cross block is staged (stride PW) in the
// first R^T's space while no sweep runs.
constexpr int QLG1 = PW * SG, QLR0 = 2 * PW * SG, QLR1 = QLR0 + PW * SR, QLEN = QLR1 + PW * SR;
// Position (0 .. 3) of each slot in the pairing of round k: 0, 1 = pair P, 2, 3 = Q,
// packed two bits per slot (slot s at bits 2 s), so that a lookup by a lane's slot
// is a shift, not a memory load (a table in memory indexed per lane took one load
// per entry).
constexpr int kQuadPosTab[3][4] = {{0, 1, 2, 3}, {0, 2, 3, 1}, {0, 2, 1, 3}};
constexpr unsigned quad_pos_bits(int k) {
    return (unsigned)kQuadPosTab[k][0] | (unsigned)kQuadPosTab[k][1] << 2 | (unsigned)kQuadPosTab[k][2] << 4 |
           (unsigned)kQuadPosTab[k][3] << 6;
}
constexpr unsigned kQuadPosBits[3] = {quad_pos_bits(0), quad_pos_bits(1), quad_pos_bits(2)};
static_assert(kQuadPosBits[0] == 0xE4u && kQuadPosBits[1] == 0x78u && kQuadPosBits[2] == 0xD8u, "slot positions");
// LDS offset of the group Gram entry (x, y) in round k's pairing: the upper
// triangle of pair P's or Q's Gram, or the cross block (P rows, Q columns).
__device__ __forceinline__ int qslot_off(int k, int x, int y) {
    const unsigned pb = k == 0 ? kQuadPosBits[0] : k == 1 ? kQuadPosBits[1] : kQuadPosBits[2];
    const int ix = (pb >> (2 * (x >> 5))) & 3, iy = (pb >> (2 * (y >> 5))) & 3;
    const int lx = 32 * (ix & 1) + (x & 31), ly = 32 * (iy & 1) + (y & 31);
    const int px = ix >> 1, py = iy >> 1;
    const int pair_off = (px ? QLG1 : 0) + min(lx, ly) * SG + max(lx, ly);
    const int cross_off = QLR0 + (px == 0 ? lx * PW + ly : ly * PW + lx);
    return px == py ? pair_off : cross_off;
}
}  // namespace

__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4))) void jac_quad_solve_kernel(const MatDev* __restrict__ mats,
                                                         MatFlags* __restrict__ flags,
                                                         const SolveItem* __restrict__ items,
                                                         int pass) {
    __shared__ __align__(16) float LS[QLEN];
    __shared__ v4f rot4[2][PW / 2];  // a step's rotations (c, s, c - 1) per pair
    __shared__ double dg[QN];
    __shared__ float mos[8];
    __shared__ double dmax_s;

    const SolveItem it = items[blockIdx.x];
    MatFlags& fl = flags[it.mat];
    if (fl.done) return;
    const MatDev& md = mats[it.mat];
    const int g = it.slot;
    int blk[4];
    quad_blocks(md.nb, pass, g, blk);
    const float tol = md.tol;
    const int tid = threadIdx.x, l = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int q = wave >> 2, w = wave & 3, pt = tid & 255;
    float* Gq = LS + q * QLG1;            // pair q's Gram
    float* RTq = LS + QLR0 + q * PW * SR;  // pair q's R^T
    float* X = LS + QLR0;                 // cross-block staging (stride PW)
    const double* part = quad_part(md, g);
    // the group's composed rotation through a buffer resource (32-bit offsets)
    const __amdgpu_buffer_rsrc_t rbuf = buf_rsrc(md.rot + (int64_t)g * (QN * QN), QN * QN * 4u);
    int* rflag = md.rot_flag + g;
    auto prow = [&](int x) { return gld(md.perm + blk[x >> 5] * kJb + (x & 31)); };

    // 1. the partials summed in split order (float64): first the diagonal, then
    //    entry e = tid + 512 k (tile e / 1024, row (e / 32) % 32, column e % 32),
    //    scaled, into round 0's pair Grams and cross block; the largest relative
    //    off-diagonal of the group (every block pair of it)
    // Split 0 of the thread's 20 entries is requested together with the diagonal
    // (one memory round trip instead of one per batch); later splits are added in
    // batches below.  Each sum is formed in split order from 0.0, as before.
    constexpr int NE = QPART / 512;
    double v0[NE];
    {
        const int b = tid >> 5, i = tid & 31;
        const int t = b == 0 ? 0 : b == 1 ? 4 : b == 2 ? 7 : 9;
        const int de = tid < QN ? t * 1024 + i * 33 : 0;
        double a = 0.0;
        a += gld(part + de);
#pragma unroll
        for (int k = 0; k < NE; ++k) v0[k] = 0.0 + gld(part + tid + 512 * k);
        for (int sp = 1; sp < it.nsplit; ++sp) a += gld(part + (int64_t)sp * QPART + de);
        if (tid < QN) dg[tid] = a;
    }
    __syncthreads();
    if (wave == 0) {
        double d = fmax(dg[l], dg[l + 64]);
        for (int o = 32; o > 0; o >>= 1) d = fmax(d, __shfl_xor(d, o));
        if (l == 0) dmax_s = d;
    }
    __syncthreads();
    const double dmax = dmax_s;
    const double scale = dmax > 0.0 ? 1.0 / dmax : 1.0;
    const double floor2d = (double)fl.floor2;
    const float floor2 = (float)(floor2d * scale);
    float mo = 0.0f;
    constexpr int KB = 5;  // entries per batch of loads
    static_assert(NE % KB == 0, "whole batches");
#pragma unroll
    for (int k0 = 0; k0 < NE; k0 += KB) {
        double v[KB];
#pragma unroll
        for (int u = 0; u < KB; ++u) v[u] = v0[k0 + u];
        for (int sp = 1; sp < it.nsplit; ++sp) {
            double t[KB];
#pragma unroll
            for (int u = 0; u < KB; ++u) t[u] = gld(part + (int64_t)sp * QPART + tid + 512 * (k0 + u));
#pragma unroll
            for (int u = 0; u < KB; ++u) v[u] += t[u];
        }
#pragma unroll
        for (int u = 0; u < KB; ++u) {
            const int e = tid + 512 * (k0 + u), t = e >> 10, i = (e >> 5) & 31, j = e & 31;
            const int x = 32 * kTi[t] + i, y = 32 * kTj[t] + j;
            if (x > y) continue;  // the lower half of a diagonal tile
            LS[qslot_off(0, x, y)] = (float)(v[u] * scale);
            if (x < y && dg[x] > floor2d && dg[y] > floor2d)
                mo = max_nan_inf(mo, (float)(fabs(v[u]) / sqrt(dg[x] * dg[y])));
            else if (x < y && !(v[u] == v[u]))
                mo = max_nan_inf(mo, (float)v[u]);
        }
    }
    for (int o = 32; o > 0; o >>= 1) mo = fmaxf(mo, __shfl_xor(mo, o));
    if (l == 0) mos[wave] = mo;
    __syncthreads();
    mo = mos[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mo = max_nan_inf(mo, mos[i]);
    if (tid == 0) atomicMax(&fl.sweep_max, __float_as_uint(mo));
    if (!(mo > tol)) {
        if (tid < QN) gst(md.cnorm + prow(tid), (float)dg[tid]);
        if (tid == 0) *rflag = 0;
        return;
    }
    // both pairs' Q^T = I before a round's sweeps (a row of stride SR is 17 vectors)
    auto rt_identity = [&]() {
        for (int e = tid; e < 2 * PW * SR / 4; e += 512) {
            const int rem = (4 * e) % (PW * SR), d = rem / SR - rem % SR;
            *(v4f*)&LS[QLR0 + 4 * e] = v4f{d == 0 ? 1.0f : 0.0f, d == 1 ? 1.0f : 0.0f,
                                           d == 2 ? 1.0f : 0.0f, d == 3 ? 1.0f : 0.0f};
        }
    };
    // the cross block into registers (thread t: row t / 8, columns 8 (t % 8) .. + 7),
    // Q^T = I for the first round
    const int ct = tid >> 3, cc0 = 8 * (tid & 7);
    float cr[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) cr[e] = X[ct * PW + cc0 + e];
    __syncthreads();
    rt_identity();
    __syncthreads();

    bool have_r = false;  // R holds the rounds so far
    int rounds = 0;
    const int lk = l >> 5, lr = l & 31;
#pragma unroll 1
    for (int k = 0; k < 3; ++k) {
        const int p0 = kQuadPairs[k][0], p1 = kQuadPairs[k][1];
        const int q0 = kQuadPairs[k][2], q1 = kQuadPairs[k][3];
        const int u0 = q == 0 ? p0 : q0, u1 = q == 0 ? p1 : q1;
        // a) any pair of the round above the threshold (current diagonal)
        float mr = 0.0f;
        for (int e = pt; e < PW * PW; e += 256) {
            const int a = e >> 6, b = e & 63;
            if (a < b) {
                const float ga = Gq[a * SG + a], gb = Gq[b * SG + b];
                if (ga > floor2 && gb > floor2)
                    mr = max_nan_inf(mr, fabsf(Gq[a * SG + b]) * __builtin_amdgcn_rsqf(ga * gb));
            }
        }
        for (int o = 32; o > 0; o >>= 1) mr = fmaxf(mr, __shfl_xor(mr, o));
        if (l == 0) mos[wave] = mr;
        __syncthreads();
        mr = mos[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) mr = fmaxf(mr, mos[i]);
        __syncthreads();
        const bool rot = mr > tol;  // workgroup-uniform
        if (rot) {
            ++rounds;
            // b) one cyclic sweep per pair (every wave runs the 63 steps); its per-lane
            //    addresses are formed here rather than kept across the other phases
            int lr_ = l, wr_ = w;
            __asm__ volatile("" : "+v"(lr_), "+s"(wr_));
            pair_sweep_q<4>(Gq, RTq, rot4[q], lr_, wr_, floor2, tol);
            __syncthreads();
            diag_to_delta<256>(RTq, pt);  // ordered before its readers by the barrier below
        }
        if (k == 2) {
            // column norms after the last round, from the pair Grams
            if (pt < PW) gst(md.cnorm + prow(qrow(u0, u1, pt)), (float)(Gq[pt * SG + pt] * dmax));
        }
        // c) the rotated pair Grams' entries (pair q, entries pt + 256 u) in registers
        float gv[PW * PW / 256];
        if (k < 2) {
#pragma unroll
            for (int u = 0; u < PW * PW / 256; ++u) {
                const int e = pt + 256 * u, a = e >> 6, b = e & 63;
                gv[u] = a <= b ? Gq[a * SG + b] : 0.0f;
            }
        }
        __syncthreads();
        // d) R <- R + R_k + R R_k with R_k = blockdiag(R_P, R_Q): for the columns of
        //    pair p, R[:, p] + R_p embedded + R[:, p] R_p, from the columns R[:, p]
        //    staged in LDS (128 x 64, stride SG, in the Grams' space); the product on
        //    the float32 matrix cores, wave w: rows 32 (w / 2) .., pair columns 32 (w % 2) ..
        //    (lane l feeds k = 2 kk + l / 32 and row / column l % 32; its outputs are
        //    rows 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32)
        if (rot) {
            float* S = LS;
            const int er = wave >> 1, ec = wave & 1;
#pragma unroll 1
            for (int pp = 0; pp < 2; ++pp) {
                const int w0 = pp == 0 ? p0 : q0, w1 = pp == 0 ? p1 : q1;
                const float* RTp = LS + QLR0 + pp * PW * SR;
                if (have_r) {
                    // stage R[:, pair columns]: thread row tid / 4, columns 16 (tid % 4) .. + 15
                    const int sxr = tid >> 2, sm = 16 * (tid & 3);
                    const int z = qrow(w0, w1, sm);
                    float r16[16];
#pragma unroll
                    for (int u = 0; u < 16; ++u) r16[u] = buf_load_f32<0>(rbuf, (sxr * QN + z + u) * 4, 0);
#pragma unroll
                    for (int u = 0; u < 16; u += 2) *(v2f*)&S[sxr * SG + sm + u] = v2f{r16[u], r16[u + 1]};
                    __syncthreads();
                }
                const int c = 32 * ec + lr;  // the lane's pair-local column
                v16f acc;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int x = 32 * er + 8 * (r >> 2) + 4 * lk + (r & 3);
                    const int lx = qloc(w0, w1, x);
                    acc[r] = (lx >= 0 ? RTp[c * SR + lx] : 0.0f) + (have_r ? S[x * SG + c] : 0.0f);
                }
                if (have_r) {
#pragma unroll 4
                    for (int kk = 0; kk < PW / 2; ++kk) {
                        const int m = 2 * kk + lk;
                        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(S[(32 * er + lr) * SG + m], RTp[c * SR + m],
                                                                   acc, 0, 0, 0);
                    }
                }
                const int y = qrow(w0, w1, c);
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    buf_store_f32<0>(acc[r], rbuf, ((32 * er + 8 * (r >> 2) + 4 * lk + (r & 3)) * QN + y) * 4, 0);
                __syncthreads();  // S read by every wave before the next pair stages
            }
            have_r = true;
        }
        if (k == 2) break;
        // e) C' = T + T R_Q, T = C + R_P^T C on the float32 matrix cores (waves 0-3,
        //    tile (w / 2, w % 2)); C staged in the first Gram's space (stride PW), T in
        //    the second's (stride SG)
        const int tr = wave >> 1, tc = wave & 1;
        v16f cacc;
        if (rot) {
            float* Cs = LS;
            float* T = LS + QLG1;
            const float* RT0 = LS + QLR0;
            const float* RT1 = LS + QLR1;
#pragma unroll
            for (int e = 0; e < 8; ++e) Cs[ct * PW + cc0 + e] = cr[e];
            __syncthreads();
            if (wave < 4) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    cacc[r] = Cs[(32 * tr + 8 * (r >> 2) + 4 * lk + (r & 3)) * PW + 32 * tc + lr];
#pragma unroll 4
                for (int kk = 0; kk < PW / 2; ++kk) {
                    const int m = 2 * kk + lk;
                    cacc = __builtin_amdgcn_mfma_f32_32x32x2f32(RT0[(32 * tr + lr) * SR + m],
                                                                Cs[m * PW + 32 * tc + lr], cacc, 0, 0, 0);
                }
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    T[(32 * tr + 8 * (r >> 2) + 4 * lk + (r & 3)) * SG + 32 * tc + lr] = cacc[r];
            }
            __syncthreads();
            if (wave < 4) {
#pragma unroll 4
                for (int kk = 0; kk < PW / 2; ++kk) {
                    const int m = 2 * kk + lk;
                    cacc = __builtin_amdgcn_mfma_f32_32x32x2f32(T[(32 * tr + lr) * SG + m],
                                                                RT1[(32 * tc + lr) * SR + m], cacc, 0, 0, 0);
                }
            }
            __syncthreads();  // T and R^T read before the space is reused
        }
        // f) the next round's pair Grams and cross block (staged, then registers): the
        //    same group Gram entries in the next pairing
#pragma unroll
        for (int u = 0; u < PW * PW / 256; ++u) {
            const int e = pt + 256 * u, a = e >> 6, b = e & 63;
            if (a <= b) LS[qslot_off(k + 1, qrow(u0, u1, a), qrow(u0, u1, b))] = gv[u];
        }
        if (rot) {
            if (wave < 4) {
                const int y = qrow(q0, q1, 32 * tc + lr);
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    LS[qslot_off(k + 1, qrow(p0, p1, 32 * tr + 8 * (r >> 2) + 4 * lk + (r & 3)), y)] = cacc[r];
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) LS[qslot_off(k + 1, qrow(p0, p1, ct), qrow(q0, q1, cc0 + e))] = cr[e];
        }
        __syncthreads();
#pragma unroll
        for (int e = 0; e < 8; ++e) cr[e] = X[ct * PW + cc0 + e];
        __syncthreads();
        rt_identity();
        __syncthreads();
    }
    if (tid == 0) {
        *rflag = have_r ? 1 : 0;
        atomicAdd(&fl.pairs_applied, 2 * rounds);
        if (have_r) atomicAdd(&fl.quads_applied, 1);
    }
}

// ---------------------------------------------------------------------------------
// Group apply: X <- X + R^T X over the group's 128 rows, columns [x0, x1) of A
// (which = 0, row stride K_ld) or V (which = 1, stride kpad) in chunks of
// kQuadCols.  R^T is split once per workgroup into three bfloat16 planes in
// MFMA operand order (96 KB of LDS); wave w owns 32 columns of a chunk and keeps
// the group's 128 rows of them in registers (16 rows of each block per lane, the
// row order of the pair apply: its B operands are its own registers); the next
// chunk's loads are in flight meanwhile.  Output tiles are formed one at a time
// over the eight 16-row k-steps and stored as x + R^T x (x itself is not changed
// until the chunk is done).
__global__ __launch_bounds__(kQuadThreads) void jac_quad_apply_kernel(const MatDev* __restrict__ mats,
                                                                  const MatFlags* __restrict__ flags,
                                                                  const QuadItem* __restrict__ items,
                                                                  int pass) {
    // [output tile][plane][16-row k-step][lane]
    __shared__ v8bf Rp[4][3][8][64];
    const QuadItem it = items[blockIdx.x];
    if (flags[it.mat].done) return;
    const MatDev& md = mats[it.mat];
    if (gld(md.rot_flag + it.group) == 0) return;
    // operand A of tile U, k-step t for lane l: R^T[32 U + l % 32][z] = R[z][32 U + l % 32]
    // at the 8 group rows z = 32 (t / 2) + apply_row(8 (t % 2) + e, l / 32); thread
    // idx handles (U, t, l) = (idx / 512, idx / 64 % 8, idx % 64) for idx = tid + 512 i.
    // All 32 of a thread's loads are issued here, before the row offsets and the
    // first chunk's loads, so that the three arrive in one memory round trip (the
    // vector-memory counter completes in order: a wait for a later load also waits
    // for every earlier one).
    static_assert(4 * kQuadThreads == 4 * 8 * 64, "four (tile, k-step, lane) entries per thread");
    const float* R = md.rot + (int64_t)it.group * (QN * QN);
    float rf[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int idx = threadIdx.x + kQuadThreads * i;
        const int U = idx >> 9, t = (idx >> 6) & 7, l = idx & 63;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            rf[i][e] = gld(R + (32 * (t >> 1) + apply_row(8 * (t & 1) + e, l >> 5)) * QN + 32 * U + (l & 31));
    }
    int blk[4];
    quad_blocks(md.nb, pass, it.group, blk);
    const int ld = it.which ? md.kpad : md.K_ld;
    const __amdgpu_buffer_rsrc_t buf = buf_rsrc(it.which ? md.V : md.A, (uint32_t)md.kpad * ld * 4u);
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int hl = lane >> 5, ll = lane & 31;
    // byte offsets row * 4 ld of the group's rows in the lanes' order: [block][lane
    // half][e] holds row apply_row(e, hl) of the block (16 per half)
    __shared__ __align__(16) unsigned int roff[4][2][16];
    if (threadIdx.x < 128) {
        const int b = threadIdx.x >> 5, h = (threadIdx.x >> 4) & 1, e = threadIdx.x & 15;
        roff[b][h][e] = (unsigned int)gld(md.perm + blk[b] * kJb + apply_row(e, h)) * (4u * ld);
    }
    __syncthreads();
    const unsigned int ll4 = 4u * ll;
    auto rows4 = [&](int b, int q) { return *(const v4u*)&roff[b][hl][4 * q]; };
    auto col0 = [&](int c) { return it.x0 + c * kQuadCols + wave * 32; };
    auto load = [&](float (&x)[4][16], int c) {
        if (col0(c) >= it.x1) return;
        const int so = __builtin_amdgcn_readfirstlane(col0(c) * 4);
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const v4u ro = rows4(b, q);
#pragma unroll
                for (int e = 0; e < 4; ++e) x[b][4 * q + e] = buf_load_f32<kBufNT>(buf, (int)(ro[e] + ll4), so);
            }
    };
    auto update = [&](const float (&x)[4][16], int c) {
        if (col0(c) >= it.x1) return;
        const int so = __builtin_amdgcn_readfirstlane(col0(c) * 4);
        v16f acc[4];
#pragma unroll
        for (int U = 0; U < 4; ++U)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[U][r] = 0.0f;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            float f[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) f[e] = x[t >> 1][8 * (t & 1) + e];
            const Split8 xs = split8(f);
#pragma unroll
            for (int U = 0; U < 4; ++U) {
                const Split8 r0{Rp[U][0][t][lane], Rp[U][1][t][lane], Rp[U][2][t][lane]};
                acc[U] = mfma_split6(r0, xs, acc[U]);
            }
        }
#pragma unroll
        for (int U = 0; U < 4; ++U)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const v4u ro = rows4(U, q);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    buf_store_f32<kBufNT>(x[U][4 * q + e] + acc[U][4 * q + e], buf, (int)(ro[e] + ll4), so);
            }
    };
    float xa[4][16], xb[4][16];
    load(xa, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int idx = threadIdx.x + kQuadThreads * i;
        const int U = idx >> 9, t = (idx >> 6) & 7, l = idx & 63;
        const Split8 sp = split8(rf[i]);
        Rp[U][0][t][l] = sp.h;
        Rp[U][1][t][l] = sp.m;
        Rp[U][2][t][l] = sp.l;
    }
    __syncthreads();
    const int n = (it.x1 - it.x0 + kQuadCols - 1) / kQuadCols;
    for (int c = 0; c < n; c += 2) {
        if (c + 1 < n) load(xb, c + 1);
        update(xa, c);
        if (c + 1 >= n) break;
        if (c + 2 < n) load(xa, c + 2);
        update(xb, c + 1);
    }
}

hipError_t launch_quad_gram(const MatDev* mats, const MatFlags* flags, const FusedItem* items, int n,
                            int pass, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(jac_quad_gram_kernel, dim3(n), dim3(512), 0, st, mats, flags, items, pass);
    return hipGetLastError();
}

hipError_t launch_quad_solve(const MatDev* mats, MatFlags* flags, const SolveItem* items, int n,
                             int pass, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(jac_quad_solve_kernel, dim3(n), dim3(512), 0, st, mats, flags, items, pass);
    return hipGetLastError();
}

hipError_t launch_quad_apply(const MatDev* mats, const MatFlags* flags, const QuadItem* items, int n,
                             int pass, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(jac_quad_apply_kernel, dim3(n), dim3(kQuadThreads), 0, st, mats, flags, items,
                       pass);
    return hipGetLastError();
}

}  // namespace scopt
