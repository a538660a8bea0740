// Host side of libscopt: the C ABI declared in include/scopt.h.
//
// Argument validation, device-state allocation (one arena per handle), work
// lists and grouped-GEMM problem tables (built once at create), and the
// stream-ordered launch sequences of the anchor update (EMA + SVD refresh)
// and of the optimizer step.  Method: papernotes.org notes on
// "Communication-Efficient LLM Adaptation over Decentralized GPU Meshes",
// "Key design 2" (anchor EMA) and "Key design 3" (SVD, Tikhonov filter,
// two-sided projection, combination), followed by AdamW.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <array>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <thread>
#include <vector>

#include "internal.hpp"
#include "scopt.h"

using namespace scopt;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

#define HIP_TRY(expr)                                                                      \
    do {                                                                                   \
        hipError_t e_ = (expr);                                                            \
        if (e_ != hipSuccess)                                                              \
            return fail(SC_ERR_HIP, "%s failed: %s (%s:%d)", #expr, hipGetErrorString(e_), \
                        __FILE__, __LINE__);                                               \
    } while (0)

constexpr int64_t kMaxDim = 65536;
constexpr int kChunk = 1024;  // elements per elementwise (EMA, AdamW) workgroup

struct DeviceGuard {
    int prev = -1;
    bool ok = false;
    explicit DeviceGuard(int dev) {
        if (hipGetDevice(&prev) == hipSuccess && hipSetDevice(dev) == hipSuccess) ok = true;
    }
    ~DeviceGuard() {
        if (prev >= 0) (void)hipSetDevice(prev);
    }
};

struct GemmGroup {
    std::vector<GemmProb> h;
    GemmProb* d = nullptr;
    int total = 0;
    bool ta = false, tb = false, abf = false, bbf = false;
    int parts = 3;  // 2: correction products (see launch_gemm)
};

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

enum ProfKind {
    PK_EMA, PK_LOAD, PK_ROWNORM, PK_INIT_FLAGS, PK_GRAM, PK_SOLVE, PK_APPLY, PK_SWEEP_END,
    PK_NORMALIZE, PK_LOWDIN, PK_FILTER, PK_PROJECTORS, PK_STEP_GEMM1, PK_STEP_GEMM2,
    PK_STEP_GEMM3, PK_ADAMW, PK_WARM, PK_SORT, PK_CHOL_GEMM, PK_CHOL, PK_POLISH_GEMM,
    PK_GRAM_E, PK_APPLY_GRAM, PK_QUAD_GRAM, PK_QUAD_SOLVE, PK_QUAD_APPLY, PK_COUNT
};
const char* const kProfNames[PK_COUNT] = {
    "ema", "jacobi_load", "rownorm", "jacobi_init", "jacobi_gram", "jacobi_solve",
    "jacobi_apply", "jacobi_sweep_end", "normalize", "lowdin_gemm", "filter", "projector_gemm",
    "step_gemm1", "step_gemm2", "step_gemm3", "combine_adamw", "warm_start", "jacobi_sort",
    "chol_syrk", "cholesky", "polish_gemm", "final_gram", "jacobi_apply_gram", "quad_gram",
    "quad_solve", "quad_apply"};

// Optional kernel timing: HIP events recorded around every launch on the
// caller's stream; totals are folded in by sc_get_kernel_times.
struct Prof {
    bool on = false;
    // serialized: every pipe on the caller's stream and each convergence poll
    // waited for (kernels timed alone); otherwise the launches keep the
    // production schedule (two pipes on their streams, non-blocking polls) and
    // each is timed on the stream it runs on
    bool serial = false;
    // per refresh, a pinned copy of the flags taken behind its last kernel; the
    // work counters of those refreshes are folded in by sc_get_kernel_times
    std::vector<MatFlags*> snaps, snap_pool;
    struct Rec {
        int kind;
        hipEvent_t a, b;
    };
    std::vector<hipEvent_t> pool;
    std::vector<Rec> recs;
    int64_t launches[PK_COUNT] = {};
    double ms[PK_COUNT] = {};
    double flops[PK_COUNT] = {};
    double bytes[PK_COUNT] = {};
};
int round_up(int x, int a) { return (x + a - 1) / a * a; }

// K-splits of a pair Gram over rows of length len (a multiple of 128): about nt
// splits (nt <= 8) of a multiple of 256 columns each, so that the fp64 folds of
// the Gram kernel see whole 256-column chunks.
// Pipelines of the refresh (one internal stream each).
constexpr int kPipes = 2;
constexpr int kMaxSplits = 8;
// Longest split of the fused apply + next Gram: each of its four waves sums its
// Gram tiles over 32 columns per 128-column chunk in float32, at most 256.
constexpr int kFusedMaxCols = 8 * kApplyCols;
int split_len(int len, int nt) { return std::max(256, round_up((len + nt - 1) / nt, 256)); }
int split_count(int len, int nt) { return (len + split_len(len, nt) - 1) / split_len(len, nt); }
// Splits per pair for a launch over `pairs` pairs: enough workgroups to fill the
// chip (about 2048), no more, since every split writes and the solve re-reads a
// 64 x 64 float64 partial.
int splits_for(int pairs) {
    return std::min(kMaxSplits, std::max(1, (2048 + pairs - 1) / std::max(pairs, 1)));
}

}  // namespace

struct sc_opt {
    int device = 0;
    int n = 0;
    sc_dtype wdt = SC_F32, gdt = SC_F32;
    sc_hparams hp{};
    std::vector<MatDev> mh;
    MatDev* md = nullptr;
    MatFlags* flags_d = nullptr;
    MatFlags* flags_h = nullptr;  // pinned
    int* status_d = nullptr;      // [0] non-finite G_mask, [1] non-finite G_anc
    int* status_h = nullptr;      // pinned copy of status_d (sc_get_stats)
    // Recorded on the caller's stream at the end of the last refresh / step, so
    // that the query calls wait for this handle's work only (not device-wide).
    hipEvent_t ev_refresh = nullptr, ev_step = nullptr;
    bool ev_refresh_rec = false, ev_step_rec = false;
    char* arena = nullptr;
    char* proj_arena = nullptr;
    Chunk* chunks_d = nullptr;
    int nchunks = 0;
    // The refresh runs as up to two pipelines ("pipes"), each over its share of
    // the matrices on its own internal stream (default priority) with its own
    // work lists, GEMM tables and progress: one pipe's MFMA-bound GEMMs and
    // latency-bound pair solves overlap the other's memory-bound sweeps, and
    // neither waits for the other's convergence checks.  Jacobi work lists come
    // in three sets: plain
    // (every matrix of the pipe, full rows), factor (every matrix; preconditioned
    // ones over their klen-long factor rows, without V) and polish (only the
    // preconditioned matrices, full rows).
    struct Lists {
        GramItem* gi = nullptr;
        int ngi = 0;
        SolveItem* si = nullptr;
        int nsi = 0;
        ApplyItem* ai = nullptr;
        int nai = 0;
        // with the fused apply: every item of ai except the A rows of the matrices
        // in fi, whose apply comes with the next round's Gram
        ApplyItem* ai_f = nullptr;
        int nai_f = 0;
        FusedItem* fi = nullptr;
        int nfi = 0;
        // with the fused apply: the V rows of the matrices in fi, two rounds per pass
        // (jac_apply_v2_kernel; columns of V in x0 / x1), and their block counts
        FusedItem* vi = nullptr;
        int nvi = 0;
        std::vector<int> vnbs;
        ApplyItem* av = nullptr;  // the same V rows one round per pass (sc_set_v_rounds 1)
        int nav = 0;
        bool all_fused = false;  // every matrix of the list has the fused apply + Gram
        // quad passes (every matrix's block count quad_capable, not polishing): group
        // Grams, group solves, group applies (A and V rows); quad_auto: also enough
        // groups per pass to fill the GPU (kQuadMinGroups)
        bool quad = false, quad_auto = false;
        FusedItem* qg = nullptr;
        int nqg = 0;
        SolveItem* qs = nullptr;
        int nqs = 0;
        QuadItem* qa = nullptr;
        int nqa = 0;
        int* mats = nullptr;
        int nmat = 0;
        int max_nb = 2;
        std::vector<int> nbs;  // distinct block counts of the list's matrices
    };
    struct Pipe {
        Lists L[3];
        std::vector<int> host_mats;
        int* mats = nullptr;  // every matrix of the pipe
        int nmat = 0;
        int* cap = nullptr;   // those with a factor phase (max(m, n) >= 2 min(m, n))
        int ncap = 0;
        SyrkItem* syrk_cap = nullptr;  // lower 128 x 128 tiles of A^T A, factor-phase matrices
        int nsyrk_cap = 0;
        SyrkItem* syrk_all = nullptr;  // the same for every matrix (final Gram)
        int nsyrk_all = 0;
        bool syrk_cap_full = true, syrk_all_full = true;  // every k a multiple of 128
        int max_kpad = 64, max_K = 128, max_k = 1, max_nbk = 0, max_klen = 0, max_t64 = 1;
        GemmGroup warm_nt, warm_nn;      // warm start: A_rows = W M^T (m >= n) or W M (m < n)
        GemmGroup factor_v;              // V rows <- diag(1/|x_j|) X^T V_prev (gated per matrix)
        GemmGroup polish_nt, polish_nn;  // A_rows = V op(M) after the factor phase
        GemmGroup lowdin_F, lowdin_eW, lowdin_W, proj;
        hipStream_t st = nullptr;
        hipEvent_t join = nullptr, poll = nullptr;
        MatFlags* flags_h = nullptr;  // pinned target of this pipe's flag polls
        // progress of the refresh in flight
        int stage = 0, which = 0, r = 0, rps = 1, max_rounds = 0, first_check = 0, poll_round = 0;
        bool pre = false, poll_pending = false;
        bool targeted = false;  // polishing sweeps restricted to the pairs the certificate marks
        bool resumed = false;   // plain sweeps resumed after the sweep-stop rule's certificate
    } pipes[kPipes];
    int npipes = 0;
    hipEvent_t fork = nullptr;
    bool have_factors = false;   // W holds orthonormal rows from a refresh / sc_set_factors
    // step GEMMs: [0] read the refresh's step operands (F, P_L, P_R, d); [1] read
    // the copy published when an asynchronous refresh starts
    GemmGroup step[2][6];
    // sc_step_noalloc: the same chain in batches over the file-scope scratch array
    struct NoAllocBatch {
        GemmGroup g[6];
    };
    std::vector<NoAllocBatch> na;
    std::string na_err;  // why the handle cannot use it ("" when it can)
    // asynchronous refresh (sc_anchor_update_async): a host worker thread drives
    // the refresh on the internal streams behind `astream`; steps issued until
    // sc_refresh_wait (or another entry point) completes it use step[1] on the
    // published operands; completion joins the worker and makes the caller's
    // stream wait for a_done
    struct PubBuf {
        float *F, *PL, *PR, *d;
    };
    std::vector<PubBuf> pub;
    char* pub_arena = nullptr;
    hipStream_t astream = nullptr;
    hipEvent_t a_ready = nullptr, a_pub = nullptr, a_done = nullptr;
    std::thread worker;
    std::atomic<bool> a_finished{false};
    bool a_pending = false;
    int a_rc = 0;
    std::string a_err;
    int64_t t = 0;
    int refreshes = 0;
    std::vector<char> stale;
    bool any_stale = false;
    bool proj_stale = false;
    bool keep_proj = false;
    bool fuse = true;                         // fused apply + next Gram where a matrix allows it
    int v_rounds = 2;                         // fused matrices' V rows: rounds per pass (1 or 2)
    float sweep_stop = 1e-4f;                 // sweep-stop rule (0 = off), see jac_sweep_end_kernel
    std::vector<std::array<char, 2>> fused;   // per matrix: fused over the factor / full rows
    int quad_mode = 1;                        // quad passes: 0 off, 1 where a list fills the GPU, 2 where allowed
    std::vector<std::array<char, 2>> quadm;   // per matrix, factor / full rows: 1 quad-capable list, 2 also filling
    int solve_waves = 0, solve_copies = 0;  // pair solve variant: 0 by the launch's pair count
    std::vector<void*> dev_allocs;
    Prof prof;
    double total_numel = 0.0;
    double ema_bytes = 0.0;    // read M, read G_anc, write M
    double adamw_bytes = 0.0;  // read G, G_filt, W, m, v; write W, m, v
};

namespace {

int upload_group(sc_opt* h, GemmGroup& g) {
    int start = 0;
    for (auto& p : g.h) {
        int tm = (p.M + kGemmBM - 1) / kGemmBM;
        p.tiles_n = (p.N + kGemmBN - 1) / kGemmBN;
        p.tile_start = start;
        start += tm * p.tiles_n;
    }
    g.total = start;
    if (g.h.empty()) return SC_OK;
    void* d = nullptr;
    HIP_TRY(hipMalloc(&d, sizeof(GemmProb) * g.h.size()));
    h->dev_allocs.push_back(d);
    g.d = (GemmProb*)d;
    HIP_TRY(hipMemcpy(g.d, g.h.data(), sizeof(GemmProb) * g.h.size(), hipMemcpyHostToDevice));
    return SC_OK;
}

GemmProb make_prob(const void* A, int lda, const void* B, int ldb, float* C, int ldc, int M, int N,
                   int K) {
    GemmProb p;
    memset(&p, 0, sizeof(p));
    p.A = A;
    p.B = B;
    p.C = C;
    p.lda = lda;
    p.ldb = ldb;
    p.ldc = ldc;
    p.M = M;
    p.N = N;
    p.K = K;
    p.alpha = 1.0f;
    p.beta = 0.0f;
    p.a_ptr = -1;
    p.b_ptr = -1;
    return p;
}

hipEvent_t prof_event(Prof& p) {
    hipEvent_t e = nullptr;
    if (!p.pool.empty()) {
        e = p.pool.back();
        p.pool.pop_back();
    } else if (hipEventCreate(&e) != hipSuccess) {
        (void)hipGetLastError();
        e = nullptr;
    }
    return e;
}

// Run `launch` (returns hipError_t); when profiling, bracket it with events.
template <typename F>
hipError_t timed(sc_opt* h, int kind, hipStream_t st, F launch) {
    if (!h->prof.on) return launch();
    hipEvent_t a = prof_event(h->prof), b = prof_event(h->prof);
    if (a) (void)hipEventRecord(a, st);
    hipError_t e = launch();
    if (b) (void)hipEventRecord(b, st);
    if (a && b) h->prof.recs.push_back(Prof::Rec{kind, a, b});
    h->prof.launches[kind] += 1;
    return e;
}

double group_flops(const GemmGroup& g) {
    double f = 0.0;
    for (const auto& p : g.h) f += 2.0 * p.M * (double)p.N * p.K;
    return f;
}

// Whether every problem of a group can load its row-major operands (A unless
// transposed, B if transposed) 8 elements at a time: rows aligned to 16 bytes
// (8 for bfloat16) and K a multiple of 8.  Caller pointers (a_ptr / b_ptr) are
// aligned by check_ptrs.
bool group_vec(const GemmGroup& g, const PtrTable& pt) {
    for (const GemmProb& p : g.h) {
        if (p.K % 8) return false;
        if (!g.ta) {
            const uintptr_t a = (uintptr_t)(p.a_ptr >= 0 ? pt.p[p.a_ptr] : p.A);
            if (p.lda % 4 || a % (g.abf ? 8 : 16)) return false;
        }
        if (g.tb) {
            const uintptr_t b = (uintptr_t)(p.b_ptr >= 0 ? pt.p[p.b_ptr] : p.B);
            if (p.ldb % 4 || b % (g.bbf ? 8 : 16)) return false;
        }
    }
    return true;
}

// Whether every problem of a group tiles exactly (M, N, K multiples of the tile).
bool group_full(const GemmGroup& g) {
    for (const GemmProb& p : g.h)
        if (p.M % kGemmBM || p.N % kGemmBN || p.K % 16) return false;
    return true;
}

int run_group(sc_opt* h, const GemmGroup& g, int kind, const PtrTable& pt, hipStream_t st) {
    if (g.h.empty()) return SC_OK;
    const bool vec = group_vec(g, pt), full = group_full(g);
    HIP_TRY(timed(h, kind, st, [&] {
        return launch_gemm(g.d, (int)g.h.size(), g.total, g.ta, g.tb, g.abf, g.bbf, vec, full, g.parts,
                           pt, st);
    }));
    if (h->prof.on) h->prof.flops[kind] += group_flops(g);
    return SC_OK;
}

int check_hp(const sc_hparams* hp) {
    if (!hp) return fail(SC_ERR_INVALID_ARG, "hparams is NULL");
    if (!(hp->tau_p >= 0.0f) || !std::isfinite(hp->tau_p))
        return fail(SC_ERR_INVALID_ARG, "tau_p must be finite and >= 0");
    if (!(hp->alpha >= 0.0f && hp->alpha <= 1.0f))
        return fail(SC_ERR_INVALID_ARG, "alpha must be in [0, 1]");
    if (!(hp->beta_anc >= 0.0f && hp->beta_anc <= 1.0f))
        return fail(SC_ERR_INVALID_ARG, "beta_anc must be in [0, 1]");
    if (!(hp->lr >= 0.0f) || !std::isfinite(hp->lr))
        return fail(SC_ERR_INVALID_ARG, "lr must be finite and >= 0");
    if (!(hp->beta1 >= 0.0f && hp->beta1 < 1.0f) || !(hp->beta2 >= 0.0f && hp->beta2 < 1.0f))
        return fail(SC_ERR_INVALID_ARG, "beta1 and beta2 must be in [0, 1)");
    if (!(hp->eps > 0.0f) || !std::isfinite(hp->eps))
        return fail(SC_ERR_INVALID_ARG, "eps must be finite and > 0");
    if (!(hp->weight_decay >= 0.0f) || !std::isfinite(hp->weight_decay))
        return fail(SC_ERR_INVALID_ARG, "weight_decay must be finite and >= 0");
    if (hp->max_sweeps < 1 || hp->max_sweeps > 1000)
        return fail(SC_ERR_INVALID_ARG, "max_sweeps must be in [1, 1000]");
    if (!(hp->jacobi_tol >= 0.0f && hp->jacobi_tol < 1.0f))
        return fail(SC_ERR_INVALID_ARG, "jacobi_tol must be in [0, 1)");
    if ((hp->sync_check != 0 && hp->sync_check != 1) || (hp->warm_start != 0 && hp->warm_start != 1) ||
        (hp->precondition != 0 && hp->precondition != 1))
        return fail(SC_ERR_INVALID_ARG, "sync_check, warm_start and precondition must be 0 or 1");
    return SC_OK;
}

int check_ptrs(const sc_opt* h, const void* const* p, sc_dtype dt, const char* what) {
    if (!p) return fail(SC_ERR_INVALID_ARG, "%s pointer array is NULL", what);
    const uintptr_t mask = dt == SC_F32 ? 15 : 7;
    for (int i = 0; i < h->n; ++i) {
        if (!p[i]) return fail(SC_ERR_INVALID_ARG, "%s[%d] is NULL", what, i);
        if ((uintptr_t)p[i] & mask)
            return fail(SC_ERR_INVALID_ARG, "%s[%d] is not %d-byte aligned", what, i,
                        (int)(mask + 1));
    }
    return SC_OK;
}

PtrTable make_table(const sc_opt* h, const void* const* p) {
    PtrTable t;
    memset(&t, 0, sizeof(t));
    if (p)
        for (int i = 0; i < h->n; ++i) t.p[i] = p[i];
    return t;
}

// ---- refresh ------------------------------------------------------------------------

enum { LIST_PLAIN = 0, LIST_FACTOR = 1, LIST_POLISH = 2 };
// STAGE_CERT: waiting for the certificate of the factor phase's A = M V;
// STAGE_CERT2: for the re-certification after selective polishing
// STAGE_CERTP: for the certificate of plain sweeps that ended on the sweep-stop rule
enum { STAGE_ROUNDS = 0, STAGE_CERT = 1, STAGE_CERT2 = 2, STAGE_DONE = 3, STAGE_CERTP = 4 };
typedef sc_opt::Pipe Pipe;

// d = s / (s + tau) and the projectors X^T diag(d) X of the pipe's matrices.
int pipe_projectors(sc_opt* h, Pipe& p, hipStream_t st) {
    HIP_TRY(timed(h, PK_FILTER, st,
                  [&] { return launch_filter(h->md, p.mats, p.nmat, h->hp.tau_p, st); }));
    return run_group(h, p.proj, PK_PROJECTORS, make_table(h, nullptr), st);
}

int build_projectors(sc_opt* h, hipStream_t st) {
    for (int q = 0; q < h->npipes; ++q) {
        int rc = pipe_projectors(h, h->pipes[q], st);
        if (rc) return rc;
    }
    h->proj_stale = false;
    return SC_OK;
}

// chol = A^T A (float64 sums) and E = its normalized off-diagonal part; with
// only_regram, for the matrices polished after failing the certificate alone.
int pipe_final_gram(sc_opt* h, Pipe& p, hipStream_t st, bool only_regram = false) {
    HIP_TRY(timed(h, PK_GRAM_E, st, [&] {
        return launch_chol_syrk(h->md, h->flags_d, p.syrk_all, p.nsyrk_all, only_regram, p.syrk_all_full, st);
    }));
    HIP_TRY(timed(h, PK_GRAM_E, st, [&] {
        return launch_gram_to_e(h->md, h->flags_d, p.mats, p.nmat, p.max_t64, only_regram, st);
    }));
    if (h->prof.on)
        for (int i : p.host_mats) {
            if (only_regram && !(h->mh[i].klen && !p.flags_h[i].done)) continue;
            const double kt = (h->mh[i].k + 127) / 128;
            h->prof.flops[PK_GRAM_E] += kt * (kt + 1) / 2 * 2.0 * 128 * 128 * h->mh[i].K_ld;
        }
    return SC_OK;
}

// Unit rows, s_j = |a_j| / |v_j|, one Loewdin step on both factors, projectors.
int pipe_finalize(sc_opt* h, Pipe& p, hipStream_t st) {
    PtrTable none = make_table(h, nullptr);
    for (int which = 0; which < 2; ++which) {
        HIP_TRY(timed(h, PK_ROWNORM, st, [&] {
            return launch_rownorm(h->md, p.mats, p.nmat, which, p.max_kpad, st);
        }));
        HIP_TRY(timed(h, PK_NORMALIZE, st, [&] {
            return launch_normalize(h->md, p.mats, h->flags_d, p.nmat, which, p.max_kpad, st);
        }));
    }
    int rc;
    // E (normalized Gram of the A-side rows, zero diagonal) comes from the final Gram
    if ((rc = run_group(h, p.lowdin_F, PK_LOWDIN, none, st))) return rc;
    if ((rc = run_group(h, p.lowdin_eW, PK_LOWDIN, none, st))) return rc;
    if ((rc = run_group(h, p.lowdin_W, PK_LOWDIN, none, st))) return rc;
    return pipe_projectors(h, p, st);
}

// Algorithmic work of the Jacobi sweeps from the device counters (profiling only):
// per active round and pair the 64x64 Gram over the row length L (2 * 64 * 64 * L
// flops, 4 * 64 * L bytes); per applied pair the update of 64 rows of the operand
// (length L) and of V (length k), 2 * 64 * 64 * (L + k) flops and
// 8 * 64 * (L + k) + 4 * 64 * 64 bytes.  In the factor phase L = klen and V is not
// touched (its k term drops out); otherwise L = K.  Per rotated pair the solve
// applies one cyclic sweep of 64 * 63 / 2 rotations, each to two rows and two
// columns of the 64 x 64 Gram and to two rows of R: 18 * 64 flops per rotation
// (vector ALU work, no HBM traffic).
void account_sweeps(sc_opt* h, const MatFlags* flags) {
    for (int i = 0; i < h->n; ++i) {
        const MatDev& m = h->mh[i];
        const MatFlags& f = flags[i];
        const double pw = kPw;
        // a matrix stops only at the end of one of its sweeps (nb - 1 rounds each)
        const double rounds[2] = {(double)f.sweep_base * (m.nb - 1),
                                  (double)(f.sweeps - f.sweep_base) * (m.nb - 1)};
        const double pairs[2] = {(double)f.pairs_pre, (double)(f.pairs_applied - f.pairs_pre)};
        const double len[2] = {(double)m.klen, (double)m.K};
        const double vlen[2] = {0.0, (double)m.k};
        // selective polishing sweeps (few pairs, unfused: each Gram from the operand,
        // rotated pairs' A and V rows) apart from the full sweeps
        const double sel_sw = f.sel_sweeps;
        const double rounds_sel = sel_sw * (m.nb - 1);
        const double sweeps[2] = {(double)f.sweep_base, (double)(f.sweeps - f.sweep_base) - sel_sw};
        const double rounds_full[2] = {rounds[0], rounds[1] - rounds_sel};
        const double pairs_full[2] = {pairs[0], pairs[1] - f.sel_rot};
        if (f.sel_sweeps > 0) {
            const double L = m.K;
            h->prof.flops[PK_SOLVE] += f.sel_rot * (pw * (pw - 1) / 2) * 18.0 * pw;
            h->prof.flops[PK_GRAM] += f.sel_pairs * 2.0 * pw * pw * L;
            h->prof.bytes[PK_GRAM] += f.sel_pairs * 4.0 * pw * L;
            h->prof.flops[PK_APPLY] += f.sel_rot * 2.0 * pw * pw * (L + m.k);
            h->prof.bytes[PK_APPLY] += f.sel_rot * (8.0 * pw * (L + m.k) + 4.0 * pw * pw);
        }
        const double quads[2] = {(double)f.quads_pre, (double)(f.quads_applied - f.quads_pre)};
        for (int ph = 0; ph < 2; ++ph) {
            const int qm = h->quadm[i][ph];
            if (h->quad_mode == 2 ? qm >= 1 : h->quad_mode == 1 ? qm == 2 : false) {
                // quad passes: every group's 128 rows read by the group Gram every pass
                // (ten 32 x 32 tiles); the solve's pair sweeps as in the pair rounds; a
                // group with a rotation has its 128 rows of the operand and of V read and
                // written once, plus R (128 x 128)
                const double qn = 4.0 * kJb;
                const double gpass = sweeps[ph] * quad_passes(m.nb) * (m.nb / 4);
                h->prof.flops[PK_QUAD_GRAM] += gpass * 10.0 * 2.0 * kJb * kJb * len[ph];
                h->prof.bytes[PK_QUAD_GRAM] += gpass * 4.0 * qn * len[ph];
                h->prof.flops[PK_QUAD_SOLVE] += pairs_full[ph] * (pw * (pw - 1) / 2) * 18.0 * pw;
                h->prof.flops[PK_QUAD_APPLY] += quads[ph] * 2.0 * qn * qn * (len[ph] + vlen[ph]);
                h->prof.bytes[PK_QUAD_APPLY] +=
                    quads[ph] * (8.0 * qn * (len[ph] + vlen[ph]) + 4.0 * qn * qn);
                continue;
            }
            h->prof.flops[PK_SOLVE] += pairs_full[ph] * (pw * (pw - 1) / 2) * 18.0 * pw;
            if (h->fuse && h->fused[i][ph]) {
                // Gram read standalone in a sweep's first round only; the fused
                // kernel reads every pair's rows every round, writes the rotated
                // ones, and forms three 32 x 32 tiles per pair of the next round
                h->prof.flops[PK_GRAM] += sweeps[ph] * (m.nb / 2) * 2.0 * pw * pw * len[ph];
                h->prof.bytes[PK_GRAM] += sweeps[ph] * (m.nb / 2) * 4.0 * pw * len[ph];
                h->prof.flops[PK_APPLY_GRAM] +=
                    pairs_full[ph] * 2.0 * pw * pw * len[ph] +
                    (rounds_full[ph] - sweeps[ph]) * (m.nb / 2) * 3.0 * 2.0 * 32 * 32 * len[ph];
                h->prof.bytes[PK_APPLY_GRAM] += rounds_full[ph] * (m.nb / 2) * 4.0 * pw * len[ph] +
                                                pairs_full[ph] * (4.0 * pw * len[ph] + 4.0 * pw * pw);
                if (vlen[ph] > 0.0) {
                    // V rows of a rotated pair read and written once per round, or
                    // once per two rounds (jac_apply_v2_kernel), plus R
                    const double vpass = h->v_rounds == 2 ? 4.0 : 8.0;
                    h->prof.flops[PK_APPLY] += pairs_full[ph] * 2.0 * pw * pw * vlen[ph];
                    h->prof.bytes[PK_APPLY] += pairs_full[ph] * (vpass * pw * vlen[ph] + 4.0 * pw * pw);
                }
            } else {
                h->prof.flops[PK_GRAM] += rounds_full[ph] * (m.nb / 2) * 2.0 * pw * pw * len[ph];
                h->prof.bytes[PK_GRAM] += rounds_full[ph] * (m.nb / 2) * 4.0 * pw * len[ph];
                h->prof.flops[PK_APPLY] += pairs_full[ph] * 2.0 * pw * pw * (len[ph] + vlen[ph]);
                h->prof.bytes[PK_APPLY] +=
                    pairs_full[ph] * (8.0 * pw * (len[ph] + vlen[ph]) + 4.0 * pw * pw);
            }
        }
    }
}

// Start of a refresh for one pipe: operand A (warm: A = M V_prev; cold: A = M),
// row norms, flags, and for the factor phase A^T A and its Cholesky factor.
int pipe_pre(sc_opt* h, Pipe& p, hipStream_t st, bool warm) {
    PtrTable none = make_table(h, nullptr);
    int rc;
    if (warm) {
        HIP_TRY(timed(h, PK_WARM, st,
                      [&] { return launch_jacobi_warm(h->md, p.mats, p.nmat, st); }));
        if ((rc = run_group(h, p.warm_nt, PK_WARM, none, st))) return rc;
        if ((rc = run_group(h, p.warm_nn, PK_WARM, none, st))) return rc;
    } else {
        HIP_TRY(timed(h, PK_LOAD, st, [&] {
            return launch_jacobi_load(h->md, p.mats, p.nmat, p.max_kpad, p.max_K + 128, st);
        }));
    }
    HIP_TRY(timed(h, PK_ROWNORM, st,
                  [&] { return launch_rownorm(h->md, p.mats, p.nmat, 0, p.max_kpad, st); }));
    HIP_TRY(timed(h, PK_INIT_FLAGS, st, [&] {
        return launch_jacobi_init_flags(h->md, p.mats, h->flags_d, p.nmat, st);
    }));
    if (p.pre) {
        // Factor phase: Jacobi on X = L, A^T A = L L^T (k-long rows, no V).
        HIP_TRY(timed(h, PK_CHOL_GEMM, st, [&] {
            return launch_chol_syrk(h->md, h->flags_d, p.syrk_cap, p.nsyrk_cap, 0, p.syrk_cap_full, st);
        }));
        HIP_TRY(timed(h, PK_CHOL, st, [&] {
            return launch_cholesky(h->md, h->flags_d, p.cap, p.ncap, p.max_nbk, p.max_klen, st);
        }));
        if (h->prof.on)
            for (int i : p.host_mats)
                if (h->mh[i].klen) {
                    const double kt = (h->mh[i].k + 127) / 128;
                    h->prof.flops[PK_CHOL_GEMM] +=
                        kt * (kt + 1) / 2 * 2.0 * 128 * 128 * h->mh[i].K_ld;
                    h->prof.flops[PK_CHOL] += std::pow((double)h->mh[i].k, 3) / 3.0;
                }
    }
    return SC_OK;
}

// Rounds of list set `which` until every matrix of the pipe is done.  The host
// polls once per `rps` rounds: a sweep of the largest matrix still in work
// (max_nb; 0 = the largest of the list).  Each matrix counts its own sweeps.
// Quad passes for this list under the handle's mode.
bool use_quad(const sc_opt* h, const sc_opt::Lists& L) {
    return h->quad_mode == 2 ? L.quad : h->quad_mode == 1 ? L.quad_auto : false;
}

void pipe_start_rounds(sc_opt* h, Pipe& p, int which, int first_check_sweeps, int max_nb = 0) {
    p.stage = STAGE_ROUNDS;
    p.which = which;
    p.r = 0;
    const int nbl = max_nb ? max_nb : p.L[which].max_nb;
    p.rps = use_quad(h, p.L[which]) ? quad_passes(nbl) : std::max(1, nbl - 1);
    const int cap = p.targeted ? std::min(kSelSweeps, h->hp.max_sweeps) : h->hp.max_sweeps;
    p.max_rounds = p.L[which].nmat ? cap * p.rps : 0;
    p.first_check = std::min(p.max_rounds, first_check_sweeps * p.rps);
    p.poll_pending = false;
}

// One Jacobi round of the pipe's current list set.
// The sweep-stop rule in the Cholesky factor phase is capped: the certificate
// that follows checks A = M V but not V, whose orthogonality comes from the
// factor's convergence (V <- normalized X^T V_prev); on the 16-block workload a
// factor sweep that saw at most 1e-4 was followed by one that saw only the
// rotation threshold, so V is as orthogonal as after a sweep that sees nothing.
constexpr float kFactorStopMax = 1e-4f;
// The sweep-stop rule for plain sweeps: only where the host polls (the
// certificate's outcome decides whether sweeps resume) and not after a resume.
// A and V are rotated together there, so the final Gram's certificate covers it.
float plain_stop(const sc_opt* h, const Pipe& p) {
    return p.which == LIST_PLAIN && h->hp.sync_check && !p.resumed ? h->sweep_stop : 0.0f;
}

float factor_stop(const sc_opt* h, const Pipe& p) {
    return p.which == LIST_FACTOR ? std::min(h->sweep_stop, kFactorStopMax) : 0.0f;
}

// One quad pass (three pair rounds over groups of four blocks) of the pipe's list.
int pipe_quad_pass(sc_opt* h, Pipe& p, hipStream_t st) {
    const sc_opt::Lists& L = p.L[p.which];
    const int r = p.r;
    bool first = false, last = false;
    for (int nb : L.nbs) {
        first = first || r % quad_passes(nb) == 0;
        last = last || r % quad_passes(nb) == quad_passes(nb) - 1;
    }
    if (first)
        HIP_TRY(timed(h, PK_SORT, st, [&] {
            return launch_jacobi_sort(h->md, h->flags_d, L.mats, L.nmat, r, 1, st);
        }));
    HIP_TRY(timed(h, PK_QUAD_GRAM, st,
                  [&] { return launch_quad_gram(h->md, h->flags_d, L.qg, L.nqg, r, st); }));
    HIP_TRY(timed(h, PK_QUAD_SOLVE, st,
                  [&] { return launch_quad_solve(h->md, h->flags_d, L.qs, L.nqs, r, st); }));
    HIP_TRY(timed(h, PK_QUAD_APPLY, st,
                  [&] { return launch_quad_apply(h->md, h->flags_d, L.qa, L.nqa, r, st); }));
    if (last)
        HIP_TRY(timed(h, PK_SWEEP_END, st, [&] {
            return launch_jacobi_sweep_end(h->md, h->flags_d, L.mats, L.nmat, r, 1, h->hp.max_sweeps,
                                           factor_stop(h, p), plain_stop(h, p), st);
        }));
    return SC_OK;
}

int pipe_round(sc_opt* h, Pipe& p, hipStream_t st) {
    const sc_opt::Lists& L = p.L[p.which];
    if (use_quad(h, L)) return pipe_quad_pass(h, p, st);
    const int r = p.r;
    // the sort acts on the first round of a matrix's sweep, the sweep end on its
    // last: launched only in rounds where some matrix of the list has one
    bool first = false, last = false;
    for (int nb : L.nbs) {
        first = first || r % (nb - 1) == 0;
        last = last || r % (nb - 1) == nb - 2;
    }
    if (first)
        HIP_TRY(timed(h, PK_SORT, st, [&] {
            return launch_jacobi_sort(h->md, h->flags_d, L.mats, L.nmat, r, 0, st);
        }));
    // with every matrix fused the standalone Gram only serves sweeps' first rounds;
    // selective polishing works on few pairs per round, each Gram from the operand
    const bool fuse = h->fuse && !p.targeted;
    if (!(fuse && L.all_fused) || first)
        HIP_TRY(timed(h, PK_GRAM, st, [&] {
            return launch_jacobi_gram(h->md, h->flags_d, L.gi, L.ngi, r, fuse ? 1 : 0, st);
        }));
    HIP_TRY(timed(h, PK_SOLVE, st,
                  [&] { return launch_jacobi_solve(h->md, h->flags_d, L.si, L.nsi, r, h->solve_waves, h->solve_copies, st); }));
    if (fuse && L.nfi) {
        if (L.nai_f)
            HIP_TRY(timed(h, PK_APPLY, st, [&] {
                return launch_jacobi_apply(h->md, h->flags_d, L.ai_f, L.nai_f, r, st);
            }));
        // V rows two rounds at a time: a sweep's odd rounds and its last round
        bool vround = false;
        for (int nb : L.vnbs) vround = vround || (r % (nb - 1)) % 2 == 1 || r % (nb - 1) == nb - 2;
        if (h->v_rounds == 2 && L.nvi && vround)
            HIP_TRY(timed(h, PK_APPLY, st, [&] {
                return launch_jacobi_apply_v2(h->md, h->flags_d, L.vi, L.nvi, r, st);
            }));
        if (h->v_rounds == 1 && L.nav)
            HIP_TRY(timed(h, PK_APPLY, st, [&] {
                return launch_jacobi_apply(h->md, h->flags_d, L.av, L.nav, r, st);
            }));
        HIP_TRY(timed(h, PK_APPLY_GRAM, st, [&] {
            return launch_jacobi_apply_gram(h->md, h->flags_d, L.fi, L.nfi, r, st);
        }));
    } else {
        HIP_TRY(timed(h, PK_APPLY, st,
                      [&] { return launch_jacobi_apply(h->md, h->flags_d, L.ai, L.nai, r, st); }));
    }
    if (last)
        HIP_TRY(timed(h, PK_SWEEP_END, st, [&] {
            return launch_jacobi_sweep_end(h->md, h->flags_d, L.mats, L.nmat, r, 0, h->hp.max_sweeps,
                                           factor_stop(h, p), plain_stop(h, p), st);
        }));
    return SC_OK;
}

// Copy the flags to the pipe's pinned buffer behind the work queued so far and
// mark the point with an event; the host polls it without blocking the queues.
// With kernel timing on, the host waits for it at once: no rounds are queued
// past a pending check, so the launch sequence does not depend on host timing.
int pipe_poll(sc_opt* h, Pipe& p, hipStream_t st) {
    HIP_TRY(hipMemcpyAsync(p.flags_h, h->flags_d, sizeof(MatFlags) * h->n, hipMemcpyDeviceToHost,
                           st));
    HIP_TRY(hipEventRecord(p.poll, st));
    if (h->prof.on && h->prof.serial) HIP_TRY(hipEventSynchronize(p.poll));
    p.poll_pending = true;
    return SC_OK;
}

bool pipe_all_done(const sc_opt* h, const Pipe& p) {
    for (int i : p.host_mats)
        if (!p.flags_h[i].done) return false;
    return true;
}

// End of a pipe's sweeps.  After the factor phase: V from the factor, A = M V,
// the final Gram and its certificate (polled); otherwise the final Gram and the
// finalization.
// Selective polishing of the matrices that failed the certificate: mark their
// pairs with a block above the threshold, then at most kSelSweeps sweeps that
// work only on those pairs (max_nb: rounds per sweep; 0 = the list's largest).
int pipe_start_selective(sc_opt* h, Pipe& p, hipStream_t st, int max_nb) {
    HIP_TRY(timed(h, PK_INIT_FLAGS, st, [&] {
        return launch_polish_mark(h->md, h->flags_d, p.cap, p.ncap, p.L[LIST_POLISH].max_nb, st);
    }));
    p.targeted = true;
    pipe_start_rounds(h, p, LIST_POLISH, 1, max_nb);
    return SC_OK;
}

// Full polishing sweeps for the matrices the re-certification still rejects.
int pipe_start_full_polish(sc_opt* h, Pipe& p, hipStream_t st, int max_nb) {
    HIP_TRY(timed(h, PK_INIT_FLAGS, st,
                  [&] { return launch_polish_full(h->flags_d, p.cap, p.ncap, st); }));
    p.targeted = false;
    pipe_start_rounds(h, p, LIST_POLISH, 1, max_nb);
    return SC_OK;
}

// polled: the pipe's host flags show the state after its last round (a poll saw
// every matrix done), so they tell whether any plain sweeps ended on the sweep-stop rule.
int pipe_after_rounds(sc_opt* h, Pipe& p, hipStream_t st, bool polled) {
    int rc;
    if (p.which == LIST_POLISH && p.targeted) {
        // re-certify: the Gram of the selectively polished matrices again, then the
        // certificate over every factor-phase matrix (the others keep theirs)
        if ((rc = pipe_final_gram(h, p, st, true))) return rc;
        HIP_TRY(timed(h, PK_INIT_FLAGS, st,
                      [&] { return launch_certify(h->md, h->flags_d, p.cap, p.ncap, st); }));
        p.targeted = false;
        if (!h->hp.sync_check) return pipe_start_full_polish(h, p, st, 0);
        p.stage = STAGE_CERT2;
        return pipe_poll(h, p, st);
    }
    if (p.which == LIST_FACTOR) {
        // Right singular vectors of A from the factor phase: V <- diag(1/|x_j|) X^T V_prev
        // (rows), then the true operand A = M V.  A rejected matrix keeps V = V_prev and
        // gets back its unchanged operand (it runs all its sweeps in the polishing phase).
        PtrTable none = make_table(h, nullptr);
        HIP_TRY(timed(h, PK_POLISH_GEMM, st, [&] {
            return launch_factor_invnorm(h->md, h->flags_d, p.cap, p.ncap, p.max_k, st);
        }));
        if ((rc = run_group(h, p.factor_v, PK_POLISH_GEMM, none, st))) return rc;
        if ((rc = run_group(h, p.polish_nt, PK_POLISH_GEMM, none, st))) return rc;
        if ((rc = run_group(h, p.polish_nn, PK_POLISH_GEMM, none, st))) return rc;
        HIP_TRY(timed(h, PK_INIT_FLAGS, st,
                      [&] { return launch_phase2_reset(h->md, h->flags_d, p.cap, p.ncap, st); }));
        // the Gram of every final operand in float64 sums: the Loewdin step's E and the
        // certificate that A = M V is converged; only matrices failing it are polished
        if ((rc = pipe_final_gram(h, p, st))) return rc;
        HIP_TRY(timed(h, PK_INIT_FLAGS, st,
                      [&] { return launch_certify(h->md, h->flags_d, p.cap, p.ncap, st); }));
        if (!h->hp.sync_check) {
            // enqueue only: selective, then full polishing rounds for every
            // factor-phase matrix; certified ones are done, their launches exit at once
            return pipe_start_selective(h, p, st, 0);
        }
        p.stage = STAGE_CERT;
        return pipe_poll(h, p, st);
    }
    bool early = plain_stop(h, p) > 0.0f;
    if (early && polled) {
        early = false;
        for (int i : p.host_mats) early = early || p.flags_h[i].early;
    }
    if (early) {
        // plain sweeps that ended on the sweep-stop rule: the final Gram's certificate;
        // failing matrices sweep on (polled)
        if ((rc = pipe_final_gram(h, p, st))) return rc;
        HIP_TRY(timed(h, PK_INIT_FLAGS, st, [&] {
            return launch_certify_early(h->md, h->flags_d, p.L[LIST_PLAIN].mats,
                                        p.L[LIST_PLAIN].nmat, st);
        }));
        p.stage = STAGE_CERTP;
        return pipe_poll(h, p, st);
    }
    if ((rc = pipe_final_gram(h, p, st, p.which == LIST_POLISH || p.resumed))) return rc;
    if ((rc = pipe_finalize(h, p, st))) return rc;
    p.stage = STAGE_DONE;
    return SC_OK;
}

int do_refresh(sc_opt* h, hipStream_t st) {
    int rc;
    const bool warm = h->hp.warm_start && h->have_factors;
    // With kernel timing on, every pipe runs on the caller's stream so that each
    // kernel's events bracket it alone (no overlap between pipes).
    const bool split = !(h->prof.on && h->prof.serial);
    auto pst = [&](Pipe& p) { return split ? p.st : st; };
    if (split) {
        HIP_TRY(hipEventRecord(h->fork, st));
        for (int q = 0; q < h->npipes; ++q) HIP_TRY(hipStreamWaitEvent(h->pipes[q].st, h->fork, 0));
    }
    for (int q = 0; q < h->npipes; ++q) {
        Pipe& p = h->pipes[q];
        // The factor phase needs a well-conditioned Gram: from the previous factors the
        // columns of A = M V_prev are close to orthogonal.  From a cold start (A = M) a
        // graded spectrum would make most factorizations fail, so it is skipped.
        p.pre = p.ncap > 0 && warm;
        p.resumed = false;
        if ((rc = pipe_pre(h, p, pst(p), warm))) return rc;
        pipe_start_rounds(h, p, p.pre ? LIST_FACTOR : LIST_PLAIN, 4);
    }
    // Round-robin over the pipes: enqueue one round per pipe per turn, poll the
    // convergence flags once per sweep of a pipe's largest matrix (after its
    // first_check rounds) without blocking, and keep at most one sweep queued
    // beyond a pending poll.  Rounds of converged matrices exit at once.
    for (;;) {
        bool queued = false, waiting = false, active = false;
        for (int q = 0; q < h->npipes; ++q) {
            Pipe& p = h->pipes[q];
            if (p.stage == STAGE_DONE) continue;
            active = true;
            hipStream_t ps = pst(p);
            if (p.poll_pending) {
                const hipError_t e = hipEventQuery(p.poll);
                if (e == hipErrorNotReady) {
                    waiting = true;
                } else if (e != hipSuccess) {
                    return fail(SC_ERR_HIP, "hipEventQuery: %s", hipGetErrorString(e));
                } else {
                    p.poll_pending = false;
                    const bool all = pipe_all_done(h, p);
                    if (p.stage == STAGE_CERTP) {
                        if (all) {
                            if ((rc = pipe_finalize(h, p, ps))) return rc;
                            p.stage = STAGE_DONE;
                        } else {
                            // sweeps on for the matrices the certificate rejected
                            p.resumed = true;
                            pipe_start_rounds(h, p, LIST_PLAIN, 1);
                        }
                        queued = true;
                        continue;
                    }
                    if (p.stage == STAGE_CERT || p.stage == STAGE_CERT2) {
                        if (all) {
                            if ((rc = pipe_finalize(h, p, ps))) return rc;
                            p.stage = STAGE_DONE;
                        } else {
                            // polish the matrices that failed the certificate: first
                            // selectively, then (re-certification failed) in full
                            int nb = 2;
                            for (int i : p.host_mats)
                                if (h->mh[i].klen && !p.flags_h[i].done)
                                    nb = std::max(nb, h->mh[i].nb);
                            rc = p.stage == STAGE_CERT ? pipe_start_selective(h, p, ps, nb)
                                                       : pipe_start_full_polish(h, p, ps, nb);
                            if (rc) return rc;
                        }
                        queued = true;
                        continue;
                    }
                    if (all || p.r >= p.max_rounds) {
                        if ((rc = pipe_after_rounds(h, p, ps, all))) return rc;
                        queued = true;
                        continue;
                    }
                }
            }
            if (p.stage != STAGE_ROUNDS) continue;
            if (p.r < p.max_rounds && (!p.poll_pending || p.r < p.poll_round + p.rps)) {
                if ((rc = pipe_round(h, p, ps))) return rc;
                p.r += 1;
                queued = true;
                if (h->hp.sync_check && !p.poll_pending && p.r >= p.first_check &&
                    p.r % p.rps == 0 && p.r < p.max_rounds) {
                    if ((rc = pipe_poll(h, p, ps))) return rc;
                    p.poll_round = p.r;
                }
            } else if (p.r >= p.max_rounds && !p.poll_pending) {
                if ((rc = pipe_after_rounds(h, p, ps, false))) return rc;
                queued = true;
            }
        }
        if (!active) break;
        if (!queued && waiting) {
            // nothing to queue: block until the oldest pending poll completes
            for (int q = 0; q < h->npipes; ++q)
                if (h->pipes[q].poll_pending) {
                    HIP_TRY(hipEventSynchronize(h->pipes[q].poll));
                    break;
                }
        }
    }
    if (split)
        for (int q = 0; q < h->npipes; ++q) {
            HIP_TRY(hipEventRecord(h->pipes[q].join, h->pipes[q].st));
            HIP_TRY(hipStreamWaitEvent(st, h->pipes[q].join, 0));
        }
    if (h->prof.on) {
        // the work counters of this refresh, copied behind it without a host wait
        MatFlags* snap = nullptr;
        if (!h->prof.snap_pool.empty()) {
            snap = h->prof.snap_pool.back();
            h->prof.snap_pool.pop_back();
        } else {
            void* q = nullptr;
            HIP_TRY(hipHostMalloc(&q, sizeof(MatFlags) * h->n, hipHostMallocDefault));
            snap = (MatFlags*)q;
        }
        h->prof.snaps.push_back(snap);
        HIP_TRY(hipMemcpyAsync(snap, h->flags_d, sizeof(MatFlags) * h->n, hipMemcpyDeviceToHost, st));
    }
    HIP_TRY(hipEventRecord(h->ev_refresh, st));
    h->ev_refresh_rec = true;
    h->proj_stale = false;
    h->have_factors = true;
    h->refreshes += 1;
    for (auto& s : h->stale) s = 0;
    h->any_stale = false;
    return SC_OK;
}

// ---- asynchronous refresh ---------------------------------------------------------------

int build_step_groups(sc_opt* h, int set);

// Published copy of the step operands (F, P_L, P_R, d), the step tables that
// read it, and the stream and events of the asynchronous refresh; allocated at
// the first sc_anchor_update_async.
int ensure_async(sc_opt* h) {
    if (h->pub_arena) return SC_OK;
    const size_t f = sizeof(float);
    std::vector<size_t> off(4 * (size_t)h->n);
    size_t total = 0;
    auto take = [&](size_t bytes) {
        const size_t o = total;
        total += align_up(bytes, 256);
        return o;
    };
    for (int i = 0; i < h->n; ++i) {
        const MatDev& m = h->mh[i];
        off[4 * i + 0] = take((size_t)m.k * m.K_ld * f);
        off[4 * i + 1] = take(m.PL ? (size_t)m.m * m.m * f : 0);
        off[4 * i + 2] = take(m.PR ? (size_t)m.n * m.n * f : 0);
        off[4 * i + 3] = take((size_t)m.kpad * f);
    }
    void* a = nullptr;
    if (hipMalloc(&a, total) != hipSuccess) {
        (void)hipGetLastError();
        return fail(SC_ERR_OOM, "device allocation of %zu bytes (published step operands) failed", total);
    }
    h->pub_arena = (char*)a;
    HIP_TRY(hipMemset(h->pub_arena, 0, total));
    h->pub.resize(h->n);
    for (int i = 0; i < h->n; ++i) {
        const MatDev& m = h->mh[i];
        h->pub[i].F = (float*)(h->pub_arena + off[4 * i + 0]);
        h->pub[i].PL = m.PL ? (float*)(h->pub_arena + off[4 * i + 1]) : nullptr;
        h->pub[i].PR = m.PR ? (float*)(h->pub_arena + off[4 * i + 2]) : nullptr;
        h->pub[i].d = (float*)(h->pub_arena + off[4 * i + 3]);
    }
    HIP_TRY(hipStreamCreateWithFlags(&h->astream, hipStreamNonBlocking));
    HIP_TRY(hipEventCreateWithFlags(&h->a_ready, hipEventDisableTiming));
    HIP_TRY(hipEventCreateWithFlags(&h->a_pub, hipEventDisableTiming));
    HIP_TRY(hipEventCreateWithFlags(&h->a_done, hipEventDisableTiming));
    return build_step_groups(h, 1);
}

// Copy the step operands in use into the published set (stream st).
int publish_step_operands(sc_opt* h, hipStream_t st) {
    const size_t f = sizeof(float);
    for (int i = 0; i < h->n; ++i) {
        const MatDev& m = h->mh[i];
        HIP_TRY(hipMemcpyAsync(h->pub[i].F, m.F, (size_t)m.k * m.K_ld * f, hipMemcpyDeviceToDevice, st));
        if (m.PL)
            HIP_TRY(hipMemcpyAsync(h->pub[i].PL, m.PL, (size_t)m.m * m.m * f, hipMemcpyDeviceToDevice, st));
        if (m.PR)
            HIP_TRY(hipMemcpyAsync(h->pub[i].PR, m.PR, (size_t)m.n * m.n * f, hipMemcpyDeviceToDevice, st));
        HIP_TRY(hipMemcpyAsync(h->pub[i].d, m.d, (size_t)m.kpad * f, hipMemcpyDeviceToDevice, st));
    }
    return SC_OK;
}

// End an asynchronous refresh: join its host thread (which returns once the
// whole refresh is queued), then order stream st after it (host_wait: block the
// host until it has run) and report its result.  No-op when none is pending.
int finish_async(sc_opt* h, hipStream_t st, bool host_wait) {
    if (!h->a_pending) return SC_OK;
    h->worker.join();
    h->a_pending = false;
    if (h->a_rc != SC_OK) {
        g_err = h->a_err;
        return h->a_rc;
    }
    if (host_wait)
        HIP_TRY(hipEventSynchronize(h->a_done));
    else
        HIP_TRY(hipStreamWaitEvent(st, h->a_done, 0));
    return SC_OK;
}

// ---- construction -------------------------------------------------------------------------

// Step GEMM tables of one operand set: set 0 reads the refresh's F, P_L, P_R
// and d, set 1 the copy published for an asynchronous refresh.  Executed chain
// (fewer flops than U D U^T G V D V^T left to right): square G_filt = P_L (G P_R);
// tall G_filt = F^T ((D F G) P_R); wide G_filt = (P_L (G F^T D)) F.
// Step GEMM problems of matrix i (see build_step_groups) into the six groups g,
// with the intermediates Y and T at the given addresses.
void add_step_probs(GemmGroup* g, int i, const MatDev& m, const float* F, const float* PL,
                    const float* PR, const float* d, float* Y, float* T) {
    GemmProb p;
    if (m.m == m.n) {
        p = make_prob(nullptr, m.n, PR, m.n, T, m.n, m.m, m.n, m.n);  // T = G P_R
        p.a_ptr = i;
        g[0].h.push_back(p);
        p = make_prob(PL, m.m, T, m.n, m.Gfilt, m.n, m.m, m.n, m.m);  // G_filt = P_L T
        g[3].h.push_back(p);
    } else if (m.tall) {
        p = make_prob(F, m.K_ld, nullptr, m.n, Y, m.k, m.k, m.n, m.m);  // Y = D F G
        p.b_ptr = i;
        p.row_scale = d;
        g[1].h.push_back(p);
        p = make_prob(Y, m.k, PR, m.n, T, m.k, m.k, m.n, m.n);  // T = Y P_R
        g[3].h.push_back(p);
        p = make_prob(F, m.K_ld, T, m.k, m.Gfilt, m.n, m.m, m.n, m.k);  // G_filt = F^T T
        g[4].h.push_back(p);
    } else {
        p = make_prob(nullptr, m.n, F, m.K_ld, Y, m.k, m.m, m.k, m.n);  // Y = G F^T D
        p.a_ptr = i;
        p.col_scale = d;
        g[2].h.push_back(p);
        p = make_prob(PL, m.m, Y, m.k, T, m.k, m.m, m.k, m.m);  // T = P_L Y
        g[3].h.push_back(p);
        p = make_prob(T, m.k, F, m.K_ld, m.Gfilt, m.n, m.m, m.n, m.k);  // G_filt = T F
        g[5].h.push_back(p);
    }
}

void init_step_groups(GemmGroup* g, bool gbf) {
    for (int q = 0; q < 6; ++q) g[q] = GemmGroup{};
    g[0].abf = gbf;  // square: A = G
    g[1].bbf = gbf;  // tall: B = G
    g[2].tb = true;  // wide: A = G, B = F^T
    g[2].abf = gbf;
    g[4].ta = true;
}

// Step GEMM tables of one operand set: set 0 reads the refresh's F, P_L, P_R
// and d, set 1 the copy published for an asynchronous refresh.  Executed chain
// (fewer flops than U D U^T G V D V^T left to right): square G_filt = P_L (G P_R);
// tall G_filt = F^T ((D F G) P_R); wide G_filt = (P_L (G F^T D)) F.
int build_step_groups(sc_opt* h, int set) {
    GemmGroup* g = h->step[set];
    init_step_groups(g, h->gdt == SC_BF16);
    for (int i = 0; i < h->n; ++i) {
        const MatDev& m = h->mh[i];
        const float* F = set ? h->pub[i].F : m.F;
        const float* PL = set ? h->pub[i].PL : m.PL;
        const float* PR = set ? h->pub[i].PR : m.PR;
        const float* d = set ? h->pub[i].d : m.d;
        add_step_probs(g, i, m, F, PL, PR, d, m.Y, m.T);
    }
    int rc;
    for (int q = 0; q < 6; ++q)
        if ((rc = upload_group(h, g[q]))) return rc;
    return SC_OK;
}

// ---- the allocation-free step (sc_step_noalloc) ------------------------------------

// The step intermediates Y and T of sc_step_noalloc live in this file-scope
// device array instead of the handle's memory.  Every GPU holds its own copy.
// In host code the name only stands in for the symbol: the device address comes
// from hipGetSymbolAddress, once per device (scratch_address), and only that
// address is passed to kernels.
constexpr size_t kNoAllocScratchBytes = (size_t)128 << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on device dev (which must be current).
int scratch_address(int dev, char** out) {
    if (dev < 0 || dev >= kMaxDevices)
        return fail(SC_ERR_NO_DEVICE, "device %d beyond the %d the library tracks", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            (void)hipGetLastError();
            return fail(SC_ERR_HIP, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
        }
        g_scratch_ptr[dev] = p;
    }
    *out = (char*)g_scratch_ptr[dev];
    return SC_OK;
}

// Step tables of sc_step_noalloc: matrices in handle order, cut into batches
// whose Y and T fit the scratch array together; each batch runs the chain's
// stages before the next reuses the array.  A matrix whose intermediates alone
// exceed it leaves the entry point unusable for the handle (na_err says why).
int build_noalloc_groups(sc_opt* h) {
    char* base = nullptr;
    int rc;
    if ((rc = scratch_address(h->device, &base))) return rc;
    h->na.clear();
    h->na_err.clear();
    size_t used = kNoAllocScratchBytes;  // forces a first batch
    for (int i = 0; i < h->n; ++i) {
        const MatDev& m = h->mh[i];
        const size_t kk = align_up((size_t)m.k * m.k * sizeof(float), 256);
        const size_t need = (m.m == m.n ? 1 : 2) * kk;
        if (need > kNoAllocScratchBytes) {
            char buf[256];
            snprintf(buf, sizeof(buf),
                     "matrix %d (%d x %d) needs %zu bytes of step intermediates, more than the %zu "
                     "bytes of the allocation-free step's scratch (4 min(rows, cols)^2 bytes for a square matrix, twice that otherwise)",
                     i, m.m, m.n, need, kNoAllocScratchBytes);
            h->na_err = buf;
            h->na.clear();
            return SC_OK;
        }
        if (used + need > kNoAllocScratchBytes) {
            h->na.emplace_back();
            init_step_groups(h->na.back().g, h->gdt == SC_BF16);
            used = 0;
        }
        float* T = (float*)(base + used);
        float* Y = m.m == m.n ? nullptr : (float*)(base + used + kk);
        add_step_probs(h->na.back().g, i, m, m.F, m.PL, m.PR, m.d, Y, T);
        used += need;
    }
    for (auto& b : h->na)
        for (int q = 0; q < 6; ++q)
            if ((rc = upload_group(h, b.g[q]))) return rc;
    return SC_OK;
}


int build(sc_opt* h, const int64_t* rows, const int64_t* cols) {
    const int n = h->n;
    h->mh.resize(n);
    h->fused.assign(n, std::array<char, 2>{0, 0});
    h->quadm.assign(n, std::array<char, 2>{0, 0});
    // layout pass: sizes of every buffer, carved from one arena
    std::vector<size_t> off;
    size_t total = 0;
    auto take = [&](size_t bytes) {
        size_t o = total;
        total += align_up(bytes ? bytes : 1, 256);
        return o;
    };
    struct Offs {
        size_t Manc, madam, vadam, A, V, F, W, PL, PR, s, d, norm2, Gfilt, Y, T, E, invn, gram, rot,
            rflag, perm, cnorm, chol, bmax;
    };
    std::vector<Offs> o(n);
    for (int i = 0; i < n; ++i) {
        MatDev& m = h->mh[i];
        memset(&m, 0, sizeof(m));
        m.m = (int)rows[i];
        m.n = (int)cols[i];
        m.tall = m.m >= m.n;
        m.K = std::max(m.m, m.n);
        m.k = std::min(m.m, m.n);
        m.kpad = round_up(m.k, kPw);
        m.K_ld = round_up(m.K, 128);
        m.nb = m.kpad / kJb;
        // Pairs are rotated above 16 * 2^-24.  Float32 sweeps leave relative
        // off-diagonals of about that size behind (rounding of the Gram and of the
        // rotations), so the last few pairs above it reappear in every sweep; the
        // sweeps therefore stop once a sweep's largest ratio is within the usual
        // one-sided Jacobi bound 2^-24 sqrt(K) (K float32 terms per inner
        // product), floored at the rotation threshold.  A given jacobi_tol sets both.
        const double eps = 5.9604644775390625e-08;
        m.tol = h->hp.jacobi_tol > 0.0f ? h->hp.jacobi_tol : (float)(16.0 * eps);
        m.tol_conv = h->hp.jacobi_tol > 0.0f
                         ? h->hp.jacobi_tol
                         : (float)(eps * std::max(16.0, std::sqrt((double)m.K)));
        m.numel = (int64_t)m.m * m.n;
        // Cholesky-preconditioned when the operand is at least twice as long as wide
        // Cholesky factor phase for operands at least twice as long as wide: their
        // singular values stay away from zero, so the Gram A^T A loses nothing
        // (square operands keep the plain sweeps: A^T A squares their condition
        // number and the factor phase then needs more sweeps, not fewer)
        m.klen = (h->hp.precondition && m.K >= 2 * m.k) ? round_up(m.k, 128) : 0;
        // Operands with a factor phase rotate pairs above 8 * 2^-24: the certificate of
        // A = M V sees the factor's residual off-diagonals amplified by the condition
        // number (E(A) ~ kappa E(X)); rotating down to half the plain threshold leaves
        // room for kappa up to ~10 at the steady state of the 16-block workload, whose
        // long matrices then pass the certificate without polishing (pass 639-645 ->
        // 616-623 ms; 4 or 6 * 2^-24 rotate more noise for no gain, 10-12 let some fail).
        if (m.klen && !(h->hp.jacobi_tol > 0.0f)) m.tol = (float)(8.0 * eps);
        m.nsplit = split_count(m.K_ld, kMaxSplits);  // capacity of the partial buffer
        if (m.klen) m.nsplit = std::max(m.nsplit, split_count(m.klen, kMaxSplits));
        // quad passes: group Gram splits of at most kQuadGramCols columns
        if (quad_capable(m.nb)) m.nsplit = std::max(m.nsplit, (m.K_ld + kQuadGramCols - 1) / kQuadGramCols);
        const size_t f = sizeof(float);
        const size_t mn = (size_t)m.numel * f;
        const size_t kk = (size_t)m.k * m.k * f;
        o[i].Manc = take(mn);
        o[i].madam = take(mn);
        o[i].vadam = take(mn);
        o[i].A = take((size_t)m.kpad * m.K_ld * f);
        o[i].V = take((size_t)m.kpad * m.kpad * f);
        o[i].F = take((size_t)m.k * m.K_ld * f);
        o[i].W = take(kk);
        o[i].PL = take(m.m <= m.n ? (size_t)m.m * m.m * f : 0);
        o[i].PR = take(m.m >= m.n ? (size_t)m.n * m.n * f : 0);
        o[i].s = take((size_t)m.kpad * f);
        o[i].d = take((size_t)m.kpad * f);
        o[i].norm2 = take((size_t)m.kpad * sizeof(double));
        o[i].Gfilt = take(mn);
        o[i].Y = take(kk);
        o[i].T = take(kk);
        o[i].E = take(kk);
        o[i].invn = take((size_t)m.kpad * f);
        // pair partials [nb/2][nsplit][64][64]; quad passes per group [nsplit][10][32][32]
        // and the group's 128 x 128 float32 Gram
        o[i].gram = take(std::max((size_t)(m.nb / 2) * m.nsplit * kPw * kPw,
                                  quad_capable(m.nb) ? (size_t)(m.nb / 4) * (m.nsplit * 10 * 1024 + 8192) : 0) *
                         sizeof(double));
        // two buffers (round parity): V rows take two rounds' rotations per pass
        o[i].rot = take((size_t)2 * (m.nb / 2) * kPw * kPw * f);
        o[i].rflag = take((size_t)2 * (m.nb / 2) * sizeof(int));
        o[i].perm = take((size_t)m.kpad * sizeof(int));
        o[i].cnorm = take((size_t)m.kpad * sizeof(float));
        o[i].chol = take((size_t)m.k * m.k * sizeof(double));
        const bool sel = m.klen && m.kpad <= kSelMaxK;
        o[i].bmax = take(sel ? (size_t)m.nb * m.nb * sizeof(float) : 0);
    }
    void* arena = nullptr;
    if (hipMalloc(&arena, total) != hipSuccess) {
        (void)hipGetLastError();
        return fail(SC_ERR_OOM, "device allocation of %zu bytes failed", total);
    }
    h->arena = (char*)arena;
    // Zero everything: anchor momentum, moments and factors start at zero, so
    // until the first refresh d = 0 and G_filt = 0.
    HIP_TRY(hipMemset(h->arena, 0, total));
    for (int i = 0; i < n; ++i) {
        MatDev& m = h->mh[i];
        char* b = h->arena;
        m.Manc = (float*)(b + o[i].Manc);
        m.madam = (float*)(b + o[i].madam);
        m.vadam = (float*)(b + o[i].vadam);
        m.A = (float*)(b + o[i].A);
        m.V = (float*)(b + o[i].V);
        m.F = (float*)(b + o[i].F);
        m.W = (float*)(b + o[i].W);
        m.PL = m.m <= m.n ? (float*)(b + o[i].PL) : nullptr;
        m.PR = m.m >= m.n ? (float*)(b + o[i].PR) : nullptr;
        m.s = (float*)(b + o[i].s);
        m.d = (float*)(b + o[i].d);
        m.norm2 = (double*)(b + o[i].norm2);
        m.Gfilt = (float*)(b + o[i].Gfilt);
        m.Gproj = nullptr;
        m.Y = (float*)(b + o[i].Y);
        m.T = (float*)(b + o[i].T);
        m.E = (float*)(b + o[i].E);
        m.invn = (float*)(b + o[i].invn);
        m.gram = (double*)(b + o[i].gram);
        m.rot = (float*)(b + o[i].rot);
        m.rot_flag = (int*)(b + o[i].rflag);
        m.perm = (int*)(b + o[i].perm);
        m.cnorm = (float*)(b + o[i].cnorm);
        m.chol = (double*)(b + o[i].chol);
        m.bmax = (m.klen && m.kpad <= kSelMaxK) ? (float*)(b + o[i].bmax) : nullptr;
    }
    void* p = nullptr;
    HIP_TRY(hipMalloc(&p, sizeof(MatDev) * n));
    h->dev_allocs.push_back(p);
    h->md = (MatDev*)p;
    HIP_TRY(hipMemcpy(h->md, h->mh.data(), sizeof(MatDev) * n, hipMemcpyHostToDevice));
    HIP_TRY(hipMalloc(&p, sizeof(MatFlags) * n));
    h->dev_allocs.push_back(p);
    h->flags_d = (MatFlags*)p;
    HIP_TRY(hipMemset(h->flags_d, 0, sizeof(MatFlags) * n));
    HIP_TRY(hipHostMalloc(&p, sizeof(MatFlags) * n, hipHostMallocDefault));
    h->flags_h = (MatFlags*)p;
    memset(h->flags_h, 0, sizeof(MatFlags) * n);
    HIP_TRY(hipMalloc(&p, 4 * sizeof(int)));
    h->dev_allocs.push_back(p);
    h->status_d = (int*)p;
    HIP_TRY(hipMemset(h->status_d, 0, 4 * sizeof(int)));
    HIP_TRY(hipHostMalloc(&p, 4 * sizeof(int), hipHostMallocDefault));
    h->status_h = (int*)p;
    HIP_TRY(hipEventCreateWithFlags(&h->ev_refresh, hipEventDisableTiming));
    HIP_TRY(hipEventCreateWithFlags(&h->ev_step, hipEventDisableTiming));

    // work lists
    std::vector<Chunk> ch;
    for (int i = 0; i < n; ++i) {
        const MatDev& m = h->mh[i];
        for (int64_t off0 = 0; off0 < m.numel; off0 += kChunk)
            ch.push_back(Chunk{i, off0, (int)std::min<int64_t>(kChunk, m.numel - off0)});
    }
    // Pipes.  Per-round work of a matrix: its pairs times the row length swept
    // (operand plus V).  When matrices with a factor phase and plain ones each
    // carry at least a quarter of the work, each kind forms a pipe: the factor
    // pipe's Gram SYRK, Cholesky and V/A GEMMs then overlap the plain pipe's
    // sweeps instead of running beside the same phase of an identical pipe
    // (measured 1.6% faster per pass than an even split on the 16-block
    // workload).  Otherwise matrices are dealt by decreasing work to the less
    // loaded pipe.
    auto work = [&](int i) {
        const MatDev& m = h->mh[i];
        return (double)m.kpad * ((m.klen ? m.klen : m.K_ld) + m.kpad);
    };
    std::vector<int> gm[kPipes];
    double wcap = 0.0, wall = 0.0;
    for (int i = 0; i < n; ++i) {
        wall += work(i);
        if (h->mh[i].klen) wcap += work(i);
    }
    if (kPipes >= 2 && wcap >= 0.25 * wall && wcap <= 0.75 * wall) {
        for (int i = 0; i < n; ++i) gm[h->mh[i].klen ? 0 : 1].push_back(i);
    } else {
        std::vector<int> order(n);
        for (int i = 0; i < n; ++i) order[i] = i;
        std::stable_sort(order.begin(), order.end(),
                         [&](int x, int y) { return work(x) > work(y); });
        double load[kPipes] = {};
        for (int i : order) {
            int g = 0;
            for (int q = 1; q < kPipes; ++q)
                if (load[q] < load[g]) g = q;
            gm[g].push_back(i);
            load[g] += work(i);
        }
        for (auto& v : gm) std::sort(v.begin(), v.end());
    }
    auto upload = [&](auto& vec, auto** dst, int* cnt) -> int {
        *cnt = (int)vec.size();
        void* q = nullptr;
        HIP_TRY(hipMalloc(&q, sizeof(vec[0]) * std::max<size_t>(vec.size(), 1)));
        h->dev_allocs.push_back(q);
        *dst = (typename std::remove_reference<decltype(**dst)>::type*)q;
        if (!vec.empty())
            HIP_TRY(hipMemcpy(q, vec.data(), sizeof(vec[0]) * vec.size(), hipMemcpyHostToDevice));
        return SC_OK;
    };
    int rc;
    if ((rc = upload(ch, &h->chunks_d, &h->nchunks))) return rc;
    h->npipes = 0;
    while (h->npipes < kPipes && !gm[h->npipes].empty()) ++h->npipes;
    for (int g = 0; g < h->npipes; ++g) {
        Pipe& P = h->pipes[g];
        P.host_mats = gm[g];
        for (int which = 0; which < 3; ++which) {
            std::vector<GramItem> gi;
            std::vector<SolveItem> si;
            std::vector<ApplyItem> ai, ai_f, av;
            bool any_unfused = false;
            std::vector<FusedItem> fi, vi, qg;
            std::vector<SolveItem> qs;
            std::vector<QuadItem> qa;
            std::vector<int> mats;
            auto& L = P.L[which];
            // quad passes: every matrix of the list quad-capable (polishing keeps the
            // pair rounds: its selective sweeps work on marked block pairs)
            bool quad = which != LIST_POLISH;
            int qgroups = 0;  // groups of a quad pass over the list
            for (int i : gm[g])
                if (which != LIST_POLISH || h->mh[i].klen) {
                    quad = quad && quad_capable(h->mh[i].nb);
                    qgroups += h->mh[i].nb / 4;
                }
            const bool qfill = qgroups >= kQuadMinGroups;
            int pairs = 0;
            for (int i : gm[g])
                if (which != LIST_POLISH || h->mh[i].klen) pairs += h->mh[i].nb / 2;
            const int nt = splits_for(pairs);
            for (int i : gm[g]) {
                const MatDev& m = h->mh[i];
                if (which == LIST_POLISH && !m.klen) continue;  // preconditioned matrices only
                const int len = (which == LIST_FACTOR && m.klen) ? m.klen : m.K_ld;
                int sl = split_len(len, nt), ns = split_count(len, nt);
                // the fused apply + next Gram: power-of-two block counts of four or
                // more (two XOR rounds close groups of four blocks) whose splits
                // fit kFusedMaxCols (more, shorter splits when needed)
                bool fuse = false;
                if (m.nb >= 4 && (m.nb & (m.nb - 1)) == 0) {
                    const int ntf = std::min(kMaxSplits,
                                             std::max(nt, (len + kFusedMaxCols - 1) / kFusedMaxCols));
                    if (split_len(len, ntf) <= kFusedMaxCols) {
                        sl = split_len(len, ntf);
                        ns = split_count(len, ntf);
                        fuse = true;
                    }
                }
                h->fused[i][which == LIST_FACTOR && m.klen ? 0 : 1] = fuse;
                any_unfused = any_unfused || !fuse;
                const bool vrows = !(which == LIST_FACTOR && m.klen);  // V moves outside the factor phase
                h->quadm[i][which == LIST_FACTOR && m.klen ? 0 : 1] = quad ? (qfill ? 2 : 1) : 0;
                if (quad) {
                    // group Gram splits: whole rows when the list's groups fill the chip,
                    // else up to one per kQuadGramCols columns
                    const int qns = std::min((len + kQuadGramCols - 1) / kQuadGramCols,
                                             std::max(1, (kQuadGramFill + qgroups - 1) / std::max(qgroups, 1)));
                    const int qsl = round_up((len + qns - 1) / qns, 128);
                    const int span = kQuadRun * kQuadCols;
                    for (int grp = 0; grp < m.nb / 4; ++grp) {
                        for (int sp = 0; sp < qns; ++sp)
                            qg.push_back(FusedItem{i, grp, sp, sp * qsl, std::min(len, (sp + 1) * qsl)});
                        qs.push_back(SolveItem{i, grp, qns});
                        for (int x0 = 0; x0 < len; x0 += span)
                            qa.push_back(QuadItem{i, grp, 0, x0, std::min(len, x0 + span)});
                        if (vrows)
                            for (int x0 = 0; x0 < m.kpad; x0 += span)
                                qa.push_back(QuadItem{i, grp, 1, x0, std::min(m.kpad, x0 + span)});
                    }
                }
                if (fuse)
                    for (int grp = 0; grp < m.nb / 4; ++grp) {
                        for (int sp = 0; sp < ns; ++sp)
                            fi.push_back(FusedItem{i, grp, sp, sp * sl, std::min(len, (sp + 1) * sl)});
                        if (vrows)
                            for (int x0 = 0; x0 < m.kpad; x0 += kV2Run * kV2Cols)
                                vi.push_back(FusedItem{i, grp, 0, x0, std::min(m.kpad, x0 + kV2Run * kV2Cols)});
                    }
                if (fuse && vrows &&
                    std::find(L.vnbs.begin(), L.vnbs.end(), m.nb) == L.vnbs.end())
                    L.vnbs.push_back(m.nb);
                mats.push_back(i);
                L.max_nb = std::max(L.max_nb, m.nb);
                if (std::find(L.nbs.begin(), L.nbs.end(), m.nb) == L.nbs.end()) L.nbs.push_back(m.nb);
                for (int s = 0; s < m.nb / 2; ++s) {
                    for (int sp = 0; sp < ns; ++sp)
                        gi.push_back(GramItem{i, s, sp, sp * sl, std::min(len, (sp + 1) * sl),
                                              fuse ? 1 : 0});
                    si.push_back(SolveItem{i, s, ns});
                    const int nca = (len + kApplyCols - 1) / kApplyCols;
                    for (int c = 0; c < nca; c += kApplyRun) {
                        ai.push_back(ApplyItem{i, s, 0, c, std::min(kApplyRun, nca - c)});
                        if (!fuse) ai_f.push_back(ai.back());
                    }
                    if (!vrows) continue;  // no V in the factor phase
                    const int ncv = (m.kpad + kApplyCols - 1) / kApplyCols;
                    for (int c = 0; c < ncv; c += kApplyRun) {
                        ai.push_back(ApplyItem{i, s, 1, c, std::min(kApplyRun, ncv - c)});
                        (fuse ? av : ai_f).push_back(ai.back());
                    }
                }
            }
            if ((rc = upload(gi, &L.gi, &L.ngi))) return rc;
            if ((rc = upload(si, &L.si, &L.nsi))) return rc;
            if ((rc = upload(ai, &L.ai, &L.nai))) return rc;
            if ((rc = upload(ai_f, &L.ai_f, &L.nai_f))) return rc;
            if ((rc = upload(fi, &L.fi, &L.nfi))) return rc;
            if ((rc = upload(vi, &L.vi, &L.nvi))) return rc;
            if ((rc = upload(av, &L.av, &L.nav))) return rc;
            if ((rc = upload(qg, &L.qg, &L.nqg))) return rc;
            if ((rc = upload(qs, &L.qs, &L.nqs))) return rc;
            if ((rc = upload(qa, &L.qa, &L.nqa))) return rc;
            L.quad = quad && !mats.empty();
            L.quad_auto = L.quad && qfill;
            L.all_fused = !mats.empty() && !any_unfused;
            if ((rc = upload(mats, &L.mats, &L.nmat))) return rc;
        }
        std::vector<int> cap;
        std::vector<SyrkItem> sy, sa;
        for (int i : gm[g]) {
            const MatDev& m = h->mh[i];
            P.max_kpad = std::max(P.max_kpad, m.kpad);
            P.max_K = std::max(P.max_K, m.K_ld);
            P.max_k = std::max(P.max_k, m.k);
            P.max_t64 = std::max(P.max_t64, (m.k + 63) / 64);
            const int kt = (m.k + 127) / 128;
            for (int ti = 0; ti < kt; ++ti)
                for (int tj = 0; tj <= ti; ++tj) sa.push_back(SyrkItem{i, ti, tj});
            P.syrk_all_full = P.syrk_all_full && m.k % 128 == 0;
            if (m.klen) {
                P.syrk_cap_full = P.syrk_cap_full && m.k % 128 == 0;
                cap.push_back(i);
                P.max_nbk = std::max(P.max_nbk, (m.k + 63) / 64);
                P.max_klen = std::max(P.max_klen, m.klen);
                for (int ti = 0; ti < kt; ++ti)
                    for (int tj = 0; tj <= ti; ++tj) sy.push_back(SyrkItem{i, ti, tj});
            }
        }
        if ((rc = upload(gm[g], &P.mats, &P.nmat))) return rc;
        if ((rc = upload(cap, &P.cap, &P.ncap))) return rc;
        if ((rc = upload(sy, &P.syrk_cap, &P.nsyrk_cap))) return rc;
        if ((rc = upload(sa, &P.syrk_all, &P.nsyrk_all))) return rc;
        HIP_TRY(hipStreamCreateWithFlags(&P.st, hipStreamNonBlocking));
        HIP_TRY(hipEventCreateWithFlags(&P.join, hipEventDisableTiming));
        HIP_TRY(hipEventCreateWithFlags(&P.poll, hipEventDisableTiming));
        void* q = nullptr;
        HIP_TRY(hipHostMalloc(&q, sizeof(MatFlags) * n, hipHostMallocDefault));
        P.flags_h = (MatFlags*)q;
        memset(P.flags_h, 0, sizeof(MatFlags) * n);
    }
    HIP_TRY(hipEventCreateWithFlags(&h->fork, hipEventDisableTiming));
    std::vector<int> pipe_of(n, 0);
    for (int g = 0; g < h->npipes; ++g)
        for (int i : gm[g]) pipe_of[i] = g;

    // GEMM problem tables
    for (int g = 0; g < h->npipes; ++g) {
        // E X of the Loewdin step: a correction of size |E| (<= the convergence
        // threshold per entry) added to X, formed from two bfloat16 parts per operand
        h->pipes[g].lowdin_F.parts = 2;
        h->pipes[g].lowdin_W.parts = 2;
        h->pipes[g].lowdin_eW.tb = true;
        h->pipes[g].proj.ta = true;
        h->pipes[g].warm_nt.tb = true;
        h->pipes[g].polish_nt.tb = true;
    }
    for (int i = 0; i < n; ++i) {
        MatDev& m = h->mh[i];
        Pipe& P = h->pipes[pipe_of[i]];
        // Loewdin re-orthogonalization of the unit rows of A (-> F) and V (-> W):
        //   E = X X^T with zero diagonal;  X_out = X - 0.5 E X
        // (E of the A side is formed by final_gram before the rows are normalized)
        GemmProb p = make_prob(m.E, m.k, m.A, m.K_ld, m.F, m.K_ld, m.k, m.K_ld, m.k);
        p.Cin = m.A;
        p.ldcin = m.K_ld;
        p.alpha = -0.5f;
        p.beta = 1.0f;
        P.lowdin_F.h.push_back(p);
        p = make_prob(m.V, m.kpad, m.V, m.kpad, m.E, m.k, m.k, m.k, m.k);
        p.flags = GF_ZERO_DIAG;
        P.lowdin_eW.h.push_back(p);
        p = make_prob(m.E, m.k, m.V, m.kpad, m.W, m.k, m.k, m.k, m.k);
        p.Cin = m.V;
        p.ldcin = m.kpad;
        p.alpha = -0.5f;
        p.beta = 1.0f;
        P.lowdin_W.h.push_back(p);
        // warm start: rows of A = W op(M): m >= n: a_j = M w_j; m < n: a_j = M^T w_j
        if (m.tall) {
            p = make_prob(m.W, m.k, m.Manc, m.n, m.A, m.K_ld, m.k, m.m, m.n);
            P.warm_nt.h.push_back(p);
        } else {
            p = make_prob(m.W, m.k, m.Manc, m.n, m.A, m.K_ld, m.k, m.n, m.m);
            P.warm_nn.h.push_back(p);
        }
        if (m.klen) {
            // after the factor phase: V rows = scaled rows of X^T times W (= V_prev),
            // only where the factorization was accepted; then A_rows = V op(M)
            p = make_prob(m.A, m.K_ld, m.W, m.k, m.V, m.kpad, m.k, m.k, m.k);
            p.row_scale = m.invn;
            p.gate = &h->flags_d[i].precond;
            P.factor_v.h.push_back(p);
            if (m.tall) {
                p = make_prob(m.V, m.kpad, m.Manc, m.n, m.A, m.K_ld, m.k, m.m, m.n);
                P.polish_nt.h.push_back(p);
            } else {
                p = make_prob(m.V, m.kpad, m.Manc, m.n, m.A, m.K_ld, m.k, m.n, m.m);
                P.polish_nn.h.push_back(p);
            }
        }
        // projectors X^T diag(d) X
        const bool square = m.m == m.n;
        if (square) {
            p = make_prob(m.F, m.K_ld, m.F, m.K_ld, m.PL, m.m, m.m, m.m, m.k);
            p.k_scale = m.d;
            P.proj.h.push_back(p);
        }
        p = make_prob(m.W, m.k, m.W, m.k, m.tall ? m.PR : m.PL, m.k, m.k, m.k, m.k);
        p.k_scale = m.d;
        P.proj.h.push_back(p);
    }
    for (int g = 0; g < h->npipes; ++g) {
        Pipe& P = h->pipes[g];
        for (GemmGroup* gg : {&P.warm_nt, &P.warm_nn, &P.factor_v, &P.polish_nt, &P.polish_nn,
                              &P.lowdin_F, &P.lowdin_eW, &P.lowdin_W, &P.proj})
            if ((rc = upload_group(h, *gg))) return rc;
    }
    if ((rc = build_step_groups(h, 0))) return rc;
    if ((rc = build_noalloc_groups(h))) return rc;
    h->stale.assign(n, 0);
    const double gsz = h->gdt == SC_BF16 ? 2.0 : 4.0, wsz = h->wdt == SC_BF16 ? 2.0 : 4.0;
    for (int i = 0; i < n; ++i) h->total_numel += (double)h->mh[i].numel;
    h->ema_bytes = h->total_numel * (8.0 + gsz);
    h->adamw_bytes = h->total_numel * (gsz + 4.0 + 2.0 * wsz + 16.0);
    HIP_TRY(hipDeviceSynchronize());
    return SC_OK;
}

// Block the host until the handle's last refresh and last step (and, through
// its internal streams, any refresh work still in flight) have run.
int wait_handle(sc_opt* h) {
    if (h->ev_refresh_rec) HIP_TRY(hipEventSynchronize(h->ev_refresh));
    if (h->ev_step_rec) HIP_TRY(hipEventSynchronize(h->ev_step));
    for (int q = 0; q < h->npipes; ++q)
        if (h->pipes[q].st) HIP_TRY(hipStreamSynchronize(h->pipes[q].st));
    if (h->astream) HIP_TRY(hipStreamSynchronize(h->astream));
    return SC_OK;
}

// Copy the device flags and status words to their pinned host copies (after
// wait_handle) on an internal stream.
int read_flags(sc_opt* h) {
    hipStream_t q = h->pipes[0].st;
    HIP_TRY(hipMemcpyAsync(h->flags_h, h->flags_d, sizeof(MatFlags) * h->n, hipMemcpyDeviceToHost, q));
    HIP_TRY(hipMemcpyAsync(h->status_h, h->status_d, 4 * sizeof(int), hipMemcpyDeviceToHost, q));
    HIP_TRY(hipStreamSynchronize(q));
    return SC_OK;
}

void release(sc_opt* h) {
    if (!h) return;
    DeviceGuard g(h->device);
    if (h->worker.joinable()) h->worker.join();
    // the handle's own work only: its last refresh and step, its internal streams
    (void)wait_handle(h);
    (void)hipGetLastError();
    for (hipEvent_t e : {h->ev_refresh, h->ev_step})
        if (e) (void)hipEventDestroy(e);
    if (h->status_h) (void)hipHostFree(h->status_h);
    if (h->astream) (void)hipStreamDestroy(h->astream);
    for (hipEvent_t e : {h->a_ready, h->a_pub, h->a_done})
        if (e) (void)hipEventDestroy(e);
    if (h->pub_arena) (void)hipFree(h->pub_arena);
    for (auto& r : h->prof.recs) {
        (void)hipEventDestroy(r.a);
        (void)hipEventDestroy(r.b);
    }
    for (hipEvent_t e : h->prof.pool) (void)hipEventDestroy(e);
    for (MatFlags* f : h->prof.snaps) (void)hipHostFree(f);
    for (MatFlags* f : h->prof.snap_pool) (void)hipHostFree(f);
    for (auto& P : h->pipes) {
        if (P.st) (void)hipStreamDestroy(P.st);
        if (P.join) (void)hipEventDestroy(P.join);
        if (P.poll) (void)hipEventDestroy(P.poll);
        if (P.flags_h) (void)hipHostFree(P.flags_h);
    }
    if (h->fork) (void)hipEventDestroy(h->fork);
    for (void* p : h->dev_allocs) (void)hipFree(p);
    if (h->arena) (void)hipFree(h->arena);
    if (h->proj_arena) (void)hipFree(h->proj_arena);
    if (h->flags_h) (void)hipHostFree(h->flags_h);
    delete h;
}

int check_handle(sc_opt* h) {
    if (!h) return fail(SC_ERR_INVALID_ARG, "handle is NULL");
    return SC_OK;
}

int check_idx(sc_opt* h, int idx) {
    if (idx < 0 || idx >= h->n) return fail(SC_ERR_INVALID_ARG, "matrix index %d out of range", idx);
    return SC_OK;
}

// Timing families of the six step GEMM groups.
const int kStepKinds[6] = {PK_STEP_GEMM1, PK_STEP_GEMM1, PK_STEP_GEMM1,
                           PK_STEP_GEMM2, PK_STEP_GEMM3, PK_STEP_GEMM3};
int step_adamw(sc_opt* h, void* const* W, const void* const* G_mask, hipStream_t st);

}  // namespace

extern "C" {

void sc_default_hparams(sc_hparams* hp) {
    if (!hp) return;
    hp->tau_p = 1e-3f;
    hp->alpha = 0.3f;
    hp->beta_anc = 0.9f;
    hp->lr = 2e-5f;
    hp->beta1 = 0.9f;
    hp->beta2 = 0.999f;
    hp->eps = 1e-8f;
    hp->weight_decay = 0.01f;
    hp->max_sweeps = 30;
    hp->jacobi_tol = 0.0f;
    hp->sync_check = 1;
    hp->warm_start = 1;
    hp->precondition = 1;
}

const char* sc_last_error(void) { return g_err.c_str(); }

int sc_opt_create(sc_handle* out, int n_mats, const int64_t* rows, const int64_t* cols,
                  sc_dtype w_dtype, sc_dtype g_dtype, const sc_hparams* hp, int device) {
    g_err.clear();
    if (!out) return fail(SC_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    if (n_mats < 1 || n_mats > kMaxPtrs)
        return fail(SC_ERR_INVALID_ARG, "n_mats must be in [1, %d]", kMaxPtrs);
    if (!rows || !cols) return fail(SC_ERR_INVALID_ARG, "rows/cols is NULL");
    for (int i = 0; i < n_mats; ++i)
        if (rows[i] < 1 || cols[i] < 1 || rows[i] > kMaxDim || cols[i] > kMaxDim)
            return fail(SC_ERR_SHAPE, "matrix %d has shape %lld x %lld (allowed 1..%lld)", i,
                        (long long)rows[i], (long long)cols[i], (long long)kMaxDim);
    if ((w_dtype != SC_F32 && w_dtype != SC_BF16) || (g_dtype != SC_F32 && g_dtype != SC_BF16))
        return fail(SC_ERR_INVALID_ARG, "unknown dtype");
    int rc = check_hp(hp);
    if (rc) return rc;
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || ndev <= 0) {
        (void)hipGetLastError();
        return fail(SC_ERR_NO_DEVICE, "no HIP device");
    }
    if (device < 0 || device >= ndev)
        return fail(SC_ERR_NO_DEVICE, "device %d out of range (%d devices)", device, ndev);
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, device) != hipSuccess)
        return fail(SC_ERR_NO_DEVICE, "cannot query device %d", device);
    if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        return fail(SC_ERR_NO_DEVICE, "device %d is %s; libscopt is built for gfx950", device,
                    prop.gcnArchName);
    DeviceGuard guard(device);
    if (!guard.ok) return fail(SC_ERR_NO_DEVICE, "cannot select device %d", device);
    sc_opt* h = new (std::nothrow) sc_opt();
    if (!h) return fail(SC_ERR_OOM, "host allocation failed");
    h->device = device;
    h->n = n_mats;
    h->wdt = w_dtype;
    h->gdt = g_dtype;
    h->hp = *hp;
    rc = build(h, rows, cols);
    if (rc) {
        std::string msg = g_err;
        release(h);
        g_err = msg;
        return rc;
    }
    *out = h;
    return SC_OK;
}

int sc_opt_destroy(sc_handle h) {
    release(h);
    return SC_OK;
}

int sc_anchor_update(sc_handle h, const void* const* G_anc, void* stream) {
    int rc;
    if ((rc = check_handle(h))) return rc;
    if ((rc = check_ptrs(h, G_anc, h->gdt, "G_anc"))) return rc;
    DeviceGuard g(h->device);
    hipStream_t st = (hipStream_t)stream;
    if ((rc = finish_async(h, st, false))) return rc;
    PtrTable pt = make_table(h, G_anc);
    HIP_TRY(timed(h, PK_EMA, st, [&] {
        return launch_ema(h->md, h->chunks_d, h->nchunks, pt, h->gdt == SC_BF16, h->hp.beta_anc,
                          h->status_d + 1, st);
    }));
    if (h->prof.on) h->prof.bytes[PK_EMA] += h->ema_bytes;
    return do_refresh(h, st);
}

int sc_refresh(sc_handle h, void* stream) {
    int rc;
    if ((rc = check_handle(h))) return rc;
    DeviceGuard g(h->device);
    if ((rc = finish_async(h, (hipStream_t)stream, false))) return rc;
    return do_refresh(h, (hipStream_t)stream);
}

int sc_anchor_update_async(sc_handle h, const void* const* G_anc, void* stream) {
    int rc;
    if ((rc = check_handle(h))) return rc;
    if ((rc = check_ptrs(h, G_anc, h->gdt, "G_anc"))) return rc;
    if (h->prof.on)
        return fail(SC_ERR_INVALID_ARG, "asynchronous refresh is not available while kernel timing is on");
    DeviceGuard g(h->device);
    hipStream_t st = (hipStream_t)stream;
    if ((rc = finish_async(h, st, false))) return rc;
    if ((rc = ensure_async(h))) return rc;
    // the operands the steps use until the refresh ends: current tau, then copied
    if (h->proj_stale && (rc = build_projectors(h, st))) return rc;
    HIP_TRY(hipEventRecord(h->a_ready, st));
    HIP_TRY(hipStreamWaitEvent(h->astream, h->a_ready, 0));
    if ((rc = publish_step_operands(h, h->astream))) return rc;
    HIP_TRY(hipEventRecord(h->a_pub, h->astream));
    HIP_TRY(hipStreamWaitEvent(st, h->a_pub, 0));
    PtrTable pt = make_table(h, G_anc);
    HIP_TRY(launch_ema(h->md, h->chunks_d, h->nchunks, pt, h->gdt == SC_BF16, h->hp.beta_anc,
                       h->status_d + 1, h->astream));
    h->any_stale = false;  // the refresh below covers every matrix
    h->a_rc = SC_OK;
    h->a_err.clear();
    h->a_finished.store(false, std::memory_order_relaxed);
    h->a_pending = true;
    try {
        h->worker = std::thread([h] {
            DeviceGuard dg(h->device);
            int r = do_refresh(h, h->astream);
            if (r == SC_OK) {
                const hipError_t e = hipEventRecord(h->a_done, h->astream);
                if (e != hipSuccess) r = fail(SC_ERR_HIP, "hipEventRecord: %s", hipGetErrorString(e));
            }
            h->a_rc = r;
            if (r != SC_OK) h->a_err = g_err;
            h->a_finished.store(true, std::memory_order_release);
        });
    } catch (...) {
        h->a_pending = false;
        return fail(SC_ERR_HIP, "could not start the refresh thread");
    }
    return SC_OK;
}

int sc_refresh_wait(sc_handle h, void* stream) {
    int rc;
    if ((rc = check_handle(h))) return rc;
    DeviceGuard g(h->device);
    return finish_async(h, (hipStream_t)stream, false);
}

int sc_refresh_pending(sc_handle h, int* pending) {
    int rc;
    if ((rc = check_handle(h))) return rc;
    if (!pending) return fail(SC_ERR_INVALID_ARG, "pending is NULL");
    *pending = h->a_pending && !h->a_finished.load(std::memory_order_acquire) ? 1 : 0;
    return SC_OK;
}

int sc_step(sc_handle h, void* const* W, const void* const* G_mask, void* stream) {
    int rc;
    if ((rc = check_handle(h))) return rc;
    if ((rc = check_ptrs(h, (const void* const*)W, h->wdt, "W"))) return rc;
    if ((rc = check_ptrs(h, G_mask, h->gdt, "G_mask"))) return rc;
    DeviceGuard g(h->device);
    hipStream_t st = (hipStream_t)stream;
    // until an asynchronous refresh is completed (sc_refresh_wait), steps read the
    // operands published when it started, whether or not it has finished: the
    // factors a step uses do not depend on timing
    if (!h->a_pending) {
        if (h->any_stale) {
            if ((rc = do_refresh(h, st))) return rc;
        }
        if (h->proj_stale) {
            if ((rc = build_projectors(h, st))) return rc;
        }
    }
    PtrTable gt = make_table(h, G_mask);
    const GemmGroup* sg = h->step[h->a_pending ? 1 : 0];
    for (int q = 0; q < 6; ++q)
        if ((rc = run_group(h, sg[q], kStepKinds[q], gt, st))) return rc;
    return step_adamw(h, W, G_mask, st);
}

int sc_step_noalloc(sc_handle h, void* const* W, const void* const* G_mask, void* stream) {
    int rc;
    if ((rc = check_handle(h))) return rc;
    if ((rc = check_ptrs(h, (const void* const*)W, h->wdt, "W"))) return rc;
    if ((rc = check_ptrs(h, G_mask, h->gdt, "G_mask"))) return rc;
    if (!h->na_err.empty()) return fail(SC_ERR_SHAPE, "%s", h->na_err.c_str());
    if (h->a_pending)
        return fail(SC_ERR_INVALID_ARG,
                    "an asynchronous refresh is pending: complete it with sc_refresh_wait first");
    if (h->prof.on)
        return fail(SC_ERR_INVALID_ARG, "kernel timing is on: it creates events (sc_profile(h, 0))");
    DeviceGuard g(h->device);
    hipStream_t st = (hipStream_t)stream;
    // a refresh or projector rebuild allocates nothing
    if (h->any_stale && (rc = do_refresh(h, st))) return rc;
    if (h->proj_stale && (rc = build_projectors(h, st))) return rc;
    PtrTable gt = make_table(h, G_mask);
    for (const auto& b : h->na)
        for (int q = 0; q < 6; ++q)
            if ((rc = run_group(h, b.g[q], kStepKinds[q], gt, st))) return rc;
    return step_adamw(h, W, G_mask, st);
}

}  // extern "C"

namespace {
// The combination and AdamW of a step, after its GEMM chain has written G_filt.
int step_adamw(sc_opt* h, void* const* W, const void* const* G_mask, hipStream_t st) {
    PtrTable gt = make_table(h, G_mask);
    PtrTable wt = make_table(h, (const void* const*)W);
    const int64_t t = h->t + 1;
    const double lr = h->hp.lr, b1 = h->hp.beta1, b2 = h->hp.beta2;
    const double bc1 = 1.0 - std::pow(b1, (double)t);
    const double bc2 = 1.0 - std::pow(b2, (double)t);
    const float step_size = (float)(lr / bc1);
    const float inv_sqrt_bc2 = (float)(1.0 / std::sqrt(bc2));
    const float lr_wd = (float)(lr * (double)h->hp.weight_decay);
    HIP_TRY(timed(h, PK_ADAMW, st, [&] {
        return launch_combine_adamw(h->md, h->chunks_d, h->nchunks, wt, gt, h->wdt == SC_BF16,
                                    h->gdt == SC_BF16, h->hp.alpha, h->hp.beta1, h->hp.beta2,
                                    h->hp.eps, step_size, inv_sqrt_bc2, lr_wd,
                                    h->keep_proj ? 1 : 0, h->status_d, st);
    }));
    if (h->prof.on)
        h->prof.bytes[PK_ADAMW] += h->adamw_bytes + (h->keep_proj ? 4.0 * h->total_numel : 0.0);
    HIP_TRY(hipEventRecord(h->ev_step, st));
    h->ev_step_rec = true;
    h->t = t;
    return SC_OK;
}
}  // namespace

extern "C" {

int sc_set_lr(sc_handle h, float lr) {
    int rc;
    if ((rc = check_handle(h))) return rc;
    if (!(lr >= 0.0f) || !std::isfinite(lr)) return fail(SC_ERR_INVALID_ARG, "lr must be >= 0");
    h->hp.lr = lr;
    return SC_OK;
}

int sc_set_tau(sc_handle h, float tau_p) {
    int rc;
    if ((rc = check_handle(h))) return rc;
    if (!(tau_p >= 0.0f) || !std::isfinite(tau_p))
        return fail(SC_ERR_INVALID_ARG, "tau_p must be finite and >= 0");
    {
        DeviceGuard g(h->device);
        if ((rc = finish_async(h, nullptr, true))) return rc;
    }
    h->hp.tau_p = tau_p;
    h->proj_stale = true;
    return SC_OK;
}

int sc_set_state(sc_handle h, int idx, int kind, const float* src, void* stream) {
    int rc;
    if ((rc = check_handle(h)) || (rc = check_idx(h, idx))) return rc;
    if (!src) return fail(SC_ERR_INVALID_ARG, "src is NULL");
    const MatDev& m = h->mh[idx];
    float* dst = kind == SC_STATE_M_ANC ? m.Manc
                 : kind == SC_STATE_ADAM_M ? m.madam
                 : kind == SC_STATE_ADAM_V ? m.vadam
                                           : nullptr;
    if (!dst) return fail(SC_ERR_INVALID_ARG, "unknown state kind %d", kind);
    DeviceGuard g(h->device);
    if ((rc = finish_async(h, (hipStream_t)stream, false))) return rc;
    HIP_TRY(hipMemcpyAsync(dst, src, sizeof(float) * m.numel, hipMemcpyDeviceToDevice,
                           (hipStream_t)stream));
    if (kind == SC_STATE_M_ANC) {
        h->stale[idx] = 1;
        h->any_stale = true;
    }
    return SC_OK;
}

int sc_get_state(sc_handle h, int idx, int kind, float* dst, void* stream) {
    int rc;
    if ((rc = check_handle(h)) || (rc = check_idx(h, idx))) return rc;
    if (!dst) return fail(SC_ERR_INVALID_ARG, "dst is NULL");
    const MatDev& m = h->mh[idx];
    const float* src = kind == SC_STATE_M_ANC ? m.Manc
                       : kind == SC_STATE_ADAM_M ? m.madam
                       : kind == SC_STATE_ADAM_V ? m.vadam
                                                 : nullptr;
    if (!src) return fail(SC_ERR_INVALID_ARG, "unknown state kind %d", kind);
    DeviceGuard g(h->device);
    if ((rc = finish_async(h, (hipStream_t)stream, false))) return rc;
    HIP_TRY(hipMemcpyAsync(dst, src, sizeof(float) * m.numel, hipMemcpyDeviceToDevice,
                           (hipStream_t)stream));
    return SC_OK;
}

int sc_set_step(sc_handle h, int64_t t) {
    int rc;
    if ((rc = check_handle(h))) return rc;
    if (t < 0) return fail(SC_ERR_INVALID_ARG, "step count must be >= 0");
    h->t = t;
    return SC_OK;
}

int sc_get_step(sc_handle h, int64_t* t) {
    int rc;
    if ((rc = check_handle(h))) return rc;
    if (!t) return fail(SC_ERR_INVALID_ARG, "t is NULL");
    *t = h->t;
    return SC_OK;
}

int sc_set_factors(sc_handle h, int idx, const float* U, const float* s, const float* V,
                   void* stream) {
    int rc;
    if ((rc = check_handle(h)) || (rc = check_idx(h, idx))) return rc;
    if (!U || !s || !V) return fail(SC_ERR_INVALID_ARG, "U, s and V must be non-NULL");
    const MatDev& m = h->mh[idx];
    DeviceGuard g(h->device);
    if ((rc = finish_async(h, (hipStream_t)stream, false))) return rc;
    hipStream_t st = (hipStream_t)stream;
    // A-side (rows of F, length K): U for m >= n, V for m < n; the other side -> W.
    const float* fa = m.tall ? U : V;
    const float* wa = m.tall ? V : U;
    const int frows = m.tall ? m.m : m.n;  // K
    const int wrows = m.tall ? m.n : m.m;  // k
    HIP_TRY(hipMemsetAsync(m.F, 0, sizeof(float) * (size_t)m.k * m.K_ld, st));
    HIP_TRY(launch_transpose(fa, frows, m.k, m.k, m.F, m.K_ld, st));
    HIP_TRY(launch_transpose(wa, wrows, m.k, m.k, m.W, m.k, st));
    HIP_TRY(hipMemsetAsync(m.s, 0, sizeof(float) * m.kpad, st));
    HIP_TRY(hipMemcpyAsync(m.s, s, sizeof(float) * m.k, hipMemcpyDeviceToDevice, st));
    h->stale[idx] = 0;
    h->any_stale = false;
    for (char c : h->stale) h->any_stale = h->any_stale || c;
    // other matrices may still hold zero factors: warm start only once every
    // matrix has had factors installed or computed
    h->have_factors = h->have_factors || h->n == 1;
    return build_projectors(h, st);
}

int sc_get_factors(sc_handle h, int idx, float* U, float* s, float* V, void* stream) {
    int rc;
    if ((rc = check_handle(h)) || (rc = check_idx(h, idx))) return rc;
    const MatDev& m = h->mh[idx];
    DeviceGuard g(h->device);
    if ((rc = finish_async(h, (hipStream_t)stream, false))) return rc;
    hipStream_t st = (hipStream_t)stream;
    float* fa = m.tall ? U : V;
    float* wa = m.tall ? V : U;
    if (fa) HIP_TRY(launch_transpose(m.F, m.k, m.tall ? m.m : m.n, m.K_ld, fa, m.k, st));
    if (wa) HIP_TRY(launch_transpose(m.W, m.k, m.k, m.k, wa, m.k, st));
    if (s) HIP_TRY(hipMemcpyAsync(s, m.s, sizeof(float) * m.k, hipMemcpyDeviceToDevice, st));
    return SC_OK;
}

int sc_set_solve_waves(sc_handle h, int waves, int copies) {
    int rc;
    if ((rc = check_handle(h))) return rc;
    if (waves != 0 && waves != 1 && waves != 2 && waves != 4 && waves != 8)
        return fail(SC_ERR_INVALID_ARG, "waves must be 0, 1, 2, 4 or 8 (got %d)", waves);
    if (copies < 0 || copies > 2 || (waves == 1 && copies == 2))
        return fail(SC_ERR_INVALID_ARG, "copies must be 0, 1 or 2, and 0 or 1 for one wave (got %d)",
                    copies);
    DeviceGuard g(h->device);
    if ((rc = finish_async(h, nullptr, true))) return rc;
    h->solve_waves = waves;
    h->solve_copies = copies;
    return SC_OK;
}

int sc_set_fused_gram(sc_handle h, int enable) {
    int rc;
    if ((rc = check_handle(h))) return rc;
    DeviceGuard g(h->device);
    if ((rc = finish_async(h, nullptr, true))) return rc;
    h->fuse = enable != 0;
    return SC_OK;
}

int sc_set_v_rounds(sc_handle h, int rounds) {
    int rc;
    if ((rc = check_handle(h))) return rc;
    if (rounds != 1 && rounds != 2) return fail(SC_ERR_INVALID_ARG, "rounds must be 1 or 2");
    DeviceGuard g(h->device);
    if ((rc = finish_async(h, nullptr, true))) return rc;
    h->v_rounds = rounds;
    return SC_OK;
}

int sc_set_sweep_stop(sc_handle h, float stop) {
    int rc;
    if ((rc = check_handle(h))) return rc;
    if (!(stop >= 0.0f && stop < 1.0f)) return fail(SC_ERR_INVALID_ARG, "stop must be in [0, 1)");
    DeviceGuard g(h->device);
    if ((rc = finish_async(h, nullptr, true))) return rc;
    h->sweep_stop = stop;
    return SC_OK;
}

int sc_set_quad(sc_handle h, int mode) {
    int rc;
    if ((rc = check_handle(h))) return rc;
    if (mode < 0 || mode > 2) return fail(SC_ERR_INVALID_ARG, "quad mode must be 0, 1 or 2");
    DeviceGuard g(h->device);
    if ((rc = finish_async(h, nullptr, true))) return rc;
    h->quad_mode = mode;
    return SC_OK;
}

int sc_keep_proj(sc_handle h, int enable) {
    int rc;
    if ((rc = check_handle(h))) return rc;
    DeviceGuard g(h->device);
    if ((rc = finish_async(h, nullptr, true))) return rc;
    if (enable && !h->proj_arena) {
        size_t total = 0;
        std::vector<size_t> offs(h->n);
        for (int i = 0; i < h->n; ++i) {
            offs[i] = total;
            total += align_up((size_t)h->mh[i].numel * sizeof(float), 256);
        }
        void* p = nullptr;
        if (hipMalloc(&p, total) != hipSuccess) {
            (void)hipGetLastError();
            return fail(SC_ERR_OOM, "device allocation of %zu bytes failed", total);
        }
        h->proj_arena = (char*)p;
        if ((rc = wait_handle(h))) return rc;
        HIP_TRY(hipMemset(p, 0, total));
        for (int i = 0; i < h->n; ++i) h->mh[i].Gproj = (float*)(h->proj_arena + offs[i]);
        HIP_TRY(hipMemcpy(h->md, h->mh.data(), sizeof(MatDev) * h->n, hipMemcpyHostToDevice));
    }
    h->keep_proj = enable && h->proj_arena;
    return SC_OK;
}

int sc_get_filtered(sc_handle h, int idx, float* G_filt, float* G_proj, void* stream) {
    int rc;
    if ((rc = check_handle(h)) || (rc = check_idx(h, idx))) return rc;
    const MatDev& m = h->mh[idx];
    if (G_proj && !m.Gproj) return fail(SC_ERR_INVALID_ARG, "G_proj is not kept (sc_keep_proj)");
    DeviceGuard g(h->device);
    if ((rc = finish_async(h, (hipStream_t)stream, false))) return rc;
    hipStream_t st = (hipStream_t)stream;
    if (G_filt)
        HIP_TRY(hipMemcpyAsync(G_filt, m.Gfilt, sizeof(float) * m.numel, hipMemcpyDeviceToDevice,
                               st));
    if (G_proj)
        HIP_TRY(hipMemcpyAsync(G_proj, m.Gproj, sizeof(float) * m.numel, hipMemcpyDeviceToDevice,
                               st));
    return SC_OK;
}

int sc_get_stats(sc_handle h, sc_stats* out, int* per_mat_sweeps) {
    int rc;
    if ((rc = check_handle(h))) return rc;
    if (!out) return fail(SC_ERR_INVALID_ARG, "out is NULL");
    DeviceGuard g(h->device);
    if ((rc = finish_async(h, nullptr, true))) return rc;
    if ((rc = wait_handle(h)) || (rc = read_flags(h))) return rc;
    const int* status = h->status_h;
    memset(out, 0, sizeof(*out));
    out->n_mats = h->n;
    out->step = h->t;
    out->refreshes = h->refreshes;
    for (int i = 0; i < h->n; ++i) {
        const MatFlags& f = h->flags_h[i];
        out->sweeps_max = std::max(out->sweeps_max, f.sweeps);
        if (h->refreshes > 0 && !f.converged) out->not_converged += 1;
        out->factor_sweeps_max = std::max(out->factor_sweeps_max, f.sweep_base);
        out->factor_rejected += f.chol_fail;
        if (per_mat_sweeps) per_mat_sweeps[i] = f.sweeps;
    }
    out->nonfinite_grad = status[0] != 0;
    out->nonfinite_anchor = status[1] != 0;
    return SC_OK;
}

int sc_get_sweep_counts(sc_handle h, int* total, int* factor) {
    int rc;
    if ((rc = check_handle(h))) return rc;
    DeviceGuard g(h->device);
    if ((rc = finish_async(h, nullptr, true))) return rc;
    if ((rc = wait_handle(h)) || (rc = read_flags(h))) return rc;
    for (int i = 0; i < h->n; ++i) {
        if (total) total[i] = h->flags_h[i].sweeps;
        if (factor) factor[i] = h->flags_h[i].sweep_base;
    }
    return SC_OK;
}

int sc_profile(sc_handle h, int enable) {
    int rc;
    if ((rc = check_handle(h))) return rc;
    DeviceGuard g(h->device);
    if (enable < 0 || enable > 2) return fail(SC_ERR_INVALID_ARG, "enable must be 0, 1 or 2");
    if ((rc = finish_async(h, nullptr, true))) return rc;
    if (!h->prof.recs.empty() || !h->prof.snaps.empty()) {
        if ((rc = wait_handle(h))) return rc;
        for (auto& r : h->prof.recs) HIP_TRY(hipEventSynchronize(r.b));
        for (auto& r : h->prof.recs) {
            h->prof.pool.push_back(r.a);
            h->prof.pool.push_back(r.b);
        }
        h->prof.recs.clear();
        for (MatFlags* f : h->prof.snaps) h->prof.snap_pool.push_back(f);
        h->prof.snaps.clear();
    }
    for (int k = 0; k < PK_COUNT; ++k) {
        h->prof.launches[k] = 0;
        h->prof.ms[k] = h->prof.flops[k] = h->prof.bytes[k] = 0.0;
    }
    h->prof.on = enable != 0;
    h->prof.serial = enable == 2;
    return SC_OK;
}

int sc_get_kernel_times(sc_handle h, sc_kernel_time* out, int max_entries, int* count) {
    int rc;
    if ((rc = check_handle(h))) return rc;
    if (!count || (max_entries > 0 && !out))
        return fail(SC_ERR_INVALID_ARG, "out/count is NULL");
    DeviceGuard g(h->device);
    if ((rc = finish_async(h, nullptr, true))) return rc;
    if ((rc = wait_handle(h))) return rc;
    for (MatFlags* f : h->prof.snaps) {
        account_sweeps(h, f);
        h->prof.snap_pool.push_back(f);
    }
    h->prof.snaps.clear();
    for (auto& r : h->prof.recs) HIP_TRY(hipEventSynchronize(r.b));
    for (auto& r : h->prof.recs) {
        float ms = 0.0f;
        if (hipEventElapsedTime(&ms, r.a, r.b) == hipSuccess) h->prof.ms[r.kind] += ms;
        else (void)hipGetLastError();
        h->prof.pool.push_back(r.a);
        h->prof.pool.push_back(r.b);
    }
    h->prof.recs.clear();
    int n = 0;
    for (int k = 0; k < PK_COUNT; ++k) {
        if (h->prof.launches[k] == 0) continue;
        if (n < max_entries) {
            sc_kernel_time& t = out[n];
            memset(&t, 0, sizeof(t));
            snprintf(t.name, sizeof(t.name), "%s", kProfNames[k]);
            t.launches = h->prof.launches[k];
            t.total_ms = h->prof.ms[k];
            t.flops = h->prof.flops[k];
            t.bytes = h->prof.bytes[k];
        }
        ++n;
    }
    *count = n;
    return SC_OK;
}

}  // extern "C"

// ---- in-graph activation mask ----------------------------------------------------------

namespace {
uint64_t host_mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

int check_mask_sizes(int64_t T, int H, int K) {
    if (T < 0 || H < 1 || H > kMaskMaxH || K < 0 || K > H)
        return fail(SC_ERR_INVALID_ARG, "mask sizes out of range (T %lld, H %d, K %d; 1 <= H <= %d, 0 <= K <= H)",
                    (long long)T, H, K, kMaskMaxH);
    if (T > (int64_t)1 << 40) return fail(SC_ERR_INVALID_ARG, "T too large");
    return SC_OK;
}
}  // namespace

extern "C" {

int sc_mask_keep_count(int H, float p, int* K) {
    if (!K) return fail(SC_ERR_INVALID_ARG, "K is NULL");
    if (H < 1 || !(p >= 0.0f && p <= 1.0f)) return fail(SC_ERR_INVALID_ARG, "need H >= 1 and p in [0, 1]");
    *K = (int)std::floor((1.0 - (double)p) * H + 0.5);
    return SC_OK;
}

int sc_mask_seed(uint64_t layer, uint64_t step, uint64_t batch, uint64_t* seed) {
    if (!seed) return fail(SC_ERR_INVALID_ARG, "seed is NULL");
    const uint64_t g = 0x9E3779B97F4A7C15ull;
    uint64_t s = host_mix64((layer + 1) * g);
    s = host_mix64(s ^ ((step + 1) * g));
    *seed = host_mix64(s ^ ((batch + 1) * g));
    return SC_OK;
}

int sc_mask_indices(uint64_t seed, int64_t T, int H, int K, int32_t* idx, void* stream) {
    int rc;
    if ((rc = check_mask_sizes(T, H, K))) return rc;
    if (T > 0 && K > 0 && !idx) return fail(SC_ERR_INVALID_ARG, "idx is NULL");
    HIP_TRY(launch_mask_indices(seed, T, H, K, idx, (hipStream_t)stream));
    return SC_OK;
}

int sc_mask_pack(sc_dtype dtype, const void* x, const int32_t* idx, int64_t T, int H, int K, void* packed,
                 void* stream) {
    int rc;
    if ((rc = check_mask_sizes(T, H, K))) return rc;
    if (dtype != SC_F32 && dtype != SC_BF16) return fail(SC_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
    if (T > 0 && K > 0 && (!x || !idx || !packed)) return fail(SC_ERR_INVALID_ARG, "NULL pointer");
    HIP_TRY(launch_mask_pack(dtype == SC_BF16, x, idx, T, H, K, packed, (hipStream_t)stream));
    return SC_OK;
}

int sc_mask_unpack(sc_dtype dtype, const void* packed, const int32_t* idx, int64_t T, int H, int K, void* x,
                   void* stream) {
    int rc;
    if ((rc = check_mask_sizes(T, H, K))) return rc;
    if (dtype != SC_F32 && dtype != SC_BF16) return fail(SC_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
    if (T > 0 && (!x || (K > 0 && (!idx || !packed)))) return fail(SC_ERR_INVALID_ARG, "NULL pointer");
    HIP_TRY(launch_mask_unpack(dtype == SC_BF16, packed, idx, T, H, K, x, (hipStream_t)stream));
    return SC_OK;
}

}  // extern "C"
