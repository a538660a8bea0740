/*
 * scopt.h -- C ABI of the spectral-correction AdamW optimizer for AMD MI355X
 * (gfx950), implemented with hand-written HIP kernels in libscopt.so.
 *
 * The method (papernotes.org notes on "Communication-Efficient LLM Adaptation
 * over Decentralized GPU Meshes", arXiv 2609.14339):
 *   - "Key design 2" (asynchronous dual circuit): the fast circuit keeps a
 *     separate anchor momentum per weight matrix, updated with each delayed,
 *     unmasked anchor gradient by an EMA with coefficient beta_anc;
 *   - "Key design 3" (spectral-correction optimizer): SVD of the anchor
 *     momentum M = U S V^T, Tikhonov response d_i = s_i / (s_i + tau_p), the
 *     two-sided projection X = U^T G V, the filter X_filt = diag(d) X diag(d),
 *     the reconstruction G_filt = U X_filt V^T and the convex combination
 *     G_proj = alpha G_mask + (1 - alpha) G_filt;
 *   - "Overall framework" and "Training strategy": the result feeds AdamW
 *     (defaults tau_p = 1e-3, alpha = 0.3, beta_anc = 0.9, lr 2e-5).
 *
 * Conventions shared by every entry point
 *   - Matrices are row-major [rows][cols] (PyTorch's [out, in]), contiguous.
 *   - "device pointer": memory on the handle's device (hipMalloc'ed by the
 *     caller, e.g. a torch tensor's data_ptr()); "host pointer": CPU memory.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  Calls
 *     that take a stream enqueue work on it; the caller keeps inputs alive and
 *     unmodified until that work is done (usual stream ordering).  One
 *     exception, on by default: with sc_hparams.sync_check = 1,
 *     sc_anchor_update and sc_refresh (and sc_step when it has to refresh stale
 *     factors) poll the Jacobi convergence flags from the host so that no
 *     sweep beyond convergence is queued, and so block the calling thread
 *     until the refresh is within about one sweep of its end on the device
 *     (the 112-matrix 1B-shape workload: most of the refresh's device time).
 *     With sync_check = 0 they only enqueue (a fixed sweep budget whose
 *     rounds exit at once on converged matrices); sc_anchor_update_async moves
 *     the polling to a library thread.
 *   - Return value: SC_OK (0) or a negative SC_ERR_* code; sc_last_error()
 *     gives a message for the calling thread.  Arguments are validated before
 *     any GPU work is enqueued; an invalid call changes nothing.
 *   - A handle is not thread-safe; calls on one handle must be serialized.
 *   - The library owns all optimizer state (anchor momentum, SVD factors,
 *     filter, AdamW moments) and frees it in sc_opt_destroy.
 */
#ifndef SCOPT_H
#define SCOPT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SC_OK 0
#define SC_ERR_INVALID_ARG (-1) /* null pointer, bad index, bad hyper-parameter */
#define SC_ERR_SHAPE (-2)       /* non-positive or too large matrix shape */
#define SC_ERR_OOM (-3)         /* device memory allocation failed */
#define SC_ERR_HIP (-4)         /* a HIP runtime call failed */
#define SC_ERR_NO_DEVICE (-5)   /* no usable gfx950 device with that index */

typedef struct sc_opt* sc_handle;

typedef enum { SC_F32 = 0, SC_BF16 = 1 } sc_dtype;

typedef struct {
    float tau_p;        /* Tikhonov threshold tau_p ("Key design 3"), >= 0 */
    float alpha;        /* convex-combination weight of G_mask, in [0, 1] */
    float beta_anc;     /* anchor EMA coefficient ("Key design 2"), in [0, 1] */
    float lr;           /* AdamW learning rate, >= 0 */
    float beta1, beta2; /* AdamW moment coefficients, in [0, 1) */
    float eps;          /* AdamW epsilon (added outside the square root), > 0 */
    float weight_decay; /* decoupled weight decay, scaled by lr, >= 0 */
    int max_sweeps;     /* Jacobi sweep cap per refresh, >= 1 (e.g. 30) */
    float jacobi_tol;   /* rotation and convergence threshold on |a_p.a_q| / (|a_p||a_q|);
                           0 = default: rotate above 16 * 2^-24 (8 * 2^-24 for operands
                           with a Cholesky factor phase, max >= 2 min of rows, cols), stop
                           after a sweep whose largest ratio is
                           <= 2^-24 * max(16, sqrt(max(rows, cols))) */
    int sync_check;     /* 1: poll convergence flags on the host, queue no sweep past
                           convergence (blocks the caller, see above);
                           0: enqueue only: every phase of the refresh queues
                           max_sweeps sweeps (plain or factor phase, then the
                           polishing of factor-phase matrices that fail the Gram
                           certificate); a matrix's rounds exit at once after its
                           convergence, so choose max_sweeps near the sweeps needed */
    int warm_start;     /* 1: a refresh starts its sweeps from the previous factors
                           (A = M V_prev); 0: always from A = M, V = I */
    int precondition;   /* 1: for matrices with max(rows, cols) >= 2 min(rows, cols) the
                           sweeps first run on the k x k Cholesky factor L of the Gram
                           A^T A = L L^T (the right singular vectors of A are the left
                           ones of L; rows k instead of K long, no accumulated
                           rotations), then polish on A = M V until converged; a
                           matrix whose factorization is rejected runs the plain
                           sweeps.  Used by refreshes that start from previous
                           factors (warm_start = 1). */
} sc_hparams;

/* Fill `hp` with the defaults of the pages' training strategy:
 * tau_p 1e-3, alpha 0.3, beta_anc 0.9, lr 2e-5, betas (0.9, 0.999), eps 1e-8,
 * weight_decay 0.01, max_sweeps 30, jacobi_tol 0 (default), sync_check 1,
 * warm_start 1, precondition 1. */
void sc_default_hparams(sc_hparams* hp);

/* Create an optimizer over n_mats weight matrices of shapes rows[i] x cols[i]
 * (host arrays).  w_dtype: storage type of the weights W; g_dtype: type of
 * the masked gradients G_mask and the anchor gradients G_anc.  Anchor
 * momentum, SVD factors and AdamW moments are float32.  The anchor momentum
 * starts at zero, so until the first refresh d = 0 and G_filt = 0.
 * device: HIP device index.  On success *out receives the handle.
 * Errors: INVALID_ARG (null pointers, n_mats < 1, bad hyper-parameters),
 * SHAPE (rows/cols < 1 or > 65536), NO_DEVICE, OOM, HIP. */
int sc_opt_create(sc_handle* out, int n_mats, const int64_t* rows, const int64_t* cols,
                  sc_dtype w_dtype, sc_dtype g_dtype, const sc_hparams* hp, int device);

/* Free every device allocation of the handle, after waiting for the handle's
 * queued work as sc_get_stats does.  NULL is accepted. */
int sc_opt_destroy(sc_handle h);

/* Anchor arrival ("Key design 2"): for every matrix i,
 *   M_anc_i <- beta_anc * M_anc_i + (1 - beta_anc) * G_anc[i]
 * then refresh the thin SVD of M_anc_i (one-sided block Jacobi on the GPU),
 * the filter d and the projection operands used by sc_step.
 * G_anc: host array of n_mats device pointers to row-major rows x cols
 * matrices of g_dtype; read only. */
int sc_anchor_update(sc_handle h, const void* const* G_anc, void* stream);

/* Recompute SVD, filter and projection operands from the current anchor
 * momentum without an EMA update (used after sc_set_state of the anchor
 * momentum; sc_step calls it by itself when the factors are stale). */
int sc_refresh(sc_handle h, void* stream);

/* Asynchronous anchor arrival: the same EMA and refresh as sc_anchor_update,
 * run beside the steps that follow, so that the steps need not wait for it
 * ("Key design 2": the anchor circuit runs beside the fast replicas).  The
 * EMA and the refresh are ordered after the work already queued on `stream`
 * and run on the library's internal streams, driven by a host
 * thread of the library; the call returns at once (`stream` only waits for a
 * device copy of the operands the steps use).  Until the refresh is completed
 * by sc_refresh_wait, every sc_step uses the factors, filter and projectors of
 * the previous refresh (tau as set at this call), however far the refresh has
 * got: which factors a step uses never depends on timing.  sc_refresh_wait
 * orders its stream after the refresh and switches the following steps to the
 * new factors; every other entry point except sc_step, sc_set_lr,
 * sc_set_step, sc_get_step and sc_refresh_pending completes a pending refresh
 * the same way first (with a host wait where it takes no stream).
 * G_anc: as for sc_anchor_update; the matrices must stay valid and unchanged
 * until the refresh has been completed.  A second call while one is pending
 * completes the pending one first.  SC_ERR_INVALID_ARG while kernel timing is on
 * (sc_profile).  The copy of the step operands takes about as much device
 * memory as the weights (allocated at the first call, kept by the handle). */
int sc_anchor_update_async(sc_handle h, const void* const* G_anc, void* stream);

/* Complete a pending asynchronous refresh: join the library's host thread (it
 * returns once the refresh is fully queued), make `stream` wait for the
 * refresh's device work, and switch later steps to its factors; reports the
 * refresh's error, if any.  SC_OK when none is pending. */
int sc_refresh_wait(sc_handle h, void* stream);

/* *pending = 1 while the host thread of a pending asynchronous refresh is still
 * queueing it, else 0 (then sc_refresh_wait returns without blocking the host;
 * the device work may still be running). */
int sc_refresh_pending(sc_handle h, int* pending);

/* One optimizer step ("Key design 3" and AdamW): for every matrix i
 *   G_filt = U diag(d) (U^T G V) diag(d) V^T,  G_proj = alpha G + (1-alpha) G_filt,
 *   t <- t + 1; AdamW(W_i, G_proj) in place.
 * W: host array of n_mats device pointers to row-major w_dtype matrices,
 * updated in place.  G_mask: host array of n_mats device pointers (g_dtype),
 * read only. */
int sc_step(sc_handle h, void* const* W, const void* const* G_mask, void* stream);

/* sc_step without allocations, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same step and the same results, but the GEMM chain's
 * intermediates live in a file-scope device array of the library, 128 MiB per
 * GPU, held from the library's first use of that GPU until the process ends,
 * instead of the handle's memory; the matrices run in batches whose
 * intermediates fit it.  The call allocates nothing (no hipMalloc, no events,
 * no library routine that allocates).  Every handle on a GPU shares that
 * GPU's array: calls on one GPU whose work overlaps (other streams, other
 * threads) race on it and must be ordered by the caller; the array keeps the
 * last call's contents.  Arguments as sc_step.  Errors: SC_ERR_SHAPE when one
 * matrix's intermediates exceed the array (4 min(rows, cols)^2 bytes for a
 * square matrix, twice that otherwise: min(rows, cols) above 5792 or 4096),
 * before any GPU work; SC_ERR_INVALID_ARG while an asynchronous refresh is
 * pending or kernel timing is on.  Stale factors are refreshed first, as by
 * sc_step. */
int sc_step_noalloc(sc_handle h, void* const* W, const void* const* G_mask, void* stream);

/* Change the learning rate used by later steps (e.g. a cosine schedule). */
int sc_set_lr(sc_handle h, float lr);

/* Change tau_p; d and the projection operands are rebuilt from the cached
 * singular values before the next step (no new SVD). */
int sc_set_tau(sc_handle h, float tau_p);

#define SC_STATE_M_ANC 0  /* anchor momentum, rows x cols float32 */
#define SC_STATE_ADAM_M 1 /* AdamW first moment, rows x cols float32 */
#define SC_STATE_ADAM_V 2 /* AdamW second moment, rows x cols float32 */

/* Copy one state tensor of matrix idx from/to a caller device buffer of
 * rows x cols float32 (stream ordered).  Setting the anchor momentum marks
 * that matrix's factors stale; the next sc_step refreshes them. */
int sc_set_state(sc_handle h, int idx, int kind, const float* src, void* stream);
int sc_get_state(sc_handle h, int idx, int kind, float* dst, void* stream);

/* AdamW step count t (number of sc_step calls so far). */
int sc_set_step(sc_handle h, int64_t t);
int sc_get_step(sc_handle h, int64_t* t);

/* Install given SVD factors of matrix idx instead of computing them:
 * U (rows x r), s (r), V (cols x r) device float32 buffers, r = min(rows, cols),
 * row-major; U and V must have orthonormal columns.  d and the projection
 * operands are built from them as after a refresh.  For checkpoint restore
 * and for testing the projection stage on its own. */
int sc_set_factors(sc_handle h, int idx, const float* U, const float* s, const float* V,
                   void* stream);

/* Export the current factors of matrix idx (same layout as sc_set_factors).
 * The singular triplets are in no particular order. */
int sc_get_factors(sc_handle h, int idx, float* U, float* s, float* V, void* stream);

/* Variant of the 64-column pair solve of the Jacobi sweeps: `waves` = 1, 2, 4
 * or 8 wavefronts per pair, `copies` = 1 or 2 copies of the pair's Gram and
 * rotation in LDS (two copies: one barrier per step but half as many pairs
 * per CU).  0 picks per launch by its number of pairs: up to 512 pairs 8
 * waves and 2 copies, else 4 waves and 1 copy.  A tuning and test knob: every
 * variant computes the same rotations in the same order and gives
 * bit-identical results.  Other values, or copies 2 with one wave:
 * SC_ERR_INVALID_ARG.  Waits for a pending asynchronous refresh. */
int sc_set_solve_waves(sc_handle h, int waves, int copies);

/* Fused rotation apply + next-round pair Gram in the Jacobi sweeps (enabled by
 * default): for matrices with a power-of-two number of 32-column blocks (four
 * or more) the apply of each round also forms the next round's pair Grams from
 * the rotated rows (bfloat16 matrix cores, each float split exactly into three
 * parts, six part products), saving one read of the operand per round.
 * enable = 0 computes every round's Gram from the operand with float32
 * products; the two agree to float32 rounding, not bit for bit.  Waits for a
 * pending asynchronous refresh. */
int sc_set_fused_gram(sc_handle h, int enable);

/* Rotations of the V rows (the right factor accumulated in the Jacobi sweeps)
 * in the fused sweeps: rounds = 2 (default) applies each pair of consecutive
 * rounds of a sweep in one pass over V (V does not feed the sweeps, so a
 * round's V update can wait for the next round's), rounds = 1 one pass per
 * round.  Same products in the same order: V is bit-identical either way.
 * Other values: SC_ERR_INVALID_ARG.  Waits for a pending asynchronous refresh.
 * A schedule of the thin SVD of the anchor momentum ("Key design 3" of the
 * papernotes.org notes); it changes no result. */
int sc_set_v_rounds(sc_handle h, int rounds);

/* Sweep-stop rule of the Jacobi sweeps (default 1e-4): a matrix's sweeps also
 * end after a sweep whose largest relative off-diagonal |a_p.a_q| / (|a_p||a_q|)
 * was at most `stop` (convergence is quadratic by then, so the next sweep would
 * rotate almost nothing), and a certificate over the final operand's Gram checks
 * the result: after the Cholesky factor phase the one of A = M V (pairs above
 * the convergence threshold are polished), after plain sweeps the final Gram's
 * (a matrix above the threshold sweeps on; applied only with sync_check, whose
 * polls read the outcome).  In the factor phase the value is capped at 1e-4:
 * that certificate does not cover V, which is as orthogonal as the factor's
 * rows are converged.  stop = 0 turns the rule off (sweeps end only on a
 * sweep that saw nothing above the threshold).  SC_ERR_INVALID_ARG unless
 * 0 <= stop < 1.  Waits for a pending asynchronous refresh.  A schedule of the
 * thin SVD of the anchor momentum ("Key design 3" of the papernotes.org notes);
 * the results meet the same convergence threshold either way. */
int sc_set_sweep_stop(sc_handle h, float stop);

/* Quad passes of the Jacobi sweeps (mode 1, the default): for matrices whose column-block
 * count nb (k rounded up to 64, over 32) is 4, 16, 64 or 256, the nb - 1 pair
 * rounds of a sweep are taken three at a time: the masks of the XOR rounds
 * split into lines {m0, m1, m0 ^ m1}, whose three rounds pair blocks inside
 * groups of four, so one pass per line forms each group's 128 x 128 Gram,
 * solves the three rounds' block pairs in LDS (the next round's Gram from the
 * rotated one) and applies their product to the group's rows: one read of the
 * operand for the Gram and one read and write for the rotation per three
 * rounds.  Every block pair is still solved once per sweep, in another order;
 * the results meet the same convergence threshold.  A list of matrices (a
 * refresh pipeline's plain or factor-phase set) runs quad passes only when all
 * its block counts allow it; mode 1 also requires at least 256 groups of four
 * blocks per pass (a group's three rounds run in sequence, so fewer groups leave
 * the GPU idle), mode 2 takes them wherever the block counts allow, mode 0
 * keeps the pair rounds.  Polishing sweeps keep the pair rounds.  Other modes:
 * SC_ERR_INVALID_ARG.  Waits for a pending asynchronous refresh.  A schedule
 * of the thin SVD of the anchor momentum ("Key design 3" of the papernotes.org
 * notes). */
int sc_set_quad(sc_handle h, int mode);

/* Keep G_proj of each step (costs one more store per element in the AdamW
 * pass and rows x cols floats per matrix). */
int sc_keep_proj(sc_handle h, int enable);

/* Copy the last step's G_filt and (if sc_keep_proj was enabled) G_proj of
 * matrix idx into caller device buffers of rows x cols float32; either may be
 * NULL. */
int sc_get_filtered(sc_handle h, int idx, float* G_filt, float* G_proj, void* stream);

typedef struct {
    int n_mats;
    int64_t step;          /* AdamW step count t */
    int refreshes;         /* SVD refreshes done */
    int sweeps_max;        /* most Jacobi sweeps any matrix needed in the last refresh */
    int not_converged;     /* matrices whose last refresh hit max_sweeps or met a
                              non-finite operand */
    int nonfinite_grad;    /* 1 if a non-finite G_mask value was seen by a step */
    int nonfinite_anchor;  /* 1 if a non-finite G_anc value was seen by an EMA */
    int factor_sweeps_max; /* most sweeps any matrix ran on its Cholesky factor (last refresh) */
    int factor_rejected;   /* matrices whose Cholesky factorization was rejected (last refresh) */
} sc_stats;

/* Wait (host) for the handle's own queued work -- its last refresh and last
 * step, on the streams they were queued on, and its internal streams; not
 * device-wide -- and report counters.  not_converged counts matrices whose
 * last refresh hit max_sweeps or met a non-finite operand (NaN or infinity in
 * the anchor momentum: their factors are not finite).
 * per_mat_sweeps: optional host array of n_mats ints receiving the sweeps of
 * each matrix in the last refresh (factor and polishing sweeps together). */
int sc_get_stats(sc_handle h, sc_stats* out, int* per_mat_sweeps);

/* Wait for the handle's work as sc_get_stats does and copy per-matrix sweep counts
 * of the last refresh into host arrays of n_mats ints (either may be NULL):
 * total[i] all sweeps, factor[i] the sweeps run on the Cholesky factor (0 when
 * the matrix was not preconditioned or its factorization was rejected). */
int sc_get_sweep_counts(sc_handle h, int* total, int* factor);

/* Kernel timing for measurement: when enabled, every kernel launch of the
 * handle is bracketed by a pair of HIP events on the stream it runs on (small
 * host overhead per launch).  enable = 1: the launches keep their production
 * schedule (the refresh split over two internal streams whose kernels overlap,
 * convergence polls that do not block), so a timed run is the production run
 * and each launch's time includes sharing the GPU with the other stream's
 * kernels; the work counters of each refresh are copied behind it and folded
 * in by sc_get_kernel_times.  enable = 2: serialized, every kernel alone on the
 * caller's stream and each convergence poll waited for (slower pass; kernel
 * times without overlap).  enable = 0: off.  Any change resets the totals.
 * SC_ERR_INVALID_ARG for other values. */
int sc_profile(sc_handle h, int enable);

typedef struct {
    char name[32];     /* kernel family, e.g. "jacobi_gram", "step_gemm1", "combine_adamw" */
    int64_t launches;  /* launches timed */
    double total_ms;   /* summed event time of those launches */
    double flops;      /* algorithmic floating-point operations of those launches */
    double bytes;      /* algorithmic HBM bytes of those launches (streaming kernels) */
} sc_kernel_time;

/* Wait for the timed launches' events, fold finished timings in, and copy up to
 * max_entries per-family records to `out` (host array); *count receives the
 * number of families with at least one launch. */
int sc_get_kernel_times(sc_handle h, sc_kernel_time* out, int max_entries, int* count);

/* Message of the last error on the calling thread ("" if none). */
const char* sc_last_error(void);

/* ---- In-graph activation mask ("Key design 1") ----------------------------------
 * At a pipeline boundary each of T tokens keeps K of its H hidden dimensions;
 * the kept set is a deterministic function of (layer, step, batch), so sender
 * and receiver rebuild it locally and only the K kept values per token travel;
 * the gradient of the masked states travels back through the same set.  Token
 * i keeps the K dimensions j with the smallest u = mix64(seed + (i*H + j + 1) *
 * 0x9E3779B97F4A7C15) (ties to the smaller j), in ascending order; mix64 is the
 * SplitMix64 output function.  These calls need no handle.  Limits: 1 <= H <=
 * 4096, 0 <= K <= H, T >= 0; T = 0 or K = 0 queues nothing (unpack with K = 0
 * writes zeros); pack and unpack clamp index entries outside [0, H) into it
 * (valid index sets come from sc_mask_indices).  Errors: SC_ERR_INVALID_ARG for bad sizes, a NULL pointer or an
 * unknown dtype, before any GPU work. */

/* K = floor((1 - p) * H + 1/2) kept dimensions per token at mask rate p in [0, 1]. */
int sc_mask_keep_count(int H, float p, int* K);

/* The mask seed of (layer, step, batch):
 * mix64(mix64(mix64((layer+1)*G) ^ (step+1)*G) ^ (batch+1)*G), G = 0x9E3779B97F4A7C15,
 * 64-bit wrapping arithmetic. */
int sc_mask_seed(uint64_t layer, uint64_t step, uint64_t batch, uint64_t* seed);

/* idx: device int32 [T][K], written with the kept dimensions of each token. */
int sc_mask_indices(uint64_t seed, int64_t T, int H, int K, int32_t* idx, void* stream);

/* packed[i][k] = x[i][idx[i][k]]: x device [T][H] of dtype, packed device [T][K]. */
int sc_mask_pack(sc_dtype dtype, const void* x, const int32_t* idx, int64_t T, int H, int K,
                 void* packed, void* stream);

/* x[i][j] = packed[i][k] where idx[i][k] = j, else 0: the masked states (forward,
 * receiver) or the masked gradient (backward, sender; packed = the packed
 * gradient).  x device [T][H] of dtype, overwritten. */
int sc_mask_unpack(sc_dtype dtype, const void* packed, const int32_t* idx, int64_t T, int H, int K,
                   void* x, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SCOPT_H */
