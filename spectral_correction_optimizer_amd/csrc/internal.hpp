// Internal structures of libscopt shared by the host orchestration (api.cpp)
// and the kernel launchers (elementwise.hip, gemm.hip, jacobi.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace scopt {

constexpr int kMaxPtrs = 128;  // matrices per launch when pointers travel as kernel arguments
constexpr int kJb = 32;        // Jacobi column-block width b; a pair block holds 2b = 64 columns
constexpr int kPw = 2 * kJb;   // pair width
constexpr int kApplyCols = 128;            // columns per rotation-apply workgroup
constexpr int kApplyThreads = 2 * kApplyCols;  // a 64-lane wave updates 32 columns
constexpr int kApplyRun = 4;  // column chunks per rotation-apply workgroup (pipelined)
constexpr int kV2Cols = 256;  // V columns per chunk of the two-round V apply (8 waves x 32)
constexpr int kV2Threads = 8 * 64;
constexpr int kV2Run = 4;     // chunks per two-round V apply workgroup
// Quad passes (quad.hip): three pair rounds of one pass over groups of four blocks
constexpr int kQuadCols = 256;  // columns per chunk of the group apply (8 waves x 32)
constexpr int kQuadThreads = 8 * 64;
constexpr int kQuadRun = 4;     // chunks per group-apply workgroup
constexpr int kQuadGramCols = 1024;  // column split of the group Gram when the groups are few
constexpr int kQuadGramFill = 512;   // group Gram workgroups per pass that fill the chip
// A list runs quad passes only with at least this many groups per pass: a group's
// three rounds run in sequence on one CU, so fewer groups leave the chip idle (one
// 2048 x 2048 matrix, 16 groups: 63.6 ms per pass against 46.6 in pair rounds; one
// Llama-3.2-1B block, 56 groups: 87.9 against 79.7; 16 blocks, 512 + 896: 590
// against 625).
constexpr int kQuadMinGroups = 256;
// Block counts whose pair rounds split into quad passes: powers of four from 4 to 256.
__host__ __device__ inline bool quad_capable(int nb) {
    return nb == 4 || nb == 16 || nb == 64 || nb == 256;
}
__host__ __device__ inline int quad_passes(int nb) { return (nb - 1) / 3; }

// Caller pointers of one call (weights / gradients), passed by value.
struct PtrTable {
    const void* p[kMaxPtrs];
};

// Per-matrix geometry and device buffers (device-visible copy in MatDev[]).
struct MatDev {
    int m, n;        // weight shape, row-major [m][n]
    int K, k;        // Jacobi operand A is K x k with K = max(m,n), k = min(m,n)
    int kpad;        // k rounded up to a multiple of 2b
    int K_ld;        // row stride of A and F: K rounded up to a multiple of 128
    int nb;          // kpad / b column blocks
    int tall;        // 1 when m >= n (A = M), 0 when m < n (A = M^T)
    int64_t numel;   // m * n
    float* Manc;     // [m][n] anchor momentum
    float* madam;    // [m][n] AdamW first moment
    float* vadam;    // [m][n] AdamW second moment
    float* A;        // [kpad][K_ld] Jacobi operand, rows = columns of A (zero padded)
    float* V;        // [kpad][kpad] accumulated rotations, rows = columns of V_A
    float* F;        // [k][K_ld] final A-side singular vectors (rows), unit norm
    float* W;        // [k][k] final accumulated-side singular vectors (rows)
    float* PL;       // [m][m] left projector U D U^T (square or wide)
    float* PR;       // [n][n] right projector V D V^T (square or tall)
    float* s;        // [kpad] singular values
    float* d;        // [kpad] Tikhonov response
    double* norm2;   // [kpad] squared row norms (scratch)
    int* perm;       // [kpad] Jacobi column order: logical position -> physical row of A / V
    float* cnorm;    // [kpad] squared column norms by physical row (sweep-start ordering)
    float* Gfilt;    // [m][n] filtered gradient of the last step
    float* Gproj;    // [m][n] combined gradient (only when kept), else null
    float* Y;        // [k][k] step intermediate
    float* T;        // [k][k] step intermediate
    float* E;        // [k][k] refresh scratch (Gram of factors, scaled copies)
    float* invn;     // [kpad] refresh scratch: inverse row norms of the factor-phase X
    double* gram;    // [nb/2][nsplit][2b][2b] split partial Gram blocks
    float* rot;      // [2][nb/2][2b][2b] R = Q - I of each pair, by round parity
    int* rot_flag;   // [2][nb/2] 1 when the pair's rotation must be applied
    int nsplit;      // K-splits of a pair Gram (room in `gram`; a phase may use fewer)
    int klen;        // row length of the Cholesky-factor operand: k rounded up to 128 (0: none)
    float tol;       // a pair is rotated when |a_p.a_q| / (|a_p| |a_q|) > tol
    float tol_conv;  // a sweep whose largest such ratio is <= tol_conv ends the sweeps
    int pad1;
    double* chol;    // [k][k] Gram of A, then its Cholesky factor (lower triangle); klen > 0 only
    float* bmax;     // [nb][nb] selective polishing: largest |E_ij| per block pair (klen > 0
                     // and kpad <= kSelMaxK only, else null)
};

// Per-matrix device flags / counters.
struct MatFlags {
    unsigned int sweep_max;  // max relative off-diagonal seen this sweep (float bits)
    int converged;           // 1 once a sweep saw nothing above tolerance
    int sweeps;              // sweeps done in the current refresh
    int done;                // converged or sweep cap reached
    float floor2;            // squared column-norm floor: columns below are zero
    int pairs_applied;       // pair rotations applied (work accounting)
    int sweep_base;          // sweeps done before the current phase (the cap counts from here)
    int precond;             // 1 while the sweeps run on the Cholesky factor (short rows)
    int chol_fail;           // 1 when the Gram's Cholesky factorization was rejected
    int pairs_pre;           // pairs_applied at the end of the factor phase
    unsigned int check_off;  // largest |a_p.a_q| / (|a_p| |a_q|) of the final operand (float bits)
    int regram;              // 1 when the certificate failed: polished, its final Gram is redone
    int sel;                 // 1 while polishing sweeps work only on the pairs bmax marks
    int sel_pairs;           // pair Grams solved in selective sweeps (work accounting)
    int sel_rot;             // pairs rotated in selective sweeps (work accounting)
    int sel_sweeps;          // selective sweeps run
    int early;               // 1 when plain sweeps ended on the sweep-stop rule (certificate pending)
    int quads_applied;       // quad passes: groups whose composed rotation was applied
    int quads_pre;           // quads_applied at the end of the factor phase
};

// Selective polishing: largest k (and kpad) whose inverse column order fits the
// marking kernel's LDS, and the sweep cap of the selective phase.
constexpr int kSelMaxK = 4096;
constexpr int kSelSweeps = 3;

// ---- work items ------------------------------------------------------------------

// operand columns [x0, x1) of one split; fused: the matrix's Grams after the first
// round of a sweep come from jac_apply_gram_kernel
struct GramItem { int mat, slot, split, x0, x1, fused; };
struct SolveItem { int mat, slot, nsplit; };
// which: 0 = A rows, 1 = V rows; chunks [chunk, chunk + nchunk) of kApplyCols columns
struct ApplyItem { int mat, slot, which, chunk, nchunk; };
// quad passes: group apply of group `group`, A rows (which = 0) or V rows (1), columns [x0, x1)
struct QuadItem { int mat, group, which, x0, x1; };
// fused apply + next Gram: four-block group of a power-of-two block count over
// operand columns [x0, x1) of split `split` (at most 8 chunks of kApplyCols)
struct FusedItem { int mat, group, split, x0, x1; };
struct Chunk { int mat; int64_t off; int len; };    // elementwise chunk of one matrix
struct SyrkItem { int mat, ti, tj; };               // lower 128 x 128 tile (ti >= tj) of A^T A

// ---- grouped GEMM ----------------------------------------------------------------

enum { GF_ZERO_DIAG = 1 };

struct GemmProb {
    const void* A;   // M x K (or K x M when transposed), element type of the launch
    const void* B;   // K x N (or N x K when transposed)
    float* C;        // M x N float32 output
    const float* Cin;  // optional, out = alpha*acc + beta*Cin
    const float* row_scale;  // optional scale of output row i
    const float* col_scale;  // optional scale of output column j
    const float* k_scale;    // optional scale of B's reduction index (row of B)
    int M, N, K;
    int lda, ldb, ldc, ldcin;
    float alpha, beta;
    int flags;
    int a_ptr, b_ptr;  // >= 0: take A (B) from the call's PtrTable entry
    int tiles_n, tile_start;
    const int* gate;   // optional: the problem is skipped when *gate == 0
};

// Launch one grouped GEMM over `probs` (device array, nprob entries, tile
// prefix filled); ta/tb: operand stored transposed; a_bf16/b_bf16: operand
// element type; vec: every problem's row-major operands (A unless ta, B if
// tb) have 16-byte aligned rows (8 for bfloat16) and K a multiple of 8.
// full: every problem's M, N and K are multiples of the 256 x 128 x 16 tile (no
// clamped addresses or zeroed elements).
// parts: 3 = float32-level products (six bfloat16 part products); 2 = three part
// products, for correction terms only (float32 operands, neither transposed).
// ptrs: caller pointers referenced by a_ptr/b_ptr.
hipError_t launch_gemm(const GemmProb* probs_dev, int nprob, int total_tiles, bool ta, bool tb,
                       bool a_bf16, bool b_bf16, bool vec, bool full, int parts, const PtrTable& ptrs,
                       hipStream_t st);
constexpr int kGemmBM = 256, kGemmBN = 128;

// ---- elementwise -------------------------------------------------------------------

hipError_t launch_ema(const MatDev* mats, const Chunk* chunks, int nchunks, const PtrTable& g,
                      bool g_bf16, float beta, int* nonfinite, hipStream_t st);
hipError_t launch_combine_adamw(const MatDev* mats, const Chunk* chunks, int nchunks,
                                const PtrTable& w, const PtrTable& g, bool w_bf16, bool g_bf16,
                                float alpha, float beta1, float beta2, float eps,
                                float step_size, float inv_sqrt_bc2, float lr_wd, int keep_proj,
                                int* nonfinite, hipStream_t st);
// The per-matrix passes below run over nmat matrices: mat_idx[0 .. nmat) (device
// list) or, with mat_idx == nullptr, matrices 0 .. nmat - 1.
// A <- M (copy or transpose), V <- I.
hipError_t launch_jacobi_load(const MatDev* mats, const int* mat_idx, int nmat, int max_kpad,
                              int max_K, hipStream_t st);
// Warm start: V <- previous W (padded with identity), zero padding rows of A.
hipError_t launch_jacobi_warm(const MatDev* mats, const int* mat_idx, int nmat, hipStream_t st);
// norm2[j] = sum_x X[j][x]^2 (fp64) for the rows of A (which=0) or V (which=1)
hipError_t launch_rownorm(const MatDev* mats, const int* mat_idx, int nmat, int which, int max_kpad,
                          hipStream_t st);
// floor2 = (2^-24)^2 * sum_j norm2[j]; clears sweep flags
hipError_t launch_jacobi_init_flags(const MatDev* mats, const int* mat_idx, MatFlags* flags,
                                    int nmat, hipStream_t st);
// Normalize rows of A (which=0, in place, s) or V (which=1, in place).
hipError_t launch_normalize(const MatDev* mats, const int* mat_idx, const MatFlags* flags,
                            int nmat, int which, int max_kpad, hipStream_t st);
hipError_t launch_filter(const MatDev* mats, const int* mat_idx, int nmat, float tau,
                         hipStream_t st);

// ---- Jacobi sweeps -------------------------------------------------------------------

hipError_t launch_jacobi_gram(const MatDev* mats, const MatFlags* flags, const GramItem* gi,
                              int ngi, int round, int skip_fused, hipStream_t st);
// Pair solve variants: waves = 1, 2, 4 or 8 wavefronts per pair; copies = 1 or
// 2 copies of G and R^T in LDS (one wavefront: one copy).  0 picks by the
// launch's pair count: up to kSolveSmallMax pairs eight waves and two copies
// (two pairs per CU), else four waves and one copy (four pairs per CU).  All
// variants give identical results.
constexpr int kSolveSmallMax = 512;
int solve_waves_for(int nsi);
hipError_t launch_jacobi_solve(const MatDev* mats, MatFlags* flags, const SolveItem* si, int nsi,
                               int round, int waves, int copies, hipStream_t st);
hipError_t launch_jacobi_apply_gram(const MatDev* mats, const MatFlags* flags, const FusedItem* fi,
                                   int nfi, int round, hipStream_t st);
hipError_t launch_jacobi_apply(const MatDev* mats, const MatFlags* flags, const ApplyItem* ai,
                               int nai, int round, hipStream_t st);
// V rows of power-of-two block counts: in a sweep's odd rounds the rotations of
// that round and the one before in one pass, in its last round that round's;
// other rounds return at once.  Items: FusedItem with x0 / x1 columns of V (runs
// of kV2Run chunks of kV2Cols), group < nb / 4.
hipError_t launch_jacobi_apply_v2(const MatDev* mats, const MatFlags* flags, const FusedItem* vi,
                                  int nvi, int round, hipStream_t st);
// Quad passes (quad.hip) of the matrices whose block count is quad_capable: pass
// `pass` of the list, each matrix at pass % quad_passes(nb) of its sweep.
// gram: the group Grams (items: group, split, operand columns x0 .. x1, at most
// kQuadGramCols, multiples of 128); solve: the three rounds of each group (items:
// slot = group, nsplit = the matrix's splits); apply: the composed rotations.
hipError_t launch_quad_gram(const MatDev* mats, const MatFlags* flags, const FusedItem* items, int n,
                            int pass, hipStream_t st);
hipError_t launch_quad_solve(const MatDev* mats, MatFlags* flags, const SolveItem* items, int n,
                             int pass, hipStream_t st);
hipError_t launch_quad_apply(const MatDev* mats, const MatFlags* flags, const QuadItem* items, int n,
                             int pass, hipStream_t st);
// At a matrix's sweep start: order its columns by decreasing norm (perm).  quad:
// the list runs quad passes (quad_passes(nb) per sweep instead of nb - 1 rounds).
hipError_t launch_jacobi_sort(const MatDev* mats, const MatFlags* flags, const int* mat_idx,
                              int nmat, int round, int quad, hipStream_t st);
// A sweep that saw nothing above tol_conv ends a matrix's sweeps; so does one that
// saw at most stop_factor (factor phase) or stop_plain (plain sweeps; early = 1,
// the final Gram's certificate decides): 0 turns the rule off.
hipError_t launch_jacobi_sweep_end(const MatDev* mats, MatFlags* flags, const int* mat_idx,
                                   int nmat, int round, int quad, int max_sweeps, float stop_factor,
                                   float stop_plain, hipStream_t st);

// ---- Cholesky preconditioning of tall operands ------------------------------------------

// chol = A^T A (lower 128 x 128 tiles listed in items), float64 sums; full: every
// listed matrix's k is a multiple of 128.
hipError_t launch_chol_syrk(const MatDev* mats, const MatFlags* flags, const SyrkItem* items,
                            int nitems, int only_regram, bool full, hipStream_t st);
// chol = L L^T (in place, lower triangle) for the matrices in mat_idx; on success the
// rows of A become the columns of L (length klen) and precond = 1, else chol_fail = 1
// and done = 1 (the matrix sits the factor phase out).  max_nbk: largest ceil(k / 64),
// max_klen: largest klen.
hipError_t launch_cholesky(const MatDev* mats, MatFlags* flags, const int* mat_idx, int nmat,
                           int max_nbk, int max_klen, hipStream_t st);
// E[i][j] = c_ij / sqrt(c_ii c_jj) (i != j; 0 on the diagonal and for columns at
// the zero floor) from the float64 Gram in md.chol (lower triangle, from
// launch_chol_syrk), for the matrices in mat_idx; the largest |E_ij| goes to
// check_off.  max_t64: largest ceil(k / 64).
hipError_t launch_gram_to_e(const MatDev* mats, MatFlags* flags, const int* mat_idx, int nmat,
                            int max_t64, int only_regram, hipStream_t st);
// For the matrices in mat_idx: converged and done when check_off <= tol_conv,
// otherwise not done (polishing sweeps follow) and check_off cleared.
hipError_t launch_certify(const MatDev* mats, MatFlags* flags, const int* mat_idx, int nmat,
                          hipStream_t st);
// For the matrices in mat_idx whose plain sweeps ended on the sweep-stop rule
// (early): kept when check_off <= tol_conv, else not done, regram = 1 (more
// sweeps follow, then their final Gram again); early cleared.
hipError_t launch_certify_early(const MatDev* mats, MatFlags* flags, const int* mat_idx, int nmat,
                                hipStream_t st);
// inv[j] = 1 / sqrt(cnorm[j]) for j < k of the accepted matrices (into md.Y):
// row scales that make V = L^T-phase vectors x W_prev orthonormal.
hipError_t launch_factor_invnorm(const MatDev* mats, const MatFlags* flags, const int* mat_idx,
                                 int nmat, int max_k, hipStream_t st);
// Start of the polishing phase for the matrices in mat_idx (A already recomputed).
hipError_t launch_phase2_reset(const MatDev* mats, MatFlags* flags, const int* mat_idx, int nmat,
                               hipStream_t st);
// Selective polishing of the matrices in mat_idx that failed the certificate
// (not done): bmax from the certificate's E in the current column order, then
// sel = 1.  max_nb: largest block count.
hipError_t launch_polish_mark(const MatDev* mats, MatFlags* flags, const int* mat_idx, int nmat,
                              int max_nb, hipStream_t st);
// After selective polishing failed its re-certification: sel = 0, so that full
// polishing sweeps follow for the matrices that are not done.
hipError_t launch_polish_full(MatFlags* flags, const int* mat_idx, int nmat, hipStream_t st);

// dst[c * ld_dst + r] = src[r * ld_src + c] for r < rows, c < cols
hipError_t launch_transpose(const float* src, int rows, int cols, int ld_src, float* dst,
                            int ld_dst, hipStream_t st);


// ---- in-graph activation mask (mask.hip) ------------------------------------------
constexpr int kMaskMaxH = 4096;  // hidden sizes up to 4096 (LDS: 48 KB per token sort)
hipError_t launch_mask_indices(uint64_t seed, int64_t T, int H, int K, int32_t* idx, hipStream_t st);
hipError_t launch_mask_pack(bool bf16, const void* x, const int32_t* idx, int64_t T, int H, int K,
                            void* packed, hipStream_t st);
hipError_t launch_mask_unpack(bool bf16, const void* packed, const int32_t* idx, int64_t T, int H, int K,
                              void* x, hipStream_t st);

}  // namespace scopt
