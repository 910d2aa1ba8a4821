/*
 * muon_ns.h -- C ABI of the MI355X (gfx950) Muon / Newton-Schulz optimizer-step library.
 *
 * Method source: the page "Dion3: Full-stack orthogonal updates" (arXiv 2608.11612).
 *   - Muon step: section "Muon Update Rule", Eq. (1), with polar(X) of Definition 1.
 *   - NorMuon: section "NorMuon Variant", Eq. (2).
 *   - Standard quintic Newton-Schulz: section "Standard Newton-Schulz".
 *   - Gram Newton-Schulz: section "1. Gram Newton-Schulz", Theorem 2, restart,
 *     Algorithm 3.
 *   - Fractional row selection: section "3. Dion3 Update Rule", Algorithm 4.
 *
 * General rules for every entry point
 *   - Every pointer is a DEVICE pointer unless its comment says (host).
 *   - Matrices are dense, row-major, contiguous: element (i, j) of a rows x cols matrix
 *     is at offset i*cols + j; a batch of B such matrices is B consecutive matrices.
 *   - Device pointers must be 16-byte aligned; the workspace must be 256-byte aligned.
 *   - Sizes: 1 <= rows, cols <= 65536 and rows*cols <= 2^31 - 1; the Newton-Schulz iterate
 *     (rows and cols each rounded up to a multiple of 256, and 256 more elements per row,
 *     in either of its two layouts) must stay below 2 GiB (2 bytes per element for
 *     MNS_BF16, 4 for MNS_F32), else MNS_ERR_SHAPE.
 *   - Storage dtype (mns_dtype): MNS_BF16 (W, G, X, O stored as bfloat16) or MNS_F32.
 *     Momentum M and NorMuon state v are always float32.
 *   - Ownership: the caller owns every buffer, including the workspace, whose size the
 *     matching *_workspace_size call returns. The library allocates no device memory,
 *     keeps no state between calls (apart from an open profiling session, see the end of
 *     this file) and is reentrant; calls on different streams must use different
 *     workspaces. The one exception is ns_orthogonalize_noalloc: its calls on one GPU
 *     share a static scratch array and must not overlap.
 *   - Errors: arguments are validated synchronously, before anything is enqueued, and
 *     reported as an mns_status; nothing is enqueued when a call returns an error other
 *     than MNS_ERR_HIP. MNS_ERR_HIP means a kernel launch failed (the stream may hold
 *     part of the call's work). No C++ exception crosses this boundary.
 *   - Streams: every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream). Nothing synchronises; the results are ready when the stream reaches them.
 *   - Graph capture: a call may be recorded into a HIP graph by capturing `stream` (it only
 *     enqueues kernels: no memset, allocation, synchronisation or host read of device
 *     data). A replay repeats the call with the pointers, sizes and hyperparameters given
 *     at capture time. Do not capture while a profiling session is open. The Dion3 page
 *     (section "3. Dion3 Update Rule", its implementation details) captures the step in a
 *     graph to remove launch overhead at small scales.
 *   - A zero input matrix yields a zero orthogonalised output (W unchanged), not an error.
 */
#ifndef MUON_NS_H
#define MUON_NS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mns_status {
  MNS_OK = 0,
  MNS_ERR_NULL = 1,        /* a required pointer is NULL */
  MNS_ERR_SHAPE = 2,       /* a size is out of range */
  MNS_ERR_DTYPE = 3,       /* unknown storage dtype */
  MNS_ERR_PARAM = 4,       /* a hyperparameter or alignment is invalid */
  MNS_ERR_WORKSPACE = 5,   /* workspace NULL, misaligned or smaller than required */
  MNS_ERR_HIP = 6          /* a HIP launch failed */
} mns_status;

typedef enum mns_dtype { MNS_F32 = 0, MNS_BF16 = 1 } mns_dtype;

typedef enum mns_ns_kind {
  MNS_NS_STANDARD = 0,     /* quintic NS on the rectangular iterate ("Standard Newton-Schulz") */
  MNS_NS_GRAM = 1          /* Gram NS on the small n x n side (Theorem 2 + restarts) */
} mns_ns_kind;

/* One weight matrix and its optimizer state (rows x cols, row-major).
 *   W  in/out  storage dtype       weights, updated in place
 *   M  in/out  float32             momentum, updated in place
 *   G  in      storage dtype       gradient
 *   v  in/out  float32 [rows]      NorMuon second moment per stored row; may be NULL
 *                                  when NorMuon is off */
typedef struct mns_matrix {
  void* W;
  float* M;
  const void* G;
  float* v;
  int64_t rows;
  int64_t cols;
} mns_matrix;

/* Hyperparameters of one optimizer step (Eq. (1), Eq. (2), Algorithm 4).
 *   mu, lr        momentum coefficient and learning rate, used as given (a Dion3 caller
 *                 applies the learning-rate transfer rule lr' = lr / sqrt(f) itself)
 *   T, abc        T >= 1 Newton-Schulz iterations; abc (host) holds 3*T floats
 *                 a_1, b_1, c_1, a_2, ... of the odd quintics p_t(x) = a x + b x^3 + c x^5
 *   kind          mns_ns_kind
 *   restart_mask  Gram NS only: bit t set (2 <= t <= min(T, 31)) = restart before iteration t
 *                 (X <- Q X, Gram matrix recomputed, Q <- I). Must be 0 for standard NS.
 *   normuon       0 = Muon update W -= lr * O; 1 = NorMuon (Eq. 2) with beta2, eps
 *   row_fraction  Dion3 f in (0, 1]: 1 = every row (plain Muon/NorMuon); f < 1 selects the
 *                 k = ceil(f * rows) rows of M + G with the largest l1 norm (ties: lower
 *                 row index), orthogonalises only those rows and decays only them by mu
 *                 (error feedback), so M then holds mu*Mhat + (M - Mhat)
 *   dtype         mns_dtype of W and G for every matrix of the call */
typedef struct mns_hparams {
  float mu;
  float lr;
  int32_t T;
  const float* abc;
  int32_t kind;
  uint32_t restart_mask;
  int32_t normuon;
  float beta2;
  float eps;
  double row_fraction;
  int32_t dtype;
} mns_hparams;

/* Human-readable name of a status code (static string, never NULL). */
const char* mns_status_string(int status);

/* Library version: major*10000 + minor*100 + patch. */
int mns_version(void);

/* Workspace bytes muon_step needs for this matrix list and these hyperparameters.
 * Same validation as muon_step except for the device pointers (which may be NULL here). */
mns_status mns_step_workspace_size(const mns_matrix* mats, int count, const mns_hparams* hp,
                                   size_t* bytes /* (host) out */);

/* One optimizer step over `count` matrices (Eq. (1); Eq. (2) when hp->normuon;
 * Algorithm 4 when hp->row_fraction < 1).
 *   mats (host) array of `count` matrices, each with its own buffers; matrices of equal
 *   shape are processed together in batched launches.
 * Per matrix, in order: M <- mu M + G (Dion3: M <- M + G, then selection); X_0 = M/||M||_F;
 * O = NS_T(X_0) by hp->kind, run on the short side (a tall matrix is transposed);
 * W <- W - lr * O, or NorMuon's W <- W - lr (||O||_F/||Ohat||_F) Ohat with v updated;
 * W is rounded once to its dtype from the float32 value. */
mns_status muon_step(const mns_matrix* mats, int count, const mns_hparams* hp,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes for ns_orthogonalize / gram_ns_orthogonalize on `batch` matrices. */
mns_status mns_ns_workspace_size(int dtype, int64_t batch, int64_t rows, int64_t cols,
                                 int kind, size_t* bytes /* (host) out */);

/* Standard quintic Newton-Schulz ("Standard Newton-Schulz"): for each of `batch`
 * rows x cols matrices X, O = NS_T(X / ||X||_F) in X's dtype and shape. The iteration
 * runs on the short side; X and O may not overlap. */
mns_status ns_orthogonalize(const void* X, void* O, int dtype, int64_t batch, int64_t rows,
                            int64_t cols, int T, const float* abc /* (host) 3*T */,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Gram Newton-Schulz (Theorem 2 with the restarts of Algorithm 3): the same result as
 * ns_orthogonalize in exact arithmetic, computed on the n x n Gram side
 * (n = min(rows, cols)); restart_mask as in mns_hparams (Algorithm 3 uses 1u << 3). */
mns_status gram_ns_orthogonalize(const void* X, void* O, int dtype, int64_t batch,
                                 int64_t rows, int64_t cols, int T,
                                 const float* abc /* (host) 3*T */, uint32_t restart_mask,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* Allocation-free variant of ns_orthogonalize, for callers that cannot allocate device
 * memory or pass a workspace: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc. The same standard quintic Newton-Schulz as ns_orthogonalize, with
 * every scratch buffer carved from a 64 MiB array of device memory inside the library (one
 * per GPU, held until the process ends); the caller passes only X and O. Nothing is
 * allocated, and no library routine that allocates is called.
 *   Sizes: a batch runs in chunks of up to 32 matrices that fit the array; a problem whose
 *   single-matrix buffers exceed 64 MiB (about 2 x 2 iterates of rows x cols plus two
 *   short-side squares, each dimension rounded up to 256 and widened by 256; for bfloat16 up
 *   to e.g. 2048 x 2048 or 1024 x 4096) returns MNS_ERR_WORKSPACE before anything is enqueued.
 *   Other arguments and errors as ns_orthogonalize; the result equals its result up to the
 *   order of split-k partial sums (bit-identical when the chunking and split-k scratch agree).
 *   Device: the array used is the current device's; `stream` (if not NULL) must belong to
 *   the current device, else MNS_ERR_PARAM.
 *   Concurrency: every call on one GPU uses that GPU's single array, which keeps the last
 *   call's contents (each call writes every word before reading it). Calls that may overlap
 *   on one GPU -- on different streams, or from different threads -- race; serialise them. */
mns_status ns_orthogonalize_noalloc(const void* X, void* O, int dtype, int64_t batch,
                                    int64_t rows, int64_t cols, int T,
                                    const float* abc /* (host) 3*T */, void* stream);

/* Workspace bytes for normuon_scale. */
mns_status mns_normuon_workspace_size(int64_t batch, int64_t rows, int64_t cols,
                                      size_t* bytes /* (host) out */);

/* NorMuon normalisation (Eq. 2) of an orthogonalised update, in place:
 * v_i <- beta2 v_i + (1 - beta2) (1/cols) sum_j O_ij^2; Ohat_ij = O_ij / (sqrt(v_i) + eps);
 * O <- (||O||_F / ||Ohat||_F) Ohat (0 when ||Ohat||_F = 0), per matrix of the batch.
 *   O  in/out  dtype [batch][rows][cols];   v  in/out  float32 [batch][rows]
 * Arithmetic is float32; O is rounded once to its dtype. */
mns_status normuon_scale(void* O, int dtype, int64_t batch, int64_t rows, int64_t cols,
                         float* v, float beta2, float eps, void* workspace,
                         size_t workspace_bytes, void* stream);

/* ---- Instrumentation ---------------------------------------------------------------------
 * Between mns_profile_begin() and mns_profile_end() every kernel launch the library makes is
 * bracketed by a pair of hipEvents recorded on the launch's stream. mns_profile_end() waits
 * for those events and writes one entry per kernel (in order of first launch): the launch
 * count, the summed event time in milliseconds and the summed algorithmic work of those
 * launches -- FLOPs for the GEMMs (a symmetric product counted at half the dense 2MNK, as the
 * page prices a symmetric GEMM) and HBM bytes for the elementwise and reduction kernels.
 * Process-global, not thread-safe; meant for benchmarks. Costs one event pair per launch.
 *   out      (host) array of `capacity` entries; entries beyond `capacity` are dropped
 *   count    (host) out: number of distinct kernels seen
 * mns_profile_end returns MNS_ERR_PARAM when no session is open, MNS_ERR_HIP when an event
 * could not be created or read. */
typedef struct mns_kernel_stat {
  char name[64];
  int64_t launches;
  double ms;
  double flops;
  double bytes;
} mns_kernel_stat;

mns_status mns_profile_begin(void);
mns_status mns_profile_end(mns_kernel_stat* out, int capacity, int* count);

/* Cache flush for the session's HBM timings: while the session is open, every launch that
 * reports no FLOPs and at least 16 MiB of algorithmic bytes (the elementwise and reduction
 * kernels) is preceded, outside its event pair, by a kernel that writes `bytes` bytes of
 * zeros over `buffer` (device memory the caller owns, 16-byte aligned; 1 GiB or more evicts
 * the 256 MB Infinity Cache), so that the timed launch reads its operands from HBM rather
 * than from a cache an earlier kernel filled. buffer = NULL or bytes = 0 turns it off;
 * mns_profile_end turns it off. MNS_ERR_PARAM when no session is open or `buffer` is
 * misaligned. The flush launches are not recorded. */
mns_status mns_profile_set_flush(void* buffer, size_t bytes);

#ifdef __cplusplus
}
#endif

#endif /* MUON_NS_H */
