// Internal declarations shared by the library's translation units (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mns {

// Type of the Newton-Schulz iterate and of the Gram-side matrices on the device.
// bfloat16 storage runs the iteration in float16 with float32 accumulation (the stabilised
// Gram NS casts in float16; a bfloat16 iterate loses too much precision); float32 storage
// runs it in float32 end to end.
enum class Elem { F16 = 0, F32 = 1 };

// Storage type of caller buffers (W, G, X, O).
enum class Store { F32 = 0, BF16 = 1 };

inline int elem_bytes(Elem e) { return e == Elem::F16 ? 2 : 4; }

// Caller pointers of up to kMaxPack same-shape matrices, passed by value as a kernel
// argument (no device-side pointer table, nothing to upload).
constexpr int kMaxPack = 32;
struct PtrPack {
  void* p[kMaxPack];
};

// Every NS-side matrix in the workspace is zero-padded to multiples of this size, so the
// GEMM kernels run on whole tiles with no bounds checks; zero padding is invariant under
// every product and polynomial the iterations form.
constexpr int kPad = 256;
inline int64_t pad_up(int64_t x) { return (x + kPad - 1) / kPad * kPad; }

// Row pitch of every padded NS-side buffer: its padded width plus kLdPad elements. With a
// power-of-two pitch the rows of one operand tile fall on the same few memory channels;
// the extra 256 elements spread them (the 4096x16384 X X^T and the 1024-wide Gram-side
// products run 4-5 % faster; a short-K dense product over the same buffers runs 5 % slower,
// other shapes within 1 %). The pad columns are never read.
constexpr int64_t kLdPad = 256;
__host__ __device__ inline int64_t padded_ld(int64_t width_p) { return width_p + kLdPad; }

// ---------------------------------------------------------------------------------------
// GEMM (gemm.hip): C = alpha * A B^T + beta * D + gamma * I
//   A: M x K, B: N x K, both row-major with k contiguous (lda, ldb). D, C: M x N row-major;
//   Ct (optional): the same result written transposed (N x M, ldct). Batched over
//   blockIdx.z with element strides.
//   sym: M == N, the result is known to be symmetric; only tiles on or above the diagonal
//   are computed and each is also stored mirrored (within a diagonal tile the upper
//   triangle is mirrored), so C is exactly symmetric. Ct must be null.
//   M, N, K must be multiples of kPad; at least one of C, Ct is given.
// ---------------------------------------------------------------------------------------
struct GemmDesc {
  Elem elem = Elem::F16;
  const void* A = nullptr; int64_t lda = 0, sA = 0;
  const void* B = nullptr; int64_t ldb = 0, sB = 0;
  const void* D = nullptr; int64_t ldd = 0, sD = 0;
  void* C = nullptr; int64_t ldc = 0, sC = 0;
  void* Ct = nullptr; int64_t ldct = 0, sCt = 0;
  int M = 0, N = 0, K = 0, batch = 1;
  float alpha = 1.f, beta = 0.f, gamma = 0.f;
  int diag_limit = 0;          // gamma is added at (i, i) for i < diag_limit
  bool sym = false;
  float* partial = nullptr;    // scratch for split-k partial sums (may be null: no split)
  size_t partial_bytes = 0;
  // Row sums of squares of the written output (dense products only): the pass that stores C
  // (C^T when C is null) also writes, for every output row r < rowsq_rows and 64-column chunk
  // c of that row, rowsq[(b * chunks + c) * rowsq_rows + r] = sum of the squares of the 64
  // values as stored (chunks = output row length / 64).
  float* rowsq = nullptr;
  int rowsq_rows = 0;
  // B given k-major: B[k][n] (K x N, row pitch ldb) instead of B[n][k] -- the iterate X read
  // as it is stored, so no transposed copy is needed. Dense float16 products on 256 x 256 or
  // 128 x 128 tiles only (gemm_kmajor_ok).
  bool b_kmajor = false;
};

// Scratch the GEMM may use for split-k partial sums (part of the caller's workspace).
constexpr size_t kGemmScratchBytes = size_t(64) << 20;
hipError_t gemm(const GemmDesc& d, hipStream_t s);
// Name of the kernel instantiation gemm() launches for this descriptor.
const char* gemm_name(const GemmDesc& d);
// Whether gemm() can take this (dense) product's B operand k-major (GemmDesc::b_kmajor).
bool gemm_kmajor_ok(const GemmDesc& d);

// ---------------------------------------------------------------------------------------
// Elementwise / reduction kernels (elementwise.hip). All are deterministic: fixed
// reduction orders, no floating-point atomics.
// ---------------------------------------------------------------------------------------

// Blocks of the momentum / sum-of-squares kernels for a matrix of `elems` elements.
int norm_blocks(int64_t elems);

// M <- mu M + G over `count` same-size matrices; partials[b * nblk + blk] = partial sum of
// the new M^2 (squares summed in float64: no underflow or overflow for any float32 M).
hipError_t momentum(const PtrPack& M, const PtrPack& G, Store g_store, int count,
                    int64_t elems, float mu, double* partials, hipStream_t s);

// partials of sum X^2 for X of storage type `st` (X_b = X + b * elems), float64.
hipError_t sumsq(const void* X, Store st, int count, int64_t elems, double* partials,
                 hipStream_t s);

// xscale[b] = S / sqrt(sum_blk partials[b * nblk + blk]), 0 for a zero matrix.
hipError_t finalize_scale(const double* partials, int nblk, int count, float S, float* xscale,
                          hipStream_t s);

// The normalised iterate in both layouts, zero padded: S (rows_p x cols_p, pitch
// padded_ld(cols_p)) = xscale * src and T (cols_p x rows_p, pitch padded_ld(rows_p)) = its
// transpose; src is rows x cols (float32 when src_f32, else storage `st`). src pointers: a
// pack (per matrix) or, when pack == nullptr, base + b * rows * cols. Outputs are batched
// with stride rows_p * padded_ld(cols_p) and cols_p * padded_ld(rows_p). S or T may be null:
// that layout is not written.
hipError_t normalize(const PtrPack* pack, const void* base, bool src_f32, Store st, int count,
                     int64_t rows, int64_t cols, const float* xscale, Elem e, void* S, void* T,
                     int64_t rows_p, int64_t cols_p, hipStream_t s);

// O (rows x cols, storage st) = inv_s * X, X in the stored layout (rows_p x cols_p, pitch
// padded_ld(cols_p), Elem).
hipError_t export_output(const void* X, Elem e, int64_t rows_p, int64_t cols_p, int count,
                         int64_t rows, int64_t cols, float inv_s, void* O, Store st,
                         hipStream_t s);

// Per row of a caller matrix O (rows x cols, storage st), the sum of its squares:
// part[b][0][row]. (Inside muon_step the NS result's row sums come from the GEMM epilogue,
// GemmDesc::rowsq.)
hipError_t row_sumsq_stored(const void* O, Store st, int count, int64_t rows, int64_t cols,
                            float* part, hipStream_t s);

// NorMuon (Eq. 2) per matrix: r_i = inv_s2 * sum_chunk part; v <- beta2 v + (1-beta2) r/cols;
// d_i = 1/(sqrt(v)+eps); ratio = sqrt(sum r / sum r d^2); rowscale_i = ratio d_i out_scale.
// rowidx (nullable): v index of row i. v pointers per matrix in the pack (or v_base +
// b * v_stride when pack is null). fin: scratch of count * 2 * normuon_blocks(rows) doubles
// (per-block sums of the row-parallel stage).
int normuon_blocks(int64_t rows);
hipError_t normuon_finalize(const float* part, int chunks, int count, int64_t rows,
                            int64_t cols, const PtrPack* v_pack, float* v_base,
                            int64_t v_stride, const int32_t* rowidx, float beta2, float eps,
                            float inv_s2, float out_scale, float* rowscale, double* fin,
                            hipStream_t s);

// Writes zeros over `bytes` (rounded down to 16) of device memory p (16-byte aligned): the
// cache flush of the profiling session's HBM timings.
hipError_t cache_flush(void* p, size_t bytes, hipStream_t s);

// rowscale[b][i] = value (plain Muon: every row scaled alike).
hipError_t fill(float* p, int64_t n, float value, hipStream_t s);

// W[rowidx[i]][j] -= lr * rowscale[i] * X[i][j]  (X in the stored layout, rows_p x cols_p,
// pitch padded_ld(cols_p); rowidx null = identity).
hipError_t weight_update(const PtrPack& W, Store st, int count, int64_t rows, int64_t cols,
                         const void* X, Elem e, int64_t rows_p, int64_t cols_p,
                         const float* rowscale, const int32_t* rowidx, int64_t rowidx_stride,
                         float lr, hipStream_t s);

// O[b][i][j] *= rowscale[b][i] in place (storage st).
hipError_t rowscale_apply(void* O, Store st, int count, int64_t rows, int64_t cols,
                          const float* rowscale, hipStream_t s);

// Dion3 (Algorithm 4): M <- M + G with per-row l1 norms and sums of squares of the new M.
hipError_t momentum_l1(const PtrPack& M, const PtrPack& G, Store g_store, int count,
                       int64_t rows, int64_t cols, float* l1, double* l2sq, hipStream_t s);
// S[b][rank] = row for the k rows of largest l1 (ties: lower index first), and
// xscale[b] = Spow / ||M[S,:]||_F from the selected rows' sums of squares (0 for a zero block).
hipError_t topk_rows(const float* l1, const double* l2sq, int count, int64_t rows, int64_t k,
                     float Spow, int32_t* S, float* xscale, hipStream_t s);
// The normalised iterate of the selected rows, like normalize() with row r of the source
// being M[S[r]] (float32), and in the same pass M[S[r]][:] *= mu.
hipError_t gather_normalize(const PtrPack& M, int count, int64_t k, int64_t cols,
                            const int32_t* S, float mu, const float* xscale, Elem e, void* X,
                            void* Xt, int64_t rows_p, int64_t cols_p, hipStream_t s);

}  // namespace mns
