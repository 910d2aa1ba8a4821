// MFMA GEMM for the Newton-Schulz products on gfx950 (CDNA4).
//
//   C = alpha * A B^T + beta * D + gamma * I        (float32 accumulation)
//
// The page "Dion3: Full-stack orthogonal updates" prices every Newton-Schulz step as GEMMs
// (section "Standard Newton-Schulz", FLOP analysis) and computes the symmetric ones --
// X X^T, A^2 and the Gram-side products -- with kernels that only form the tiles of one
// triangle and copy them to the mirrored position (section "2. Symmetric GEMM Kernels").
// This kernel does the same on CDNA4: in `sym` mode the grid enumerates the tiles on or
// above the diagonal, and each tile is stored twice (directly and transposed); inside a
// diagonal tile only the upper triangle is kept and mirrored, so the result is exactly
// symmetric. The a X + (b A + c A^2) X and Z = a I + b R + c R^2 updates use the fused
// epilogue (alpha, beta * D, gamma * I).
//
// Products are "NT" (both operands row-major with k contiguous), except that the dense
// float16 products on 256 x 256 and 128 x 128 tiles can take B k-major (B[k][n]): the
// rectangular products P X and Q X then read the iterate X as it is stored, its k-tiles
// staged by DMA as 512- or 256-byte rows and turned into MFMA fragments by the transposing
// LDS read
// (ds_read_b64_tr_b16), and no transposed copy of X is ever written. Elsewhere they read X
// through its transposed copy, which their epilogue writes beside X (C and C^T).
//
// Layout / pipeline:
//   * WGM x WGN wave64s; block tile BM x BN, wave tile (BM/WGM) x (BN/WGN) of 32 x 32
//     MFMA fragments (v_mfma_f32_32x32x16_f16, or 32x32x2f32 for float32).
//   * k-tile = 128 bytes per row (64 halves / 32 floats). Both operand tiles sit in LDS as
//     [row][k] in 16-byte chunks, double buffered, with chunk c of row r stored at
//     c ^ ((r ^ ((r >> 3) & 3)) & 7): a fragment read (32 rows, one chunk) is conflict-free,
//     and rows 32 apart share the pattern, so the fragments of one k-step sit at fixed
//     offsets from one address.
//   * Global -> LDS is a buffer load with the LDS-DMA bit (buffer_load_dwordx4 ... lds):
//     no staging registers and no LDS store instructions. Each wave instruction fills
//     1 KB = 8 LDS rows; the lane -> global chunk mapping applies the swizzle.
//   * Pipeline (k-step = 16 halves / 4 floats of k, four per k-tile): fragments are read one
//     k-step ahead of the MFMAs that use them. The barrier of k-tile k comes before its last
//     k-step, whose fragments are already in registers, so buffer k % 2 is free at that
//     point and the load of k-tile k+2 starts into it: two k-tiles are in flight with two
//     buffers, one barrier per k-tile. Each wave's share of a k-tile load (8 DMA
//     instructions at 256x256) goes out in two halves, one instruction after each of the
//     first MFMAs of the last k-step of k-tile k (just after its barrier) and of the first
//     k-step of k-tile k+1, so it has most of a k-tile to land before the next barrier.
//   * A diagonal tile of a symmetric product whose two operands are one matrix (X X^T, A A)
//     loads only its A k-tiles and reads the B fragments from them, and skips the MFMAs of the
//     fragments wholly below the diagonal (that part of a diagonal tile is never stored); the
//     waves take the tile's regions in an order that leaves each SIMD at most 10 of its 16
//     fragments. Results are bit-identical to the full tile's.
//   * MFMA operand roles are swapped (the B tile feeds the MFMA's A input), so each lane's
//     accumulators hold 4 consecutive output columns of one row.
//   * The epilogue stages the finished tile once in the (then idle) LDS, as [m][n], and
//     writes every output as 16-byte row chunks: C from its rows, C^T and the mirrored tile
//     from its columns through the transposing LDS read (4 rows x 16 columns per 16 lanes
//     become 16 columns of 4). On request the pass that writes the stored layout also sums
//     the squares of each output row per 64-column chunk (NorMuon's row statistics, Eq. (2)),
//     from the values as stored.
//   * Work decomposition: whole rounds of tiles (one block per tile, one round = one block
//     per CU slot); when the last round would be less than half full, its tiles are split
//     along k so that round is full. Split blocks write float32 partial sums; a later launch
//     adds each tile's partials in a fixed order (a wide reduction launch first when they
//     are many) and runs the same epilogue on the sums (deterministic, no inter-block
//     waiting).
//   * Small grids (64 x 64 tiles) run k_gemm_kw instead: the four waves of a block split the
//     block's k-range, each with its own LDS stages and no barrier in the k loop, and add
//     their partial tiles in wave order before the same epilogue (gemm_epilogue.inc, which
//     both kernels expand inline).
#include "mns_internal.h"

#include <type_traits>

namespace mns {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kChunks = 8;   // 16-byte chunks per LDS row (one 128-byte k-tile)
constexpr int kBufferFlags = 0x00020000;   // buffer resource word 3: raw loads, gfx9 family

template <typename T>
struct Traits;

template <>
struct Traits<_Float16> {
  static constexpr int VEC = 8;   // elements per 16-byte chunk
  static constexpr int BK = 64;   // elements per k-tile
  __device__ static __forceinline__ void mma(floatx16& acc, u32x4 a, u32x4 b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, a),
                                                 __builtin_bit_cast(half8, b), acc, 0, 0, 0);
  }
};

template <>
struct Traits<float> {
  static constexpr int VEC = 4;
  static constexpr int BK = 32;
  // A 16-byte chunk holds 4 consecutive k; lanes 0-31 and 32-63 hold neighbouring chunks,
  // so MFMA p (K = 2) reduces over k = {p, 4 + p} of the 8-k step.
  __device__ static __forceinline__ void mma(floatx16& acc, u32x4 a, u32x4 b) {
#pragma unroll
    for (int p = 0; p < 4; ++p)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[p]), __uint_as_float(b[p]),
                                                 acc, 0, 0, 0);
  }
};

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kChunks + (chunk ^ ((row ^ ((row >> 3) & 3)) & 7));
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = bytes > 0x7FFFFFFFLL ? 0x7FFFFFFF : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, kBufferFlags);
}

// 16-byte-per-lane global -> LDS copy: lane l's 16 bytes land at dst + 16 l (dst is the
// wave-uniform LDS base, carried in M0). Kept out of lambdas: the host pass of a kernel
// must not see the LDS address-space cast.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, u32x4* dst, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, voff, soff, 0, 0);
}

// s_waitcnt immediate (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[15:14]).
constexpr int kWaitVm0Lgkm0 = 0x0070;     // vmcnt(0) lgkmcnt(0)
// vmcnt(n) alone (n < 64): at most n of this wave's vector-memory operations outstanding
constexpr int wait_vm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x70 | 0xF00; }

__device__ __forceinline__ void block_sync() {
  // All of this wave's LDS-DMA writes and LDS accesses are done, then the workgroup meets.
  // No memory fence: the DMA traffic is ordered by the explicit counters.
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(kWaitVm0Lgkm0);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

struct GemmArgs {
  const void* A; const void* B; const void* D;
  void* C;  void* Ct;
  int64_t lda, ldb, ldd, ldc, ldct;
  int64_t sA, sB, sD, sC, sCt;
  int M, N, K;
  float alpha, beta, gamma;
  int diag_limit;
  int tiles_n;      // N / BN (dense grid) or tiles per side (sym)
  int group;        // tile rows per group of the dense tile order
  int tiles_per_batch;
  int full_blocks;  // blocks that own a whole tile; tiles beyond are split
  int split;        // k-parts per split tile
  float* partial;   // split partial sums, BM*BN floats per (tile, part)
  int fix_parts;    // parts the epilogue launch adds (split, or 1 after k_reduce_parts)
  float* rowsq;     // per-row sums of squares of the stored output (or null)
  int rowsq_rows, rowsq_chunks;
};

// Sum of the squares of one 16-byte chunk of stored output values, added over the RS_L
// consecutive lanes that hold one 64-column chunk of an output row (fixed shuffle order); the
// first of them writes the chunk's sum.
template <typename T, int RS_L>
__device__ __forceinline__ void rowsq_chunk(const u32x4& v, const GemmArgs& p, int64_t bz,
                                            int chunk, int row) {
  const T* e = reinterpret_cast<const T*>(&v);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < (int)(16 / sizeof(T)); ++i) {
    const float x = (float)e[i];
    s += x * x;
  }
#pragma unroll
  for (int o = RS_L / 2; o > 0; o >>= 1) s += __shfl_down(s, o, RS_L);
  if ((threadIdx.x % RS_L) == 0 && row < p.rowsq_rows)
    p.rowsq[(bz * p.rowsq_chunks + chunk) * p.rowsq_rows + row] = s;
}

template <typename T>
__device__ __forceinline__ void load4(const T* p, float* v);
template <>
__device__ __forceinline__ void load4<_Float16>(const _Float16* p, float* v) {
  typedef _Float16 half4 __attribute__((ext_vector_type(4)));
  const half4 h = *reinterpret_cast<const half4*>(p);
  v[0] = (float)h.x; v[1] = (float)h.y; v[2] = (float)h.z; v[3] = (float)h.w;
}
template <>
__device__ __forceinline__ void load4<float>(const float* p, float* v) {
  const float4 f = *reinterpret_cast<const float4*>(p);
  v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
}


// The product: whole tiles with their epilogue, and the k-parts of split tiles (float32
// partial sums, finished by k_tail_epilogue).
template <typename T, int BM, int BN, int WGM, int WGN, bool SYM, bool KB = false>
__global__ __launch_bounds__(64 * WGM * WGN) void k_gemm(GemmArgs p) {
  using Tr = Traits<T>;
  constexpr int NW = WGM * WGN, NT = 64 * NW;
  constexpr int VEC = Tr::VEC, BK = Tr::BK, ES = (int)sizeof(T);
  constexpr int WM = BM / WGM, WN = BN / WGN, FM = WM / 32, FN = WN / 32;
  constexpr int A_INST = BM / 8 / NW;     // LDS-DMA instructions per wave per k-tile, A
  constexpr int B_INST = BN / 8 / NW;
  constexpr int STAGE = (BM + BN) * kChunks;   // u32x4 per LDS stage
  static_assert(A_INST >= 1 && B_INST >= 1 && FM >= 1 && FN >= 1, "tile too small");
  static_assert(BM * BN * ES <= 2 * STAGE * 16, "epilogue tile must fit the stage buffers");
  static_assert(!KB || (!SYM && (BN == 256 || BN == 128) && ES == 2 && WN == 64 && FN == 2),
                "k-major B: dense float16 tiles of 256 or 128 columns, 64-column wave tiles");
  // k-major B: a k-row of the tile is BN * 2 bytes (KCH 16-byte chunks); one DMA instruction
  // (1 KB) fills KRI k-rows.
  constexpr int KCH = BN / 8, KRI = 64 / KCH, KRB = BN * 2;

  __shared__ u32x4 lds[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: LDS-DMA bases stay scalar

  // Block -> (tile, k-range, partial slot); see the work decomposition above.
  // Tile order. Workgroups go round-robin to the 8 XCDs (L2 domains); whole-tile blocks are
  // remapped so each XCD walks a contiguous range of logical tiles, ordered in groups of
  // p.group tile rows (column-major inside a group), so the CUs of one XCD share A and B rows
  // (dense and symmetric grids alike).
  const int KT = p.K / BK;
  int lin = blockIdx.x, k_begin = 0, k_end = KT, slot = -1;
  if (lin < p.full_blocks) {
    const int q = p.full_blocks / 8;
    if (lin < 8 * q) lin = (lin % 8) * q + lin / 8;
  } else {
    const int r = lin - p.full_blocks, part = r % p.split;
    lin = p.full_blocks + r / p.split;
    slot = r;
    k_begin = (int)((int64_t)part * KT / p.split);
    k_end = (int)((int64_t)(part + 1) * KT / p.split);
  }
  // The decode is uniform over the block; state it, so k offsets stay in scalar registers.
  lin = __builtin_amdgcn_readfirstlane(lin);
  slot = __builtin_amdgcn_readfirstlane(slot);
  k_begin = __builtin_amdgcn_readfirstlane(k_begin);
  k_end = __builtin_amdgcn_readfirstlane(k_end);
  const int64_t bz = lin / p.tiles_per_batch;
  int t = lin % p.tiles_per_batch;
  int tm, tn;
  if (SYM) {
    // Upper-triangle tiles (tm <= tn) in groups of p.group tile rows, column by column
    // inside a group, like the dense order.
    const int tt = p.tiles_n;
    int g0 = 0;
    tm = tn = 0;
    for (;;) {
      const int gs = tt - g0 < p.group ? tt - g0 : p.group;
      const int cnt = gs * tt - gs * g0 - gs * (gs - 1) / 2;
      if (t < cnt) {
        for (int c = g0;; ++c) {
          const int rows = c - g0 + 1 < gs ? c - g0 + 1 : gs;
          if (t < rows) { tm = g0 + t; tn = c; break; }
          t -= rows;
        }
        break;
      }
      t -= cnt;
      g0 += gs;
    }
  } else {
    const int tiles_m = p.M / BM;
    const int per_group = p.group * p.tiles_n;
    const int g = t / per_group, l = t % per_group;
    const int first = g * p.group;
    const int gsize = tiles_m - first < p.group ? tiles_m - first : p.group;
    tm = first + l % gsize;
    tn = l / gsize;
  }
  const int m0 = tm * BM, n0 = tn * BN;

  // Buffer resources based at this block's first A row / B row; reads past the batch slice
  // return zero instead of faulting.
  const char* Abase = static_cast<const char*>(p.A) + (bz * p.sA + (int64_t)m0 * p.lda) * ES;
  // k-major B (KB): B[k][n] with row pitch ldb; the block's columns start at n0.
  const char* Bbase = static_cast<const char*>(p.B) +
                      (bz * p.sB + (KB ? (int64_t)n0 : (int64_t)n0 * p.ldb)) * ES;
  const __amdgpu_buffer_rsrc_t rA = make_rsrc(Abase, ((int64_t)(p.M - m0) * p.lda) * ES);
  const __amdgpu_buffer_rsrc_t rB =
      make_rsrc(Bbase, (KB ? (int64_t)p.K * p.ldb - n0 : (int64_t)(p.N - n0) * p.ldb) * ES);

  // A diagonal tile of a symmetric product whose operands are one matrix (X X^T, A A): its A
  // and B k-tiles are the same rows, so only A is loaded and the B fragments are read from the
  // A stage; fragments wholly below the diagonal are never stored (the row pass keeps the upper
  // triangle, the mirror is made from it), so their MFMAs are skipped. Waves get the 128 x 64
  // regions in a permuted order that pairs, on each SIMD (waves w and w + 4), a region with
  // much of the upper triangle and one with little: at most 10 of 16 fragments per SIMD.
  constexpr bool kDiagOK = SYM && !KB && BM == 256 && BN == 256 && WGM == 2 && WGN == 4;
  const bool diag_same = kDiagOK && slot < 0 && tm == tn && p.A == p.B && p.sA == p.sB &&
                         p.lda == p.ldb;
  // Region r = wm * WGN + wn; wave w takes nibble w of 0x06547132 (waves 0-3: regions 2, 3, 1, 7
  // with 8, 8, 7, 7 fragments on or above the diagonal; waves 4-7: regions 4, 5, 6, 0 with
  // 0, 0, 3, 3).
  const int reg = diag_same ? (int)((0x06547132u >> (4 * wave)) & 0xFu) : wave;
  const int wm = reg / WGN, wn = reg % WGN;
  uint32_t keep = 0u;   // bit m: fragment (m / FN, m % FN) of this wave is on or above the diagonal
#pragma unroll
  for (int m = 0; m < FM * FN; ++m)
    keep |= (uint32_t)(wm * FM + m / FN <= wn * FN + m % FN) << m;
  keep = __builtin_amdgcn_readfirstlane(keep);

  // Lane -> (LDS row, physical chunk) of one DMA instruction: row r0 + lane/8, chunk
  // lane%8, which holds logical k-chunk (lane%8) ^ f(row).
  int offA[A_INST], offB[B_INST];
#pragma unroll
  for (int i = 0; i < A_INST; ++i) {
    const int row = (wave * A_INST + i) * 8 + (lane >> 3);
    const int ch = (lane & 7) ^ ((row ^ ((row >> 3) & 3)) & 7);
    offA[i] = (row * (int)p.lda + ch * VEC) * ES;
  }
#pragma unroll
  for (int i = 0; i < B_INST; ++i) {
    if constexpr (KB) {
      // k-major: one instruction fills KRI k-rows of the tile; 16-byte chunk c of k-row r sits
      // at c ^ 4 (r % 4), so that a transposing read (4 k-rows x 64 bytes per 32 lanes)
      // touches 16 distinct chunk positions, i.e. all 64 banks once.
      const int kr = KRI * (wave * B_INST + i) + lane / KCH;
      const int c = (lane % KCH) ^ (4 * (kr & 3));
      offB[i] = (kr * (int)p.ldb + 8 * c) * ES;
    } else {
      const int row = (wave * B_INST + i) * 8 + (lane >> 3);
      const int ch = (lane & 7) ^ ((row ^ ((row >> 3) & 3)) & 7);
      offB[i] = (row * (int)p.ldb + ch * VEC) * ES;
    }
  }
  // k offset of k-tile kt in the B rows (bytes, scalar)
  auto b_koff = [&](int kt) { return KB ? kt * BK * (int)p.ldb * ES : kt * BK * ES; };

  auto issue = [&](int kt, int buf, auto dg) {
    const int so = kt * BK * ES;
#pragma unroll
    for (int i = 0; i < A_INST; ++i)
      dma16(rA, &lds[buf * STAGE + (wave * A_INST + i) * 8 * kChunks], offA[i], so);
    if constexpr (!decltype(dg)::value) {
#pragma unroll
      for (int i = 0; i < B_INST; ++i)
        dma16(rB, &lds[buf * STAGE + (BM + (wave * B_INST + i) * 8) * kChunks], offB[i],
              b_koff(kt));
    }
  };

  floatx16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int arow = wm * WM + (lane & 31);
  const int brow = (diag_same ? 0 : BM) + wn * WN + (lane & 31);
  u32x4 af[2][FM], bf[2][FN];
  auto load_frags = [&](int buf, int ks, int slot) {
    const int ch = 2 * ks + (lane >> 5);
#pragma unroll
    for (int i = 0; i < FM; ++i) af[slot][i] = lds[buf * STAGE + swz(arow + 32 * i, ch)];
    if constexpr (!KB) {
#pragma unroll
      for (int j = 0; j < FN; ++j) bf[slot][j] = lds[buf * STAGE + swz(brow + 32 * j, ch)];
    }
  };
  // k-major B fragments through ds_read_b64_tr_b16: within each 16-lane group (G = lane / 16)
  // lane 4s + a points at the 8 bytes of k-row 8 (G / 2) + s (+ 4 for the second read) and
  // columns n .. n+3, n = wn WN + 32 j + 16 (G % 2) + 4 a; the read hands lane 4a + b the
  // four k-values of column n + b, so each lane ends with 8 consecutive k of its column --
  // the fragment the MFMA's A input expects. The loads are inline asm that waits for them
  // itself (the compiler cannot see that they do not touch the buffer the DMA is filling, and
  // would otherwise wait for every outstanding DMA first); the outputs are early-clobber and
  // the fragments the preceding MFMAs read are inputs, so none of those registers is reused
  // while the MFMAs may still read it.
  uint32_t b_addr[2] = {0u, 0u};
  if constexpr (KB) {
    const uint32_t lbase = (uint32_t)(uintptr_t)(lds_void*)&lds[0];
    const int G = lane >> 4, sq = (lane & 15) >> 2, a4 = lane & 3;
    const int kb = 8 * (G >> 1) + sq;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = wn * WN + 32 * j + 16 * (G & 1) + 4 * a4;
      b_addr[j] = lbase + BM * 128 + kb * KRB + ((n >> 3) ^ (4 * (kb & 3))) * 16 + (n & 7) * 2;
    }
  }
  auto load_b = [&](int buf, int ks, int slot) {
    if constexpr (KB) {
      typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
      u32x2 t00, t01, t10, t11;
      const uint32_t o = (uint32_t)(buf * STAGE * 16 + ks * 16 * KRB);
      const uint32_t a0 = b_addr[0] + o, a1 = b_addr[1] + o;
      const int ps = slot ^ 1;
      // the second read of each pair is 4 k-rows further (offset 4 KRB)
      static_assert(FM == 4 || FM == 2, "fragment inputs below");
      const u32x4 pa2 = af[ps][FM > 2 ? 2 : 0], pa3 = af[ps][FM > 2 ? 3 : 1];
      asm volatile(
          "ds_read_b64_tr_b16 %0, %4\n\t"
          "ds_read_b64_tr_b16 %1, %4 offset:%c12\n\t"
          "ds_read_b64_tr_b16 %2, %5\n\t"
          "ds_read_b64_tr_b16 %3, %5 offset:%c12\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(t00), "=&v"(t01), "=&v"(t10), "=&v"(t11)
          : "v"(a0), "v"(a1), "v"(af[ps][0]), "v"(af[ps][1]), "v"(pa2), "v"(pa3),
            "v"(bf[ps][0]), "v"(bf[ps][1]), "i"(4 * KRB));
      bf[slot][0] = u32x4{t00.x, t00.y, t01.x, t01.y};
      bf[slot][1] = u32x4{t10.x, t10.y, t11.x, t11.y};
    } else {
      (void)buf; (void)ks; (void)slot;
    }
  };

  // Partial sums of a split tile, in fragment order: the float4 (i, j, g) of thread tid,
  // acc[i][j][4g .. 4g+3], at ((i * FN + j) * 4 + g) * NT + tid (coalesced both ways).
  constexpr int TILE_F4 = FM * FN * 4 * NT;
  {
    // The scheduling fences keep each k-step's order as written: the next k-step's LDS reads
    // go out before this k-step's MFMAs, which then cover their latency, and a k-tile's DMA
    // instructions go out one at a time between MFMAs (a burst of them fills the vector
    // memory queue and stalls the waves that issued it).
    constexpr int KS = kChunks / 2;
    static_assert(KS == 4, "four k-steps per k-tile");
    const int KL = k_end - k_begin;
    // DMA instruction q of a k-tile (q < A_INST: A row block q, else B row block q - A_INST).
    constexpr int NI = A_INST + B_INST;
    constexpr int NP0 = NI / 2, NP1 = NI - NP0;
    auto dma_one = [&](int kt, int buf, int q, auto dg) {
      const int so = kt * BK * ES;
      if (decltype(dg)::value && q >= A_INST) return;
      if (q < A_INST)
        dma16(rA, &lds[buf * STAGE + (wave * A_INST + q) * 8 * kChunks], offA[q], so);
      else
        dma16(rB, &lds[buf * STAGE + (BM + (wave * B_INST + q - A_INST) * 8) * kChunks],
              offB[q - A_INST], b_koff(kt));
    };
    // One k-step: the MFMAs of fragment slot s with DMA instructions q0 .. q0+nq-1 of k-tile
    // kt spread between them (after every RR-th MFMA).
    auto kstep = [&](int s, int kt, int buf, int q0, auto nq_c, auto dg) {
      constexpr int NQ = decltype(nq_c)::value;
      constexpr bool DG = decltype(dg)::value;
      constexpr int NM = FM * FN;
      constexpr int RR = NM / (NQ + 1) > 0 ? NM / (NQ + 1) : 1;
      // DMA instruction q goes out after MFMA pos(q) = min((q + 1) RR, NM) - 1.
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        if (!DG || ((keep >> m) & 1u)) Tr::mma(acc[m / FN][m % FN], bf[s][m % FN], af[s][m / FN]);
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
          const int pos = (q + 1) * RR < NM ? (q + 1) * RR - 1 : NM - 1;
          if (pos == m) dma_one(kt, buf, q0 + q, dg);
        }
      }
      if constexpr (!DG && NQ > 0) {
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
#pragma unroll
          for (int q = 0; q < NQ; ++q) {
            const int pos = (q + 1) * RR < NM ? (q + 1) * RR - 1 : NM - 1;
            if (pos == m) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
          }
        }
      }
    };
    using I0 = std::integral_constant<int, 0>;
    using IP0 = std::integral_constant<int, NP0>;
    using IP1 = std::integral_constant<int, NP1>;
    // k-tile kl from buffer kl % 2. DMA of k-tile kl+1 (buffer b ^ 1): its first half went
    // out in the previous k-tile's last k-step, its second half goes out during k-step 0
    // here; the barrier before k-step 3 waits for it, and the first half of k-tile kl+2
    // follows the barrier.
    auto body = [&](int kl, auto has1, auto has2, auto dg) {
      const int b = kl & 1;
      // This k-tile's first fragments were read a whole k-step ago: waiting for them here is
      // free and leaves only the next k-step's reads pending below.
      __builtin_amdgcn_s_waitcnt(0xC07F);
      load_frags(b, 1, 1);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (decltype(has1)::value) kstep(0, k_begin + kl + 1, b ^ 1, NP0, IP1{}, dg);
      else kstep(0, 0, 0, 0, I0{}, dg);
      __builtin_amdgcn_sched_barrier(0);
      load_b(b, 1, 1);
      load_frags(b, 2, 0);
      __builtin_amdgcn_sched_barrier(0);
      kstep(1, 0, 0, 0, I0{}, dg);
      __builtin_amdgcn_sched_barrier(0);
      load_b(b, 2, 0);
      load_frags(b, 3, 1);
      __builtin_amdgcn_sched_barrier(0);
      kstep(0, 0, 0, 0, I0{}, dg);
      __builtin_amdgcn_sched_barrier(0);
      load_b(b, 3, 1);
      // k-tile kl+1 has landed and every wave's reads of buffer b are done.
      block_sync();
      load_frags(b ^ 1, 0, 0);   // after the last k-tile: a harmless read of the idle buffer
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (decltype(has2)::value) kstep(1, k_begin + kl + 2, b, 0, IP0{}, dg);
      else kstep(1, 0, 0, 0, I0{}, dg);
      __builtin_amdgcn_sched_barrier(0);
      load_b(b ^ 1, 0, 0);   // after the last k-tile: a harmless read of the idle buffer
    };
    using T1 = std::true_type;
    using F1 = std::false_type;
    auto run = [&](auto dg) {
      issue(k_begin, 0, dg);
      if (KL > 1) {
#pragma unroll
        for (int q = 0; q < NP0; ++q) dma_one(k_begin + 1, 1, q, dg);
      }
      block_sync();
      load_frags(0, 0, 0);
      load_b(0, 0, 0);
      int kl = 0;
      for (; kl + 2 < KL; ++kl) body(kl, T1{}, T1{}, dg);
      if (kl + 1 < KL) body(kl++, T1{}, F1{}, dg);
      body(kl, F1{}, F1{}, dg);
    };
    if constexpr (kDiagOK) {
      if (diag_same) run(T1{});
      else run(F1{});
    } else {
      run(F1{});
    }
    if (slot >= 0) {
      floatx4* P = reinterpret_cast<floatx4*>(p.partial) + (int64_t)slot * TILE_F4;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            floatx4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * g + e];
            P[((i * FN + j) * 4 + g) * NT + tid] = v;
          }
      return;
    }
    block_sync();
  }

  // ---- epilogue: v = alpha acc + beta D + gamma I, staged through LDS ----
  {
    T* tile = reinterpret_cast<T*>(&lds[0]);
#include "gemm_epilogue.inc"
  }
}

// Sums the k-parts of every split tile into its part 0, in part order (the same float32
// additions for every run): one thread per float4, tile_f4 / 256 blocks per tile.
__global__ __launch_bounds__(256) void k_reduce_parts(floatx4* partial, int split, int tile_f4) {
  const int chunks = tile_f4 / 256;
  const int tile = blockIdx.x / chunks, c = blockIdx.x % chunks;
  floatx4* P = partial + (int64_t)tile * split * tile_f4 + c * 256 + threadIdx.x;
  floatx4 v = P[0];
  int part = 1;
  for (; part + 4 <= split; part += 4) {
    const floatx4 a = P[(int64_t)part * tile_f4], b = P[(int64_t)(part + 1) * tile_f4];
    const floatx4 c2 = P[(int64_t)(part + 2) * tile_f4], d = P[(int64_t)(part + 3) * tile_f4];
    v += a;
    v += b;
    v += c2;
    v += d;
  }
  for (; part < split; ++part) v += P[(int64_t)part * tile_f4];
  P[0] = v;
}

// Logical tile `lin` of the grid order -> (tile row, tile column, batch entry); the same
// order as the product kernel's decode.
template <bool SYM, int BM>
__device__ __forceinline__ void tile_coords(const GemmArgs& p, int lin, int& tm, int& tn,
                                            int64_t& bz) {
  bz = lin / p.tiles_per_batch;
  int t = lin % p.tiles_per_batch;
  if (SYM) {
    // Upper-triangle tiles (tm <= tn) in groups of p.group tile rows, column by column
    // inside a group, like the dense order.
    const int tt = p.tiles_n;
    int g0 = 0;
    tm = tn = 0;
    for (;;) {
      const int gs = tt - g0 < p.group ? tt - g0 : p.group;
      const int cnt = gs * tt - gs * g0 - gs * (gs - 1) / 2;
      if (t < cnt) {
        for (int c = g0;; ++c) {
          const int rows = c - g0 + 1 < gs ? c - g0 + 1 : gs;
          if (t < rows) { tm = g0 + t; tn = c; break; }
          t -= rows;
        }
        break;
      }
      t -= cnt;
      g0 += gs;
    }
  } else {
    const int tiles_m = p.M / BM;
    const int per_group = p.group * p.tiles_n;
    const int g = t / per_group, l = t % per_group;
    const int first = g * p.group;
    const int gsize = tiles_m - first < p.group ? tiles_m - first : p.group;
    tm = first + l % gsize;
    tn = l / gsize;
  }
}

// Epilogue of the split tail tiles on 64 x 64 sub-tiles (BM/64 x BN/64 blocks of 256 threads
// per tile): each thread sums four float4 of partial sums (the product kernel's fragment
// order, p.fix_parts parts in part order), applies alpha, beta D and gamma I, and the sub-tile
// leaves through LDS as 16-byte rows of C and, transposed, of C^T or of the mirrored tile.
// Spreading a tile over many CUs keeps the tail's epilogue from running on only a few.
template <typename T, int BM, int BN, int WGM, int WGN, bool SYM>
__global__ __launch_bounds__(256) void k_tail_epilogue(GemmArgs p) {
  constexpr int NT = 64 * WGM * WGN;          // threads of the product kernel
  constexpr int WM = BM / WGM, WN = BN / WGN, FN = WN / 32;
  constexpr int ES = (int)sizeof(T), EPC = 16 / ES, SUB = 64, CPR = SUB / EPC;
  constexpr int TILE_F4 = BM * BN / 4;
  constexpr int SUBS_N = BN / SUB, SUBS = (BM / SUB) * SUBS_N;
  static_assert(BM % SUB == 0 && BN % SUB == 0, "whole sub-tiles");
  typedef T t4 __attribute__((ext_vector_type(4)));
  typedef T tv __attribute__((ext_vector_type(EPC)));   // one 16-byte chunk
  __shared__ __align__(16) T tile[SUB][SUB + EPC];
  const int ti = blockIdx.x / SUBS, sub = blockIdx.x % SUBS;
  const int sm = (sub / SUBS_N) * SUB, sn = (sub % SUBS_N) * SUB;
  int tm, tn;
  int64_t bz;
  tile_coords<SYM, BM>(p, p.full_blocks + ti, tm, tn, bz);
  const int m0 = tm * BM, n0 = tn * BN;
  const floatx4* P = reinterpret_cast<const floatx4*>(p.partial) + (int64_t)ti * p.split * TILE_F4;
  const T* Dg = p.D ? static_cast<const T*>(p.D) + bz * p.sD : nullptr;
  // element (ml, nl .. nl+3) of the tile is float4 ((i FN + j) 4 + g) NT + ftid of a part
  const int ml = sm + (threadIdx.x & 63);
  const int wm = ml / WM, i = (ml % WM) / 32, lo = ml % 32;
  // D for the four pieces first, under one test (not one test per piece).
  float d[4][4] = {};
  if (Dg) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      load4<T>(Dg + (int64_t)(m0 + ml) * p.ldd + n0 + sn + 4 * ((threadIdx.x >> 6) + 4 * k), d[k]);
  }
  // The four pieces' partial sums, part by part: each part's four loads go out together (the
  // additions per element stay in part order). A part loop inside each piece waited once per
  // load.
  int64_t idx[4];
  floatx4 acc[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int nl = sn + 4 * ((threadIdx.x >> 6) + 4 * k);
    const int wn = nl / WN, j = (nl % WN) / 32, g = (nl % 32) / 8, hi = (nl % 8) / 4;
    idx[k] = ((int64_t)(i * FN + j) * 4 + g) * NT + (wm * WGN + wn) * 64 + hi * 32 + lo;
    acc[k] = P[idx[k]];
  }
  for (int part = 1; part < p.fix_parts; ++part) {
    floatx4 q[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) q[k] = P[(int64_t)part * TILE_F4 + idx[k]];
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[k] += q[k];
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int nl = sn + 4 * ((threadIdx.x >> 6) + 4 * k);
    t4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float v = p.alpha * acc[k][e] + p.beta * d[k][e];
      if (m0 + ml == n0 + nl + e && m0 + ml < p.diag_limit) v += p.gamma;
      o[e] = (T)v;
    }
    *reinterpret_cast<t4*>(&tile[ml - sm][nl - sn]) = o;
  }
  __syncthreads();
  const bool diag_tile = SYM && tm == tn;
  if (SYM || p.C) {
    T* Cg = static_cast<T*>(p.C) + bz * p.sC;
    for (int q = threadIdx.x; q < SUB * CPR; q += 256) {
      const int r = q / CPR, c = q % CPR;
      const int gm = sm + r, gn = sn + c * EPC;
      const tv v = *reinterpret_cast<const tv*>(&tile[r][c * EPC]);
      T* dst = Cg + (int64_t)(m0 + gm) * p.ldc + n0 + gn;
      if (!diag_tile || gn >= gm) {
        *reinterpret_cast<tv*>(dst) = v;
      } else if (gn + EPC > gm) {
#pragma unroll
        for (int e = 0; e < EPC; ++e)
          if (gm <= gn + e) dst[e] = v[e];
      }
      if (!SYM && p.rowsq)
        rowsq_chunk<T, CPR>(__builtin_bit_cast(u32x4, v), p, bz, (n0 + sn) / SUB, m0 + gm);
    }
  }
  if (SYM || p.Ct) {
    T* Tg;
    int64_t ldt;
    if (SYM) {
      Tg = static_cast<T*>(p.C) + bz * p.sC;
      ldt = p.ldc;
    } else {
      Tg = static_cast<T*>(p.Ct) + bz * p.sCt;
      ldt = p.ldct;
    }
    for (int q = threadIdx.x; q < SUB * CPR; q += 256) {
      const int r = q / CPR, c = q % CPR;       // output row: tile column sn + r
      const int gn = sn + r, gm = sm + c * EPC;
      tv vs;
#pragma unroll
      for (int e = 0; e < EPC; ++e) vs[e] = tile[c * EPC + e][r];
      T* dst = Tg + (int64_t)(n0 + gn) * ldt + m0 + gm;
      if (!diag_tile || gm + EPC <= gn) {
        *reinterpret_cast<tv*>(dst) = vs;
      } else if (gm < gn) {
#pragma unroll
        for (int e = 0; e < EPC; ++e)
          if (gm + e < gn) dst[e] = vs[e];
      }
      if (!SYM && p.rowsq && !p.C)
        rowsq_chunk<T, CPR>(__builtin_bit_cast(u32x4, vs), p, bz, (m0 + sm) / SUB, n0 + gn);
    }
  }
}

int cu_count() {
  static int n = 0;
  if (n == 0) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      n = v;
    else
      n = 256;
  }
  return n;
}

// Small grids (64 x 64 tiles, few tiles per CU): the four waves of a block split the block's
// k-range among themselves (wave w takes k-tiles w, w + 4, ...), each computing the whole
// 64 x 64 tile from its own double-buffered LDS stages with no barriers in the k loop; the four
// partial tiles are then added in wave order through LDS, each wave keeping the quarter the
// 2 x 2 wave layout gives it, and the usual epilogue (or partial-sum store) follows. A k loop
// of KL k-tiles takes about KL / 4 steps of load latency instead of KL.
template <typename T, bool SYM>
__global__ __launch_bounds__(256) void k_gemm_kw(GemmArgs p) {
  using Tr = Traits<T>;
  constexpr int BM = 64, BN = 64, NT = 256;
  constexpr int VEC = Tr::VEC, BK = Tr::BK, ES = (int)sizeof(T);
  constexpr int ROWS = BM + BN;                 // LDS rows of one stage (A rows, then B rows)
  constexpr int WSTAGE = ROWS * kChunks;        // u32x4 per stage
  constexpr int INST = ROWS / 8;                // DMA instructions per wave per k-tile
  __shared__ u32x4 lds[4 * 2 * WSTAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  const int KT = p.K / BK;
  int lin = blockIdx.x, k_begin = 0, k_end = KT, slot = -1;
  if (lin < p.full_blocks) {
    const int q = p.full_blocks / 8;
    if (lin < 8 * q) lin = (lin % 8) * q + lin / 8;
  } else {
    const int r = lin - p.full_blocks, part = r % p.split;
    lin = p.full_blocks + r / p.split;
    slot = r;
    k_begin = (int)((int64_t)part * KT / p.split);
    k_end = (int)((int64_t)(part + 1) * KT / p.split);
  }
  lin = __builtin_amdgcn_readfirstlane(lin);
  slot = __builtin_amdgcn_readfirstlane(slot);
  k_begin = __builtin_amdgcn_readfirstlane(k_begin);
  k_end = __builtin_amdgcn_readfirstlane(k_end);
  int tm, tn;
  int64_t bz;
  tile_coords<SYM, BM>(p, lin, tm, tn, bz);
  const int m0 = tm * BM, n0 = tn * BN;

  const char* Abase = static_cast<const char*>(p.A) + (bz * p.sA + (int64_t)m0 * p.lda) * ES;
  const char* Bbase = static_cast<const char*>(p.B) + (bz * p.sB + (int64_t)n0 * p.ldb) * ES;
  const __amdgpu_buffer_rsrc_t rA = make_rsrc(Abase, ((int64_t)(p.M - m0) * p.lda) * ES);
  const __amdgpu_buffer_rsrc_t rB = make_rsrc(Bbase, ((int64_t)(p.N - n0) * p.ldb) * ES);
  // instruction i fills LDS rows 8i .. 8i+7 of the wave's stage (rows < BM: A, else B)
  int off[INST];
#pragma unroll
  for (int i = 0; i < INST; ++i) {
    const int row = i * 8 + (lane >> 3);
    const int ch = (lane & 7) ^ ((row ^ ((row >> 3) & 3)) & 7);
    off[i] = row < BM ? (row * (int)p.lda + ch * VEC) * ES
                      : ((row - BM) * (int)p.ldb + ch * VEC) * ES;
  }
  u32x4* const wlds = lds + wave * 2 * WSTAGE;
  auto issue = [&](int kt, int st) {
    const int so = kt * BK * ES;
#pragma unroll
    for (int i = 0; i < INST; ++i)
      dma16(i * 8 < BM ? rA : rB, &wlds[st * WSTAGE + i * 8 * kChunks], off[i], so);
  };

  floatx16 acc4[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc4[i][j][e] = 0.f;
  u32x4 af[2][2], bf[2][2];
  auto load_frags = [&](int st, int ks, int sl) {
    const int ch = 2 * ks + (lane >> 5);
#pragma unroll
    for (int i = 0; i < 2; ++i) af[sl][i] = wlds[st * WSTAGE + swz(32 * i + (lane & 31), ch)];
#pragma unroll
    for (int j = 0; j < 2; ++j) bf[sl][j] = wlds[st * WSTAGE + swz(BM + 32 * j + (lane & 31), ch)];
  };
  auto mma_step = [&](int sl) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) Tr::mma(acc4[i][j], bf[sl][j], af[sl][i]);
  };

  // This wave's k-tiles: k_begin + wave + 4 j, j < nk. Two are in flight: the load of the
  // wave's k-tile j+2 goes into stage j % 2 once the last k-step of k-tile j is in registers.
  const int KL = k_end - k_begin;
  const int nk = KL > wave ? (KL - wave + 3) / 4 : 0;
  constexpr int KS = kChunks / 2;
  if (nk > 0) {
    issue(k_begin + wave, 0);
    if (nk > 1) {
      issue(k_begin + wave + 4, 1);
      __builtin_amdgcn_s_waitcnt(wait_vm(INST));   // k-tile 0 has landed
    } else {
      __builtin_amdgcn_s_waitcnt(kWaitVm0Lgkm0);
    }
    asm volatile("" ::: "memory");
    load_frags(0, 0, 0);
    for (int j = 0; j < nk; ++j) {
      const int st = j & 1;
#pragma unroll
      for (int ks = 0; ks < KS - 1; ++ks) {
        load_frags(st, ks + 1, (ks + 1) & 1);
        mma_step(ks & 1);
      }
      // k-step 3's fragments in registers, so stage st is free; k-tile j+1 must have landed
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
      asm volatile("" ::: "memory");
      if (j + 2 < nk) {
        issue(k_begin + wave + 4 * (j + 2), st);
        __builtin_amdgcn_s_waitcnt(wait_vm(INST));   // k-tile j+1 has landed
      } else {
        __builtin_amdgcn_s_waitcnt(kWaitVm0Lgkm0);
      }
      asm volatile("" ::: "memory");
      if (j + 1 < nk) load_frags(st ^ 1, 0, 0);
      mma_step((KS - 1) & 1);
    }
  }

  // Sum the four partial tiles in wave order; wave w keeps fragment (w / 2, w % 2).
  block_sync();
  floatx4* ex = reinterpret_cast<floatx4*>(lds);   // [owner][source][g][lane]
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int owner = 2 * i + j;
      if (owner == wave) continue;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        floatx4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc4[i][j][4 * g + e];
        ex[((owner * 4 + wave) * 4 + g) * 64 + lane] = v;
      }
    }
  block_sync();
  floatx16 acc[1][1];
  {
    const int wi = wave >> 1, wj = wave & 1;
    floatx16 own;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        if (i == wi && j == wj) own = acc4[i][j];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      floatx4 sum;
#pragma unroll
      for (int src = 0; src < 4; ++src) {
        floatx4 v;
        if (src == wave) {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = own[4 * g + e];
        } else {
          v = ex[((wave * 4 + src) * 4 + g) * 64 + lane];
        }
        sum = src == 0 ? v : sum + v;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[0][0][4 * g + e] = sum[e];
    }
  }

  if (slot >= 0) {
    // partial sums in the fragment order of the 2 x 2 layout (what k_tail_epilogue reads)
    floatx4* P = reinterpret_cast<floatx4*>(p.partial) + (int64_t)slot * (4 * NT);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      floatx4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = acc[0][0][4 * g + e];
      P[g * NT + tid] = v;
    }
    return;
  }
  if constexpr (SYM) {
    // Symmetric tile: each wave stores its 32 x 32 quarter straight from registers, no LDS
    // staging and no barrier: the upper triangle (diagonal included) to C as 4-element row
    // pieces, and its strictly upper part mirrored, where 32 lanes write 32 consecutive
    // elements of one row of C. The same values and the same triangle rule as the LDS-staged
    // epilogue.
    typedef T t4 __attribute__((ext_vector_type(4)));
    const int wm = wave >> 1, wn = wave & 1;
    const int ml = wm * 32 + (lane & 31);
    const T* Dg = p.D ? static_cast<const T*>(p.D) + bz * p.sD : nullptr;
    T* Cg = static_cast<T*>(p.C) + bz * p.sC;
    const bool diag_tile = tm == tn;
    // D for all four pieces first, under one test: loads placed between the stores below
    // would each wait for the one before (the stores may alias D as far as the compiler knows).
    float d[4][4] = {};
    if (Dg) {
#pragma unroll
      for (int g = 0; g < 4; ++g)
        load4<T>(Dg + (int64_t)(m0 + ml) * p.ldd + n0 + wn * 32 + 8 * g + 4 * (lane >> 5), d[g]);
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int nl = wn * 32 + 8 * g + 4 * (lane >> 5);
      t4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float v = p.alpha * acc[0][0][4 * g + e] + p.beta * d[g][e];
        if (m0 + ml == n0 + nl + e && m0 + ml < p.diag_limit) v += p.gamma;
        o[e] = (T)v;
      }
      T* dst = Cg + (int64_t)(m0 + ml) * p.ldc + n0 + nl;
      if (!diag_tile || nl >= ml) {
        *reinterpret_cast<t4*>(dst) = o;
      } else if (nl + 3 >= ml) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (nl + e >= ml) dst[e] = o[e];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (!diag_tile || ml < nl + e) Cg[(int64_t)(n0 + nl + e) * p.ldc + m0 + ml] = o[e];
    }
  } else {
    block_sync();
    constexpr int WM = 32, WN = 32, FM = 1, FN = 1;   // the 2 x 2 wave layout
    const int wm = wave >> 1, wn = wave & 1;
    T* tile = reinterpret_cast<T*>(&lds[0]);
#include "gemm_epilogue.inc"
  }
}

template <typename T, int BM, int BN, int WGM, int WGN, bool SYM, bool KW = false,
          bool KB = false>
hipError_t launch(const GemmDesc& d, hipStream_t s) {
  GemmArgs a;
  a.A = d.A; a.B = d.B; a.D = d.D; a.C = d.C; a.Ct = d.Ct;
  a.lda = d.lda; a.ldb = d.ldb; a.ldd = d.ldd; a.ldc = d.ldc; a.ldct = d.ldct;
  a.sA = d.sA; a.sB = d.sB; a.sD = d.sD; a.sC = d.sC; a.sCt = d.sCt;
  a.M = d.M; a.N = d.N; a.K = d.K;
  a.alpha = d.alpha; a.beta = d.beta; a.gamma = d.gamma;
  a.diag_limit = d.diag_limit;
  a.rowsq = d.rowsq;
  a.rowsq_rows = d.rowsq_rows;
  a.rowsq_chunks = (d.C ? d.N : d.M) / 64;
  a.group = 4;
  if (SYM) {
    const int t = d.M / BM;
    a.tiles_n = t;
    a.tiles_per_batch = t * (t + 1) / 2;
  } else {
    a.tiles_n = d.N / BN;
    a.tiles_per_batch = (d.M / BM) * (d.N / BN);
  }
  // Rounds of whole tiles over the CU slots (one 256-tile block per CU, two 128-tile blocks,
  // one 64-tile block of k_gemm_kw); a tail round less than half full is split along k (at
  // least 8 k-tiles per part).
  const int64_t total = (int64_t)a.tiles_per_batch * d.batch;
  const int slots = cu_count() * (KW || BM >= 256 ? 1 : BM >= 128 ? 2 : 4);
  const int64_t rounds = total / slots, tail = total % slots;
  const int KT = d.K / Traits<T>::BK;
  int split = 1;
  if (tail > 0 && tail <= slots / 2 && d.partial) {
    int64_t sp = slots / tail;
    if (sp > KT / 8) sp = KT / 8;
    const int64_t per = (int64_t)BM * BN * 4;
    while (sp > 1 && tail * sp * per > (int64_t)d.partial_bytes) --sp;
    if (sp > 1) split = (int)sp;
  }
  a.split = split;
  a.partial = d.partial;
  a.fix_parts = split;
  a.full_blocks = (int)(split > 1 ? rounds * slots : total);
  const unsigned blocks = (unsigned)(a.full_blocks + (split > 1 ? tail * split : 0));
  if constexpr (KW)
    hipLaunchKernelGGL((k_gemm_kw<T, SYM>), dim3(blocks), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((k_gemm<T, BM, BN, WGM, WGN, SYM, KB>), dim3(blocks), dim3(64 * WGM * WGN), 0,
                       s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || split < 2) return e;
  // The tail epilogue (one block per 64 x 64 sub-tile) sums the parts itself when they are
  // few (at most 8, 128 KiB per block); more are first summed by a wide reduction launch.
  constexpr int tile_f4 = BM * BN / 4;
  static_assert(tile_f4 % 256 == 0, "whole reduce blocks per tile");
  a.fix_parts = split;
  if (split > 8) {
    hipLaunchKernelGGL(k_reduce_parts, dim3((unsigned)(tail * (tile_f4 / 256))), dim3(256), 0, s,
                       reinterpret_cast<floatx4*>(a.partial), split, tile_f4);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    a.fix_parts = 1;
  }
  hipLaunchKernelGGL((k_tail_epilogue<T, BM, BN, WGM, WGN, SYM>),
                     dim3((unsigned)(tail * (BM / 64) * (BN / 64))), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename T, int BT, int WGM, int WGN>
hipError_t dispatch_tile(const GemmDesc& d, hipStream_t s) {
  if (d.sym) return launch<T, BT, BT, WGM, WGN, true>(d, s);
  return launch<T, BT, BT, WGM, WGN, false>(d, s);
}

// Tiles per batch entry of a BT x BT grid (upper triangle for sym).
int64_t tiles_of(const GemmDesc& d, int bt) {
  const int64_t tm = d.M / bt, tn = d.N / bt;
  return d.sym ? tm * (tm + 1) / 2 : tm * tn;
}

// 256 x 256 tiles when they give at least two rounds of blocks over the CUs, or one round
// when K is long (>= 4096: the split tail then has k-tiles enough); 64 x 64 (the k-split
// kernel) when 128 x 128 tiles would not even fill a quarter of the CUs; else 128 x 128.
// Float32 uses the same rule without the 256 x 256 step.
int tile_for(const GemmDesc& d) {
  if (d.elem == Elem::F32) return tiles_of(d, 128) * d.batch * 4 < cu_count() ? 64 : 128;
  if (tiles_of(d, 256) * d.batch >= (d.K >= 4096 ? 1 : 2) * cu_count()) return 256;
  if (tiles_of(d, 128) * d.batch * 4 < cu_count()) return 64;
  return 128;
}

}  // namespace

hipError_t gemm(const GemmDesc& d, hipStream_t s) {
  if (d.M % kPad || d.N % kPad || d.K % kPad || d.batch < 1) return hipErrorInvalidValue;
  if (d.sym && (d.M != d.N || !d.C || d.Ct)) return hipErrorInvalidValue;
  if (!d.sym && !d.C && !d.Ct) return hipErrorInvalidValue;
  if (d.rowsq && (d.sym || d.rowsq_rows < 0)) return hipErrorInvalidValue;
  if (d.b_kmajor) {
    if (!gemm_kmajor_ok(d)) return hipErrorInvalidValue;
    if (tile_for(d) == 256) return launch<_Float16, 256, 256, 2, 4, false, false, true>(d, s);
    return launch<_Float16, 128, 128, 2, 2, false, false, true>(d, s);
  }
  if (d.elem == Elem::F32) {
    if (tile_for(d) == 64) {
      if (d.sym) return launch<float, 64, 64, 2, 2, true, true>(d, s);
      return launch<float, 64, 64, 2, 2, false, true>(d, s);
    }
    return dispatch_tile<float, 128, 2, 2>(d, s);
  }
  const int bt = tile_for(d);
  if (bt == 256) return dispatch_tile<_Float16, 256, 2, 4>(d, s);
  if (bt == 64) {
    if (d.sym) return launch<_Float16, 64, 64, 2, 2, true, true>(d, s);
    return launch<_Float16, 64, 64, 2, 2, false, true>(d, s);
  }
  return dispatch_tile<_Float16, 128, 2, 2>(d, s);
}

bool gemm_kmajor_ok(const GemmDesc& d) {
  if (d.elem != Elem::F16 || d.sym) return false;
  const int bt = tile_for(d);
  return bt == 256 || bt == 128;
}

const char* gemm_name(const GemmDesc& d) {
  if (d.elem == Elem::F32) {
    if (tile_for(d) == 64) return d.sym ? "gemm_sym_f32_64" : "gemm_nt_f32_64";
    return d.sym ? "gemm_sym_f32_128" : "gemm_nt_f32_128";
  }
  switch (tile_for(d)) {
    case 256: return d.sym ? "gemm_sym_f16_256" : "gemm_nt_f16_256";
    case 64: return d.sym ? "gemm_sym_f16_64" : "gemm_nt_f16_64";
    default: return d.sym ? "gemm_sym_f16_128" : "gemm_nt_f16_128";
  }
}

}  // namespace mns
