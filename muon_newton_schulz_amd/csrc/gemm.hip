// MFMA GEMM for the Newton-Schulz products on gfx950 (CDNA4).
//
//   C = alpha * A op(B) + beta * D + gamma * I        (float32 accumulation)
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
// Layout / tiling:
//   * 256 threads = 4 wave64s in a 2 x 2 grid; block tile BM x BN, wave tile BM/2 x BN/2 of
//     32 x 32 MFMA fragments (v_mfma_f32_32x32x16_f16, or 32x32x2f32 for float32).
//   * k-tile = 128 bytes per row (64 halves / 32 floats). Both operands sit in LDS as
//     [row][k] in 16-byte chunks, double buffered, with chunk c of row r stored at
//     c ^ ((r ^ (r >> 3)) & 7): fragment reads (32 rows, one chunk) and the transposed
//     writes below hit distinct bank groups.
//   * A and a k-contiguous B are copied chunk by chunk. An n-contiguous B ([K][N], the X
//     of B X) is loaded as VEC x VEC blocks (VEC = elements per 16 bytes) and transposed in
//     registers before the LDS store, so the MFMA always reads k-contiguous chunks.
//   * MFMA operand roles are swapped (the B tile feeds the MFMA's A input), so each lane's
//     accumulators hold 4 consecutive output columns of one row: vector stores along N.
#include "mns_internal.h"

namespace mns {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kChunks = 8;   // 16-byte chunks per LDS row (one 128-byte k-tile)

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
  return row * kChunks + (chunk ^ ((row ^ (row >> 3)) & 7));
}

struct GemmArgs {
  const void* A; const void* B; void* C; const void* D;
  int64_t lda, ldb, ldc, ldd;
  int64_t sA, sB, sC, sD;
  int M, N, K;
  float alpha, beta, gamma;
  int diag_limit;
  int tiles_n;      // N / BN (dense grid) or tiles per side (sym)
  int group;        // tile rows per group of the dense tile order
};

template <typename T>
__device__ __forceinline__ void store4(T* p, const float* v);
template <>
__device__ __forceinline__ void store4<_Float16>(_Float16* p, const float* v) {
  half4 h = {(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
  *reinterpret_cast<half4*>(p) = h;
}
template <>
__device__ __forceinline__ void store4<float>(float* p, const float* v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}

template <typename T>
__device__ __forceinline__ void load4(const T* p, float* v);
template <>
__device__ __forceinline__ void load4<_Float16>(const _Float16* p, float* v) {
  const half4 h = *reinterpret_cast<const half4*>(p);
  v[0] = (float)h.x; v[1] = (float)h.y; v[2] = (float)h.z; v[3] = (float)h.w;
}
template <>
__device__ __forceinline__ void load4<float>(const float* p, float* v) {
  const float4 f = *reinterpret_cast<const float4*>(p);
  v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
}

// Block tile BM x BN computed by WGM x WGN waves (wave tile BM/WGM x BN/WGN).
template <typename T, int BM, int BN, int WGM, int WGN, bool BKMAJ, bool SYM>
__global__ __launch_bounds__(64 * WGM * WGN) void k_gemm(GemmArgs p) {
  using Tr = Traits<T>;
  constexpr int NT = 64 * WGM * WGN;
  constexpr int VEC = Tr::VEC, BK = Tr::BK;
  constexpr int WM = BM / WGM, WN = BN / WGN, FM = WM / 32, FN = WN / 32;
  constexpr int A_LD = BM * kChunks / NT;                  // A chunks per thread
  constexpr int BK_LD = BN * kChunks / NT;                 // k-major B chunks per thread
  // [K][N] operand: a thread loads 4 k-rows x VEC n-columns (4 x 16 bytes) per k-tile.
  constexpr int NN_JOBS = (BK / 4) * (BN / VEC);
  constexpr int B_REGS = BKMAJ ? BK_LD : 4;
  static_assert(A_LD >= 1 && BK_LD >= 1 && FM >= 1 && FN >= 1, "tile too small");
  static_assert(BKMAJ || NN_JOBS == NT, "[K][N] loader assumes one 4-row job per thread");

  __shared__ u32x4 lds[2][(BM + BN) * kChunks];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;

  // Tile order. Workgroups go round-robin to the 8 XCDs (L2 domains); remap so each XCD
  // walks a contiguous range of logical tiles, and order those in groups of p.group tile
  // rows (column-major inside a group), so the CUs of one XCD share A rows and B columns.
  int t = blockIdx.x;
  {
    const int q = (int)gridDim.x / 8;
    if (t < 8 * q) t = (t % 8) * q + t / 8;
  }
  int tm, tn;
  if (SYM) {
    tm = 0;
    while (t >= p.tiles_n - tm) { t -= p.tiles_n - tm; ++tm; }
    tn = tm + t;
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
  const int64_t bz = blockIdx.z;
  const T* Ag = static_cast<const T*>(p.A) + bz * p.sA + (int64_t)m0 * p.lda;
  const T* Bg = static_cast<const T*>(p.B) + bz * p.sB +
                (BKMAJ ? (int64_t)n0 * p.ldb : (int64_t)n0);

  // [K][N] job of this thread: 16-bit types alternate the 8-byte half of the k-chunk
  // between neighbouring lanes, which keeps the 8-byte LDS writes conflict-free.
  int nn_c = 0, nn_kq = 0;
  if (!BKMAJ) {
    if (VEC == 8) {
      nn_c = (tid >> 1) % (BN / VEC);
      nn_kq = 2 * ((tid >> 1) / (BN / VEC)) + (tid & 1);
    } else {
      nn_c = tid % (BN / VEC);
      nn_kq = tid / (BN / VEC);
    }
  }

  u32x4 ra[A_LD];
  u32x4 rb[B_REGS];

  auto load_global = [&](int kt) {
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
      const int q = tid + NT * i, row = q / kChunks, ch = q % kChunks;
      ra[i] = *reinterpret_cast<const u32x4*>(Ag + (int64_t)row * p.lda + k0 + ch * VEC);
    }
    if (BKMAJ) {
#pragma unroll
      for (int i = 0; i < BK_LD; ++i) {
        const int q = tid + NT * i, row = q / kChunks, ch = q % kChunks;
        rb[i] = *reinterpret_cast<const u32x4*>(Bg + (int64_t)row * p.ldb + k0 + ch * VEC);
      }
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        rb[r] = *reinterpret_cast<const u32x4*>(Bg + (int64_t)(k0 + 4 * nn_kq + r) * p.ldb +
                                               nn_c * VEC);
    }
  };

  auto store_lds = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
      const int q = tid + NT * i, row = q / kChunks, ch = q % kChunks;
      lds[buf][swz(row, ch)] = ra[i];
    }
    if (BKMAJ) {
#pragma unroll
      for (int i = 0; i < BK_LD; ++i) {
        const int q = tid + NT * i, row = q / kChunks, ch = q % kChunks;
        lds[buf][swz(BM + row, ch)] = rb[i];
      }
    } else if (VEC == 8) {
      // 4 k-rows x 8 n-columns of 16-bit values -> for each column e, 4 consecutive k
      // (8 bytes) into half (nn_kq & 1) of k-chunk nn_kq / 2 of LDS row n.
      unsigned* base = reinterpret_cast<unsigned*>(&lds[buf][0]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = e >> 1;
        const unsigned r0 = rb[0][d], r1 = rb[1][d], r2 = rb[2][d], r3 = rb[3][d];
        unsigned w0, w1;
        if (e & 1) {
          w0 = (r0 >> 16) | (r1 & 0xFFFF0000u);
          w1 = (r2 >> 16) | (r3 & 0xFFFF0000u);
        } else {
          w0 = (r0 & 0xFFFFu) | (r1 << 16);
          w1 = (r2 & 0xFFFFu) | (r3 << 16);
        }
        const int row = BM + nn_c * 8 + e;
        unsigned* dst = base + 4 * swz(row, nn_kq >> 1) + 2 * (nn_kq & 1);
        *reinterpret_cast<uint2*>(dst) = make_uint2(w0, w1);
      }
    } else {
      // 4 k-rows x 4 n-columns of float32 -> one 16-byte k-chunk per column.
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        u32x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = rb[q][e];
        lds[buf][swz(BM + nn_c * 4 + e, nn_kq)] = o;
      }
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
  const int brow = BM + wn * WN + (lane & 31);
  u32x4 af[2][FM], bf[2][FN];
  auto load_frags = [&](int buf, int ks, int slot) {
    const int ch = 2 * ks + (lane >> 5);
#pragma unroll
    for (int i = 0; i < FM; ++i) af[slot][i] = lds[buf][swz(arow + 32 * i, ch)];
#pragma unroll
    for (int j = 0; j < FN; ++j) bf[slot][j] = lds[buf][swz(brow + 32 * j, ch)];
  };

  // Pipeline: LDS holds tile kt (being read) and receives tile kt+1 from registers at the
  // top of iteration kt; the registers are then refilled with tile kt+2, so every global
  // load has a whole iteration of MFMA work to arrive.
  const int KT = p.K / BK;
  load_global(0);
  store_lds(0);
  if (KT > 1) load_global(1);
  __syncthreads();

  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    load_frags(cur, 0, 0);
    if (kt + 1 < KT) store_lds(cur ^ 1);
    if (kt + 2 < KT) load_global(kt + 2);
#pragma unroll
    for (int ks = 0; ks < kChunks / 2; ++ks) {
      if (ks + 1 < kChunks / 2) load_frags(cur, ks + 1, (ks + 1) & 1);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) Tr::mma(acc[i][j], bf[ks & 1][j], af[ks & 1][i]);
    }
    __syncthreads();
  }

  // Epilogue. acc[i][j][4g + e] is C[m][n + e] with m = row of the A tile (lane & 31) and
  // n = 8g + 4 (lane >> 5) within the 32 x 32 fragment.
  T* Cg = static_cast<T*>(p.C) + bz * p.sC;
  const T* Dg = p.D ? static_cast<const T*>(p.D) + bz * p.sD : nullptr;
  const bool diag_tile = SYM && (tm == tn);
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int m = m0 + wm * WM + 32 * i + (lane & 31);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * WN + 32 * j + 8 * g + 4 * (lane >> 5);
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = p.alpha * acc[i][j][4 * g + e];
        if (Dg) {
          float d[4];
          load4<T>(Dg + (int64_t)m * p.ldd + n, d);
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] += p.beta * d[e];
        }
        if (p.gamma != 0.f && m < p.diag_limit && m >= n && m < n + 4) v[m - n] += p.gamma;
        if (!SYM) {
          store4<T>(Cg + (int64_t)m * p.ldc + n, v);
        } else if (!diag_tile) {
          store4<T>(Cg + (int64_t)m * p.ldc + n, v);
#pragma unroll
          for (int e = 0; e < 4; ++e) Cg[(int64_t)(n + e) * p.ldc + m] = (T)v[e];
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (m <= n + e) Cg[(int64_t)m * p.ldc + n + e] = (T)v[e];
            if (m < n + e) Cg[(int64_t)(n + e) * p.ldc + m] = (T)v[e];
          }
        }
      }
    }
  }
}

template <typename T, int BM, int BN, int WGM, int WGN, bool BKMAJ, bool SYM>
hipError_t launch(const GemmDesc& d, hipStream_t s) {
  GemmArgs a;
  a.A = d.A; a.B = d.B; a.C = d.C; a.D = d.D;
  a.lda = d.lda; a.ldb = d.ldb; a.ldc = d.ldc; a.ldd = d.ldd;
  a.sA = d.sA; a.sB = d.sB; a.sC = d.sC; a.sD = d.sD;
  a.M = d.M; a.N = d.N; a.K = d.K;
  a.alpha = d.alpha; a.beta = d.beta; a.gamma = d.gamma;
  a.diag_limit = d.diag_limit;
  a.group = 4;
  unsigned tiles;
  if (SYM) {
    const int t = d.M / BM;
    a.tiles_n = t;
    tiles = (unsigned)(t * (t + 1) / 2);
  } else {
    a.tiles_n = d.N / BN;
    tiles = (unsigned)((d.M / BM) * (d.N / BN));
  }
  hipLaunchKernelGGL((k_gemm<T, BM, BN, WGM, WGN, BKMAJ, SYM>), dim3(tiles, 1, d.batch),
                     dim3(64 * WGM * WGN), 0, s, a);
  return hipGetLastError();
}

template <typename T, int BT, int WGM, int WGN>
hipError_t dispatch_tile(const GemmDesc& d, hipStream_t s) {
  if (d.sym) return launch<T, BT, BT, WGM, WGN, true, true>(d, s);
  if (d.b_kmajor) return launch<T, BT, BT, WGM, WGN, true, false>(d, s);
  return launch<T, BT, BT, WGM, WGN, false, false>(d, s);
}

}  // namespace

// 256 x 256 tiles when they give at least two waves of blocks over the 256 CUs.
static int tile_for(const GemmDesc& d) {
  if (d.elem == Elem::F32) return 128;
  const int64_t t256 = d.sym ? (int64_t)(d.M / 256) * (d.M / 256 + 1) / 2
                             : (int64_t)(d.M / 256) * (d.N / 256);
  return t256 * d.batch >= 512 ? 256 : 128;
}

hipError_t gemm(const GemmDesc& d, hipStream_t s) {
  if (d.M % kPad || d.N % kPad || d.K % kPad || d.batch < 1) return hipErrorInvalidValue;
  if (d.sym && (d.M != d.N || !d.b_kmajor)) return hipErrorInvalidValue;
  if (d.elem == Elem::F32) return dispatch_tile<float, 128, 2, 2>(d, s);
  if (tile_for(d) == 256) return dispatch_tile<_Float16, 256, 2, 4>(d, s);
  return dispatch_tile<_Float16, 128, 2, 2>(d, s);
}

const char* gemm_name(const GemmDesc& d) {
  const bool f32 = d.elem == Elem::F32;
  const bool t256 = tile_for(d) == 256;
  if (d.sym) return f32 ? "gemm_sym_f32_128" : (t256 ? "gemm_sym_f16_256" : "gemm_sym_f16_128");
  if (d.b_kmajor) return f32 ? "gemm_nt_f32_128" : (t256 ? "gemm_nt_f16_256" : "gemm_nt_f16_128");
  return f32 ? "gemm_nn_f32_128" : (t256 ? "gemm_nn_f16_256" : "gemm_nn_f16_128");
}

}  // namespace mns
