// HBM-bound kernels of the Muon step on gfx950: momentum with Frobenius partial sums,
// normalisation into the padded Newton-Schulz iterate, NorMuon statistics, the fused
// weight update, and Dion3's row selection. All reductions run in a fixed order (no
// floating-point atomics), so every result is bitwise reproducible.
//
// Method: page "Dion3: Full-stack orthogonal updates" -- Eq. (1) (momentum, weight update),
// section "Standard Newton-Schulz" (X_0 = X / ||X||_F), Eq. (2) (NorMuon, in float32 as the
// page's implementation notes state), Algorithm 4 (l1 selection, error feedback).
#include "mns_internal.h"

#include <math.h>

namespace mns {
namespace {

constexpr int kThreads = 256;
constexpr int kIter = 8;                      // float4 vectors per thread per block

// ---- scalar conversions -------------------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Round-to-nearest-even float32 -> bfloat16 (bfloat16 is the upper half of binary32:
// add half an ulp of the kept part, plus one when the kept part is odd, and truncate).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return 0x7FC0u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Load 4 consecutive storage elements (bfloat16 bits or float32) as float32.
template <typename TS>
__device__ __forceinline__ float4 load4(const TS* p, int64_t i);
template <>
__device__ __forceinline__ float4 load4<float>(const float* p, int64_t i) {
  return *reinterpret_cast<const float4*>(p + i);
}
template <>
__device__ __forceinline__ float4 load4<uint16_t>(const uint16_t* p, int64_t i) {
  uint2 v = *reinterpret_cast<const uint2*>(p + i);
  return make_float4(bf16_to_f32(v.x & 0xFFFFu), bf16_to_f32(v.x >> 16),
                     bf16_to_f32(v.y & 0xFFFFu), bf16_to_f32(v.y >> 16));
}
template <>
__device__ __forceinline__ float4 load4<_Float16>(const _Float16* p, int64_t i) {
  typedef _Float16 h4 __attribute__((ext_vector_type(4)));
  h4 v = *reinterpret_cast<const h4*>(p + i);
  return make_float4((float)v.x, (float)v.y, (float)v.z, (float)v.w);
}

template <typename TS>
__device__ __forceinline__ float load1(const TS* p, int64_t i);
template <>
__device__ __forceinline__ float load1<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load1<uint16_t>(const uint16_t* p, int64_t i) {
  return bf16_to_f32(p[i]);
}
template <>
__device__ __forceinline__ float load1<_Float16>(const _Float16* p, int64_t i) {
  return (float)p[i];
}

template <typename TS>
__device__ __forceinline__ void store4(TS* p, int64_t i, float4 v);
template <>
__device__ __forceinline__ void store4<float>(float* p, int64_t i, float4 v) {
  *reinterpret_cast<float4*>(p + i) = v;
}
template <>
__device__ __forceinline__ void store4<uint16_t>(uint16_t* p, int64_t i, float4 v) {
  uint2 o;
  o.x = f32_to_bf16(v.x) | (f32_to_bf16(v.y) << 16);
  o.y = f32_to_bf16(v.z) | (f32_to_bf16(v.w) << 16);
  *reinterpret_cast<uint2*>(p + i) = o;
}
template <>
__device__ __forceinline__ void store4<_Float16>(_Float16* p, int64_t i, float4 v) {
  typedef _Float16 h4 __attribute__((ext_vector_type(4)));
  h4 o = {(_Float16)v.x, (_Float16)v.y, (_Float16)v.z, (_Float16)v.w};
  *reinterpret_cast<h4*>(p + i) = o;
}

template <typename TS>
__device__ __forceinline__ void store1(TS* p, int64_t i, float v);
template <>
__device__ __forceinline__ void store1<float>(float* p, int64_t i, float v) { p[i] = v; }
template <>
__device__ __forceinline__ void store1<uint16_t>(uint16_t* p, int64_t i, float v) {
  p[i] = (uint16_t)f32_to_bf16(v);
}
template <>
__device__ __forceinline__ void store1<_Float16>(_Float16* p, int64_t i, float v) {
  p[i] = (_Float16)v;
}

// ---- deterministic block reductions (fixed shuffle tree, then waves in order) --------------

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_down(v, o, 64);
  return v;  // valid in lane 0
}

// Sum over the block; the result is valid in thread 0 only.
template <typename T, int NT>
__device__ __forceinline__ T block_sum(T v, T* sh) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) sh[w] = v;
  __syncthreads();
  T r = 0;
  if (threadIdx.x == 0) {
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) r += sh[i];
  }
  __syncthreads();
  return r;
}

// ---- a1: momentum M <- mu M + G, partial sums of M^2 (Eq. 1) --------------------------------

template <typename TG>
__global__ __launch_bounds__(kThreads) void k_momentum(PtrPack Mp, PtrPack Gp, int64_t elems,
                                                       float mu, float* partials, int nblk) {
  __shared__ float sh[kThreads / 64];
  const int b = blockIdx.y;
  float* m = static_cast<float*>(Mp.p[b]);
  const TG* g = static_cast<const TG*>(Gp.p[b]);
  const int64_t nvec = elems / 4;
  float acc = 0.f;
#pragma unroll
  for (int it = 0; it < kIter; ++it) {
    const int64_t v = ((int64_t)blockIdx.x * kIter + it) * kThreads + threadIdx.x;
    if (v < nvec) {
      float4 mv = load4<float>(m, 4 * v);
      const float4 gv = load4<TG>(g, 4 * v);
      mv.x = fmaf(mu, mv.x, gv.x);
      mv.y = fmaf(mu, mv.y, gv.y);
      mv.z = fmaf(mu, mv.z, gv.z);
      mv.w = fmaf(mu, mv.w, gv.w);
      store4<float>(m, 4 * v, mv);
      acc += mv.x * mv.x + mv.y * mv.y + mv.z * mv.z + mv.w * mv.w;
    }
  }
  if (blockIdx.x == gridDim.x - 1 && threadIdx.x < 4) {
    const int64_t e = nvec * 4 + threadIdx.x;
    if (e < elems) {
      const float mv = fmaf(mu, m[e], load1<TG>(g, e));
      m[e] = mv;
      acc += mv * mv;
    }
  }
  const float s = block_sum<float, kThreads>(acc, sh);
  if (threadIdx.x == 0) partials[(int64_t)b * nblk + blockIdx.x] = s;
}

// ---- partial sums of X^2 for a stored matrix (X / ||X||_F of standard NS) ------------------

template <typename TX>
__global__ __launch_bounds__(kThreads) void k_sumsq(const TX* X, int64_t elems, float* partials,
                                                    int nblk) {
  __shared__ float sh[kThreads / 64];
  const int b = blockIdx.y;
  const TX* x = X + (int64_t)b * elems;
  const int64_t nvec = elems / 4;
  float acc = 0.f;
#pragma unroll
  for (int it = 0; it < kIter; ++it) {
    const int64_t v = ((int64_t)blockIdx.x * kIter + it) * kThreads + threadIdx.x;
    if (v < nvec) {
      const float4 xv = load4<TX>(x, 4 * v);
      acc += xv.x * xv.x + xv.y * xv.y + xv.z * xv.z + xv.w * xv.w;
    }
  }
  if (blockIdx.x == gridDim.x - 1 && threadIdx.x < 4) {
    const int64_t e = nvec * 4 + threadIdx.x;
    if (e < elems) {
      const float xv = load1<TX>(x, e);
      acc += xv * xv;
    }
  }
  const float s = block_sum<float, kThreads>(acc, sh);
  if (threadIdx.x == 0) partials[(int64_t)b * nblk + blockIdx.x] = s;
}

// ---- a2: 1/||M||_F (times the iterate's storage scale) ----------------------------------------

__global__ __launch_bounds__(kThreads) void k_finalize_scale(const float* partials, int nblk,
                                                             float S, float* xscale) {
  __shared__ double sh[kThreads / 64];
  const int b = blockIdx.x;
  double acc = 0.0;
  for (int i = threadIdx.x; i < nblk; i += kThreads) acc += (double)partials[(int64_t)b * nblk + i];
  const double s = block_sum<double, kThreads>(acc, sh);
  if (threadIdx.x == 0) xscale[b] = s > 0.0 ? (float)((double)S / sqrt(s)) : 0.f;
}

// ---- a2: X_0 = scale * M, in both layouts, zero padded -------------------------------------

// One block per 64 x 64 tile of the padded source: the scaled tile goes to S (same
// layout as the source, 8-byte row chunks) and, through LDS, to T transposed.
template <typename TS, typename TX>
__global__ __launch_bounds__(kThreads) void k_normalize(PtrPack src, const TS* base, int64_t rows,
                                                        int64_t cols, const float* xscale, TX* S,
                                                        TX* T, int64_t rows_p, int64_t cols_p) {
  __shared__ float tile[64][65];
  const int b = blockIdx.z;
  const TS* s = base ? base + (int64_t)b * rows * cols : static_cast<const TS*>(src.p[b]);
  const int64_t lds = padded_ld(cols_p), ldt = padded_ld(rows_p);
  TX* so = S + (int64_t)b * rows_p * lds;
  TX* to = T + (int64_t)b * cols_p * ldt;
  const float sc = xscale[b];
  const int64_t r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const bool vec_ok = (cols % 4) == 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int lr = ty + 16 * i;
    const int64_t r = r0 + lr, c = c0 + 4 * tx;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (r < rows) {
      if (vec_ok && c + 4 <= cols) {
        v = load4<TS>(s, r * cols + c);
      } else {
        float t4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) t4[e] = (c + e < cols) ? load1<TS>(s, r * cols + c + e) : 0.f;
        v = make_float4(t4[0], t4[1], t4[2], t4[3]);
      }
    }
    v.x *= sc; v.y *= sc; v.z *= sc; v.w *= sc;
    store4<TX>(so, r * lds + c, v);
    tile[lr][4 * tx + 0] = v.x;
    tile[lr][4 * tx + 1] = v.y;
    tile[lr][4 * tx + 2] = v.z;
    tile[lr][4 * tx + 3] = v.w;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int lc = ty + 16 * i;
    const float4 v = make_float4(tile[4 * tx + 0][lc], tile[4 * tx + 1][lc], tile[4 * tx + 2][lc],
                                 tile[4 * tx + 3][lc]);
    store4<TX>(to, (c0 + lc) * ldt + r0 + 4 * tx, v);
  }
}

// ---- O (caller layout) = inv_s * iterate in the stored layout ------------------------------

template <typename TX, typename TO>
__global__ __launch_bounds__(kThreads) void k_export(const TX* X, int64_t rows_p, int64_t cols_p,
                                                     int64_t rows, int64_t cols, float inv_s,
                                                     TO* O) {
  const int b = blockIdx.z;
  const int64_t ldx = padded_ld(cols_p);
  const TX* x = X + (int64_t)b * rows_p * ldx;
  TO* o = O + (int64_t)b * rows * cols;
  const int64_t c0 = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * 4;
  if (c0 >= cols) return;
  const bool vec_ok = (cols % 4) == 0;
  for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) {
    float4 v = load4<TX>(x, r * ldx + c0);
    v.x *= inv_s; v.y *= inv_s; v.z *= inv_s; v.w *= inv_s;
    if (vec_ok) {
      store4<TO>(o, r * cols + c0, v);
    } else {
      const float t[4] = {v.x, v.y, v.z, v.w};
      for (int e = 0; e < 4 && c0 + e < cols; ++e) store1<TO>(o, r * cols + c0 + e, t[e]);
    }
  }
}

// ---- NorMuon statistics: per stored row, partial sums of O^2 -------------------------------

// One block per 256 x 256 tile of the iterate in the stored layout: partial sums of each
// row's squares over the tile's 256 columns -> part[chunk = tile column][row].
template <typename TX>
__global__ __launch_bounds__(kThreads) void k_row_sumsq_x(const TX* X, int64_t rows_p,
                                                          int64_t cols_p, int64_t rows,
                                                          float* part) {
  constexpr int TPR = 64;                 // one wave per 256-wide row segment (4 per thread)
  constexpr int RPI = kThreads / TPR;     // rows per iteration
  const int b = blockIdx.z;
  const int64_t ldx = padded_ld(cols_p);
  const TX* x = X + (int64_t)b * rows_p * ldx;
  const int64_t r0 = (int64_t)blockIdx.y * 256, c = (int64_t)blockIdx.x * 256 + (threadIdx.x % TPR) * 4;
  const int64_t chunks = cols_p / 256;
  float* out = part + (int64_t)b * chunks * rows + (int64_t)blockIdx.x * rows;
  for (int it = 0; it < 256 / RPI; ++it) {
    const int64_t r = r0 + it * RPI + threadIdx.x / TPR;
    const float4 v = load4<TX>(x, r * ldx + c);
    float s = v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    s = wave_sum(s);
    if ((threadIdx.x % TPR) == 0 && r < rows) out[r] = s;
  }
}

// Caller-layout O (rows x cols): one block per row, part[b][0][row].
template <typename TO>
__global__ __launch_bounds__(kThreads) void k_row_sumsq_stored(const TO* O, int64_t rows,
                                                               int64_t cols, float* part) {
  __shared__ float sh[kThreads / 64];
  const int b = blockIdx.y;
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
    const TO* o = O + ((int64_t)b * rows + r) * cols;
    float acc = 0.f;
    for (int64_t j = threadIdx.x; j < cols; j += kThreads) {
      const float v = load1<TO>(o, j);
      acc += v * v;
    }
    const float s = block_sum<float, kThreads>(acc, sh);
    if (threadIdx.x == 0) part[(int64_t)b * rows + r] = s;
  }
}

// ---- a7: NorMuon (Eq. 2) v update and the per-row step scale --------------------------------

constexpr int kFinThreads = 1024;

__global__ __launch_bounds__(kFinThreads) void k_normuon_finalize(
    const float* part, int chunks, int64_t rows, int64_t cols, PtrPack vp, float* v_base,
    int64_t v_stride, const int32_t* rowidx, float beta2, float eps, float inv_s2,
    float out_scale, float* rowscale) {
  __shared__ double sh[kFinThreads / 64];
  __shared__ float ratio_sh;
  const int b = blockIdx.x;
  float* v = v_base ? v_base + (int64_t)b * v_stride : static_cast<float*>(vp.p[b]);
  const float* pt = part + (int64_t)b * chunks * rows;
  const int32_t* ri = rowidx ? rowidx + (int64_t)b * rows : nullptr;
  float* rs = rowscale + (int64_t)b * rows;
  const float inv_cols = 1.0f / (float)cols;
  double s_o = 0.0, s_h = 0.0;
  for (int64_t i = threadIdx.x; i < rows; i += kFinThreads) {
    float r = 0.f;
    for (int c = 0; c < chunks; ++c) r += pt[(int64_t)c * rows + i];
    r *= inv_s2;
    const int64_t vi = ri ? (int64_t)ri[i] : i;
    const float vn = fmaf(beta2, v[vi], (1.0f - beta2) * (r * inv_cols));
    v[vi] = vn;
    const float d = 1.0f / (sqrtf(vn) + eps);
    rs[i] = d;
    s_o += (double)r;
    s_h += (double)r * (double)d * (double)d;
  }
  const double to = block_sum<double, kFinThreads>(s_o, sh);
  const double th = block_sum<double, kFinThreads>(s_h, sh);
  if (threadIdx.x == 0) ratio_sh = th > 0.0 ? (float)sqrt(to / th) : 0.f;
  __syncthreads();
  const float scale = ratio_sh * out_scale;
  for (int64_t i = threadIdx.x; i < rows; i += kFinThreads) rs[i] = rs[i] * scale;
}

__global__ __launch_bounds__(kThreads) void k_fill(float* p, int64_t n, float value) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * kThreads)
    p[i] = value;
}

// ---- a7: fused weight update W <- W - lr * rowscale_i * O_ij, one rounding ------------------

template <typename TW, typename TX>
__global__ __launch_bounds__(kThreads) void k_wupdate(PtrPack Wp, int64_t rows, int64_t cols,
                                                      const TX* X, int64_t rows_p, int64_t cols_p,
                                                      const float* rowscale,
                                                      const int32_t* rowidx,
                                                      int64_t rowidx_stride, float lr) {
  const int b = blockIdx.z;
  TW* w = static_cast<TW*>(Wp.p[b]);
  const int64_t ldx = padded_ld(cols_p);
  const TX* x = X + (int64_t)b * rows_p * ldx;
  const float* rs = rowscale + (int64_t)b * rows;
  const int32_t* ri = rowidx ? rowidx + (int64_t)b * rowidx_stride : nullptr;
  const int64_t c0 = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * 4;
  if (c0 >= cols) return;
  const bool vec_ok = (cols % 4) == 0;
  for (int64_t p = blockIdx.y; p < rows; p += gridDim.y) {
    const int64_t wr = ri ? (int64_t)ri[p] : p;
    const float k = -lr * rs[p];
    const float4 o = load4<TX>(x, p * ldx + c0);
    if (vec_ok) {
      float4 wv = load4<TW>(w, wr * cols + c0);
      wv.x = fmaf(k, o.x, wv.x);
      wv.y = fmaf(k, o.y, wv.y);
      wv.z = fmaf(k, o.z, wv.z);
      wv.w = fmaf(k, o.w, wv.w);
      store4<TW>(w, wr * cols + c0, wv);
    } else {
      const float t[4] = {o.x, o.y, o.z, o.w};
      for (int e = 0; e < 4 && c0 + e < cols; ++e) {
        const int64_t idx = wr * cols + c0 + e;
        store1<TW>(w, idx, fmaf(k, t[e], load1<TW>(w, idx)));
      }
    }
  }
}

template <typename TO>
__global__ __launch_bounds__(kThreads) void k_rowscale_apply(TO* O, int64_t rows, int64_t cols,
                                                             const float* rowscale) {
  const int b = blockIdx.z;
  TO* o = O + (int64_t)b * rows * cols;
  const float* rs = rowscale + (int64_t)b * rows;
  for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) {
    const float k = rs[r];
    for (int64_t j = (int64_t)blockIdx.x * kThreads + threadIdx.x; j < cols;
         j += (int64_t)gridDim.x * kThreads) {
      const int64_t idx = r * cols + j;
      store1<TO>(o, idx, k * load1<TO>(o, idx));
    }
  }
}

// ---- a8: Dion3 selection (Algorithm 4) ------------------------------------------------------

template <typename TG>
__global__ __launch_bounds__(kThreads) void k_momentum_l1(PtrPack Mp, PtrPack Gp, int64_t rows,
                                                          int64_t cols, float* l1) {
  __shared__ float sh[kThreads / 64];
  const int b = blockIdx.y;
  float* m = static_cast<float*>(Mp.p[b]);
  const TG* g = static_cast<const TG*>(Gp.p[b]);
  const bool vec_ok = (cols % 4) == 0;
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
    float acc = 0.f;
    if (vec_ok) {
      for (int64_t j = (int64_t)threadIdx.x * 4; j < cols; j += kThreads * 4) {
        float4 mv = load4<float>(m, r * cols + j);
        const float4 gv = load4<TG>(g, r * cols + j);
        mv.x += gv.x; mv.y += gv.y; mv.z += gv.z; mv.w += gv.w;
        store4<float>(m, r * cols + j, mv);
        acc += fabsf(mv.x) + fabsf(mv.y) + fabsf(mv.z) + fabsf(mv.w);
      }
    } else {
      for (int64_t j = threadIdx.x; j < cols; j += kThreads) {
        const float mv = m[r * cols + j] + load1<TG>(g, r * cols + j);
        m[r * cols + j] = mv;
        acc += fabsf(mv);
      }
    }
    const float s = block_sum<float, kThreads>(acc, sh);
    if (threadIdx.x == 0) l1[(int64_t)b * rows + r] = s;
  }
}

// rank_i = #{j : l1_j > l1_i or (l1_j == l1_i and j < i)}: a strict total order, so the k
// rows of rank < k are the top-k with ties resolved towards the lower index. A NaN norm is
// ordered below every number, which keeps the ranks a permutation (every S slot written).
constexpr int kTopkChunk = 4096;

__device__ __forceinline__ float topk_key(float x) { return isnan(x) ? -INFINITY : x; }

__global__ __launch_bounds__(kThreads) void k_topk(const float* l1, int64_t rows, int64_t k,
                                                   int32_t* S) {
  __shared__ float keys[kTopkChunk];
  const int b = blockIdx.y;
  const float* key = l1 + (int64_t)b * rows;
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const float ki = i < rows ? topk_key(key[i]) : 0.f;
  int64_t rank = 0;
  for (int64_t c0 = 0; c0 < rows; c0 += kTopkChunk) {
    const int64_t len = rows - c0 < kTopkChunk ? rows - c0 : kTopkChunk;
    __syncthreads();
    for (int64_t t = threadIdx.x; t < len; t += kThreads) keys[t] = topk_key(key[c0 + t]);
    __syncthreads();
    for (int64_t t = 0; t < len; ++t) {
      const float kj = keys[t];
      const int64_t j = c0 + t;
      rank += (kj > ki || (kj == ki && j < i)) ? 1 : 0;
    }
  }
  if (i < rows && rank < k) S[(int64_t)b * k + rank] = (int32_t)i;
}

__global__ __launch_bounds__(kThreads) void k_gather_decay(PtrPack Mp, int64_t cols, int64_t k,
                                                           const int32_t* S, float mu, float* Msel,
                                                           float* partials) {
  __shared__ float sh[kThreads / 64];
  const int b = blockIdx.y;
  float* m = static_cast<float*>(Mp.p[b]);
  for (int64_t p = blockIdx.x; p < k; p += gridDim.x) {
    const int64_t src = S[(int64_t)b * k + p];
    float* row = m + src * cols;
    float* dst = Msel + ((int64_t)b * k + p) * cols;
    float acc = 0.f;
    for (int64_t j = threadIdx.x; j < cols; j += kThreads) {
      const float v = row[j];
      dst[j] = v;
      row[j] = mu * v;
      acc += v * v;
    }
    const float s = block_sum<float, kThreads>(acc, sh);
    if (threadIdx.x == 0) partials[(int64_t)b * k + p] = s;
  }
}

inline hipError_t last() { return hipGetLastError(); }

inline unsigned grid_rows(int64_t rows) { return (unsigned)(rows < 65535 ? rows : 65535); }

}  // namespace

// ---------------------------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------------------------

int norm_blocks(int64_t elems) {
  const int64_t nvec = elems / 4;
  int64_t nb = (nvec + (int64_t)kThreads * kIter - 1) / ((int64_t)kThreads * kIter);
  return (int)(nb < 1 ? 1 : nb);
}

hipError_t momentum(const PtrPack& M, const PtrPack& G, Store g_store, int count, int64_t elems,
                    float mu, float* partials, hipStream_t s) {
  const int nblk = norm_blocks(elems);
  dim3 grid(nblk, count);
  if (g_store == Store::BF16)
    hipLaunchKernelGGL(k_momentum<uint16_t>, grid, dim3(kThreads), 0, s, M, G, elems, mu, partials, nblk);
  else
    hipLaunchKernelGGL(k_momentum<float>, grid, dim3(kThreads), 0, s, M, G, elems, mu, partials, nblk);
  return last();
}

hipError_t sumsq(const void* X, Store st, int count, int64_t elems, float* partials, hipStream_t s) {
  const int nblk = norm_blocks(elems);
  dim3 grid(nblk, count);
  if (st == Store::BF16)
    hipLaunchKernelGGL(k_sumsq<uint16_t>, grid, dim3(kThreads), 0, s,
                       static_cast<const uint16_t*>(X), elems, partials, nblk);
  else
    hipLaunchKernelGGL(k_sumsq<float>, grid, dim3(kThreads), 0, s, static_cast<const float*>(X),
                       elems, partials, nblk);
  return last();
}

hipError_t finalize_scale(const float* partials, int nblk, int count, float S, float* xscale,
                          hipStream_t s) {
  hipLaunchKernelGGL(k_finalize_scale, dim3(count), dim3(kThreads), 0, s, partials, nblk, S, xscale);
  return last();
}

template <typename TS, typename TX>
static void launch_normalize(const PtrPack* pack, const void* base, int count, int64_t rows,
                             int64_t cols, const float* xscale, void* S, void* T, int64_t rows_p,
                             int64_t cols_p, hipStream_t s) {
  PtrPack pk = {};
  if (pack) pk = *pack;
  dim3 grid((unsigned)(cols_p / 64), (unsigned)(rows_p / 64), count);
  hipLaunchKernelGGL((k_normalize<TS, TX>), grid, dim3(kThreads), 0, s, pk,
                     static_cast<const TS*>(base), rows, cols, xscale, static_cast<TX*>(S),
                     static_cast<TX*>(T), rows_p, cols_p);
}

hipError_t normalize(const PtrPack* pack, const void* base, bool src_f32, Store st, int count,
                     int64_t rows, int64_t cols, const float* xscale, Elem e, void* S, void* T,
                     int64_t rows_p, int64_t cols_p, hipStream_t s) {
  const bool f32src = src_f32 || st == Store::F32;
  if (e == Elem::F16) {
    if (f32src) launch_normalize<float, _Float16>(pack, base, count, rows, cols, xscale, S, T, rows_p, cols_p, s);
    else launch_normalize<uint16_t, _Float16>(pack, base, count, rows, cols, xscale, S, T, rows_p, cols_p, s);
  } else {
    if (f32src) launch_normalize<float, float>(pack, base, count, rows, cols, xscale, S, T, rows_p, cols_p, s);
    else launch_normalize<uint16_t, float>(pack, base, count, rows, cols, xscale, S, T, rows_p, cols_p, s);
  }
  return last();
}

template <typename TX, typename TO>
static void launch_export(const void* X, int64_t rows_p, int64_t cols_p, int count, int64_t rows,
                          int64_t cols, float inv_s, void* O, hipStream_t s) {
  dim3 grid((unsigned)((cols + 4 * kThreads - 1) / (4 * kThreads)), grid_rows(rows), count);
  hipLaunchKernelGGL((k_export<TX, TO>), grid, dim3(kThreads), 0, s, static_cast<const TX*>(X),
                     rows_p, cols_p, rows, cols, inv_s, static_cast<TO*>(O));
}

hipError_t export_output(const void* X, Elem e, int64_t rows_p, int64_t cols_p, int count,
                         int64_t rows, int64_t cols, float inv_s, void* O, Store st, hipStream_t s) {
  if (e == Elem::F16) {
    if (st == Store::BF16) launch_export<_Float16, uint16_t>(X, rows_p, cols_p, count, rows, cols, inv_s, O, s);
    else launch_export<_Float16, float>(X, rows_p, cols_p, count, rows, cols, inv_s, O, s);
  } else {
    if (st == Store::BF16) launch_export<float, uint16_t>(X, rows_p, cols_p, count, rows, cols, inv_s, O, s);
    else launch_export<float, float>(X, rows_p, cols_p, count, rows, cols, inv_s, O, s);
  }
  return last();
}

hipError_t row_sumsq_x(const void* X, Elem e, int64_t rows_p, int64_t cols_p, int count,
                       int64_t rows, int64_t cols, float* part, hipStream_t s) {
  (void)cols;
  dim3 grid((unsigned)(cols_p / 256), (unsigned)(rows_p / 256), count);
  if (e == Elem::F16)
    hipLaunchKernelGGL(k_row_sumsq_x<_Float16>, grid, dim3(kThreads), 0, s,
                       static_cast<const _Float16*>(X), rows_p, cols_p, rows, part);
  else
    hipLaunchKernelGGL(k_row_sumsq_x<float>, grid, dim3(kThreads), 0, s,
                       static_cast<const float*>(X), rows_p, cols_p, rows, part);
  return last();
}

hipError_t row_sumsq_stored(const void* O, Store st, int count, int64_t rows, int64_t cols,
                            float* part, hipStream_t s) {
  dim3 grid(grid_rows(rows), count);
  if (st == Store::BF16)
    hipLaunchKernelGGL(k_row_sumsq_stored<uint16_t>, grid, dim3(kThreads), 0, s,
                       static_cast<const uint16_t*>(O), rows, cols, part);
  else
    hipLaunchKernelGGL(k_row_sumsq_stored<float>, grid, dim3(kThreads), 0, s,
                       static_cast<const float*>(O), rows, cols, part);
  return last();
}

hipError_t normuon_finalize(const float* part, int chunks, int count, int64_t rows, int64_t cols,
                            const PtrPack* v_pack, float* v_base, int64_t v_stride,
                            const int32_t* rowidx, float beta2, float eps, float inv_s2,
                            float out_scale, float* rowscale, hipStream_t s) {
  PtrPack vp = {};
  if (v_pack) vp = *v_pack;
  hipLaunchKernelGGL(k_normuon_finalize, dim3(count), dim3(kFinThreads), 0, s, part, chunks, rows,
                     cols, vp, v_base, v_stride, rowidx, beta2, eps, inv_s2, out_scale, rowscale);
  return last();
}

hipError_t fill(float* p, int64_t n, float value, hipStream_t s) {
  int64_t blocks = (n + kThreads - 1) / kThreads;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(k_fill, dim3((unsigned)blocks), dim3(kThreads), 0, s, p, n, value);
  return last();
}

template <typename TW, typename TX>
static void launch_wupdate(const PtrPack& W, int count, int64_t rows, int64_t cols, const void* X,
                           int64_t rows_p, int64_t cols_p, const float* rowscale,
                           const int32_t* rowidx, int64_t rowidx_stride, float lr, hipStream_t s) {
  dim3 grid((unsigned)((cols + 4 * kThreads - 1) / (4 * kThreads)), grid_rows(rows), count);
  hipLaunchKernelGGL((k_wupdate<TW, TX>), grid, dim3(kThreads), 0, s, W, rows, cols,
                     static_cast<const TX*>(X), rows_p, cols_p, rowscale, rowidx, rowidx_stride, lr);
}

hipError_t weight_update(const PtrPack& W, Store st, int count, int64_t rows, int64_t cols,
                         const void* X, Elem e, int64_t rows_p, int64_t cols_p,
                         const float* rowscale, const int32_t* rowidx, int64_t rowidx_stride,
                         float lr, hipStream_t s) {
  if (e == Elem::F16) {
    if (st == Store::BF16) launch_wupdate<uint16_t, _Float16>(W, count, rows, cols, X, rows_p, cols_p, rowscale, rowidx, rowidx_stride, lr, s);
    else launch_wupdate<float, _Float16>(W, count, rows, cols, X, rows_p, cols_p, rowscale, rowidx, rowidx_stride, lr, s);
  } else {
    if (st == Store::BF16) launch_wupdate<uint16_t, float>(W, count, rows, cols, X, rows_p, cols_p, rowscale, rowidx, rowidx_stride, lr, s);
    else launch_wupdate<float, float>(W, count, rows, cols, X, rows_p, cols_p, rowscale, rowidx, rowidx_stride, lr, s);
  }
  return last();
}

hipError_t rowscale_apply(void* O, Store st, int count, int64_t rows, int64_t cols,
                          const float* rowscale, hipStream_t s) {
  dim3 grid((unsigned)((cols + kThreads - 1) / kThreads < 64 ? (cols + kThreads - 1) / kThreads : 64),
            grid_rows(rows), count);
  if (st == Store::BF16)
    hipLaunchKernelGGL(k_rowscale_apply<uint16_t>, grid, dim3(kThreads), 0, s,
                       static_cast<uint16_t*>(O), rows, cols, rowscale);
  else
    hipLaunchKernelGGL(k_rowscale_apply<float>, grid, dim3(kThreads), 0, s, static_cast<float*>(O),
                       rows, cols, rowscale);
  return last();
}

hipError_t momentum_l1(const PtrPack& M, const PtrPack& G, Store g_store, int count, int64_t rows,
                       int64_t cols, float* l1, hipStream_t s) {
  dim3 grid(grid_rows(rows), count);
  if (g_store == Store::BF16)
    hipLaunchKernelGGL(k_momentum_l1<uint16_t>, grid, dim3(kThreads), 0, s, M, G, rows, cols, l1);
  else
    hipLaunchKernelGGL(k_momentum_l1<float>, grid, dim3(kThreads), 0, s, M, G, rows, cols, l1);
  return last();
}

hipError_t topk_rows(const float* l1, int count, int64_t rows, int64_t k, int32_t* S, hipStream_t s) {
  dim3 grid((unsigned)((rows + kThreads - 1) / kThreads), count);
  hipLaunchKernelGGL(k_topk, grid, dim3(kThreads), 0, s, l1, rows, k, S);
  return last();
}

hipError_t gather_decay(const PtrPack& M, int count, int64_t cols, int64_t k, const int32_t* S,
                        float mu, float* Msel, float* partials, hipStream_t s) {
  dim3 grid(grid_rows(k), count);
  hipLaunchKernelGGL(k_gather_decay, grid, dim3(kThreads), 0, s, M, cols, k, S, mu, Msel, partials);
  return last();
}

}  // namespace mns
