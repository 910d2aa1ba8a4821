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

// 8 consecutive elements (16 bytes of bfloat16/float16, 32 of float32) as two float4.
struct f8 {
  float4 lo, hi;
};
template <typename TS>
__device__ __forceinline__ f8 load8(const TS* p, int64_t i) {
  return {load4<TS>(p, i), load4<TS>(p, i + 4)};
}
template <>
__device__ __forceinline__ f8 load8<uint16_t>(const uint16_t* p, int64_t i) {
  const uint4 v = *reinterpret_cast<const uint4*>(p + i);
  return {make_float4(bf16_to_f32(v.x & 0xFFFFu), bf16_to_f32(v.x >> 16), bf16_to_f32(v.y & 0xFFFFu),
                      bf16_to_f32(v.y >> 16)),
          make_float4(bf16_to_f32(v.z & 0xFFFFu), bf16_to_f32(v.z >> 16), bf16_to_f32(v.w & 0xFFFFu),
                      bf16_to_f32(v.w >> 16))};
}
template <>
__device__ __forceinline__ f8 load8<_Float16>(const _Float16* p, int64_t i) {
  typedef _Float16 h8 __attribute__((ext_vector_type(8)));
  const h8 v = *reinterpret_cast<const h8*>(p + i);
  return {make_float4((float)v[0], (float)v[1], (float)v[2], (float)v[3]),
          make_float4((float)v[4], (float)v[5], (float)v[6], (float)v[7])};
}

template <typename TS>
__device__ __forceinline__ void store8(TS* p, int64_t i, const f8& v) {
  store4<TS>(p, i, v.lo);
  store4<TS>(p, i + 4, v.hi);
}
template <>
__device__ __forceinline__ void store8<uint16_t>(uint16_t* p, int64_t i, const f8& v) {
  uint4 o;
  o.x = f32_to_bf16(v.lo.x) | (f32_to_bf16(v.lo.y) << 16);
  o.y = f32_to_bf16(v.lo.z) | (f32_to_bf16(v.lo.w) << 16);
  o.z = f32_to_bf16(v.hi.x) | (f32_to_bf16(v.hi.y) << 16);
  o.w = f32_to_bf16(v.hi.z) | (f32_to_bf16(v.hi.w) << 16);
  *reinterpret_cast<uint4*>(p + i) = o;
}
template <>
__device__ __forceinline__ void store8<_Float16>(_Float16* p, int64_t i, const f8& v) {
  typedef _Float16 h8 __attribute__((ext_vector_type(8)));
  const h8 o = {(_Float16)v.lo.x, (_Float16)v.lo.y, (_Float16)v.lo.z, (_Float16)v.lo.w,
                (_Float16)v.hi.x, (_Float16)v.hi.y, (_Float16)v.hi.z, (_Float16)v.hi.w};
  *reinterpret_cast<h8*>(p + i) = o;
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

// Sum of the squares of four float32 values, squared and added in float64.
__device__ __forceinline__ double sq4(const float4& v) {
  const double x = v.x, y = v.y, z = v.z, w = v.w;
  return x * x + y * y + z * z + w * w;
}

// ---- a1: momentum M <- mu M + G, partial sums of M^2 (Eq. 1) --------------------------------
// The squares are summed in float64: ||M||_F stays exact in range for any float32 M (squares
// of |M| < 1e-19 underflow in float32, of |M| > 2e19 overflow), and the method is scale-free.

template <typename TG>
__global__ __launch_bounds__(kThreads) void k_momentum(PtrPack Mp, PtrPack Gp, int64_t elems,
                                                       float mu, double* partials, int nblk) {
  __shared__ double sh[kThreads / 64];
  const int b = blockIdx.y;
  float* m = static_cast<float*>(Mp.p[b]);
  const TG* g = static_cast<const TG*>(Gp.p[b]);
  const int64_t nvec = elems / 4;
  double acc = 0.0;
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
      acc += sq4(mv);
    }
  }
  if (blockIdx.x == gridDim.x - 1 && threadIdx.x < 4) {
    const int64_t e = nvec * 4 + threadIdx.x;
    if (e < elems) {
      const float mv = fmaf(mu, m[e], load1<TG>(g, e));
      m[e] = mv;
      acc += (double)mv * (double)mv;
    }
  }
  const double s = block_sum<double, kThreads>(acc, sh);
  if (threadIdx.x == 0) partials[(int64_t)b * nblk + blockIdx.x] = s;
}

// ---- partial sums of X^2 for a stored matrix (X / ||X||_F of standard NS) ------------------

template <typename TX>
__global__ __launch_bounds__(kThreads) void k_sumsq(const TX* X, int64_t elems, double* partials,
                                                    int nblk) {
  __shared__ double sh[kThreads / 64];
  const int b = blockIdx.y;
  const TX* x = X + (int64_t)b * elems;
  const int64_t nvec = elems / 4;
  double acc = 0.0;
  // Every load first, unguarded (a vector past the end re-reads the last one), then the sums
  // in the same order as before: a load guarded by its own test, with its use in the same
  // block, made each load wait for the one before.
  if (nvec > 0) {
    float4 xv[kIter];
#pragma unroll
    for (int it = 0; it < kIter; ++it) {
      const int64_t v = ((int64_t)blockIdx.x * kIter + it) * kThreads + threadIdx.x;
      xv[it] = load4<TX>(x, 4 * (v < nvec ? v : nvec - 1));
    }
#pragma unroll
    for (int it = 0; it < kIter; ++it) {
      const int64_t v = ((int64_t)blockIdx.x * kIter + it) * kThreads + threadIdx.x;
      if (v < nvec) acc += sq4(xv[it]);
    }
  }
  if (blockIdx.x == gridDim.x - 1 && threadIdx.x < 4) {
    const int64_t e = nvec * 4 + threadIdx.x;
    if (e < elems) {
      const float xv = load1<TX>(x, e);
      acc += (double)xv * (double)xv;
    }
  }
  const double s = block_sum<double, kThreads>(acc, sh);
  if (threadIdx.x == 0) partials[(int64_t)b * nblk + blockIdx.x] = s;
}

// ---- a2: 1/||M||_F (times the iterate's storage scale) ----------------------------------------

__global__ __launch_bounds__(kThreads) void k_finalize_scale(const double* partials, int nblk,
                                                             float S, float* xscale) {
  __shared__ double sh[kThreads / 64];
  const int b = blockIdx.x;
  double acc = 0.0;
  // unrolled so several loads are in flight; the additions keep their order
#pragma unroll 8
  for (int i = threadIdx.x; i < nblk; i += kThreads) acc += partials[(int64_t)b * nblk + i];
  const double s = block_sum<double, kThreads>(acc, sh);
  if (threadIdx.x == 0) xscale[b] = s > 0.0 ? (float)((double)S / sqrt(s)) : 0.f;
}

// ---- a2: X_0 = scale * M, in both layouts, zero padded -------------------------------------

// One block per 64 x 128 tile of the padded source: each thread scales 8 consecutive
// columns of 4 rows and stores them to S as 16-byte chunks; the tile passes through LDS
// (float32, padded rows: conflict-free column reads) and leaves transposed to T, again as
// 16-byte chunks of 8 elements.
constexpr int kNormRows = 64, kNormCols = 128;

// GATHER (Dion3, Algorithm 4): row r of the iterate is source row rowidx[b][r] of the float32
// momentum, which is also decayed in place (M[S,:] <- mu M[S,:]) from the values just read.
template <typename TS, typename TX, bool GATHER>
__global__ __launch_bounds__(kThreads) void k_normalize(PtrPack src, const TS* base, int64_t rows,
                                                        int64_t cols, const float* xscale, TX* S,
                                                        TX* T, int64_t rows_p, int64_t cols_p,
                                                        const int32_t* rowidx, float mu) {
  __shared__ float tile[kNormRows][kNormCols + 1];
  const int b = blockIdx.z;
  const TS* s = base ? base + (int64_t)b * rows * cols : static_cast<const TS*>(src.p[b]);
  const int64_t lds = padded_ld(cols_p), ldt = padded_ld(rows_p);
  TX* so = S + (int64_t)b * rows_p * lds;
  TX* to = T + (int64_t)b * cols_p * ldt;
  const float sc = xscale[b];
  const int64_t r0 = (int64_t)blockIdx.y * kNormRows, c0 = (int64_t)blockIdx.x * kNormCols;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;   // 16 x 8 columns, 16 rows per pass
  const int64_t c = c0 + 8 * tx;
  const bool vec_ok = (cols % 8) == 0;
  // Source offsets, then every load, then the decayed rows (as in k_normalize_rows: a load
  // after a store to the same array would wait for it).
  constexpr int NV = kNormRows / 16;
  const bool full = vec_ok && c + 8 <= cols;
  f8 v[NV];
  int64_t soff[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int64_t r = r0 + ty + 16 * i;
    soff[i] = r < rows ? (GATHER ? (int64_t)rowidx[(int64_t)b * rows + r] : r) * cols + c : -1;
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    v[i] = {make_float4(0.f, 0.f, 0.f, 0.f), make_float4(0.f, 0.f, 0.f, 0.f)};
    if (soff[i] < 0) continue;
    if (full) {
      v[i] = load8<TS>(s, soff[i]);
    } else {
      float t8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) t8[e] = (c + e < cols) ? load1<TS>(s, soff[i] + e) : 0.f;
      v[i] = {make_float4(t8[0], t8[1], t8[2], t8[3]), make_float4(t8[4], t8[5], t8[6], t8[7])};
    }
  }
  if constexpr (GATHER) {
    // M[S,:] <- mu M[S,:]
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      if (soff[i] < 0) continue;
      const f8 w = v[i];
      if (full) {
        store8<float>(const_cast<float*>(s), soff[i],
                      {make_float4(mu * w.lo.x, mu * w.lo.y, mu * w.lo.z, mu * w.lo.w),
                       make_float4(mu * w.hi.x, mu * w.hi.y, mu * w.hi.z, mu * w.hi.w)});
      } else {
        const float t8[8] = {w.lo.x, w.lo.y, w.lo.z, w.lo.w, w.hi.x, w.hi.y, w.hi.z, w.hi.w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (c + e < cols) const_cast<float*>(s)[soff[i] + e] = mu * t8[e];
      }
    }
  }
#pragma unroll
  for (int i = 0; i < kNormRows / 16; ++i) {
    const int lr = ty + 16 * i;
    f8 w = v[i];
    w.lo.x *= sc; w.lo.y *= sc; w.lo.z *= sc; w.lo.w *= sc;
    w.hi.x *= sc; w.hi.y *= sc; w.hi.z *= sc; w.hi.w *= sc;
    if (S) store8<TX>(so, (r0 + lr) * lds + c, w);
    float* t = &tile[lr][8 * tx];
    t[0] = w.lo.x; t[1] = w.lo.y; t[2] = w.lo.z; t[3] = w.lo.w;
    t[4] = w.hi.x; t[5] = w.hi.y; t[6] = w.hi.z; t[7] = w.hi.w;
  }
  if (!T) return;   // only the straight layout wanted (the same for every thread)
  __syncthreads();
  // T rows c0 .. c0+kNormCols-1, kNormRows elements (chunks of 8) each
  constexpr int CPT = kNormRows / 8;
#pragma unroll
  for (int i = 0; i < kNormCols * kNormRows / 8 / kThreads; ++i) {
    const int q = threadIdx.x + kThreads * i;
    const int lc = q / CPT, ch = q % CPT;
    f8 w;
    w.lo = make_float4(tile[8 * ch + 0][lc], tile[8 * ch + 1][lc], tile[8 * ch + 2][lc],
                       tile[8 * ch + 3][lc]);
    w.hi = make_float4(tile[8 * ch + 4][lc], tile[8 * ch + 5][lc], tile[8 * ch + 6][lc],
                       tile[8 * ch + 7][lc]);
    store8<TX>(to, (c0 + lc) * ldt + r0 + 8 * ch, w);
  }
}

// The straight layout alone (no transposed copy wanted: the products read X as stored): a
// streaming pass, one thread per two 8-element vectors of the padded iterate (block-strided,
// so a wave's loads and stores are contiguous), with non-temporal loads of the source and
// stores of the iterate: each is touched once here, and the cache hints keep the stream from
// displacing other lines (on this part the float32 -> float16 mix runs ~20 % faster so).
typedef float f4v __attribute__((ext_vector_type(4)));
typedef unsigned int u4v __attribute__((ext_vector_type(4)));

template <typename TS>
__device__ __forceinline__ f8 load8_nt(const TS* p, int64_t i);
template <>
__device__ __forceinline__ f8 load8_nt<float>(const float* p, int64_t i) {
  const f4v a = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(p + i));
  const f4v b = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(p + i + 4));
  return {make_float4(a.x, a.y, a.z, a.w), make_float4(b.x, b.y, b.z, b.w)};
}
template <>
__device__ __forceinline__ f8 load8_nt<uint16_t>(const uint16_t* p, int64_t i) {
  const u4v v = __builtin_nontemporal_load(reinterpret_cast<const u4v*>(p + i));
  return {make_float4(bf16_to_f32(v.x & 0xFFFFu), bf16_to_f32(v.x >> 16), bf16_to_f32(v.y & 0xFFFFu),
                      bf16_to_f32(v.y >> 16)),
          make_float4(bf16_to_f32(v.z & 0xFFFFu), bf16_to_f32(v.z >> 16), bf16_to_f32(v.w & 0xFFFFu),
                      bf16_to_f32(v.w >> 16))};
}

template <typename TX>
__device__ __forceinline__ void store8_nt(TX* p, int64_t i, const f8& v);
template <>
__device__ __forceinline__ void store8_nt<_Float16>(_Float16* p, int64_t i, const f8& v) {
  typedef _Float16 h8 __attribute__((ext_vector_type(8)));
  const h8 o = {(_Float16)v.lo.x, (_Float16)v.lo.y, (_Float16)v.lo.z, (_Float16)v.lo.w,
                (_Float16)v.hi.x, (_Float16)v.hi.y, (_Float16)v.hi.z, (_Float16)v.hi.w};
  __builtin_nontemporal_store(o, reinterpret_cast<h8*>(p + i));
}
template <>
__device__ __forceinline__ void store8_nt<float>(float* p, int64_t i, const f8& v) {
  const f4v a = {v.lo.x, v.lo.y, v.lo.z, v.lo.w}, b = {v.hi.x, v.hi.y, v.hi.z, v.hi.w};
  __builtin_nontemporal_store(a, reinterpret_cast<f4v*>(p + i));
  __builtin_nontemporal_store(b, reinterpret_cast<f4v*>(p + i + 4));
}

constexpr int kRowIter = 2;   // 8-element vectors per thread

template <typename TS, typename TX, bool GATHER>
__global__ __launch_bounds__(kThreads) void k_normalize_rows(PtrPack src, const TS* base,
                                                             int64_t rows, int64_t cols,
                                                             const float* xscale, TX* S,
                                                             int64_t rows_p, int64_t cols_p,
                                                             const int32_t* rowidx, float mu) {
  const int b = blockIdx.y;
  const TS* s = base ? base + (int64_t)b * rows * cols : static_cast<const TS*>(src.p[b]);
  const int64_t lds = padded_ld(cols_p);
  TX* so = S + (int64_t)b * rows_p * lds;
  const float sc = xscale[b];
  const int64_t vpr = cols_p / 8;                  // vectors per padded row
  const int64_t nvec = rows_p * vpr;
  const bool vec_ok = (cols % 8) == 0;
  const int64_t v0 = (int64_t)blockIdx.x * kThreads * kRowIter + threadIdx.x;
  // Source offsets first (with a row index, all of the thread's index loads go out together),
  // then every load, and only then the decayed rows written back: a load placed after a store
  // to the same array would wait for that store, one latency per vector.
  f8 v[kRowIter];
  int64_t dst[kRowIter], soff[kRowIter];
#pragma unroll
  for (int it = 0; it < kRowIter; ++it) {
    const int64_t vi = v0 + (int64_t)it * kThreads;
    dst[it] = -1;
    soff[it] = -1;
    if (vi < nvec) {
      const int64_t r = vi / vpr, c = 8 * (vi % vpr);
      dst[it] = r * lds + c;
      if (r < rows && c < cols)
        soff[it] = (GATHER ? (int64_t)rowidx[(int64_t)b * rows + r] : r) * cols + c;
    }
  }
#pragma unroll
  for (int it = 0; it < kRowIter; ++it) {
    v[it] = {make_float4(0.f, 0.f, 0.f, 0.f), make_float4(0.f, 0.f, 0.f, 0.f)};
    if (soff[it] < 0) continue;
    if (vec_ok) {
      v[it] = load8_nt<TS>(s, soff[it]);
    } else {
      const int64_t c = 8 * ((v0 + (int64_t)it * kThreads) % vpr);
      float t8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) t8[e] = (c + e < cols) ? load1<TS>(s, soff[it] + e) : 0.f;
      v[it] = {make_float4(t8[0], t8[1], t8[2], t8[3]), make_float4(t8[4], t8[5], t8[6], t8[7])};
    }
  }
  if constexpr (GATHER) {
    // M[S,:] <- mu M[S,:] (the selected rows' decay)
#pragma unroll
    for (int it = 0; it < kRowIter; ++it) {
      if (soff[it] < 0) continue;
      const f8 w = v[it];
      if (vec_ok) {
        store8<float>(const_cast<float*>(s), soff[it],
                      {make_float4(mu * w.lo.x, mu * w.lo.y, mu * w.lo.z, mu * w.lo.w),
                       make_float4(mu * w.hi.x, mu * w.hi.y, mu * w.hi.z, mu * w.hi.w)});
      } else {
        const int64_t c = 8 * ((v0 + (int64_t)it * kThreads) % vpr);
        const float t8[8] = {w.lo.x, w.lo.y, w.lo.z, w.lo.w, w.hi.x, w.hi.y, w.hi.z, w.hi.w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (c + e < cols) const_cast<float*>(s)[soff[it] + e] = mu * t8[e];
      }
    }
  }
#pragma unroll
  for (int it = 0; it < kRowIter; ++it) {
    if (dst[it] < 0) continue;
    f8 w = v[it];
    w.lo.x *= sc; w.lo.y *= sc; w.lo.z *= sc; w.lo.w *= sc;
    w.hi.x *= sc; w.hi.y *= sc; w.hi.z *= sc; w.hi.w *= sc;
    store8_nt<TX>(so, dst[it], w);
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

// ---- NorMuon statistics of a caller matrix (normuon_scale): per row, the sum of O^2 --------

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

// Stage 1, 64 rows per block of four waves: r_i = inv_s2 * sum over chunks of part, the v
// update, d_i = 1/(sqrt(v_i) + eps) into rowscale, and per block the float64 sums of r_i and
// r_i d_i^2 (the squared norms of O and of O-hat) into fin[b][0 / 1][block]. Wave q sums the
// chunks c = q (mod 4) of its lane's row in increasing order (the chunks past the last whole
// group of four go to wave 0), each load 64 consecutive rows of one chunk, and the row sum is
// (s0 + s1) + (s2 + s3): a fixed order, the same additions as one thread keeping four partial
// sums.
constexpr int kRowsPerBlock = 64;

__global__ __launch_bounds__(kThreads) void k_normuon_rows(
    const float* part, int chunks, int64_t rows, int64_t cols, PtrPack vp, float* v_base,
    int64_t v_stride, const int32_t* rowidx, float beta2, float eps, float inv_s2,
    float* rowscale, double* fin) {
  static_assert(kThreads == 4 * kRowsPerBlock, "four waves of 64 rows");
  __shared__ float part_sh[4][kRowsPerBlock];
  __shared__ double sh[kThreads / 64];
  const int b = blockIdx.y, nblk = gridDim.x;
  const int q = threadIdx.x / kRowsPerBlock, lane = threadIdx.x % kRowsPerBlock;
  const int64_t i = (int64_t)blockIdx.x * kRowsPerBlock + lane;
  const bool live = i < rows;
  float acc = 0.f;
  if (live) {
    const float* pt = part + (int64_t)b * chunks * rows + i;
    const int full = chunks - chunks % 4;
#pragma unroll 8
    for (int c = q; c < full; c += 4) acc += pt[(int64_t)c * rows];
    if (q == 0)
      for (int c = full; c < chunks; ++c) acc += pt[(int64_t)c * rows];
  }
  part_sh[q][lane] = acc;
  __syncthreads();
  double s_o = 0.0, s_h = 0.0;
  if (live && q == 0) {
    float* v = v_base ? v_base + (int64_t)b * v_stride : static_cast<float*>(vp.p[b]);
    const float r = ((part_sh[0][lane] + part_sh[1][lane]) + (part_sh[2][lane] + part_sh[3][lane])) * inv_s2;
    const int64_t vi = rowidx ? (int64_t)rowidx[(int64_t)b * rows + i] : i;
    const float vn = fmaf(beta2, v[vi], (1.0f - beta2) * (r * (1.0f / (float)cols)));
    v[vi] = vn;
    const float d = 1.0f / (sqrtf(vn) + eps);
    rowscale[(int64_t)b * rows + i] = d;
    s_o = (double)r;
    s_h = (double)r * (double)d * (double)d;
  }
  const double to = block_sum<double, kThreads>(s_o, sh);
  const double th = block_sum<double, kThreads>(s_h, sh);
  if (threadIdx.x == 0) {
    fin[((int64_t)b * 2 + 0) * nblk + blockIdx.x] = to;
    fin[((int64_t)b * 2 + 1) * nblk + blockIdx.x] = th;
  }
}

// Stage 2, one block per matrix: ratio = sqrt(sum r / sum r d^2) = ||O|| / ||O-hat|| from the
// block sums (0 for a zero matrix), and rowscale_i = ratio * d_i * out_scale.
__global__ __launch_bounds__(kThreads) void k_normuon_ratio(const double* fin, int nblk,
                                                            int64_t rows, float out_scale,
                                                            float* rowscale) {
  __shared__ double sh[kThreads / 64];
  __shared__ float scale_sh;
  const int b = blockIdx.x;
  double s_o = 0.0, s_h = 0.0;
#pragma unroll 4
  for (int k = threadIdx.x; k < nblk; k += kThreads) {
    s_o += fin[((int64_t)b * 2 + 0) * nblk + k];
    s_h += fin[((int64_t)b * 2 + 1) * nblk + k];
  }
  const double to = block_sum<double, kThreads>(s_o, sh);
  const double th = block_sum<double, kThreads>(s_h, sh);
  if (threadIdx.x == 0) scale_sh = (th > 0.0 ? (float)sqrt(to / th) : 0.f) * out_scale;
  __syncthreads();
  const float scale = scale_sh;
  float* rs = rowscale + (int64_t)b * rows;
#pragma unroll 4
  for (int64_t i = threadIdx.x; i < rows; i += kThreads) rs[i] = rs[i] * scale;
}

// Cache flush for timings: zeros written over a large scratch buffer with 16-byte stores.
__global__ __launch_bounds__(kThreads) void k_flush(uint4* p, int64_t n16) {
  const uint4 z = make_uint4(0u, 0u, 0u, 0u);
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n16;
       i += (int64_t)gridDim.x * kThreads)
    p[i] = z;
}

__global__ __launch_bounds__(kThreads) void k_fill(float* p, int64_t n, float value) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * kThreads)
    p[i] = value;
}

// ---- a7: fused weight update W <- W - lr * rowscale_i * O_ij, one rounding ------------------

// Each thread updates 8 consecutive columns of kWuRows rows (all loads issued first); one row
// per thread, one block row per matrix row, measured fastest (a one-shot grid).
constexpr int kWuRows = 1;

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
  const int64_t c0 = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * 8;
  if (c0 >= cols) return;
  const bool vec_ok = (cols % 8) == 0;
  for (int64_t p0 = (int64_t)blockIdx.y * kWuRows; p0 < rows; p0 += (int64_t)gridDim.y * kWuRows) {
    if (vec_ok && p0 + kWuRows <= rows) {
      f8 o[kWuRows], wv[kWuRows];
      int64_t wr[kWuRows];
#pragma unroll
      for (int q = 0; q < kWuRows; ++q) {
        wr[q] = ri ? (int64_t)ri[p0 + q] : p0 + q;
        o[q] = load8<TX>(x, (p0 + q) * ldx + c0);
        wv[q] = load8<TW>(w, wr[q] * cols + c0);
      }
#pragma unroll
      for (int q = 0; q < kWuRows; ++q) {
        const float k = -lr * rs[p0 + q];
        wv[q].lo.x = fmaf(k, o[q].lo.x, wv[q].lo.x);
        wv[q].lo.y = fmaf(k, o[q].lo.y, wv[q].lo.y);
        wv[q].lo.z = fmaf(k, o[q].lo.z, wv[q].lo.z);
        wv[q].lo.w = fmaf(k, o[q].lo.w, wv[q].lo.w);
        wv[q].hi.x = fmaf(k, o[q].hi.x, wv[q].hi.x);
        wv[q].hi.y = fmaf(k, o[q].hi.y, wv[q].hi.y);
        wv[q].hi.z = fmaf(k, o[q].hi.z, wv[q].hi.z);
        wv[q].hi.w = fmaf(k, o[q].hi.w, wv[q].hi.w);
        store8<TW>(w, wr[q] * cols + c0, wv[q]);
      }
    } else {
      for (int64_t p = p0; p < rows && p < p0 + kWuRows; ++p) {
        const int64_t r = ri ? (int64_t)ri[p] : p;
        const float k = -lr * rs[p];
        for (int e = 0; e < 8 && c0 + e < cols; ++e) {
          const int64_t idx = r * cols + c0 + e;
          store1<TW>(w, idx, fmaf(k, load1<TX>(x, p * ldx + c0 + e), load1<TW>(w, idx)));
        }
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
                                                          int64_t cols, float* l1, double* l2sq) {
  __shared__ float sh[kThreads / 64];
  __shared__ double dsh[kThreads / 64];
  const int b = blockIdx.y;
  float* m = static_cast<float*>(Mp.p[b]);
  const TG* g = static_cast<const TG*>(Gp.p[b]);
  const bool vec_ok = (cols % 4) == 0;
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
    float acc = 0.f;
    double acc2 = 0.0;   // float64 squares, as in k_momentum
    if (vec_ok) {
      for (int64_t j = (int64_t)threadIdx.x * 4; j < cols; j += kThreads * 4) {
        float4 mv = load4<float>(m, r * cols + j);
        const float4 gv = load4<TG>(g, r * cols + j);
        mv.x += gv.x; mv.y += gv.y; mv.z += gv.z; mv.w += gv.w;
        store4<float>(m, r * cols + j, mv);
        acc += fabsf(mv.x) + fabsf(mv.y) + fabsf(mv.z) + fabsf(mv.w);
        acc2 += sq4(mv);
      }
    } else {
      for (int64_t j = threadIdx.x; j < cols; j += kThreads) {
        const float mv = m[r * cols + j] + load1<TG>(g, r * cols + j);
        m[r * cols + j] = mv;
        acc += fabsf(mv);
        acc2 += (double)mv * (double)mv;
      }
    }
    const float s = block_sum<float, kThreads>(acc, sh);
    const double s2 = block_sum<double, kThreads>(acc2, dsh);
    if (threadIdx.x == 0) {
      l1[(int64_t)b * rows + r] = s;
      l2sq[(int64_t)b * rows + r] = s2;
    }
  }
}

// Top-k rows by l1 norm, ties towards the lower index, by radix selection on an order-
// preserving 32-bit key (one block per matrix): four 8-bit digit passes find the k-th
// largest key K and how many rows equal to K still belong to the top k; a compaction then
// writes the selected rows in ascending index order. A NaN norm is ordered below every
// number. Integer counts only, so the selection is exact and reproducible.
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;

__device__ __forceinline__ uint32_t order_key(float x) {
  if (isnan(x)) x = -INFINITY;
  if (x == 0.f) x = 0.f;                       // -0 and +0 are one value
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum over the block (kSelThreads values), deterministic.
__device__ int block_exclusive_scan(int v, int* sh) {
  // integer sums are exact, so the result does not depend on the order of the additions:
  // a shuffle scan inside each wave, then one over the wave totals
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh[w] = x;
  __syncthreads();
  if (w == 0) {
    const int tot = lane < kSelWaves ? sh[lane] : 0;
    int y = tot;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int z = __shfl_up(y, o, 64);
      if (lane >= o) y += z;
    }
    if (lane < kSelWaves) sh[64 + lane] = y - tot;
  }
  __syncthreads();
  const int res = x - v + sh[64 + w];
  __syncthreads();
  return res;
}

// Thread t owns the contiguous rows [t * per, t * per + per) in every pass. When they are at
// most kSelCache, their keys are read once into registers; otherwise each pass reads them in
// chunks of kSelCache independent loads. Either way a pass waits for one load latency per
// chunk instead of one per row, and the counts (so the selection) do not depend on which.
constexpr int kSelCache = 8;

__global__ __launch_bounds__(kSelThreads) void k_topk(const float* l1, const double* l2sq,
                                                      int64_t rows, int64_t k, int32_t* S,
                                                      float Spow, float* xscale) {
  __shared__ uint32_t hist[kSelWaves][256];
  __shared__ double dsh[kSelWaves];
  __shared__ int scan_sh[kSelThreads];
  __shared__ uint32_t sh_prefix;
  __shared__ int64_t sh_remaining;
  const int b = blockIdx.x, t = threadIdx.x, wave = t >> 6;
  const float* key = l1 + (int64_t)b * rows;
  const int64_t per = (rows + kSelThreads - 1) / kSelThreads;
  const int64_t i0 = (int64_t)t * per < rows ? (int64_t)t * per : rows;
  const int64_t i1 = i0 + per < rows ? i0 + per : rows;
  const bool cached = per <= kSelCache;
  // The loads are unguarded (an index past the thread's rows is clamped to the last row, and
  // its key set to 0 after the load): a load guarded by its own test, with its use in the same
  // block, waited for the one before.
  uint32_t kc[kSelCache];
  {
    float kf[kSelCache];
#pragma unroll
    for (int j = 0; j < kSelCache; ++j) kf[j] = key[i0 + j < rows ? i0 + j : rows - 1];
#pragma unroll
    for (int j = 0; j < kSelCache; ++j) {
      const uint32_t o = order_key(kf[j]);
      kc[j] = (cached && i0 + j < i1) ? o : 0u;
    }
  }
  // f(row, key) over this thread's rows in ascending row order
  auto for_keys = [&](auto&& f) {
    if (cached) {
#pragma unroll
      for (int j = 0; j < kSelCache; ++j)
        if (i0 + j < i1) f(i0 + j, kc[j]);
    } else {
      for (int64_t c = i0; c < i1; c += kSelCache) {
        float uf[kSelCache];
        uint32_t u[kSelCache];
#pragma unroll
        for (int j = 0; j < kSelCache; ++j) uf[j] = key[c + j < i1 ? c + j : i1 - 1];
#pragma unroll
        for (int j = 0; j < kSelCache; ++j) u[j] = order_key(uf[j]);
#pragma unroll
        for (int j = 0; j < kSelCache; ++j)
          if (c + j < i1) f(c + j, u[j]);
      }
    }
  };

  uint32_t prefix = 0, mask = 0;
  int64_t remaining = k;   // rows still to take among those whose key matches prefix on mask
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = t; i < kSelWaves * 256; i += kSelThreads) (&hist[0][0])[i] = 0u;
    __syncthreads();
    for_keys([&](int64_t, uint32_t u) {
      if ((u & mask) == prefix) atomicAdd(&hist[wave][(u >> shift) & 255u], 1u);
    });
    __syncthreads();
    if (t < 256) {
      uint32_t c = 0;
      for (int w = 0; w < kSelWaves; ++w) c += hist[w][t];
      hist[0][t] = c;
    }
    __syncthreads();
    // The digit of the k-th largest key: with digits in descending order (thread t holds
    // digit 255 - t), `above` counts the keys with a larger digit; exactly one digit has
    // above < remaining <= above + count.
    {
      const int cnt = t < 256 ? (int)hist[0][255 - t] : 0;
      const int above = block_exclusive_scan(cnt, scan_sh);
      if (t < 256 && (int64_t)above < remaining && (int64_t)above + cnt >= remaining) {
        sh_prefix = prefix | ((uint32_t)(255 - t) << shift);
        sh_remaining = remaining - above;
      }
    }
    __syncthreads();
    prefix = sh_prefix;
    remaining = sh_remaining;
    mask |= 255u << shift;
  }
  // keys > K are all taken; of the keys == K, the first `remaining` in index order
  int eq = 0;
  for_keys([&](int64_t, uint32_t u) { eq += u == prefix ? 1 : 0; });
  const int eq_before = block_exclusive_scan(eq, scan_sh);
  int sel = 0;
  {
    int e = eq_before;
    for_keys([&](int64_t, uint32_t u) {
      if (u > prefix) ++sel;
      else if (u == prefix) sel += (e++ < remaining) ? 1 : 0;
    });
  }
  int pos = block_exclusive_scan(sel, scan_sh);
  int e = eq_before;
  int32_t* out = S + (int64_t)b * k;
  const double* sq = l2sq + (int64_t)b * rows;
  double ssq = 0.0;
  for_keys([&](int64_t i, uint32_t u) {
    const bool take = u > prefix || (u == prefix && e++ < remaining);
    if (take) {
      out[pos++] = (int32_t)i;
      ssq += sq[i];
    }
  });
  // ||M[S,:]||_F from the selected rows' sums of squares (fixed order): the normalisation
  // scale of the selected block (0 for a zero block).
  const double tot = block_sum<double, kSelThreads>(ssq, dsh);
  if (t == 0) xscale[b] = tot > 0.0 ? (float)((double)Spow / sqrt(tot)) : 0.f;
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
                    float mu, double* partials, hipStream_t s) {
  const int nblk = norm_blocks(elems);
  dim3 grid(nblk, count);
  if (g_store == Store::BF16)
    hipLaunchKernelGGL(k_momentum<uint16_t>, grid, dim3(kThreads), 0, s, M, G, elems, mu, partials, nblk);
  else
    hipLaunchKernelGGL(k_momentum<float>, grid, dim3(kThreads), 0, s, M, G, elems, mu, partials, nblk);
  return last();
}

hipError_t sumsq(const void* X, Store st, int count, int64_t elems, double* partials, hipStream_t s) {
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

hipError_t finalize_scale(const double* partials, int nblk, int count, float S, float* xscale,
                          hipStream_t s) {
  hipLaunchKernelGGL(k_finalize_scale, dim3(count), dim3(kThreads), 0, s, partials, nblk, S, xscale);
  return last();
}

template <typename TS, typename TX, bool GATHER = false>
static void launch_normalize(const PtrPack* pack, const void* base, int count, int64_t rows,
                             int64_t cols, const float* xscale, void* S, void* T, int64_t rows_p,
                             int64_t cols_p, hipStream_t s, const int32_t* rowidx = nullptr,
                             float mu = 0.f) {
  PtrPack pk = {};
  if (pack) pk = *pack;
  if (!T) {
    // straight layout only: the streaming pass
    const int64_t nvec = rows_p * (cols_p / 8);
    const int64_t per = (int64_t)kThreads * kRowIter;
    dim3 grid1((unsigned)((nvec + per - 1) / per), count);
    hipLaunchKernelGGL((k_normalize_rows<TS, TX, GATHER>), grid1, dim3(kThreads), 0, s, pk,
                       static_cast<const TS*>(base), rows, cols, xscale, static_cast<TX*>(S),
                       rows_p, cols_p, rowidx, mu);
    return;
  }
  dim3 grid((unsigned)(cols_p / kNormCols), (unsigned)(rows_p / kNormRows), count);
  hipLaunchKernelGGL((k_normalize<TS, TX, GATHER>), grid, dim3(kThreads), 0, s, pk,
                     static_cast<const TS*>(base), rows, cols, xscale, static_cast<TX*>(S),
                     static_cast<TX*>(T), rows_p, cols_p, rowidx, mu);
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

int normuon_blocks(int64_t rows) { return (int)((rows + kRowsPerBlock - 1) / kRowsPerBlock); }

hipError_t normuon_finalize(const float* part, int chunks, int count, int64_t rows, int64_t cols,
                            const PtrPack* v_pack, float* v_base, int64_t v_stride,
                            const int32_t* rowidx, float beta2, float eps, float inv_s2,
                            float out_scale, float* rowscale, double* fin, hipStream_t s) {
  PtrPack vp = {};
  if (v_pack) vp = *v_pack;
  const int nblk = normuon_blocks(rows);
  hipLaunchKernelGGL(k_normuon_rows, dim3(nblk, count), dim3(kThreads), 0, s, part, chunks, rows,
                     cols, vp, v_base, v_stride, rowidx, beta2, eps, inv_s2, rowscale, fin);
  const hipError_t e = last();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_normuon_ratio, dim3(count), dim3(kThreads), 0, s, fin, nblk, rows,
                     out_scale, rowscale);
  return last();
}

hipError_t fill(float* p, int64_t n, float value, hipStream_t s) {
  int64_t blocks = (n + kThreads - 1) / kThreads;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(k_fill, dim3((unsigned)blocks), dim3(kThreads), 0, s, p, n, value);
  return last();
}

hipError_t cache_flush(void* p, size_t bytes, hipStream_t s) {
  const int64_t n16 = (int64_t)(bytes / 16);
  if (n16 < 1) return hipSuccess;
  hipLaunchKernelGGL(k_flush, dim3(8192), dim3(kThreads), 0, s, static_cast<uint4*>(p), n16);
  return last();
}

template <typename TW, typename TX>
static void launch_wupdate(const PtrPack& W, int count, int64_t rows, int64_t cols, const void* X,
                           int64_t rows_p, int64_t cols_p, const float* rowscale,
                           const int32_t* rowidx, int64_t rowidx_stride, float lr, hipStream_t s) {
  dim3 grid((unsigned)((cols + 8 * kThreads - 1) / (8 * kThreads)),
            grid_rows((rows + kWuRows - 1) / kWuRows), count);
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
                       int64_t cols, float* l1, double* l2sq, hipStream_t s) {
  dim3 grid(grid_rows(rows), count);
  if (g_store == Store::BF16)
    hipLaunchKernelGGL(k_momentum_l1<uint16_t>, grid, dim3(kThreads), 0, s, M, G, rows, cols, l1, l2sq);
  else
    hipLaunchKernelGGL(k_momentum_l1<float>, grid, dim3(kThreads), 0, s, M, G, rows, cols, l1, l2sq);
  return last();
}

hipError_t topk_rows(const float* l1, const double* l2sq, int count, int64_t rows, int64_t k,
                     float Spow, int32_t* S, float* xscale, hipStream_t s) {
  hipLaunchKernelGGL(k_topk, dim3(count), dim3(kSelThreads), 0, s, l1, l2sq, rows, k, S, Spow,
                     xscale);
  return last();
}

hipError_t gather_normalize(const PtrPack& M, int count, int64_t k, int64_t cols,
                            const int32_t* S, float mu, const float* xscale, Elem e, void* X,
                            void* Xt, int64_t rows_p, int64_t cols_p, hipStream_t s) {
  if (e == Elem::F16)
    launch_normalize<float, _Float16, true>(&M, nullptr, count, k, cols, xscale, X, Xt, rows_p,
                                            cols_p, s, S, mu);
  else
    launch_normalize<float, float, true>(&M, nullptr, count, k, cols, xscale, X, Xt, rows_p,
                                         cols_p, s, S, mu);
  return last();
}

}  // namespace mns
