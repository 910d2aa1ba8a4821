// C ABI of the Muon / Newton-Schulz step: argument validation, workspace planning and the
// drivers that sequence the kernels of one step on the caller's stream.
//
// Method: page "Dion3: Full-stack orthogonal updates" -- Eq. (1) (Muon), Eq. (2) (NorMuon),
// section "Standard Newton-Schulz", Theorem 2 and the restart of Algorithm 3 (Gram NS),
// Algorithm 4 (Dion3 row selection), section "4. Megabatched Communication" (matrices of
// one shape are processed as one batch).
#include "muon_ns.h"
#include "mns_internal.h"

#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

using namespace mns;

namespace {

// ---- instrumentation: hipEvent pairs around every launch while a session is open ----------

struct ProfRec {
  const char* name;
  hipEvent_t a, b;
  double flops, bytes;
};
// g_prof_on is read on every launch without the lock (atomic: a session toggled on another
// thread is seen cleanly); the record list and the failure flag are guarded by g_prof_mu.
std::mutex g_prof_mu;
std::atomic<bool> g_prof_on{false};
bool g_prof_failed = false;
std::vector<ProfRec> g_prof;
// Optional cache flush before the session's HBM-bound launches (mns_profile_set_flush).
void* g_flush_buf = nullptr;
size_t g_flush_bytes = 0;
constexpr double kFlushMinBytes = double(16 << 20);

template <typename F>
hipError_t timed(const char* name, double flops, double bytes, hipStream_t s, F&& launch) {
  if (!g_prof_on.load(std::memory_order_acquire)) return launch();
  {
    void* fb = nullptr;
    size_t fn = 0;
    {
      std::lock_guard<std::mutex> lk(g_prof_mu);
      fb = g_flush_buf;
      fn = g_flush_bytes;
    }
    // outside the event pair: the launch then reads its operands from HBM
    if (fb && fn && flops == 0.0 && bytes >= kFlushMinBytes) {
      const hipError_t fe = cache_flush(fb, fn, s);
      if (fe != hipSuccess) return fe;
    }
  }
  ProfRec r{name, nullptr, nullptr, flops, bytes};
  if (hipEventCreate(&r.a) != hipSuccess || hipEventCreate(&r.b) != hipSuccess) {
    if (r.a) (void)hipEventDestroy(r.a);   // the first event was made, the second was not
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof_failed = true;
    return launch();
  }
  (void)hipEventRecord(r.a, s);
  const hipError_t e = launch();
  (void)hipEventRecord(r.b, s);
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof.push_back(r);
  return e;
}

hipError_t timed_gemm(const GemmDesc& d, double flops, hipStream_t s) {
  return timed(gemm_name(d), flops, 0.0, s, [&] { return gemm(d, s); });
}



constexpr int64_t kMaxDim = 65536;
constexpr int64_t kMaxElems = 2147483647LL;
constexpr int kMaxT = 64;
constexpr int kChunk = kMaxPack;      // matrices per batched launch sequence

// Carves 256-byte aligned slices from the workspace; with a null base it only measures.
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  template <typename T>
  T* take(size_t count) {
    off = (off + 255) & ~size_t(255);
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += count * sizeof(T);
    return p;
  }
};

// Geometry of the Newton-Schulz problem for a rows x cols matrix: it runs on the short
// side (n <= m), a tall matrix through its transpose, in a zero-padded n_p x m_p iterate
// whose entries are stored times S (a power of two chosen so the float16 iterate keeps
// its entries well inside the normal range: X_0 entries ~ S/sqrt(nm), later ~ S/sqrt(m)).
struct Geo {
  int64_t rows, cols, n, m, n_p, m_p;
  int64_t rows_p, cols_p;      // stored layout, padded (the result O is kept this way)
  int64_t ld_x, ld_t, ld_q;    // row pitch of X (n_p x m_p), X^T (m_p x n_p), n_p x n_p
  bool tall;
  Elem elem;
  float S;
};

Geo make_geo(int64_t rows, int64_t cols, Store st) {
  Geo g;
  g.rows = rows;
  g.cols = cols;
  g.tall = rows > cols;
  g.n = g.tall ? cols : rows;
  g.m = g.tall ? rows : cols;
  g.n_p = pad_up(g.n);
  g.m_p = pad_up(g.m);
  g.rows_p = pad_up(rows);
  g.cols_p = pad_up(cols);
  g.ld_x = padded_ld(g.m_p);
  g.ld_t = padded_ld(g.n_p);
  g.ld_q = padded_ld(g.n_p);
  g.elem = st == Store::BF16 ? Elem::F16 : Elem::F32;
  if (g.elem == Elem::F16) {
    int e = (int)std::lround(0.5 * std::log2((double)g.m));
    if (e < 0) e = 0;
    if (e > 12) e = 12;
    g.S = std::ldexp(1.0f, e);
  } else {
    g.S = 1.0f;
  }
  return g;
}

// The iterate X (n_p x m_p, rows = the short side) feeds X X^T and, read k-major, B X and
// Q X; its transposed copy X^T (m_p x n_p) is formed only where those products cannot read X
// k-major (64 x 64 tiles, float32) and as the stored layout of a tall result. Each layout
// has a ping-pong pair.
struct NsBuffers {
  void* X[2] = {};
  void* Xt[2] = {};
  void* sq[6] = {};        // n_p x n_p scratch: standard uses 2, Gram uses 6
  float* gemm_scratch = nullptr;
  size_t gemm_scratch_bytes = 0;
  int64_t x_stride = 0, xt_stride = 0, sq_stride = 0;   // batch strides (elements)
};

// Split-k scratch the GEMMs of this geometry can use at most: (output tiles) x (k-tiles / 8)
// float32 tiles (before any cap).
size_t gemm_scratch_need(const Geo& g, int count) {
  const size_t kparts = (size_t)(g.m_p > g.n_p ? g.m_p : g.n_p) / 256;
  return (size_t)count * g.n_p * g.n_p * kparts * sizeof(float);
}

void carve_ns(Carver& cv, const Geo& g, int count, int kind, NsBuffers& b,
              size_t gemm_cap = kGemmScratchBytes) {
  const size_t es = (size_t)elem_bytes(g.elem);
  b.x_stride = g.n_p * g.ld_x;
  b.xt_stride = g.m_p * g.ld_t;
  b.sq_stride = g.n_p * g.ld_q;
  for (int i = 0; i < 2; ++i) {
    b.X[i] = cv.take<char>(es * count * b.x_stride);
    b.Xt[i] = cv.take<char>(es * count * b.xt_stride);
  }
  const int nsq = kind == MNS_NS_GRAM ? 6 : 2;
  for (int i = 0; i < nsq; ++i) b.sq[i] = cv.take<char>(es * count * b.sq_stride);
  // split-k partial sums: at most (output tiles) x (k-tiles / 8) tiles of float32, capped (a
  // smaller cap only makes the GEMMs split their tail tiles into fewer parts)
  size_t scratch = gemm_scratch_need(g, count);
  if (scratch > gemm_cap) scratch = gemm_cap;
  b.gemm_scratch = cv.take<float>(scratch / sizeof(float));
  b.gemm_scratch_bytes = scratch;
}

// Normalisation targets: the stored layout of the source is X for a wide matrix and X^T for
// a tall one; the other buffer receives the transpose.
// With km (the products read X k-major) only X is formed: null for the X^T side.
void* straight(const Geo& g, const NsBuffers& b, bool km) {
  return g.tall ? (km ? nullptr : b.Xt[0]) : b.X[0];
}
void* transposed(const Geo& g, const NsBuffers& b, bool km) {
  return g.tall ? b.X[0] : (km ? nullptr : b.Xt[0]);
}

#define MNS_HIP(expr)                               \
  do {                                              \
    if ((expr) != hipSuccess) return MNS_ERR_HIP;   \
  } while (0)

GemmDesc sym_desc(const Geo& g, int count, const NsBuffers& b, const void* A, const void* B,
                  int64_t ldab, int64_t sab, int K, void* C) {
  GemmDesc d;
  d.elem = g.elem;
  d.A = A; d.lda = ldab; d.sA = sab;
  d.B = B; d.ldb = ldab; d.sB = sab;
  d.C = C; d.ldc = g.ld_q; d.sC = b.sq_stride;
  d.M = (int)g.n_p; d.N = (int)g.n_p; d.K = K; d.batch = count;
  d.sym = true;
  d.partial = b.gemm_scratch; d.partial_bytes = b.gemm_scratch_bytes;
  return d;
}

// L X for L n_p x n_p (symmetric) and X given by its transpose Xt (m_p x n_p): written to
// C (n_p x m_p) and/or Ct (m_p x n_p).
GemmDesc left_desc(const Geo& g, int count, const NsBuffers& b, const void* L, const void* Xt,
                   void* C, void* Ct) {
  GemmDesc d;
  d.elem = g.elem;
  d.A = L; d.lda = g.ld_q; d.sA = b.sq_stride;
  d.B = Xt; d.ldb = g.ld_t; d.sB = b.xt_stride;
  d.C = C; d.ldc = g.ld_x; d.sC = b.x_stride;
  d.Ct = Ct; d.ldct = g.ld_t; d.sCt = b.xt_stride;
  d.M = (int)g.n_p; d.N = (int)g.m_p; d.K = (int)g.n_p; d.batch = count;
  d.partial = b.gemm_scratch; d.partial_bytes = b.gemm_scratch_bytes;
  return d;
}

// Whether the products L X of this geometry read the iterate X itself, k-major (float16 on
// 256 x 256 or 128 x 128 tiles): X^T is then never formed, except as the stored layout of a
// tall result.
bool kmajor_ns(const Geo& g, int count, const NsBuffers& b) {
  return gemm_kmajor_ok(left_desc(g, count, b, nullptr, nullptr, b.X[1], nullptr));
}

// L X for the iterate X[cur] (through X^T[cur], or k-major from X[cur] when km).
GemmDesc lx_desc(const Geo& g, int count, const NsBuffers& b, bool km, const void* L, int cur,
                 void* C, void* Ct) {
  GemmDesc d = left_desc(g, count, b, L, b.Xt[cur], C, Ct);
  if (km) {
    d.B = b.X[cur]; d.ldb = g.ld_x; d.sB = b.x_stride;
    d.b_kmajor = true;
  }
  return d;
}

// Optional request for the per-row sums of squares of the NS result (NorMuon's row
// statistics), taken in the epilogue of the product that writes the result: part gets the
// GemmDesc::rowsq layout (64-column chunks); done reports whether such a product ran.
struct RowSq {
  float* part = nullptr;
  int rows = 0;
  bool done = false;
};

void want_rowsq(GemmDesc& d, RowSq* rs) {
  if (!rs) return;
  d.rowsq = rs->part;
  d.rowsq_rows = rs->rows;
  rs->done = true;
}

// Standard quintic NS on the normalised iterate (b.X[0], b.Xt[0]) (section "Standard
// Newton-Schulz"): A = X X^T, B = b A + c A^2, X <- a X + B X. Returns the result in the
// stored layout (X for a wide matrix, X^T for a tall one; row pitch padded_ld(cols_p)).
mns_status run_standard(const Geo& g, int count, const NsBuffers& b, int T, const float* abc,
                        hipStream_t s, void** out, RowSq* rs) {
  int cur = 0;
  void* A = b.sq[0];
  void* B = b.sq[1];
  const float inv_s2 = 1.0f / (g.S * g.S);
  const double nn = (double)count * g.n * g.n;
  const bool km = kmajor_ns(g, count, b);
  for (int t = 0; t < T; ++t) {
    const float a = abc[3 * t], bb = abc[3 * t + 1], c = abc[3 * t + 2];
    GemmDesc gram = sym_desc(g, count, b, b.X[cur], b.X[cur], g.ld_x, b.x_stride, (int)g.m_p, A);
    gram.alpha = inv_s2;
    MNS_HIP(timed_gemm(gram, nn * g.m, s));
    const bool last = t == T - 1;
    // X is needed for the next X X^T (and, k-major, the next update); X^T only for the next
    // update when it cannot read X k-major, and as the stored layout of a tall result.
    GemmDesc upd = lx_desc(g, count, b, km, A, cur, (!last || !g.tall) ? b.X[cur ^ 1] : nullptr,
                           (last ? g.tall : !km) ? b.Xt[cur ^ 1] : nullptr);
    if (c != 0.0f) {
      // P = a I + b A + c A^2 (a on the real diagonal only, so padding stays zero), then
      // X <- P X: the same map as a X + (b A + c A^2) X, without re-reading X.
      GemmDesc poly = sym_desc(g, count, b, A, A, g.ld_q, b.sq_stride, (int)g.n_p, B);
      poly.alpha = c;
      poly.beta = bb;
      poly.D = A; poly.ldd = g.ld_q; poly.sD = b.sq_stride;
      poly.gamma = a;
      poly.diag_limit = (int)g.n;
      MNS_HIP(timed_gemm(poly, nn * g.n, s));
      upd.A = B;
    } else {
      upd.alpha = bb;
      upd.beta = a;
      upd.D = b.X[cur]; upd.ldd = g.ld_x; upd.sD = b.x_stride;   // read in C coordinates
    }
    if (last) want_rowsq(upd, rs);
    MNS_HIP(timed_gemm(upd, 2.0 * nn * g.m, s));
    cur ^= 1;
  }
  *out = g.tall ? b.Xt[cur] : b.X[cur];
  return MNS_OK;
}

// Gram Newton-Schulz (Theorem 2) with restarts (Algorithm 3): R = X X^T; per iteration
// Z = a I + b R + c R^2, R <- R Z^2 (skipped when unused), Q <- Q Z (Q_1 = Z_1);
// a restart before t forms X <- Q X, R <- X X^T, Q <- I. Output Q X (stored layout).
// Whether restart_mask asks for a restart before iteration t (bits 2..31; a 32-bit mask
// cannot name a later iteration, and a shift by 32 or more would be undefined).
inline bool restart_at(uint32_t restart_mask, int t) {
  return t >= 0 && t < 32 && ((restart_mask >> t) & 1u);
}

mns_status run_gram(const Geo& g, int count, const NsBuffers& b, int T, const float* abc,
                    uint32_t restart_mask, hipStream_t s, void** out, RowSq* rs) {
  int cur = 0;
  void* R = b.sq[0];
  void* Rt = b.sq[1];
  void* Z = b.sq[2];
  void* Z2 = b.sq[3];
  void* Q = b.sq[4];
  void* Qt = b.sq[5];
  const float inv_s2 = 1.0f / (g.S * g.S);
  const int n = (int)g.n_p;
  const double nn = (double)count * g.n * g.n;
  const bool km = kmajor_ns(g, count, b);

  GemmDesc gram = sym_desc(g, count, b, b.X[cur], b.X[cur], g.ld_x, b.x_stride, (int)g.m_p, R);
  gram.alpha = inv_s2;
  MNS_HIP(timed_gemm(gram, nn * g.m, s));
  bool q_identity = true;
  for (int t = 1; t <= T; ++t) {
    const float a = abc[3 * (t - 1)], bb = abc[3 * (t - 1) + 1], c = abc[3 * (t - 1) + 2];
    if (t > 1 && restart_at(restart_mask, t)) {
      if (!q_identity) {
        MNS_HIP(timed_gemm(lx_desc(g, count, b, km, Q, cur, b.X[cur ^ 1],
                                   km ? nullptr : b.Xt[cur ^ 1]),
                           2.0 * nn * g.m, s));
        cur ^= 1;
      }
      GemmDesc re = sym_desc(g, count, b, b.X[cur], b.X[cur], g.ld_x, b.x_stride, (int)g.m_p, R);
      re.alpha = inv_s2;
      MNS_HIP(timed_gemm(re, nn * g.m, s));
      q_identity = true;
    }
    GemmDesc zd = sym_desc(g, count, b, R, R, g.ld_q, b.sq_stride, n, Z);
    zd.alpha = c;
    zd.beta = bb;
    zd.D = R; zd.ldd = g.ld_q; zd.sD = b.sq_stride;
    zd.gamma = a;
    zd.diag_limit = (int)g.n;
    MNS_HIP(timed_gemm(zd, nn * g.n, s));
    if (t < T && !restart_at(restart_mask, t + 1)) {
      MNS_HIP(timed_gemm(sym_desc(g, count, b, Z, Z, g.ld_q, b.sq_stride, n, Z2), nn * g.n, s));
      MNS_HIP(timed_gemm(sym_desc(g, count, b, R, Z2, g.ld_q, b.sq_stride, n, Rt), nn * g.n, s));
      void* tmp = R; R = Rt; Rt = tmp;
    }
    if (q_identity) {
      void* tmp = Q; Q = Z; Z = tmp;
      q_identity = false;
    } else {
      MNS_HIP(timed_gemm(sym_desc(g, count, b, Q, Z, g.ld_q, b.sq_stride, n, Qt), nn * g.n, s));
      void* tmp = Q; Q = Qt; Qt = tmp;
    }
  }
  if (q_identity) {
    *out = g.tall ? b.Xt[cur] : b.X[cur];
  } else {
    GemmDesc fin = lx_desc(g, count, b, km, Q, cur, g.tall ? nullptr : b.X[cur ^ 1],
                           g.tall ? b.Xt[cur ^ 1] : nullptr);
    want_rowsq(fin, rs);
    MNS_HIP(timed_gemm(fin, 2.0 * nn * g.m, s));
    *out = g.tall ? b.Xt[cur ^ 1] : b.X[cur ^ 1];
  }
  return MNS_OK;
}

mns_status run_ns(const Geo& g, int count, const NsBuffers& b, int kind, int T, const float* abc,
                  uint32_t restart_mask, hipStream_t s, void** out, RowSq* rs = nullptr) {
  if (kind == MNS_NS_GRAM) return run_gram(g, count, b, T, abc, restart_mask, s, out, rs);
  return run_standard(g, count, b, T, abc, s, out, rs);
}

// ---- validation helpers --------------------------------------------------------------------

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

mns_status check_shape(int64_t batch, int64_t rows, int64_t cols) {
  if (batch < 1 || rows < 1 || cols < 1) return MNS_ERR_SHAPE;
  if (rows > kMaxDim || cols > kMaxDim || rows * cols > kMaxElems) return MNS_ERR_SHAPE;
  if (batch > kMaxElems / (rows * cols)) return MNS_ERR_SHAPE;
  return MNS_OK;
}

// The GEMMs address one padded iterate (either layout, with its row pitch) with 32-bit byte
// offsets.
mns_status check_iterate(int64_t rows, int64_t cols, Store st) {
  const int64_t rp = pad_up(rows), cp = pad_up(cols);
  const int64_t a = rp * padded_ld(cp), b = cp * padded_ld(rp);
  const int64_t bytes = (a > b ? a : b) * (st == Store::BF16 ? 2 : 4);
  return bytes <= kMaxElems ? MNS_OK : MNS_ERR_SHAPE;
}

mns_status check_dtype(int dt) {
  return (dt == MNS_F32 || dt == MNS_BF16) ? MNS_OK : MNS_ERR_DTYPE;
}

mns_status check_ns(int T, const float* abc, int kind, uint32_t restart_mask) {
  if (T < 1 || T > kMaxT) return MNS_ERR_PARAM;
  if (!abc) return MNS_ERR_NULL;
  for (int i = 0; i < 3 * T; ++i)
    if (!std::isfinite(abc[i])) return MNS_ERR_PARAM;
  if (kind != MNS_NS_STANDARD && kind != MNS_NS_GRAM) return MNS_ERR_PARAM;
  if (kind == MNS_NS_STANDARD && restart_mask != 0) return MNS_ERR_PARAM;
  // valid restart bits: 2..T
  const uint64_t allowed = ((T >= 31 ? 0xFFFFFFFFull : ((1ull << (T + 1)) - 1))) & ~3ull;
  if ((uint64_t)restart_mask & ~allowed) return MNS_ERR_PARAM;
  return MNS_OK;
}

mns_status check_ws(void* ws, size_t have, size_t need) {
  if (!ws) return MNS_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return MNS_ERR_WORKSPACE;
  if (have < need) return MNS_ERR_WORKSPACE;
  return MNS_OK;
}

int64_t k_rows(double f, int64_t rows) {
  int64_t k = (int64_t)std::ceil(f * (double)rows);
  if (k < 1) k = 1;
  if (k > rows) k = rows;
  return k;
}

// Shape groups: matrices of equal (rows, cols), in order of first appearance.
struct Group {
  int64_t rows, cols;
  std::vector<int> idx;
};

std::vector<Group> group_by_shape(const mns_matrix* mats, int count) {
  std::vector<Group> gs;
  for (int i = 0; i < count; ++i) {
    bool found = false;
    for (auto& g : gs)
      if (g.rows == mats[i].rows && g.cols == mats[i].cols) {
        g.idx.push_back(i);
        found = true;
        break;
      }
    if (!found) gs.push_back(Group{mats[i].rows, mats[i].cols, {i}});
  }
  return gs;
}

mns_status validate_step(const mns_matrix* mats, int count, const mns_hparams* hp,
                         bool need_ptrs) {
  if (!mats || !hp) return MNS_ERR_NULL;
  if (count < 1) return MNS_ERR_SHAPE;
  mns_status st = check_dtype(hp->dtype);
  if (st != MNS_OK) return st;
  st = check_ns(hp->T, hp->abc, hp->kind, hp->restart_mask);
  if (st != MNS_OK) return st;
  if (!std::isfinite(hp->mu) || !std::isfinite(hp->lr)) return MNS_ERR_PARAM;
  if (!(hp->row_fraction > 0.0 && hp->row_fraction <= 1.0)) return MNS_ERR_PARAM;
  if (hp->normuon != 0 && hp->normuon != 1) return MNS_ERR_PARAM;
  if (hp->normuon && (!(hp->beta2 >= 0.f && hp->beta2 <= 1.f) || !(hp->eps >= 0.f) ||
                      !std::isfinite(hp->eps)))
    return MNS_ERR_PARAM;
  for (int i = 0; i < count; ++i) {
    st = check_shape(1, mats[i].rows, mats[i].cols);
    if (st != MNS_OK) return st;
    st = check_iterate(mats[i].rows, mats[i].cols, hp->dtype == MNS_BF16 ? Store::BF16 : Store::F32);
    if (st != MNS_OK) return st;
    if (need_ptrs) {
      if (!mats[i].W || !mats[i].M || !mats[i].G) return MNS_ERR_NULL;
      if (hp->normuon && !mats[i].v) return MNS_ERR_NULL;
      if (!aligned(mats[i].W, 16) || !aligned(mats[i].M, 16) || !aligned(mats[i].G, 16) ||
          (mats[i].v && !aligned(mats[i].v, 4)))
        return MNS_ERR_PARAM;
    }
  }
  return MNS_OK;
}

// Workspace layout of one chunk (<= kChunk matrices of one shape) of muon_step.
struct StepWs {
  double* partials = nullptr;
  float* xscale = nullptr;
  NsBuffers ns;
  float* part = nullptr;
  float* rowscale = nullptr;
  double* fin = nullptr;
  float* l1 = nullptr;
  double* l2sq = nullptr;
  int32_t* S = nullptr;
  int nblk = 0, chunks = 0;
};

size_t carve_step(void* base, const Geo& g, int count, int64_t rows, int64_t cols, bool dion,
                  int64_t k, int kind, StepWs& w) {
  Carver cv(base);
  w.nblk = dion ? 0 : norm_blocks(rows * cols);
  w.partials = cv.take<double>((size_t)count * w.nblk);
  w.xscale = cv.take<float>((size_t)count);
  carve_ns(cv, g, count, kind, w.ns);
  w.chunks = (int)(g.cols_p / 64);                     // row-norm partials per stored row
  w.part = cv.take<float>((size_t)count * w.chunks * g.rows);
  w.rowscale = cv.take<float>((size_t)count * g.rows);
  w.fin = cv.take<double>((size_t)count * 2 * normuon_blocks(g.rows));
  if (dion) {
    w.l1 = cv.take<float>((size_t)count * rows);
    w.S = cv.take<int32_t>((size_t)count * k);
    w.l2sq = cv.take<double>((size_t)count * rows);
  }
  return cv.off + 256;
}

size_t step_bytes(const mns_matrix* mats, int count, const mns_hparams* hp) {
  const Store st = hp->dtype == MNS_BF16 ? Store::BF16 : Store::F32;
  const bool dion = hp->row_fraction < 1.0;
  size_t need = 0;
  for (const Group& gr : group_by_shape(mats, count)) {
    const int c = (int)gr.idx.size() < kChunk ? (int)gr.idx.size() : kChunk;
    const int64_t k = dion ? k_rows(hp->row_fraction, gr.rows) : gr.rows;
    const Geo g = make_geo(k, gr.cols, st);
    StepWs w;
    const size_t b = carve_step(nullptr, g, c, gr.rows, gr.cols, dion, k, hp->kind, w);
    if (b > need) need = b;
  }
  return need;
}

}  // namespace

extern "C" {

const char* mns_status_string(int status) {
  switch (status) {
    case MNS_OK: return "MNS_OK";
    case MNS_ERR_NULL: return "MNS_ERR_NULL: a required pointer is NULL";
    case MNS_ERR_SHAPE: return "MNS_ERR_SHAPE: a size is out of range";
    case MNS_ERR_DTYPE: return "MNS_ERR_DTYPE: unknown storage dtype";
    case MNS_ERR_PARAM: return "MNS_ERR_PARAM: invalid hyperparameter or alignment";
    case MNS_ERR_WORKSPACE: return "MNS_ERR_WORKSPACE: workspace NULL, misaligned or too small";
    case MNS_ERR_HIP: return "MNS_ERR_HIP: a HIP launch failed";
    default: return "unknown mns_status";
  }
}

int mns_version(void) { return 100; }

mns_status mns_step_workspace_size(const mns_matrix* mats, int count, const mns_hparams* hp,
                                   size_t* bytes) {
  if (!bytes) return MNS_ERR_NULL;
  const mns_status st = validate_step(mats, count, hp, false);
  if (st != MNS_OK) return st;
  *bytes = step_bytes(mats, count, hp);
  return MNS_OK;
}

mns_status muon_step(const mns_matrix* mats, int count, const mns_hparams* hp, void* workspace,
                     size_t workspace_bytes, void* stream) {
  mns_status st = validate_step(mats, count, hp, true);
  if (st != MNS_OK) return st;
  st = check_ws(workspace, workspace_bytes, step_bytes(mats, count, hp));
  if (st != MNS_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Store sto = hp->dtype == MNS_BF16 ? Store::BF16 : Store::F32;
  const bool dion = hp->row_fraction < 1.0;

  for (const Group& gr : group_by_shape(mats, count)) {
    const int64_t rows = gr.rows, cols = gr.cols;
    const int64_t k = dion ? k_rows(hp->row_fraction, rows) : rows;
    const Geo g = make_geo(k, cols, sto);      // the matrix NS runs on: k x cols
    for (size_t c0 = 0; c0 < gr.idx.size(); c0 += kChunk) {
      const int c = (int)((gr.idx.size() - c0) < (size_t)kChunk ? gr.idx.size() - c0 : kChunk);
      PtrPack Wp = {}, Mp = {}, Gp = {}, Vp = {};
      for (int i = 0; i < c; ++i) {
        const mns_matrix& mm = mats[gr.idx[c0 + i]];
        Wp.p[i] = mm.W;
        Mp.p[i] = mm.M;
        Gp.p[i] = const_cast<void*>(mm.G);
        Vp.p[i] = mm.v;
      }
      StepWs w;
      carve_step(workspace, g, c, rows, cols, dion, k, hp->kind, w);
      const bool km = kmajor_ns(g, c, w.ns);

      const double all = (double)c * rows * cols;      // elements of the chunk's matrices
      const double sel = (double)c * k * cols;         // elements the NS runs on
      const double es = elem_bytes(g.elem), ss = sto == Store::BF16 ? 2.0 : 4.0;
      if (!dion) {
        MNS_HIP(timed("momentum", 0, all * (8.0 + ss), s, [&] {
          return momentum(Mp, Gp, sto, c, rows * cols, hp->mu, w.partials, s); }));
        MNS_HIP(timed("finalize_scale", 0, 4.0 * c * w.nblk, s, [&] {
          return finalize_scale(w.partials, w.nblk, c, g.S, w.xscale, s); }));
        MNS_HIP(timed("normalize", 0, all * (4.0 + (km ? 1.0 : 2.0) * es), s, [&] {
          return normalize(&Mp, nullptr, true, sto, c, rows, cols, w.xscale, g.elem,
                           straight(g, w.ns, km), transposed(g, w.ns, km), g.rows_p,
                           g.cols_p, s); }));
      } else {
        MNS_HIP(timed("momentum_l1", 0, all * (8.0 + ss), s, [&] {
          return momentum_l1(Mp, Gp, sto, c, rows, cols, w.l1, w.l2sq, s); }));
        MNS_HIP(timed("topk", 0, 8.0 * c * rows + 8.0 * c * k, s, [&] {
          return topk_rows(w.l1, w.l2sq, c, rows, k, g.S, w.S, w.xscale, s); }));
        MNS_HIP(timed("gather_normalize", 0, sel * (8.0 + (km ? 1.0 : 2.0) * es), s, [&] {
          return gather_normalize(Mp, c, k, cols, w.S, hp->mu, w.xscale, g.elem,
                                  straight(g, w.ns, km), transposed(g, w.ns, km), g.rows_p,
                           g.cols_p, s); }));
      }
      void* O = nullptr;
      RowSq rs;
      rs.part = w.part;
      rs.rows = (int)k;
      st = run_ns(g, c, w.ns, hp->kind, hp->T, hp->abc, hp->restart_mask, s, &O,
                  hp->normuon ? &rs : nullptr);
      if (st != MNS_OK) return st;
      const float inv_s = 1.0f / g.S;
      if (hp->normuon) {
        // The row statistics come from the epilogue of the product that wrote the result
        // (every run ends with one: T >= 1).
        if (!rs.done) return MNS_ERR_PARAM;
        MNS_HIP(timed("normuon_finalize", 0, 4.0 * c * k * (w.chunks + 3), s, [&] {
          return normuon_finalize(w.part, w.chunks, c, k, cols, &Vp, nullptr, 0,
                                  dion ? w.S : nullptr, hp->beta2, hp->eps, inv_s * inv_s, inv_s,
                                  w.rowscale, w.fin, s); }));
      } else {
        MNS_HIP(timed("fill", 0, 4.0 * c * k, s, [&] {
          return fill(w.rowscale, (int64_t)c * k, inv_s, s); }));
      }
      MNS_HIP(timed("weight_update", 0, sel * (2.0 * ss + es) + 4.0 * c * k, s, [&] {
        return weight_update(Wp, sto, c, k, cols, O, g.elem, g.rows_p, g.cols_p, w.rowscale,
                             dion ? w.S : nullptr, k, hp->lr, s); }));
    }
  }
  return MNS_OK;
}

// ---- standalone orthogonalisation ------------------------------------------------------------

static size_t ns_bytes(const Geo& g, int c, int kind, int64_t rows, int64_t cols,
                       NsBuffers* b, double** partials, float** xscale, void* base,
                       size_t gemm_cap = kGemmScratchBytes) {
  Carver cv(base);
  NsBuffers tmp;
  NsBuffers& nb = b ? *b : tmp;
  double* p = cv.take<double>((size_t)c * norm_blocks(rows * cols));
  float* x = cv.take<float>((size_t)c);
  carve_ns(cv, g, c, kind, nb, gemm_cap);
  if (partials) *partials = p;
  if (xscale) *xscale = x;
  return cv.off + 256;
}

mns_status mns_ns_workspace_size(int dtype, int64_t batch, int64_t rows, int64_t cols, int kind,
                                 size_t* bytes) {
  if (!bytes) return MNS_ERR_NULL;
  mns_status st = check_dtype(dtype);
  if (st != MNS_OK) return st;
  st = check_shape(batch, rows, cols);
  if (st != MNS_OK) return st;
  st = check_iterate(rows, cols, dtype == MNS_BF16 ? Store::BF16 : Store::F32);
  if (st != MNS_OK) return st;
  if (kind != MNS_NS_STANDARD && kind != MNS_NS_GRAM) return MNS_ERR_PARAM;
  const Geo g = make_geo(rows, cols, dtype == MNS_BF16 ? Store::BF16 : Store::F32);
  const int c = batch < kChunk ? (int)batch : kChunk;
  *bytes = ns_bytes(g, c, kind, rows, cols, nullptr, nullptr, nullptr, nullptr);
  return MNS_OK;
}

// Argument checks shared by the orthogonalisation entry points (everything but the workspace).
static mns_status check_orthogonalize(const void* X, void* O, int dtype, int64_t batch,
                                      int64_t rows, int64_t cols, int T, const float* abc,
                                      int kind, uint32_t restart_mask) {
  mns_status st = check_dtype(dtype);
  if (st != MNS_OK) return st;
  st = check_shape(batch, rows, cols);
  if (st != MNS_OK) return st;
  st = check_iterate(rows, cols, dtype == MNS_BF16 ? Store::BF16 : Store::F32);
  if (st != MNS_OK) return st;
  if (!X || !O) return MNS_ERR_NULL;
  st = check_ns(T, abc, kind, restart_mask);
  if (st != MNS_OK) return st;
  if (!aligned(X, 16) || !aligned(O, 16)) return MNS_ERR_PARAM;
  return MNS_OK;
}

// The orthogonalisation of `batch` matrices in chunks of at most `cmax`, each chunk's
// buffers carved from `ws` (split-k scratch capped at gemm_cap): per chunk the Frobenius
// norm, the normalised iterate, T iterations (standard or Gram), and the export to O.
static mns_status run_orthogonalize(const void* X, void* O, Store sto, const Geo& g,
                                    int64_t batch, int64_t rows, int64_t cols, int T,
                                    const float* abc, int kind, uint32_t restart_mask, void* ws,
                                    int cmax, size_t gemm_cap, hipStream_t s) {
  const size_t esz = sto == Store::BF16 ? 2 : 4;
  for (int64_t b0 = 0; b0 < batch; b0 += cmax) {
    const int c = (int)((batch - b0) < cmax ? batch - b0 : cmax);
    NsBuffers nb;
    double* partials = nullptr;
    float* xscale = nullptr;
    ns_bytes(g, c, kind, rows, cols, &nb, &partials, &xscale, ws, gemm_cap);
    const bool km = kmajor_ns(g, c, nb);
    const char* xin = static_cast<const char*>(X) + (size_t)b0 * rows * cols * esz;
    char* out = static_cast<char*>(O) + (size_t)b0 * rows * cols * esz;
    const double all = (double)c * rows * cols, ss = (double)esz, es = elem_bytes(g.elem);
    const int nblk = norm_blocks(rows * cols);
    MNS_HIP(timed("sumsq", 0, all * ss, s, [&] {
      return sumsq(xin, sto, c, rows * cols, partials, s); }));
    MNS_HIP(timed("finalize_scale", 0, 4.0 * c * nblk, s, [&] {
      return finalize_scale(partials, nblk, c, g.S, xscale, s); }));
    MNS_HIP(timed("normalize", 0, all * (ss + (km ? 1.0 : 2.0) * es), s, [&] {
      return normalize(nullptr, xin, false, sto, c, rows, cols, xscale, g.elem,
                       straight(g, nb, km), transposed(g, nb, km), g.rows_p, g.cols_p, s); }));
    void* res = nullptr;
    const mns_status st = run_ns(g, c, nb, kind, T, abc, restart_mask, s, &res);
    if (st != MNS_OK) return st;
    MNS_HIP(timed("export", 0, all * (ss + es), s, [&] {
      return export_output(res, g.elem, g.rows_p, g.cols_p, c, rows, cols, 1.0f / g.S, out,
                           sto, s); }));
  }
  return MNS_OK;
}

static mns_status orthogonalize(const void* X, void* O, int dtype, int64_t batch, int64_t rows,
                                int64_t cols, int T, const float* abc, int kind,
                                uint32_t restart_mask, void* ws, size_t ws_bytes, void* stream) {
  mns_status st = check_orthogonalize(X, O, dtype, batch, rows, cols, T, abc, kind, restart_mask);
  if (st != MNS_OK) return st;
  const Store sto = dtype == MNS_BF16 ? Store::BF16 : Store::F32;
  const Geo g = make_geo(rows, cols, sto);
  const int cmax = batch < kChunk ? (int)batch : kChunk;
  st = check_ws(ws, ws_bytes, ns_bytes(g, cmax, kind, rows, cols, nullptr, nullptr, nullptr, nullptr));
  if (st != MNS_OK) return st;
  return run_orthogonalize(X, O, sto, g, batch, rows, cols, T, abc, kind, restart_mask, ws, cmax,
                           kGemmScratchBytes, static_cast<hipStream_t>(stream));
}

// ---- allocation-free standard NS (for callers that cannot allocate) ---------------------
//
// The same computation as ns_orthogonalize, with every buffer carved from one file-scope
// device array instead of a caller workspace. Each GPU the library runs on holds its own
// copy until the process ends. Host code never uses the array's name as an address: the
// first call on a device looks up that device's copy with hipGetSymbolAddress (with the
// device current) and keeps the pointer.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

static constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices] = {};

// This device's copy of `scratch` (looked up once per device). The stream, if given, must
// belong to the current device: the array's address is the current device's.
static mns_status scratch_on_current_device(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MNS_ERR_HIP;
  if (stream) {
    int sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return MNS_ERR_HIP;
    if (sdev != dev) return MNS_ERR_PARAM;
  }
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MNS_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MNS_OK;
}

// Matrices per chunk and split-k scratch cap so that one chunk's buffers fit in `scratch`:
// the largest chunk (<= kChunk) whose buffers fit with the full split-k scratch of the
// workspace path; else one matrix per chunk with what space remains for split-k parts.
// False when one matrix's buffers alone do not fit.
static bool noalloc_plan(const Geo& g, int64_t batch, int64_t rows, int64_t cols, int* cmax,
                  size_t* gemm_cap) {
  const int hi = batch < kChunk ? (int)batch : kChunk;
  for (int c = hi; c >= 1; --c) {
    if (ns_bytes(g, c, MNS_NS_STANDARD, rows, cols, nullptr, nullptr, nullptr, nullptr) <=
        kNoAllocScratchBytes) {
      *cmax = c;
      *gemm_cap = kGemmScratchBytes;
      return true;
    }
  }
  const size_t base = ns_bytes(g, 1, MNS_NS_STANDARD, rows, cols, nullptr, nullptr, nullptr,
                               nullptr, 0);
  if (base > kNoAllocScratchBytes) return false;
  *cmax = 1;
  *gemm_cap = (kNoAllocScratchBytes - base) & ~size_t(255);
  return true;
}

mns_status ns_orthogonalize_noalloc(const void* X, void* O, int dtype, int64_t batch,
                                    int64_t rows, int64_t cols, int T, const float* abc,
                                    void* stream) {
  mns_status st = check_orthogonalize(X, O, dtype, batch, rows, cols, T, abc, MNS_NS_STANDARD, 0u);
  if (st != MNS_OK) return st;
  const Store sto = dtype == MNS_BF16 ? Store::BF16 : Store::F32;
  const Geo g = make_geo(rows, cols, sto);
  int cmax = 0;
  size_t gemm_cap = 0;
  if (!noalloc_plan(g, batch, rows, cols, &cmax, &gemm_cap)) return MNS_ERR_WORKSPACE;
  void* ws = nullptr;
  st = scratch_on_current_device(static_cast<hipStream_t>(stream), &ws);
  if (st != MNS_OK) return st;
  return run_orthogonalize(X, O, sto, g, batch, rows, cols, T, abc, MNS_NS_STANDARD, 0u, ws, cmax,
                           gemm_cap, static_cast<hipStream_t>(stream));
}

mns_status ns_orthogonalize(const void* X, void* O, int dtype, int64_t batch, int64_t rows,
                            int64_t cols, int T, const float* abc, void* workspace,
                            size_t workspace_bytes, void* stream) {
  return orthogonalize(X, O, dtype, batch, rows, cols, T, abc, MNS_NS_STANDARD, 0u, workspace,
                       workspace_bytes, stream);
}

mns_status gram_ns_orthogonalize(const void* X, void* O, int dtype, int64_t batch, int64_t rows,
                                 int64_t cols, int T, const float* abc, uint32_t restart_mask,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  return orthogonalize(X, O, dtype, batch, rows, cols, T, abc, MNS_NS_GRAM, restart_mask,
                       workspace, workspace_bytes, stream);
}

// ---- standalone NorMuon ------------------------------------------------------------------------

static size_t normuon_bytes(int64_t batch, int64_t rows, float** part, float** rowscale,
                            double** fin, void* base) {
  Carver cv(base);
  float* p = cv.take<float>((size_t)batch * rows);
  float* r = cv.take<float>((size_t)batch * rows);
  double* f = cv.take<double>((size_t)batch * 2 * normuon_blocks(rows));
  if (part) *part = p;
  if (rowscale) *rowscale = r;
  if (fin) *fin = f;
  return cv.off + 256;
}

mns_status mns_normuon_workspace_size(int64_t batch, int64_t rows, int64_t cols, size_t* bytes) {
  if (!bytes) return MNS_ERR_NULL;
  const mns_status st = check_shape(batch, rows, cols);
  if (st != MNS_OK) return st;
  *bytes = normuon_bytes(batch, rows, nullptr, nullptr, nullptr, nullptr);
  return MNS_OK;
}

mns_status normuon_scale(void* O, int dtype, int64_t batch, int64_t rows, int64_t cols, float* v,
                         float beta2, float eps, void* workspace, size_t workspace_bytes,
                         void* stream) {
  mns_status st = check_dtype(dtype);
  if (st != MNS_OK) return st;
  st = check_shape(batch, rows, cols);
  if (st != MNS_OK) return st;
  if (!O || !v) return MNS_ERR_NULL;
  if (!(beta2 >= 0.f && beta2 <= 1.f) || !(eps >= 0.f) || !std::isfinite(eps)) return MNS_ERR_PARAM;
  if (!aligned(O, 16) || !aligned(v, 4)) return MNS_ERR_PARAM;
  if (batch > 65535) return MNS_ERR_SHAPE;
  st = check_ws(workspace, workspace_bytes,
                normuon_bytes(batch, rows, nullptr, nullptr, nullptr, nullptr));
  if (st != MNS_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Store sto = dtype == MNS_BF16 ? Store::BF16 : Store::F32;
  float *part = nullptr, *rowscale = nullptr;
  double* fin = nullptr;
  normuon_bytes(batch, rows, &part, &rowscale, &fin, workspace);
  const double all = (double)batch * rows * cols, ss = sto == Store::BF16 ? 2.0 : 4.0;
  MNS_HIP(timed("row_sumsq_stored", 0, all * ss, s, [&] {
    return row_sumsq_stored(O, sto, (int)batch, rows, cols, part, s); }));
  MNS_HIP(timed("normuon_finalize", 0, 4.0 * batch * rows * 4, s, [&] {
    return normuon_finalize(part, 1, (int)batch, rows, cols, nullptr, v, rows, nullptr, beta2,
                            eps, 1.0f, 1.0f, rowscale, fin, s); }));
  MNS_HIP(timed("rowscale_apply", 0, 2.0 * all * ss, s, [&] {
    return rowscale_apply(O, sto, (int)batch, rows, cols, rowscale, s); }));
  return MNS_OK;
}

mns_status mns_profile_begin(void) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (ProfRec& r : g_prof) {
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  g_prof.clear();
  g_prof_failed = false;
  g_prof_on.store(true, std::memory_order_release);
  return MNS_OK;
}

mns_status mns_profile_set_flush(void* buffer, size_t bytes) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (!g_prof_on.load()) return MNS_ERR_PARAM;
  if (buffer && !aligned(buffer, 16)) return MNS_ERR_PARAM;
  g_flush_buf = bytes ? buffer : nullptr;
  g_flush_bytes = buffer ? bytes : 0;
  return MNS_OK;
}

mns_status mns_profile_end(mns_kernel_stat* out, int capacity, int* count) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (!g_prof_on.load()) return MNS_ERR_PARAM;
  g_prof_on.store(false, std::memory_order_release);
  g_flush_buf = nullptr;
  g_flush_bytes = 0;
  std::vector<mns_kernel_stat> stats;
  bool ok = !g_prof_failed;
  for (ProfRec& r : g_prof) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess)
      ok = false;
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
    mns_kernel_stat* st = nullptr;
    for (auto& x : stats)
      if (std::strncmp(x.name, r.name, sizeof(x.name)) == 0) st = &x;
    if (!st) {
      mns_kernel_stat z = {};
      std::strncpy(z.name, r.name, sizeof(z.name) - 1);
      stats.push_back(z);
      st = &stats.back();
    }
    st->launches += 1;
    st->ms += ms;
    st->flops += r.flops;
    st->bytes += r.bytes;
  }
  g_prof.clear();
  if (count) *count = (int)stats.size();
  for (int i = 0; i < (int)stats.size() && i < capacity && out; ++i) out[i] = stats[i];
  return ok ? MNS_OK : MNS_ERR_HIP;
}

}  // extern "C"
