// C ABI of the gfx950 BaKron solver (declared in include/bakron.h).
//
// Host side only: argument checks, workspace carving, and the launch schedule
// of the solve, the recursion of "BaKron: Efficient Quantization with
// Kronecker-Factored Hessians" (arXiv 2608.06291), §3.5 Algorithm 6, over
// ranges of tile anti-diagonals. Every computation runs in the kernels of the
// .hip files; nothing here touches matrix data.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <climits>
#include <cstdint>
#include <cstring>
#include <limits>
#include <mutex>
#include <vector>

#include "bakron.h"
#include "launch.hpp"

namespace {

using namespace bk;

constexpr size_t kAlign = 256;
// largest batch of bakron_solve_batched: the grid's y extent
constexpr int64_t kMaxBatch = 65535;

inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

inline bool dtype_ok(int dtype) { return dtype == BAKRON_F32 || dtype == BAKRON_F64; }
inline size_t esize(int dtype) { return dtype == BAKRON_F64 ? 8 : 4; }
inline int64_t tiles(int64_t d) { return (d + kTile - 1) / kTile; }

// ---- solve schedule --------------------------------------------------------
struct Op {
  int32_t kind, k, mid, l;
};
enum { OP_LEAF = 0, OP_BAND1 = 2, OP_BAND2 = 3 };

// Algorithm 6 over blocks [kb, lb) of kLeafBlock tile anti-diagonals each
// (R tile anti-diagonals in all); a leaf is a whole block, one launch.
void build_schedule(int kb, int lb, int R, std::vector<Op>& ops) {
  if (lb - kb == 1) {
    const int K0 = kb * kLeafBlock;
    const int K1 = (kb + 1) * kLeafBlock < R ? (kb + 1) * kLeafBlock : R;
    ops.push_back({OP_LEAF, K0, K1, 0});
    return;
  }
  const int midb = (kb + lb) / 2;
  build_schedule(kb, midb, R, ops);
  const int k = kb * kLeafBlock, mid = midb * kLeafBlock;
  const int l = lb * kLeafBlock < R ? lb * kLeafBlock : R;
  ops.push_back({OP_BAND1, k, mid, l});
  ops.push_back({OP_BAND2, k, mid, l});
  build_schedule(midb, lb, R, ops);
}

std::vector<Op> schedule_for(int64_t m, int64_t n) {
  std::vector<Op> ops;
  if (m <= 0 || n <= 0) return ops;
  const int R = (int)(tiles(m) + tiles(n) - 1);
  const int nb = (R + kLeafBlock - 1) / kLeafBlock;
  ops.reserve(3 * (size_t)nb);
  build_schedule(0, nb, R, ops);
  return ops;
}

// leaf blocks of the schedule of an m x n solve
inline int leaf_blocks(int64_t m, int64_t n) {
  const int64_t R = tiles(m) + tiles(n) - 1;
  return (int)((R + kLeafBlock - 1) / kLeafBlock);
}

// Solve workspace, per problem: W tiles, packed L^B and L^A tiles, the
// stage-1 product M of the band products, the leaf blocks' ticket counters
// and status word, and the leaves' error copy (Mt x Nt tiles).
struct SolveLayout {
  size_t wk, lb, la, mb, sync, eb, total;
};
SolveLayout solve_layout(int dtype, int64_t m, int64_t n) {
  const size_t es = esize(dtype);
  const int64_t Mt = tiles(m), Nt = tiles(n);
  const size_t tt = (size_t)kTile * kTile * es;
  SolveLayout L;
  L.wk = align_up((size_t)(Mt * Nt) * tt);
  L.lb = align_up((size_t)(Mt * (Mt + 1) / 2) * tt);
  L.la = align_up((size_t)(Nt * (Nt + 1) / 2) * tt);
  L.mb = L.wk;
  L.sync = align_up((size_t)(leaf_blocks(m, n) + 1) * sizeof(int));
  L.eb = L.wk;
  L.total = L.wk + L.lb + L.la + L.mb + L.sync + L.eb + kAlign;
  return L;
}
// offset of the status word in a problem's workspace
inline size_t status_offset(const SolveLayout& L, int64_t m, int64_t n) {
  return L.wk + L.lb + L.la + L.mb + (size_t)leaf_blocks(m, n) * sizeof(int);
}

// Poll bound of the leaves' waits (bakron_debug_set_wait_polls).
std::atomic<int> g_wait_polls{kLeafWaitPolls};

// The status words of `batch` solves whose workspaces start at ws, lay.total
// bytes apart, once the work on `s` has finished: BAKRON_EWAIT if a leaf of any
// of them gave up waiting.
int read_wait_status(const void* ws, const SolveLayout& lay, int64_t m, int64_t n, int64_t batch,
                     hipStream_t s) {
  std::vector<int32_t> st((size_t)batch, 0);
  const char* p = static_cast<const char*>(ws) + status_offset(lay, m, n);
  if (hipMemcpy2DAsync(st.data(), sizeof(int32_t), p, lay.total, sizeof(int32_t), (size_t)batch,
                       hipMemcpyDeviceToHost, s) != hipSuccess)
    return BAKRON_EHIP;
  if (hipStreamSynchronize(s) != hipSuccess) return BAKRON_EHIP;
  for (int32_t v : st)
    if (v != 0) return BAKRON_EWAIT;
  return BAKRON_OK;
}

template <typename R>
int solve_impl(int64_t m, int64_t n, const R* W, int64_t ldw, const R* LA, int64_t ldla,
               const R* LB, int64_t ldlb, int32_t lo, int32_t hi, int32_t unb, int scale_mode,
               const R* scales, int32_t* V, int64_t ldv, R* Wt, int64_t ldwt, void* ws,
               hipStream_t s, double* op_ms = nullptr, int batch = 1,
               const BatchStrides* strides = nullptr) {
  SolveGeom g;
  g.m = m;
  g.n = n;
  g.Mt = (int)tiles(m);
  g.Nt = (int)tiles(n);
  const SolveLayout lay = solve_layout(sizeof(R) == 8 ? BAKRON_F64 : BAKRON_F32, m, n);
  // a batch: the same launches for every problem, each with its own
  // workspace of lay.total bytes (a multiple of the alignment)
  g.batch = batch;
  if (strides) g.bs = *strides;
  g.bs.ws = batch > 1 ? (int64_t)(lay.total / sizeof(R)) : 0;
  char* base = static_cast<char*>(ws);
  R* Wk = reinterpret_cast<R*>(base);
  R* LBp = reinterpret_cast<R*>(base + lay.wk);
  R* LAp = reinterpret_cast<R*>(base + lay.wk + lay.lb);
  R* Mb = reinterpret_cast<R*>(base + lay.wk + lay.lb + lay.la);
  LeafSync ls;
  ls.sync = reinterpret_cast<int*>(base + lay.wk + lay.lb + lay.la + lay.mb);
  ls.stride = batch > 1 ? (int64_t)(lay.total / sizeof(int)) : 0;
  ls.nblocks = leaf_blocks(m, n);
  ls.eb = base + lay.wk + lay.lb + lay.la + lay.mb + lay.sync;
  ls.polls = g_wait_polls.load();
  BandBuffers<R> bb;
  bb.Wk = Wk;
  bb.LBp = LBp;
  bb.LAp = LAp;
  bb.Mb = Mb;

  // the solve runs in code units: U = W / s, the factor on the scaled side
  // conjugated by the scales
  const R* scB = scale_mode == 1 ? scales : nullptr;
  const R* scA = scale_mode == 2 ? scales : nullptr;
  if (launch_pack_w<R>(g, W, ldw, scales, scale_mode, Wk, s, ls) != hipSuccess) return BAKRON_EHIP;
  if (launch_pack_l<R>(g, true, LB, ldlb, scB, LBp, s) != hipSuccess) return BAKRON_EHIP;
  if (launch_pack_l<R>(g, false, LA, ldla, scA, LAp, s) != hipSuccess) return BAKRON_EHIP;

  LeafParams<R> lp;
  lp.lo = unb ? -std::numeric_limits<R>::infinity() : (R)lo;
  lp.hi = unb ? std::numeric_limits<R>::infinity() : (R)hi;
  lp.unbounded = unb;
  lp.scale_mode = scale_mode;
  lp.scales = scales;
  lp.V = V;
  lp.ldv = ldv;
  lp.Wt = Wt;
  lp.ldwt = ldwt;

  const std::vector<Op> ops = schedule_for(m, n);
  // optional per-launch timing of every leaf and band launch (measurement
  // entry point)
  std::vector<hipEvent_t> ev;
  if (op_ms) {
    ev.assign(2 * ops.size(), nullptr);
    for (auto& e : ev)
      if (hipEventCreate(&e) != hipSuccess) {
        for (auto& d : ev)
          if (d) (void)hipEventDestroy(d);
        return BAKRON_EHIP;
      }
  }
  size_t evi = 0;
  int rc = BAKRON_OK;
  for (const Op& op : ops) {
    hipError_t e = hipSuccess;
    const bool timed = op_ms != nullptr;
    hipEvent_t e0 = timed ? ev[evi] : nullptr, e1 = timed ? ev[evi + 1] : nullptr;
    switch (op.kind) {
      case OP_LEAF:
        e = launch_leaf_rows<R>(g, op.k, op.mid, op.k / kLeafBlock, Wk, LBp, LAp, lp, ls, s, e0,
                                e1);
        break;
      case OP_BAND1:
        e = launch_node_band<R>(g, op.k, op.mid, op.l, 1, bb, s, e0, e1);
        break;
      case OP_BAND2:
        e = launch_node_band<R>(g, op.k, op.mid, op.l, 2, bb, s, e0, e1);
        break;
    }
    if (e != hipSuccess) { rc = BAKRON_EHIP; break; }
    if (timed) evi += 2;
  }
  if (op_ms) {
    if (rc == BAKRON_OK && !ev.empty() && hipEventSynchronize(ev.back()) != hipSuccess)
      rc = BAKRON_EHIP;
    if (rc == BAKRON_OK) rc = read_wait_status(ws, lay, m, n, batch, s);
    for (size_t i = 0; i < ops.size(); ++i) {
      op_ms[i] = -1.0;
      if (rc == BAKRON_OK) {
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, ev[2 * i], ev[2 * i + 1]) != hipSuccess) rc = BAKRON_EHIP;
        op_ms[i] = ms;
      }
    }
    for (auto& d : ev) (void)hipEventDestroy(d);
  }
  return rc;
}

// ---- factor ---------------------------------------------------------------
// Per side of order D: X (D^2), Y (D^2) and the per-size-class C21 Y11
// buffers (factor_tmp_layout) in doubles; one info word per side. When
// m == n both sides run in the same launches.
size_t side_bytes(int64_t D) {
  return 2 * align_up((size_t)(D * D) * 8) + align_up((size_t)factor_tmp_layout(D, nullptr) * 8);
}

constexpr int64_t kHelperMinOrder = 8192;

// Helper stream and events of one factor set (created per call; the call
// is synchronous, so they are destroyed after its final synchronisation).
struct HelperStream {
  std::vector<hipEvent_t> ev;
  FactorAux fa;
  int init(int64_t order) {
    // creating the stream and its events costs ~0.1 ms per call: measured on
    // one box, the overlap loses 7 % at order 2048 and 2-4 % at 4096, breaks
    // even at 8192 and gains 3 % at 14336
    if (order <= kHelperMinOrder) return BAKRON_OK;
    const int64_t ne = factor_helper_events(order);
    if (ne == 0) return BAKRON_OK;
    if (hipStreamCreateWithFlags(&fa.ts, hipStreamNonBlocking) != hipSuccess) {
      fa.ts = nullptr;
      return BAKRON_EHIP;
    }
    ev.assign((size_t)ne, nullptr);
    for (auto& e : ev)
      if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) return BAKRON_EHIP;
    fa.ev = ev.data();
    fa.nev = (int)ev.size();
    return BAKRON_OK;
  }
  FactorAux* get() { return fa.ts ? &fa : nullptr; }
  ~HelperStream() {
    for (auto& e : ev)
      if (e) (void)hipEventDestroy(e);
    if (fa.ts) (void)hipStreamDestroy(fa.ts);
  }
};

struct FactorLayout {
  size_t a, b, info, total;  // a, b: one side's bytes; info: 2 * batch words
};
FactorLayout factor_layout(int64_t m, int64_t n, int64_t batch = 1) {
  FactorLayout L;
  L.a = side_bytes(n);
  L.b = side_bytes(m);
  L.info = align_up(2 * (size_t)batch * sizeof(int32_t));
  L.total = (size_t)batch * (L.a + L.b) + L.info + kAlign;
  return L;
}

FactorSide carve_side(char* base, int64_t D, int32_t* info) {
  FactorSide f;
  f.X = reinterpret_cast<double*>(base);
  f.Y = reinterpret_cast<double*>(base + align_up((size_t)(D * D) * 8));
  f.Tmp = reinterpret_cast<double*>(base + 2 * align_up((size_t)(D * D) * 8));
  f.info = info;
  return f;
}

// Caller strides (elements) between the matrices of a batched factor.
struct FactorStrides {
  int64_t a, b, la, lb, da, db;
};

// Factor `batch` pairs (A, B) of orders (n, m). Workspace: the batch's A
// sides (side_bytes(n) each), then its B sides, then 2 * batch info words
// (A sides first). When m == n all 2 * batch sides form one set and share
// every launch; otherwise the A sides and the B sides are two sets.
// bad (host, nullable) receives {problem, side, pivot} of the first failure.
template <typename R>
int factor_impl(int64_t batch, int64_t m, int64_t n, const R* A, int64_t lda, const R* B,
                int64_t ldb, R* LA, int64_t ldla, R* LB, int64_t ldlb, R* dA, R* dB,
                const FactorStrides& st, void* ws, int64_t* bad, hipStream_t s) {
  const FactorLayout lay = factor_layout(m, n, batch);
  char* base = static_cast<char*>(ws);
  char* base_b = base + (size_t)batch * lay.a;
  int32_t* info = reinterpret_cast<int32_t*>(base_b + (size_t)batch * lay.b);
  const FactorSide sa = carve_side(base, n, info);
  const FactorSide sb = carve_side(base_b, m, info + batch);
  const int nb = (int)batch;
  const int64_t za = (int64_t)(lay.a / 8), zb = (int64_t)(lay.b / 8);
  // helper streams and events of this call (created here, destroyed when the
  // call returns, after the final synchronisation)
  struct Aux {
    hipStream_t st = nullptr;
    hipEvent_t ready = nullptr, done = nullptr;
    ~Aux() {
      if (ready) (void)hipEventDestroy(ready);
      if (done) (void)hipEventDestroy(done);
      if (st) (void)hipStreamDestroy(st);
    }
  } aux;
  // each set's large nodes form their C21 Y11 products on a helper stream
  HelperStream ha, hb;
  // Once anything is enqueued, an error return first waits for every stream
  // of the call, so that no kernel still uses the caller's workspace (or a
  // helper stream about to be destroyed) after the call returns.
  auto fail = [&]() {
    (void)hipStreamSynchronize(s);
    if (aux.st) (void)hipStreamSynchronize(aux.st);
    if (ha.fa.ts) (void)hipStreamSynchronize(ha.fa.ts);
    if (hb.fa.ts) (void)hipStreamSynchronize(hb.fa.ts);
    return BAKRON_EHIP;
  };
  if (ha.init(n) != BAKRON_OK) return BAKRON_EHIP;
  if (m != n && hb.init(m) != BAKRON_OK) return BAKRON_EHIP;
  if (m != n && m > 0 && n > 0) {
    if (hipStreamCreateWithFlags(&aux.st, hipStreamNonBlocking) != hipSuccess) {
      aux.st = nullptr;
      return BAKRON_EHIP;
    }
    if (hipEventCreateWithFlags(&aux.ready, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&aux.done, hipEventDisableTiming) != hipSuccess)
      return BAKRON_EHIP;
  }
  if (launch_fill_i32(info, 2 * batch, INT_MAX, s) != hipSuccess) return fail();
  if (n > 0 && launch_load_reversed<R>(n, A, lda, st.a, sa.X, za, nb, s) != hipSuccess)
    return fail();
  if (m > 0 && launch_load_reversed<R>(m, B, ldb, st.b, sb.X, zb, nb, s) != hipSuccess)
    return fail();
  if (m == n) {
    // the B sides follow the A sides at the same stride: one set of 2 * batch
    if (factor_cholesky_inverse(n, FactorSet{sa, za, 2 * nb}, s, ha.get()) != hipSuccess)
      return fail();
  } else if (m > 0 && n > 0) {
    // orders differ, so the sides cannot share launches: the B set runs on a
    // stream of this call, concurrently with the A set (both sequences are
    // launch- and latency-bound and leave most of the GPU idle)
    if (hipEventRecord(aux.ready, s) != hipSuccess ||
        hipStreamWaitEvent(aux.st, aux.ready, 0) != hipSuccess)
      return fail();
    if (factor_cholesky_inverse(m, FactorSet{sb, zb, nb}, aux.st, hb.get()) != hipSuccess)
      return fail();
    if (hipEventRecord(aux.done, aux.st) != hipSuccess) return fail();
    if (factor_cholesky_inverse(n, FactorSet{sa, za, nb}, s, ha.get()) != hipSuccess)
      return fail();
    if (hipStreamWaitEvent(s, aux.done, 0) != hipSuccess) return fail();
  } else {
    if (factor_cholesky_inverse(n, FactorSet{sa, za, nb}, s, ha.get()) != hipSuccess)
      return fail();
    if (factor_cholesky_inverse(m, FactorSet{sb, zb, nb}, s, hb.get()) != hipSuccess)
      return fail();
  }
  if (n > 0 &&
      launch_store_normalized<R>(n, sa.Y, za, LA, ldla, st.la, dA, st.da, nb, s) != hipSuccess)
    return fail();
  if (m > 0 &&
      launch_store_normalized<R>(m, sb.Y, zb, LB, ldlb, st.lb, dB, st.db, nb, s) != hipSuccess)
    return fail();
  std::vector<int32_t> hinfo((size_t)(2 * batch), INT_MAX);
  if (hipMemcpyAsync(hinfo.data(), info, hinfo.size() * sizeof(int32_t), hipMemcpyDeviceToHost,
                     s) != hipSuccess)
    return fail();
  if (hipStreamSynchronize(s) != hipSuccess) return fail();
  for (int64_t z = 0; z < batch; ++z)
    for (int side = 0; side < 2; ++side) {
      const int32_t v = hinfo[(size_t)(side * batch + z)];
      if (v != INT_MAX) {
        if (bad) {
          bad[0] = z;
          bad[1] = side;
          bad[2] = v;
        }
        return BAKRON_ENOTSPD;
      }
    }
  return BAKRON_OK;
}

// ---- loss -----------------------------------------------------------------
struct LossLayout {
  size_t a, b, d, be, part, total;
  int64_t nparts;
};
LossLayout loss_layout(int64_t m, int64_t n) {
  LossLayout L;
  L.a = align_up((size_t)(n * n) * 8);
  L.b = align_up((size_t)(m * m) * 8);
  L.d = align_up((size_t)(m * n) * 8);
  L.be = L.d;
  L.nparts = gemm64_num_blocks(m, m);
  L.part = align_up((size_t)(L.nparts > 0 ? L.nparts : 1) * 8);
  L.total = L.a + L.b + L.d + L.be + L.part + kAlign;
  return L;
}

// Caller strides (elements) between the problems of a batched loss.
struct LossStrides {
  int64_t w, v, s, a, b;
};

// Loss of `batch` problems; workspace regions are batch copies of the
// single-problem layout's regions.
// Workspace of `batch` losses of one shape: the float64 copies of A (one
// when every problem shares A, share_a), of B, D = W - s V and D A per
// problem, and the per-problem partial sums.
size_t loss_ws_bytes(int64_t batch, int64_t m, int64_t n, bool share_a) {
  const LossLayout lay = loss_layout(m, n);
  const size_t nb = (size_t)batch;
  return (share_a ? 1 : nb) * lay.a + nb * (lay.b + lay.d + lay.be + lay.part) + kAlign;
}

template <typename R>
int loss_impl(int64_t batch, int64_t m, int64_t n, const R* W, int64_t ldw, const int32_t* V,
              int64_t ldv, int scale_mode, const R* scales, const R* A, int64_t lda, const R* B,
              int64_t ldb, const LossStrides& st, double* loss, void* ws, hipStream_t s) {
  const LossLayout lay = loss_layout(m, n);
  const size_t nb = (size_t)batch;
  // a shared A (stride 0) is converted once and read by every problem
  const bool share_a = st.a == 0;
  const size_t na = share_a ? 1 : nb;
  char* base = static_cast<char*>(ws);
  double* A64 = reinterpret_cast<double*>(base);
  double* B64 = reinterpret_cast<double*>(base + na * lay.a);
  double* D = reinterpret_cast<double*>(base + na * lay.a + nb * lay.b);
  double* BE = reinterpret_cast<double*>(base + na * lay.a + nb * (lay.b + lay.d));
  double* part = reinterpret_cast<double*>(base + na * lay.a + nb * (lay.b + lay.d + lay.be));
  const int64_t za = share_a ? 0 : (int64_t)(lay.a / 8), zb = (int64_t)(lay.b / 8),
                zd = (int64_t)(lay.d / 8);
  const int64_t zp = (int64_t)(lay.part / 8);
  const int bt = (int)batch;
  if (launch_sym_to_f64<R>(n, A, lda, A64, s, share_a ? 1 : bt, st.a, za) != hipSuccess)
    return BAKRON_EHIP;
  if (launch_sym_to_f64<R>(m, B, ldb, B64, s, bt, st.b, zb) != hipSuccess) return BAKRON_EHIP;
  if (launch_residual_f64<R>(m, n, W, ldw, V, ldv, scale_mode, scales, D, s, bt,
                             ResidualStrides{st.w, st.v, st.s, zd}) != hipSuccess)
    return BAKRON_EHIP;
  // tr(B D A D^T) = sum_ij B_ij H_ij with H = (D A) D^T symmetric: G = D A in
  // full, then H on its lower blocks only, reduced against B with weight 2
  // below the diagonal and 1 on it (3 m n^2-type products instead of 4)
  Gemm64Args g1{};
  g1.M = m; g1.N = n; g1.K = n; g1.batch = bt;
  g1.A = D; g1.lda = n; g1.sA = zd;
  g1.B = A64; g1.ldb = n; g1.sB = za; g1.transB = 0;
  g1.C = BE; g1.ldc = n; g1.sC = zd;
  g1.alpha = 1.0; g1.beta = 0.0;
  if (launch_gemm64(g1, s) != hipSuccess) return BAKRON_EHIP;
  Gemm64Args g2{};
  g2.M = m; g2.N = m; g2.K = n; g2.batch = bt;
  g2.A = BE; g2.lda = n; g2.sA = zd;
  g2.B = D; g2.ldb = n; g2.sB = zd; g2.transB = 1;
  g2.lower_out = 1;
  g2.alpha = 1.0;
  g2.dot = B64; g2.lddot = m; g2.sDot = zb; g2.partial = part; g2.sPart = zp; g2.sym_dot = 1;
  if (launch_gemm64(g2, s) != hipSuccess) return BAKRON_EHIP;
  if (launch_sum_partials(part, gemm64_partials(g2), loss, s, bt, zp) != hipSuccess)
    return BAKRON_EHIP;
  return BAKRON_OK;
}

// ---- no-allocation solve ----------------------------------------------------
// Scratch of bakron_solve_noalloc: one array per GPU, held by that GPU from
// the library's load until the process ends. In host code `scratch` names a
// host-side stand-in, never the device memory: its per-device address comes
// from hipGetSymbolAddress, taken once per device (with that device current)
// on the entry point's first call there, and only that address is used.
static_assert(BAKRON_NOALLOC_SCRATCH_BYTES % kAlign == 0, "scratch size must keep 256-byte alignment");
static __device__ __align__(256) unsigned char scratch[BAKRON_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address (nullptr and *rc set on failure).
void* device_scratch(int* rc) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *rc = BAKRON_EHIP;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      *rc = BAKRON_EHIP;
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

const char* bakron_status_string(int status) {
  switch (status) {
    case BAKRON_OK: return "ok";
    case BAKRON_EINVAL: return "invalid argument";
    case BAKRON_ENOTSPD: return "matrix is not numerically positive definite";
    case BAKRON_EHIP: return "HIP runtime or kernel launch error";
    case BAKRON_EWAIT: return "a solve's dependency wait gave up (its results are invalid)";
    default: return "unknown status";
  }
}

int bakron_abi_version(void) { return 1; }

int bakron_tile_size(int dtype) { return dtype_ok(dtype) ? kTile : 0; }

size_t bakron_factor_workspace_bytes(int dtype, int64_t m, int64_t n) {
  if (!dtype_ok(dtype) || m < 0 || n < 0) return 0;
  return factor_layout(m, n).total;
}

int bakron_factor(int dtype, int64_t m, int64_t n, const void* A, int64_t lda, const void* B,
                  int64_t ldb, void* LA, int64_t ldla, void* LB, int64_t ldlb, void* dA, void* dB,
                  void* workspace, size_t workspace_bytes, int64_t* bad_pivot, void* stream) {
  if (bad_pivot) {
    bad_pivot[0] = -1;
    bad_pivot[1] = -1;
  }
  if (!dtype_ok(dtype) || m < 0 || n < 0) return BAKRON_EINVAL;
  if (m > INT_MAX / 2 || n > INT_MAX / 2) return BAKRON_EINVAL;
  if (m == 0 && n == 0) return BAKRON_OK;
  if (n > 0 && (!A || !LA || lda < n || ldla < n)) return BAKRON_EINVAL;
  if (m > 0 && (!B || !LB || ldb < m || ldlb < m)) return BAKRON_EINVAL;
  if (!workspace || workspace_bytes < bakron_factor_workspace_bytes(dtype, m, n))
    return BAKRON_EINVAL;
  if ((reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0) return BAKRON_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const FactorStrides st = {0, 0, 0, 0, 0, 0};
  int64_t bad3[3] = {-1, -1, -1};
  int rc;
  if (dtype == BAKRON_F32)
    rc = factor_impl<float>(1, m, n, (const float*)A, lda, (const float*)B, ldb, (float*)LA, ldla,
                            (float*)LB, ldlb, (float*)dA, (float*)dB, st, workspace, bad3, s);
  else
    rc = factor_impl<double>(1, m, n, (const double*)A, lda, (const double*)B, ldb, (double*)LA,
                             ldla, (double*)LB, ldlb, (double*)dA, (double*)dB, st, workspace,
                             bad3, s);
  if (rc == BAKRON_ENOTSPD && bad_pivot) {
    bad_pivot[0] = bad3[1];
    bad_pivot[1] = bad3[2];
  }
  return rc;
}

size_t bakron_factor_batched_workspace_bytes(int dtype, int64_t batch, int64_t m, int64_t n) {
  if (!dtype_ok(dtype) || batch < 0 || m < 0 || n < 0) return 0;
  if (batch == 0) return 0;
  const FactorLayout one = factor_layout(m, n, 1);
  if ((one.a + one.b) > (std::numeric_limits<size_t>::max() / 2) / (size_t)batch) return 0;
  return factor_layout(m, n, batch).total;
}

int bakron_factor_batched(int dtype, int64_t batch, int64_t m, int64_t n, const void* A,
                          int64_t lda, int64_t stride_a, const void* B, int64_t ldb,
                          int64_t stride_b, void* LA, int64_t ldla, int64_t stride_la, void* LB,
                          int64_t ldlb, int64_t stride_lb, void* dA, int64_t stride_da, void* dB,
                          int64_t stride_db, void* workspace, size_t workspace_bytes,
                          int64_t* bad_pivot, void* stream) {
  if (bad_pivot) bad_pivot[0] = bad_pivot[1] = bad_pivot[2] = -1;
  if (!dtype_ok(dtype) || batch < 0 || m < 0 || n < 0) return BAKRON_EINVAL;
  // both sides of every pair may share one launch: 2 * batch problems
  if (batch > kMaxBatch / 2) return BAKRON_EINVAL;
  if (m > INT_MAX / 2 || n > INT_MAX / 2) return BAKRON_EINVAL;
  if (batch == 0 || (m == 0 && n == 0)) return BAKRON_OK;
  if (n > 0 && (!A || !LA || lda < n || ldla < n)) return BAKRON_EINVAL;
  if (m > 0 && (!B || !LB || ldb < m || ldlb < m)) return BAKRON_EINVAL;
  if (stride_a < 0 || stride_b < 0) return BAKRON_EINVAL;
  if (batch > 1) {
    // outputs of different problems must not overlap
    if (n > 0 && stride_la < (n - 1) * ldla + n) return BAKRON_EINVAL;
    if (m > 0 && stride_lb < (m - 1) * ldlb + m) return BAKRON_EINVAL;
    if (dA && n > 0 && stride_da < n) return BAKRON_EINVAL;
    if (dB && m > 0 && stride_db < m) return BAKRON_EINVAL;
    const int64_t big = std::max(std::max(std::max(stride_a, stride_b), std::max(stride_la, stride_lb)),
                                 std::max(stride_da, stride_db));
    if (big > std::numeric_limits<int64_t>::max() / 2 / (batch - 1)) return BAKRON_EINVAL;
  }
  const size_t need = bakron_factor_batched_workspace_bytes(dtype, batch, m, n);
  if (!workspace || need == 0 || workspace_bytes < need) return BAKRON_EINVAL;
  if ((reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0) return BAKRON_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const FactorStrides st = {stride_a, stride_b, stride_la, stride_lb, stride_da, stride_db};
  if (dtype == BAKRON_F32)
    return factor_impl<float>(batch, m, n, (const float*)A, lda, (const float*)B, ldb, (float*)LA,
                              ldla, (float*)LB, ldlb, (float*)dA, (float*)dB, st, workspace,
                              bad_pivot, s);
  return factor_impl<double>(batch, m, n, (const double*)A, lda, (const double*)B, ldb,
                             (double*)LA, ldla, (double*)LB, ldlb, (double*)dA, (double*)dB, st,
                             workspace, bad_pivot, s);
}

size_t bakron_solve_workspace_bytes(int dtype, int64_t m, int64_t n) {
  if (!dtype_ok(dtype) || m < 0 || n < 0) return 0;
  return solve_layout(dtype, m, n).total;
}

static int solve_entry(int dtype, int64_t m, int64_t n, const void* W, int64_t ldw, const void* LA,
                       int64_t ldla, const void* LB, int64_t ldlb, int32_t alpha_lo,
                       int32_t alpha_hi, int32_t unbounded, int scale_mode, const void* scales,
                       int32_t* V, int64_t ldv, void* Wt, int64_t ldwt, void* workspace,
                       size_t workspace_bytes, void* stream, double* op_ms, int64_t n_ops) {
  if (!dtype_ok(dtype) || m < 0 || n < 0) return BAKRON_EINVAL;
  if (m > INT_MAX / 2 || n > INT_MAX / 2) return BAKRON_EINVAL;
  if (m == 0 || n == 0) return BAKRON_OK;
  if (!W || !LA || !LB || !V) return BAKRON_EINVAL;
  if (ldw < n || ldla < n || ldlb < m || ldv < n) return BAKRON_EINVAL;
  if (Wt && ldwt < n) return BAKRON_EINVAL;
  if (!unbounded && alpha_lo > alpha_hi) return BAKRON_EINVAL;
  if (scale_mode == BAKRON_SCALE_NONE) {
    if (scales) return BAKRON_EINVAL;
  } else if (scale_mode == BAKRON_SCALE_ROW || scale_mode == BAKRON_SCALE_COL) {
    if (!scales) return BAKRON_EINVAL;
  } else {
    return BAKRON_EINVAL;
  }
  if (!workspace || workspace_bytes < bakron_solve_workspace_bytes(dtype, m, n))
    return BAKRON_EINVAL;
  if ((reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0) return BAKRON_EINVAL;
  if (op_ms && n_ops != (int64_t)schedule_for(m, n).size()) return BAKRON_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == BAKRON_F32)
    return solve_impl<float>(m, n, (const float*)W, ldw, (const float*)LA, ldla,
                             (const float*)LB, ldlb, alpha_lo, alpha_hi, unbounded, scale_mode,
                             (const float*)scales, V, ldv, (float*)Wt, ldwt, workspace, s, op_ms);
  return solve_impl<double>(m, n, (const double*)W, ldw, (const double*)LA, ldla,
                            (const double*)LB, ldlb, alpha_lo, alpha_hi, unbounded, scale_mode,
                            (const double*)scales, V, ldv, (double*)Wt, ldwt, workspace, s, op_ms);
}

int bakron_solve(int dtype, int64_t m, int64_t n, const void* W, int64_t ldw, const void* LA,
                 int64_t ldla, const void* LB, int64_t ldlb, int32_t alpha_lo, int32_t alpha_hi,
                 int32_t unbounded, int scale_mode, const void* scales, int32_t* V, int64_t ldv,
                 void* Wt, int64_t ldwt, void* workspace, size_t workspace_bytes, void* stream) {
  return solve_entry(dtype, m, n, W, ldw, LA, ldla, LB, ldlb, alpha_lo, alpha_hi, unbounded,
                     scale_mode, scales, V, ldv, Wt, ldwt, workspace, workspace_bytes, stream,
                     nullptr, 0);
}

int bakron_solve_noalloc(int dtype, int64_t m, int64_t n, const void* W, int64_t ldw,
                         const void* LA, int64_t ldla, const void* LB, int64_t ldlb,
                         int32_t alpha_lo, int32_t alpha_hi, int32_t unbounded, int scale_mode,
                         const void* scales, int32_t* V, int64_t ldv, void* Wt, int64_t ldwt,
                         void* stream) {
  // the size check comes before any HIP call, so an oversized problem is
  // rejected without touching the device
  if (!dtype_ok(dtype) || m < 0 || n < 0) return BAKRON_EINVAL;
  if (m > INT_MAX / 2 || n > INT_MAX / 2) return BAKRON_EINVAL;
  if (m == 0 || n == 0) return BAKRON_OK;
  const size_t need = bakron_solve_workspace_bytes(dtype, m, n);
  if (need == 0 || need > (size_t)BAKRON_NOALLOC_SCRATCH_BYTES) return BAKRON_EINVAL;
  int rc = BAKRON_OK;
  void* ws = device_scratch(&rc);
  if (!ws) return rc;
  return solve_entry(dtype, m, n, W, ldw, LA, ldla, LB, ldlb, alpha_lo, alpha_hi, unbounded,
                     scale_mode, scales, V, ldv, Wt, ldwt, ws, (size_t)BAKRON_NOALLOC_SCRATCH_BYTES,
                     stream, nullptr, 0);
}

int bakron_solve_timed(int dtype, int64_t m, int64_t n, const void* W, int64_t ldw,
                       const void* LA, int64_t ldla, const void* LB, int64_t ldlb,
                       int32_t alpha_lo, int32_t alpha_hi, int32_t unbounded, int scale_mode,
                       const void* scales, int32_t* V, int64_t ldv, void* Wt, int64_t ldwt,
                       void* workspace, size_t workspace_bytes, void* stream, double* op_ms,
                       int64_t n_ops) {
  if (!op_ms) return BAKRON_EINVAL;
  return solve_entry(dtype, m, n, W, ldw, LA, ldla, LB, ldlb, alpha_lo, alpha_hi, unbounded,
                     scale_mode, scales, V, ldv, Wt, ldwt, workspace, workspace_bytes, stream,
                     op_ms, n_ops);
}

int bakron_solve_status(int dtype, int64_t batch, int64_t m, int64_t n, const void* workspace,
                        size_t workspace_bytes, void* stream) {
  if (!dtype_ok(dtype) || batch < 0 || batch > kMaxBatch || m < 0 || n < 0) return BAKRON_EINVAL;
  if (m > INT_MAX / 2 || n > INT_MAX / 2) return BAKRON_EINVAL;
  if (batch == 0 || m == 0 || n == 0) return BAKRON_OK;
  const SolveLayout lay = solve_layout(dtype, m, n);
  const void* ws = workspace;
  if (!ws) {
    // the no-allocation solve's scratch on the current device
    if (batch != 1 || lay.total > (size_t)BAKRON_NOALLOC_SCRATCH_BYTES) return BAKRON_EINVAL;
    int rc = BAKRON_OK;
    ws = device_scratch(&rc);
    if (!ws) return rc;
  } else if (workspace_bytes < (size_t)batch * lay.total) {
    return BAKRON_EINVAL;
  }
  return read_wait_status(ws, lay, m, n, batch, static_cast<hipStream_t>(stream));
}

int32_t bakron_debug_set_wait_polls(int32_t polls) {
  return g_wait_polls.exchange(polls < 0 ? kLeafWaitPolls : polls);
}

size_t bakron_solve_antidiag_workspace_bytes(int dtype, int64_t m, int64_t n) {
  if (!dtype_ok(dtype) || m < 0 || n < 0) return 0;
  if (m > INT_MAX / 2 || n > INT_MAX / 2) return 0;
  return antidiag_layout(esize(dtype), m, n).total;
}

int bakron_solve_antidiag(int dtype, int64_t m, int64_t n, const void* W, int64_t ldw,
                          const void* LA, int64_t ldla, const void* LB, int64_t ldlb,
                          int32_t alpha_lo, int32_t alpha_hi, int32_t unbounded, int scale_mode,
                          const void* scales, int32_t* V, int64_t ldv, void* Wt, int64_t ldwt,
                          void* workspace, size_t workspace_bytes, void* stream) {
  if (!dtype_ok(dtype) || m < 0 || n < 0) return BAKRON_EINVAL;
  if (m > INT_MAX / 2 || n > INT_MAX / 2) return BAKRON_EINVAL;
  if (m == 0 || n == 0) return BAKRON_OK;
  if (!W || !LA || !LB || !V) return BAKRON_EINVAL;
  if (ldw < n || ldla < n || ldlb < m || ldv < n) return BAKRON_EINVAL;
  if (Wt && ldwt < n) return BAKRON_EINVAL;
  if (!unbounded && alpha_lo > alpha_hi) return BAKRON_EINVAL;
  if (scale_mode == BAKRON_SCALE_NONE) {
    if (scales) return BAKRON_EINVAL;
  } else if (scale_mode == BAKRON_SCALE_ROW || scale_mode == BAKRON_SCALE_COL) {
    if (!scales) return BAKRON_EINVAL;
  } else {
    return BAKRON_EINVAL;
  }
  if (!workspace || workspace_bytes < bakron_solve_antidiag_workspace_bytes(dtype, m, n))
    return BAKRON_EINVAL;
  if ((reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0) return BAKRON_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (dtype == BAKRON_F32) {
    const float lo = unbounded ? -std::numeric_limits<float>::infinity() : (float)alpha_lo;
    const float hi = unbounded ? std::numeric_limits<float>::infinity() : (float)alpha_hi;
    e = launch_antidiag_solve<float>(m, n, (const float*)W, ldw, (const float*)LA, ldla,
                                     (const float*)LB, ldlb, lo, hi, scale_mode,
                                     (const float*)scales, V, ldv, (float*)Wt, ldwt, workspace, s);
  } else {
    const double lo = unbounded ? -std::numeric_limits<double>::infinity() : (double)alpha_lo;
    const double hi = unbounded ? std::numeric_limits<double>::infinity() : (double)alpha_hi;
    e = launch_antidiag_solve<double>(m, n, (const double*)W, ldw, (const double*)LA, ldla,
                                      (const double*)LB, ldlb, lo, hi, scale_mode,
                                      (const double*)scales, V, ldv, (double*)Wt, ldwt, workspace,
                                      s);
  }
  return e == hipSuccess ? BAKRON_OK : BAKRON_EHIP;
}

size_t bakron_solve_batched_workspace_bytes(int dtype, int64_t batch, int64_t m, int64_t n) {
  if (!dtype_ok(dtype) || batch < 0 || m < 0 || n < 0) return 0;
  const size_t one = solve_layout(dtype, m, n).total;
  if (batch > 0 && one > std::numeric_limits<size_t>::max() / (size_t)batch) return 0;
  return (size_t)batch * one;
}

int bakron_solve_batched(int dtype, int64_t batch, int64_t m, int64_t n, const void* W,
                         int64_t ldw, int64_t stride_w, const void* LA, int64_t ldla,
                         int64_t stride_la, const void* LB, int64_t ldlb, int64_t stride_lb,
                         int32_t alpha_lo, int32_t alpha_hi, int32_t unbounded, int scale_mode,
                         const void* scales, int64_t stride_s, int32_t* V, int64_t ldv,
                         int64_t stride_v, void* Wt, int64_t ldwt, int64_t stride_wt,
                         void* workspace, size_t workspace_bytes, void* stream) {
  if (!dtype_ok(dtype) || batch < 0 || m < 0 || n < 0) return BAKRON_EINVAL;
  if (batch > kMaxBatch) return BAKRON_EINVAL;
  if (m > INT_MAX / 2 || n > INT_MAX / 2) return BAKRON_EINVAL;
  if (batch == 0 || m == 0 || n == 0) return BAKRON_OK;
  if (!W || !LA || !LB || !V) return BAKRON_EINVAL;
  if (ldw < n || ldla < n || ldlb < m || ldv < n) return BAKRON_EINVAL;
  if (Wt && ldwt < n) return BAKRON_EINVAL;
  if (!unbounded && alpha_lo > alpha_hi) return BAKRON_EINVAL;
  if (scale_mode == BAKRON_SCALE_NONE) {
    if (scales) return BAKRON_EINVAL;
  } else if (scale_mode == BAKRON_SCALE_ROW || scale_mode == BAKRON_SCALE_COL) {
    if (!scales) return BAKRON_EINVAL;
  } else {
    return BAKRON_EINVAL;
  }
  // inputs may be shared (stride 0); the outputs of different problems must
  // not overlap
  if (stride_w < 0 || stride_la < 0 || stride_lb < 0 || stride_s < 0) return BAKRON_EINVAL;
  const int64_t span_v = (m - 1) * ldv + n, span_wt = Wt ? (m - 1) * ldwt + n : 0;
  if (batch > 1 && (stride_v < span_v || (Wt && stride_wt < span_wt))) return BAKRON_EINVAL;
  const int64_t top = batch - 1;
  const int64_t big = std::max(std::max(std::max(stride_w, stride_la), std::max(stride_lb, stride_s)),
                               std::max(batch > 1 ? stride_v : 0, Wt && batch > 1 ? stride_wt : 0));
  if (top > 0 && big > std::numeric_limits<int64_t>::max() / 2 / top) return BAKRON_EINVAL;
  const size_t need = bakron_solve_batched_workspace_bytes(dtype, batch, m, n);
  if (!workspace || need == 0 || workspace_bytes < need) return BAKRON_EINVAL;
  if ((reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0) return BAKRON_EINVAL;
  BatchStrides bs = {stride_w, stride_s, stride_la, stride_lb, stride_v, Wt ? stride_wt : 0, 0};
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == BAKRON_F32)
    return solve_impl<float>(m, n, (const float*)W, ldw, (const float*)LA, ldla,
                             (const float*)LB, ldlb, alpha_lo, alpha_hi, unbounded, scale_mode,
                             (const float*)scales, V, ldv, (float*)Wt, ldwt, workspace, s, nullptr,
                             (int)batch, &bs);
  return solve_impl<double>(m, n, (const double*)W, ldw, (const double*)LA, ldla,
                            (const double*)LB, ldlb, alpha_lo, alpha_hi, unbounded, scale_mode,
                            (const double*)scales, V, ldv, (double*)Wt, ldwt, workspace, s,
                            nullptr, (int)batch, &bs);
}

int64_t bakron_solve_schedule(int dtype, int64_t m, int64_t n, int32_t* ops, int64_t max_ops) {
  if (!dtype_ok(dtype) || m < 0 || n < 0 || max_ops < 0) return BAKRON_EINVAL;
  if (m > INT_MAX / 2 || n > INT_MAX / 2) return BAKRON_EINVAL;
  const std::vector<Op> sch = schedule_for(m, n);
  if (ops) {
    const int64_t cnt = (int64_t)sch.size() < max_ops ? (int64_t)sch.size() : max_ops;
    for (int64_t i = 0; i < cnt; ++i) {
      ops[4 * i + 0] = sch[i].kind;
      ops[4 * i + 1] = sch[i].k;
      ops[4 * i + 2] = sch[i].mid;
      ops[4 * i + 3] = sch[i].l;
    }
  }
  return (int64_t)sch.size();
}

size_t bakron_loss_workspace_bytes(int dtype, int64_t m, int64_t n) {
  if (!dtype_ok(dtype) || m < 0 || n < 0) return 0;
  return loss_layout(m, n).total;
}

int bakron_loss(int dtype, int64_t m, int64_t n, const void* W, int64_t ldw, const int32_t* V,
                int64_t ldv, int scale_mode, const void* scales, const void* A, int64_t lda,
                const void* B, int64_t ldb, double* loss, void* workspace, size_t workspace_bytes,
                void* stream) {
  if (!dtype_ok(dtype) || m < 0 || n < 0) return BAKRON_EINVAL;
  if (!loss) return BAKRON_EINVAL;
  if (m > 0 && n > 0) {
    if (!W || !V || !A || !B) return BAKRON_EINVAL;
    if (ldw < n || ldv < n || lda < n || ldb < m) return BAKRON_EINVAL;
  }
  if (scale_mode == BAKRON_SCALE_NONE) {
    if (scales) return BAKRON_EINVAL;
  } else if (scale_mode == BAKRON_SCALE_ROW || scale_mode == BAKRON_SCALE_COL) {
    if (!scales) return BAKRON_EINVAL;
  } else {
    return BAKRON_EINVAL;
  }
  if (!workspace || workspace_bytes < bakron_loss_workspace_bytes(dtype, m, n))
    return BAKRON_EINVAL;
  if ((reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0) return BAKRON_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (m == 0 || n == 0) {
    // empty problem: loss 0, written by the same reduction kernel over no partials
    return launch_sum_partials(nullptr, 0, loss, s) == hipSuccess ? BAKRON_OK : BAKRON_EHIP;
  }
  const LossStrides st = {0, 0, 0, 0, 0};
  if (dtype == BAKRON_F32)
    return loss_impl<float>(1, m, n, (const float*)W, ldw, V, ldv, scale_mode,
                            (const float*)scales, (const float*)A, lda, (const float*)B, ldb, st,
                            loss, workspace, s);
  return loss_impl<double>(1, m, n, (const double*)W, ldw, V, ldv, scale_mode,
                           (const double*)scales, (const double*)A, lda, (const double*)B, ldb, st,
                           loss, workspace, s);
}

size_t bakron_loss_batched_workspace_bytes(int dtype, int64_t batch, int64_t m, int64_t n) {
  if (!dtype_ok(dtype) || batch < 0 || m < 0 || n < 0) return 0;
  const size_t one = loss_layout(m, n).total;
  if (batch > 0 && one > std::numeric_limits<size_t>::max() / (size_t)batch) return 0;
  return (size_t)batch * one;
}

int bakron_loss_batched(int dtype, int64_t batch, int64_t m, int64_t n, const void* W,
                        int64_t ldw, int64_t stride_w, const int32_t* V, int64_t ldv,
                        int64_t stride_v, int scale_mode, const void* scales, int64_t stride_s,
                        const void* A, int64_t lda, int64_t stride_a, const void* B, int64_t ldb,
                        int64_t stride_b, double* loss, void* workspace, size_t workspace_bytes,
                        void* stream) {
  if (!dtype_ok(dtype) || batch < 0 || m < 0 || n < 0) return BAKRON_EINVAL;
  if (batch > kMaxBatch || m > INT_MAX / 2 || n > INT_MAX / 2) return BAKRON_EINVAL;
  if (batch == 0) return BAKRON_OK;
  if (!loss) return BAKRON_EINVAL;
  if (m > 0 && n > 0) {
    if (!W || !V || !A || !B) return BAKRON_EINVAL;
    if (ldw < n || ldv < n || lda < n || ldb < m) return BAKRON_EINVAL;
  }
  if (scale_mode == BAKRON_SCALE_NONE) {
    if (scales) return BAKRON_EINVAL;
  } else if (scale_mode == BAKRON_SCALE_ROW || scale_mode == BAKRON_SCALE_COL) {
    if (!scales) return BAKRON_EINVAL;
  } else {
    return BAKRON_EINVAL;
  }
  if (stride_w < 0 || stride_v < 0 || stride_s < 0 || stride_a < 0 || stride_b < 0)
    return BAKRON_EINVAL;
  if (batch > 1) {
    const int64_t big = std::max(std::max(std::max(stride_w, stride_v), std::max(stride_s, stride_a)),
                                 stride_b);
    if (big > std::numeric_limits<int64_t>::max() / 2 / (batch - 1)) return BAKRON_EINVAL;
  }
  const size_t need = bakron_loss_batched_workspace_bytes(dtype, batch, m, n);
  if (!workspace || need == 0 || workspace_bytes < need) return BAKRON_EINVAL;
  if ((reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0) return BAKRON_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (m == 0 || n == 0) {
    // empty problems: every loss 0, written by the same reduction over no partials
    return launch_sum_partials(nullptr, 0, loss, s, (int)batch, 0) == hipSuccess ? BAKRON_OK
                                                                                : BAKRON_EHIP;
  }
  const LossStrides st = {stride_w, stride_v, stride_s, stride_a, stride_b};
  if (dtype == BAKRON_F32)
    return loss_impl<float>(batch, m, n, (const float*)W, ldw, V, ldv, scale_mode,
                            (const float*)scales, (const float*)A, lda, (const float*)B, ldb, st,
                            loss, workspace, s);
  return loss_impl<double>(batch, m, n, (const double*)W, ldw, V, ldv, scale_mode,
                           (const double*)scales, (const double*)A, lda, (const double*)B, ldb, st,
                           loss, workspace, s);
}

// ---- block-diagonal output factor ------------------------------------------
// B = blockdiag(B_0 .. B_{h-1}) of h blocks of order b = m / h. Then B^-1 and
// its Cholesky factor are block-diagonal too, L^B[p][i] = 0 unless rows p and
// i share a block, so an error reaches only rows of its own block: the solve
// splits exactly into h problems of b x n that share L^A, and the loss into
// sum_h tr(B_h D_h A D_h^T). Each call maps onto the batched machinery (one
// set of launches for all heads), which never touches the zero blocks.

static bool heads_ok(int64_t heads, int64_t m) {
  return heads >= 1 && heads <= kMaxBatch / 2 && m % heads == 0;
}

size_t bakron_factor_blockdiag_workspace_bytes(int dtype, int64_t heads, int64_t m, int64_t n) {
  if (!dtype_ok(dtype) || m < 0 || n < 0 || !heads_ok(heads, m)) return 0;
  const size_t fa = factor_layout(0, n, 1).total;
  const size_t fb = factor_layout(m / heads, 0, heads).total;
  return fa > fb ? fa : fb;
}

int bakron_factor_blockdiag(int dtype, int64_t heads, int64_t m, int64_t n, const void* A,
                            int64_t lda, const void* B, int64_t ldb, int64_t stride_b, void* LA,
                            int64_t ldla, void* LB, int64_t ldlb, int64_t stride_lb, void* dA,
                            void* dB, void* workspace, size_t workspace_bytes,
                            int64_t* bad_pivot, void* stream) {
  if (bad_pivot) bad_pivot[0] = bad_pivot[1] = bad_pivot[2] = -1;
  if (!dtype_ok(dtype) || m < 0 || n < 0 || !heads_ok(heads, m)) return BAKRON_EINVAL;
  if (m > INT_MAX / 2 || n > INT_MAX / 2) return BAKRON_EINVAL;
  const int64_t b = m / heads;
  if (n > 0 && (!A || !LA || lda < n || ldla < n)) return BAKRON_EINVAL;
  if (b > 0 && (!B || !LB || ldb < b || ldlb < b)) return BAKRON_EINVAL;
  if (b > 0 && heads > 1 && (stride_b < 0 || stride_lb < (b - 1) * ldlb + b)) return BAKRON_EINVAL;
  if (b > 0 && heads > 1 && std::max(stride_b, stride_lb) > std::numeric_limits<int64_t>::max() / 2 / (heads - 1))
    return BAKRON_EINVAL;
  const size_t need = bakron_factor_blockdiag_workspace_bytes(dtype, heads, m, n);
  if (!workspace || workspace_bytes < need) return BAKRON_EINVAL;
  if ((reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0) return BAKRON_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const FactorStrides sta = {0, 0, 0, 0, 0, 0};
  const FactorStrides stb = {0, stride_b, 0, stride_lb, 0, b};
  int64_t bad3[3] = {-1, -1, -1};
  int rc = BAKRON_OK;
  // the input side (one factor of order n), then the h output blocks in the
  // same launches (the batched factor with no input side); both synchronous
  if (n > 0) {
    rc = dtype == BAKRON_F32
             ? factor_impl<float>(1, 0, n, (const float*)A, lda, nullptr, 1, (float*)LA, ldla,
                                  nullptr, 1, (float*)dA, nullptr, sta, workspace, bad3, s)
             : factor_impl<double>(1, 0, n, (const double*)A, lda, nullptr, 1, (double*)LA, ldla,
                                   nullptr, 1, (double*)dA, nullptr, sta, workspace, bad3, s);
    if (rc == BAKRON_ENOTSPD && bad_pivot) {
      bad_pivot[0] = 0;
      bad_pivot[1] = -1;
      bad_pivot[2] = bad3[2];
    }
    if (rc != BAKRON_OK) return rc;
  }
  if (b > 0) {
    rc = dtype == BAKRON_F32
             ? factor_impl<float>(heads, b, 0, nullptr, 1, (const float*)B, ldb, nullptr, 1,
                                  (float*)LB, ldlb, nullptr, (float*)dB, stb, workspace, bad3, s)
             : factor_impl<double>(heads, b, 0, nullptr, 1, (const double*)B, ldb, nullptr, 1,
                                   (double*)LB, ldlb, nullptr, (double*)dB, stb, workspace, bad3, s);
    if (rc == BAKRON_ENOTSPD && bad_pivot) {
      bad_pivot[0] = 1;
      bad_pivot[1] = bad3[0];
      bad_pivot[2] = bad3[2];
    }
  }
  return rc;
}

size_t bakron_solve_blockdiag_workspace_bytes(int dtype, int64_t heads, int64_t m, int64_t n) {
  if (!dtype_ok(dtype) || m < 0 || n < 0 || !heads_ok(heads, m)) return 0;
  return bakron_solve_batched_workspace_bytes(dtype, heads, m / heads, n);
}

int bakron_solve_blockdiag(int dtype, int64_t heads, int64_t m, int64_t n, const void* W,
                           int64_t ldw, const void* LA, int64_t ldla, const void* LB, int64_t ldlb,
                           int64_t stride_lb, int32_t alpha_lo, int32_t alpha_hi,
                           int32_t unbounded, int scale_mode, const void* scales, int32_t* V,
                           int64_t ldv, void* Wt, int64_t ldwt, void* workspace,
                           size_t workspace_bytes, void* stream) {
  if (!dtype_ok(dtype) || m < 0 || n < 0 || !heads_ok(heads, m)) return BAKRON_EINVAL;
  if (m > INT_MAX / 2 || n > INT_MAX / 2) return BAKRON_EINVAL;
  if (m == 0 || n == 0) return BAKRON_OK;
  if (ldw < n || ldv < n || (Wt && ldwt < n)) return BAKRON_EINVAL;
  const int64_t b = m / heads;
  // head h: rows [h b, (h + 1) b) of W, V, Wt and of the row scales; the
  // column scales and L^A are shared (stride 0)
  const int64_t ss = scale_mode == BAKRON_SCALE_ROW ? b : 0;
  return bakron_solve_batched(dtype, heads, b, n, W, ldw, b * ldw, LA, ldla, 0, LB, ldlb,
                              heads > 1 ? stride_lb : 0, alpha_lo, alpha_hi, unbounded, scale_mode,
                              scales, ss, V, ldv, b * ldv, Wt, ldwt, Wt ? b * ldwt : 0, workspace,
                              workspace_bytes, stream);
}

size_t bakron_loss_blockdiag_workspace_bytes(int dtype, int64_t heads, int64_t m, int64_t n) {
  if (!dtype_ok(dtype) || m < 0 || n < 0 || !heads_ok(heads, m)) return 0;
  return loss_ws_bytes(heads, m / heads, n, true) + align_up((size_t)heads * 8);
}

int bakron_loss_blockdiag(int dtype, int64_t heads, int64_t m, int64_t n, const void* W,
                          int64_t ldw, const int32_t* V, int64_t ldv, int scale_mode,
                          const void* scales, const void* A, int64_t lda, const void* B,
                          int64_t ldb, int64_t stride_b, double* loss, void* workspace,
                          size_t workspace_bytes, void* stream) {
  if (!dtype_ok(dtype) || m < 0 || n < 0 || !heads_ok(heads, m)) return BAKRON_EINVAL;
  if (m > INT_MAX / 2 || n > INT_MAX / 2) return BAKRON_EINVAL;
  if (!loss) return BAKRON_EINVAL;
  const int64_t b = m / heads;
  if (m > 0 && n > 0) {
    if (!W || !V || !A || !B) return BAKRON_EINVAL;
    if (ldw < n || ldv < n || lda < n || ldb < b) return BAKRON_EINVAL;
    if (heads > 1 && (stride_b < 0 || stride_b > std::numeric_limits<int64_t>::max() / 2 / (heads - 1)))
      return BAKRON_EINVAL;
  }
  if (scale_mode == BAKRON_SCALE_NONE) {
    if (scales) return BAKRON_EINVAL;
  } else if (scale_mode == BAKRON_SCALE_ROW || scale_mode == BAKRON_SCALE_COL) {
    if (!scales) return BAKRON_EINVAL;
  } else {
    return BAKRON_EINVAL;
  }
  const size_t need = bakron_loss_blockdiag_workspace_bytes(dtype, heads, m, n);
  if (!workspace || need == 0 || workspace_bytes < need) return BAKRON_EINVAL;
  if ((reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0) return BAKRON_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (m == 0 || n == 0)
    return launch_sum_partials(nullptr, 0, loss, s) == hipSuccess ? BAKRON_OK : BAKRON_EHIP;
  // per-head losses at the end of the workspace, then their sum in a fixed order
  double* per_head = reinterpret_cast<double*>(static_cast<char*>(workspace) +
                                               loss_ws_bytes(heads, b, n, true));
  const LossStrides st = {b * ldw, b * ldv, scale_mode == BAKRON_SCALE_ROW ? b : 0, 0,
                          heads > 1 ? stride_b : 0};
  const int rc =
      dtype == BAKRON_F32
          ? loss_impl<float>(heads, b, n, (const float*)W, ldw, V, ldv, scale_mode,
                             (const float*)scales, (const float*)A, lda, (const float*)B, ldb, st,
                             per_head, workspace, s)
          : loss_impl<double>(heads, b, n, (const double*)W, ldw, V, ldv, scale_mode,
                              (const double*)scales, (const double*)A, lda, (const double*)B, ldb,
                              st, per_head, workspace, s);
  if (rc != BAKRON_OK) return rc;
  return launch_sum_partials(per_head, heads, loss, s) == hipSuccess ? BAKRON_OK : BAKRON_EHIP;
}

int bakron_row_scales(int dtype, int64_t m, int64_t n, const void* W, int64_t ldw, int32_t hi,
                      void* scales, void* stream) {
  if (!dtype_ok(dtype) || m < 0 || n < 0 || hi <= 0) return BAKRON_EINVAL;
  if (m == 0) return BAKRON_OK;
  if (!scales || (n > 0 && (!W || ldw < n))) return BAKRON_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (dtype == BAKRON_F32)
    e = launch_row_scales<float>(m, n, (const float*)W, ldw, hi, (float*)scales, s);
  else
    e = launch_row_scales<double>(m, n, (const double*)W, ldw, hi, (double*)scales, s);
  return e == hipSuccess ? BAKRON_OK : BAKRON_EHIP;
}

int bakron_row_scales_mse(int dtype, int64_t m, int64_t n, const void* W, int64_t ldw,
                          int32_t alpha_lo, int32_t alpha_hi, int32_t grid, double max_shrink,
                          void* scales, void* stream) {
  if (!dtype_ok(dtype) || m < 0 || n < 0 || alpha_hi <= 0 || alpha_lo > alpha_hi)
    return BAKRON_EINVAL;
  if (grid < 0 || grid > kScaleMaxGrid) return BAKRON_EINVAL;
  if (!(max_shrink >= 0.0 && max_shrink < 1.0)) return BAKRON_EINVAL;
  if (m == 0) return BAKRON_OK;
  if (!scales || (n > 0 && (!W || ldw < n))) return BAKRON_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (dtype == BAKRON_F32)
    e = launch_row_scales_mse<float>(m, n, (const float*)W, ldw, alpha_lo, alpha_hi, alpha_hi, grid,
                                     max_shrink, (float*)scales, s);
  else
    e = launch_row_scales_mse<double>(m, n, (const double*)W, ldw, alpha_lo, alpha_hi, alpha_hi,
                                      grid, max_shrink, (double*)scales, s);
  return e == hipSuccess ? BAKRON_OK : BAKRON_EHIP;
}

int bakron_gram(int dtype, int64_t N, int64_t d, const void* X, int64_t ldx, const void* weights,
                double damp_rel, void* G, int64_t ldg, void* stream) {
  if (!dtype_ok(dtype) || N < 0 || d < 0) return BAKRON_EINVAL;
  if (N > INT_MAX || d > INT_MAX / 2) return BAKRON_EINVAL;
  if (!(damp_rel >= 0.0) || damp_rel > 1e300) return BAKRON_EINVAL;
  if (d == 0) return BAKRON_OK;
  if (!G || ldg < d) return BAKRON_EINVAL;
  if (N > 0 && (!X || ldx < d)) return BAKRON_EINVAL;
  if (N > 0) {  // G is written while X is read: the two byte ranges must be disjoint
    const size_t es = esize(dtype);
    const uintptr_t x0 = reinterpret_cast<uintptr_t>(X), g0 = reinterpret_cast<uintptr_t>(G);
    const uintptr_t x1 = x0 + ((size_t)(N - 1) * (size_t)ldx + (size_t)d) * es;
    const uintptr_t g1 = g0 + ((size_t)(d - 1) * (size_t)ldg + (size_t)d) * es;
    if (x0 < g1 && g0 < x1) return BAKRON_EINVAL;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (dtype == BAKRON_F32)
    e = launch_gram<float>(N, d, (const float*)X, ldx, (const float*)weights, damp_rel, (float*)G,
                           ldg, s);
  else
    e = launch_gram<double>(N, d, (const double*)X, ldx, (const double*)weights, damp_rel,
                            (double*)G, ldg, s);
  return e == hipSuccess ? BAKRON_OK : BAKRON_EHIP;
}

int bakron_sample_sqnorms(int dtype, int64_t N, int64_t d, const void* X, int64_t ldx, void* out,
                          void* stream) {
  if (!dtype_ok(dtype) || N < 0 || d < 0 || N > INT_MAX) return BAKRON_EINVAL;
  if (N == 0) return BAKRON_OK;
  if (!out || (d > 0 && (!X || ldx < d))) return BAKRON_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (dtype == BAKRON_F32)
    e = launch_sample_sqnorms<float>(N, d, (const float*)X, ldx, (float*)out, s);
  else
    e = launch_sample_sqnorms<double>(N, d, (const double*)X, ldx, (double*)out, s);
  return e == hipSuccess ? BAKRON_OK : BAKRON_EHIP;
}

}  // extern "C"
