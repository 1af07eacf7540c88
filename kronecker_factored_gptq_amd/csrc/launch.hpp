// Host-side launch wrappers of the gfx950 kernels (defined in the .hip files).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bk {

// Solver tile edge (elements). The same tiling serves the anti-diagonal sweep
// and the masks of the band products.
constexpr int kTile = 16;

// Element strides between consecutive problems of a batched solve (problem b
// of a launch is blockIdx.y); a stride of 0 shares one array across the batch.
struct BatchStrides {
  int64_t w;       // W
  int64_t s;       // scales
  int64_t la, lb;  // the caller's factors L^A, L^B
  int64_t v, wt;   // outputs V and Wt
  int64_t ws;      // the per-problem solve workspace, in elements
};

struct SolveGeom {
  int64_t m, n;
  int Mt, Nt;     // tiles per column / row direction
  int batch = 1;  // problems of the same shape, solved in the same launches
  BatchStrides bs = {0, 0, 0, 0, 0, 0, 0};
};

// ---- solve (solve_kernels.hip) --------------------------------------------
// Polls of the rows above before a leaf row gives up (each poll is a set of
// device-coherent loads, about a microsecond, plus a short sleep: about
// 0.1 s in all, far beyond any real wait, which is bounded by the block's own
// tiles, tens of microseconds). A give-up sets the problem's status word.
constexpr int kLeafWaitPolls = 1 << 16;
// Per-problem words of the leaf blocks: one ticket counter per leaf block,
// then the status word (nonzero: a wait gave up), `stride` ints apart, and the
// error copy eb (Mt x Nt tiles, the same stride in elements of the dtype).
struct LeafSync {
  int* sync = nullptr;
  int64_t stride = 0;
  int nblocks = 0;
  void* eb = nullptr;
  int polls = kLeafWaitPolls;
};
// Packs W (and clears ls's words when given).
template <typename R>
hipError_t launch_pack_w(const SolveGeom& g, const R* W, int64_t ldw, const R* scales,
                         int scale_mode, R* Wk, hipStream_t s, const LeafSync& ls);
// L^B (lb = true) or L^A of every problem of g's batch.
template <typename R>
hipError_t launch_pack_l(const SolveGeom& g, bool lb, const R* L, int64_t ld, const R* scales,
                         R* Lp, hipStream_t s);

template <typename R>
struct LeafParams {
  R lo, hi;
  int unbounded;
  int scale_mode;
  const R* scales;
  int32_t* V;
  int64_t ldv;
  R* Wt;
  int64_t ldwt;
};
// The leaf block [K0, K1) (the blk-th leaf block of the schedule) in one
// launch, one workgroup per tile row. ev0 / ev1 (nullable): events stamped
// with the kernel's start and end by its dispatch (for measurement).
template <typename R>
hipError_t launch_leaf_rows(const SolveGeom& g, int K0, int K1, int blk, R* Wk, const R* LBp,
                            const R* LAp, const LeafParams<R>& lp, const LeafSync& ls,
                            hipStream_t s, hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);

// Buffers of the band products: W tiles (errors on finished tiles), packed
// L^B and L^A tiles, and the stage-1 product M.
template <typename R>
struct BandBuffers {
  R* Wk;
  const R* LBp;
  const R* LAp;
  R* Mb;
};
// Internal node of the recursion over tile anti-diagonals [k, l) split at mid:
// stage 1 or 2 of the band products. ev0 / ev1 (nullable): events stamped
// with the kernel's start and end by its dispatch (for measurement).
template <typename R>
hipError_t launch_node_band(const SolveGeom& g, int k, int mid, int l, int stage,
                            const BandBuffers<R>& bb, hipStream_t s, hipEvent_t ev0 = nullptr,
                            hipEvent_t ev1 = nullptr);
// Tile anti-diagonals per leaf block (updates inside a block are left-looking).
#ifndef BK_LEAF_BLOCK
#define BK_LEAF_BLOCK 24
#endif
constexpr int kLeafBlock = BK_LEAF_BLOCK;

// ---- BaKron-antidiagonal (antidiag_kernels.hip) ----------------------------
// Workspace of the whole-matrix anti-diagonal solver (element size es): U
// (Mp x Np), the transposed factors LBt (m x Mp) and LAt (n x Np), and two
// error vectors of min(m, n) entries; Mp, Np = m, n rounded up to 64.
struct AntidiagLayout {
  int64_t Mp, Np;
  size_t u, lbt, lat, d0, d1, total;
};
inline AntidiagLayout antidiag_layout(size_t es, int64_t m, int64_t n) {
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  AntidiagLayout L;
  L.Mp = (m + 63) / 64 * 64;
  L.Np = (n + 63) / 64 * 64;
  const int64_t r = m < n ? m : n;
  L.u = 0;
  L.lbt = L.u + al((size_t)(L.Mp * L.Np) * es);
  L.lat = L.lbt + al((size_t)(m * L.Mp) * es);
  L.d0 = L.lat + al((size_t)(n * L.Np) * es);
  L.d1 = L.d0 + al((size_t)(r + 64) * es);
  L.total = L.d1 + al((size_t)(r + 64) * es) + 256;
  return L;
}
// Algorithm 3 on the whole matrix: pack, then one launch per anti-diagonal
// (m + n - 1 launches) on stream s. lo / hi: +-infinity for the unbounded
// alphabet.
template <typename R>
hipError_t launch_antidiag_solve(int64_t m, int64_t n, const R* W, int64_t ldw, const R* LA,
                                 int64_t ldla, const R* LB, int64_t ldlb, R lo, R hi,
                                 int scale_mode, const R* scales, int32_t* V, int64_t ldv, R* Wt,
                                 int64_t ldwt, void* ws, hipStream_t s);

// ---- factor (factor_kernels.hip), always float64 inside --------------------
// X = J A J for `batch` matrices: A + z * sA -> X + z * sX (elements).
template <typename R>
hipError_t launch_load_reversed(int64_t n, const R* A, int64_t lda, int64_t sA, double* X,
                                int64_t sX, int batch, hipStream_t s);
// One matrix being factored: X (n x n, ld n) holds the lower triangle of the
// (reversed) input and is overwritten with Schur complements; Y (n x n, ld n)
// receives the inverse of its Cholesky factor (lower, zeros above the
// diagonal inside 64 x 64 diagonal blocks); Tmp holds >= (n/2 + 64)^2
// doubles; *info receives the smallest failing pivot index (starts INT_MAX).
struct FactorSide {
  double* X;
  double* Y;
  double* Tmp;  // one C21 Y11 buffer per node-size class (factor_tmp_layout)
  int32_t* info;
};
// Node-size classes of the recursion (class c: orders in (64 << c, 128 << c]).
constexpr int kTmpClasses = 24;
// Doubles of the per-class C21 Y11 buffers of a factor of order n; off
// (nullable, kTmpClasses entries) receives each class's offset.
int64_t factor_tmp_layout(int64_t n, int64_t* off);
// Events the large nodes of a factor of order n take from a FactorAux.
int64_t factor_helper_events(int64_t n);
// Helper stream of a factor call and the events it hands out (the owner
// creates and destroys them; nullptr from event() means creation failed).
struct FactorAux {
  hipStream_t ts = nullptr;
  hipEvent_t* ev = nullptr;
  int nev = 0, used = 0;
  hipEvent_t event() { return used < nev ? ev[used++] : nullptr; }
};
// `count` matrices of one order factored in the same launches: side z is
// `first` with X, Y, Tmp and TmpS advanced by z * stride doubles and info by
// z words.
struct FactorSet {
  FactorSide first;
  int64_t stride;
  int count;
};
__host__ __device__ inline FactorSide factor_side(const FactorSet& f, int z) {
  FactorSide s = f.first;
  const int64_t o = (int64_t)z * f.stride;
  s.X += o;
  s.Y += o;
  s.Tmp += o;
  s.info += z;
  return s;
}
// Y = Cholesky(X)^-1 for every matrix of the set (order n), in one sequence
// of launches on s; with aux (nullable), the large nodes' C21 Y11 products run
// on aux->ts, joined back to s by events.
hipError_t factor_cholesky_inverse(int64_t n, const FactorSet& set, hipStream_t s,
                                   FactorAux* aux = nullptr);
// L (and d, nullable) of `batch` matrices: Y + z * sY -> L + z * sL, d + z * sd.
template <typename R>
hipError_t launch_store_normalized(int64_t n, const double* Y, int64_t sY, R* L, int64_t ldl,
                                   int64_t sL, R* d, int64_t sd, int batch, hipStream_t s);
hipError_t launch_fill_i32(int32_t* p, int64_t count, int32_t v, hipStream_t s);

// ---- float64 GEMM (gemm64.hip) --------------------------------------------
// C = alpha * A * op(B) + beta * C, op(B) = B (K x N) or B^T (B is N x K), for
// `batch` problems of one shape: problem z uses A + z * sA, B + z * sB,
// C + z * sC (element strides).
// lower_out: only 64x64 output blocks with block_row >= block_col are
// computed (the others are left untouched). a_lower: A is lower triangular,
// so row block r only needs k < (r + 1) * 64. b_lower: B as stored is lower
// triangular: with transB the column block c only needs k < (c + 1) * 64,
// without it only k >= c * 64.
// dot != nullptr: instead of storing C, the block's sum of alpha (A op(B)) .*
// dot is written to partial[z * sPart + block] (C unused); with sym_dot the
// elements are weighted 2 below the diagonal, 1 on it, 0 above. (Batch 1
// products of the loss's shape use a stream-K kernel with per-workgroup
// partials instead.)
struct Gemm64Args {
  int64_t M, N, K;
  const double* A;
  int64_t lda, sA;
  const double* B;
  int64_t ldb, sB;
  double* C;
  int64_t ldc, sC;
  double alpha, beta;
  int transB;
  int lower_out;
  int a_lower;
  int b_lower;
  const double* dot;
  int64_t lddot, sDot;  // problem z's dot matrix at dot + z * sDot
  double* partial;
  int64_t sPart;        // problem z's partials start at partial + z * sPart
  int batch;
  // dot epilogue of a symmetric product computed on its lower blocks only:
  // element (r, c) counts twice below the diagonal, once on it, not above
  int sym_dot;
};
hipError_t launch_gemm64(const Gemm64Args& a, hipStream_t s);
// Largest batch of one launch (the grid's z extent).
constexpr int kMaxGemmBatch = 65535;
// Two independent products: one launch when both go to the same 64 x 64 /
// 32 x 32 kernel (no dot epilogue), else two launches in order.
hipError_t launch_gemm64_pair(const Gemm64Args& a0, const Gemm64Args& a1, hipStream_t s);
// Upper bound of the partials a dot-epilogue product of this shape writes
// (per-block or per-workgroup; for workspace sizing), and the exact count a
// given product writes.
int64_t gemm64_num_blocks(int64_t M, int64_t N);
int64_t gemm64_partials(const Gemm64Args& a);

// ---- loss and scales (loss_kernels.hip) -----------------------------------
// The loss's elementwise steps for `batch` problems (grid z): A + z * sA ->
// X + z * sX, and D = W - s (.) V per problem.
template <typename R>
hipError_t launch_sym_to_f64(int64_t n, const R* A, int64_t lda, double* X, hipStream_t s,
                             int batch = 1, int64_t sA = 0, int64_t sX = 0);
struct ResidualStrides {
  int64_t w, v, s, d;
};
template <typename R>
hipError_t launch_residual_f64(int64_t m, int64_t n, const R* W, int64_t ldw, const int32_t* V,
                               int64_t ldv, int scale_mode, const R* scales, double* D,
                               hipStream_t s, int batch = 1,
                               ResidualStrides st = ResidualStrides{0, 0, 0, 0});
// out[z] = sum of partial[z * sPart .. z * sPart + count), fixed order.
hipError_t launch_sum_partials(const double* partial, int64_t count, double* out, hipStream_t s,
                               int batch = 1, int64_t sPart = 0);
template <typename R>
hipError_t launch_row_scales(int64_t m, int64_t n, const R* W, int64_t ldw, int32_t hi, R* s_out,
                             hipStream_t s);

// ---- scale search (scale_kernels.hip) -------------------------------------
// Largest candidate count - 1 of the per-row scale search.
constexpr int kScaleMaxGrid = 1024;
template <typename R>
hipError_t launch_row_scales_mse(int64_t m, int64_t n, const R* W, int64_t ldw, int32_t lo,
                                 int32_t hi, int32_t hi_code, int32_t grid, double max_shrink,
                                 R* s_out, hipStream_t s);

// ---- Kronecker factors from samples (gram_kernels.hip) ----------------------
// G = (1/N) X^T diag(w) X (w nullable = 1), then + damp_rel * mean(diag) * I;
// X is N x d (ldx), G d x d (ldg), both triangles written.
template <typename R>
hipError_t launch_gram(int64_t N, int64_t d, const R* X, int64_t ldx, const R* w, double damp_rel,
                       R* G, int64_t ldg, hipStream_t s);
// out[k] = |row k of X|^2.
template <typename R>
hipError_t launch_sample_sqnorms(int64_t N, int64_t d, const R* X, int64_t ldx, R* out,
                                 hipStream_t s);

}  // namespace bk
