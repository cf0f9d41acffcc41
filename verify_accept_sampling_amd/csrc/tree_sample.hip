// Tree sampling verification: multi-step speculative sampling over the
// siblings of a draft tree.
//
// The EAGLE-3 review (section on the full inference loop, step 4 "Strict
// Acceptance") states that sampling over the tree applies the min(1, p/q)
// test with residual correction so that the target distribution is kept.
// Sibling order follows SpecInfer's multi-step speculative sampling (Miao et
// al., ASPLOS 2024): at the current node u the children are tried in
// increasing node index against the current target distribution r; after a
// rejection r <- normalise(max(0, r - q_u)) (kept when that has no mass);
// an accepted child becomes the current node with r = p_child; the stop node
// draws one token from r by inverse CDF.
//
// Closed form used on the device.  With p = p_u and q = q_u, after i
// rejections r_i = max(0, p - C_i q) / M_i, where C_0 = 0, M_0 = 1 and,
// at each rejection, C' = C_i + M_i, F = sum_j max(0, p_j - C' q_j):
// (C_{i+1}, M_{i+1}) = (C', F) if F > 0, else (C_i, M_i).  (By induction:
// max(0, max(0, p - C q)/M - q) = max(0, p - (C + M) q)/M.)  The test of
// the (i+1)-th child x is u q(x) M_i < max(0, p(x) - C_i q(x)).  The masses
// F depend only on the node's two rows, so every one the walk could need is
// computed before it, in rounds: round i computes, for every node with more
// than i children, F at that node's C_i (rounds 1 .. max children - 1).
//
// Launches (none waits for another work-group: each reads what the kernels
// before it on the stream wrote):
//   k_tree_setup     one work-group (trees above kSmallTree nodes, or
//                    probability rows; else work-group 0 of k_tree_stats):
//                    child lists, ranks, depths, the list of nodes with
//                    children, and the children of rank >= 1 by rank, from
//                    the parent array, into the workspace;
//   k_tree_stats     (logits) the float64 statistic of both rows of every
//                    node with children, per kTreeStatChunk-element chunk;
//   k_tree_mass      one launch per round: per (request, child of rank i,
//                    8192-element chunk) the chunk's sum of
//                    max(0, p - C_i q) at its parent;
//   k_tree_walk      one wave per request: the tests, the accepted path, the
//                    outputs but the final token, and the draw state (trees
//                    of up to 64 nodes: every node's inputs in its own lane,
//                    requested together, then a walk in registers);
//   k_tree_leaf      (logits) per (request, chunk) the float32 statistic of
//                    the target row of the leaf where the walk stopped, if
//                    it stopped at a leaf (only the draw reads it);
//   k_tree_draw      per (request, chunk) the chunk's draw-weight totals;
//                    the request's last work-group (completion ticket) then
//                    picks the chunk by running total and the element by
//                    the same per-chunk scan, on one wave.
#include <algorithm>

#include "sample_device.h"

// Every product and difference below is rounded on its own: with fused
// multiply-adds the compiler could round p_j = e_p / S_p and C q_j
// differently inside max(0, p_j - C q_j), so that identical target and
// draft rows would leave a residual of rounding noise instead of the exact
// zero the empty-residual rule is about.
#pragma clang fp contract(off)

namespace specv {

// Tables k_tree_setup writes into the workspace, kMaxNodes int32 each.
enum TreeTable {
  kTabParent = 0,
  kTabNChild,    // number of children
  kTabFirst,     // lowest-index child, -1 if none
  kTabNext,      // next sibling in index order, -1 if none
  kTabRank,      // index among its siblings (0 = lowest)
  kTabDepth,
  kTabInternal,  // nodes with a child, ascending
  kTabRanked,    // children of rank >= 1, by (rank, index)
  kTabRankOff,   // kTabRanked offset of rank r (entry r - 1), r = 1 .. max rank + 1
  kTabCount
};
static_assert((size_t)kTabCount * kMaxNodes * 4 <= kTreeTableBytes, "tree tables fit their region");

__device__ __forceinline__ const int* tree_tab(const int* t, int which) {
  return t + which * kMaxNodes;
}

// Per-request draw state from the walk.
struct TreeDraw {
  int node;   // stop node
  int depth;  // its depth = accepted length
  double cf;  // C of the weights max(0, p - C q) drawn from (0: p itself)
  double cp;  // C before the last rejection (the weights if cf's have no mass)
};

// ---------------------------------------------------------------------------
// Setup
// ---------------------------------------------------------------------------

// Every table entry is computed by its own thread from the parent array in
// shared memory (O(N) per entry, N <= NMAX): no sequential pass.  Run by a
// whole work-group.
template <int NMAX>
__device__ __forceinline__ void tree_setup_block(const TreeArgsN<NMAX>& tree, int N,
                                                 int* __restrict__ tables) {
  __shared__ int par[NMAX], nch[NMAX], rank[NMAX];
  int* const t_parent = tables + kTabParent * kMaxNodes;
  for (int j = threadIdx.x; j < N; j += kThreads) par[j] = j == 0 ? -1 : tree.parent[j];
  __syncthreads();
  // Per node: its rank among its siblings (children in increasing index),
  // its next sibling, its number of children, its first child, its depth.
  for (int j = threadIdx.x; j < N; j += kThreads) {
    const int u = par[j];
    int r = 0, nx = -1, nc = 0, fc = -1;
    for (int i = 1; i < N; ++i) {
      const int pi = par[i];
      if (j > 0 && pi == u) {
        if (i < j) ++r;
        else if (i > j && nx < 0) nx = i;
      }
      if (pi == j) {
        if (fc < 0) fc = i;
        ++nc;
      }
    }
    int d = 0;
    for (int x = j; x > 0; x = par[x]) ++d;  // parents precede their children
    nch[j] = nc;
    rank[j] = r;
    t_parent[j] = u;
    tables[kTabNChild * kMaxNodes + j] = nc;
    tables[kTabFirst * kMaxNodes + j] = fc;
    tables[kTabNext * kMaxNodes + j] = nx;
    tables[kTabRank * kMaxNodes + j] = r;
    tables[kTabDepth * kMaxNodes + j] = d;
  }
  __syncthreads();
  for (int j = threadIdx.x; j < N; j += kThreads) {
    // The nodes with a child, ascending; the children of rank >= 1 grouped by rank, ascending index within a
    // rank; rank r's offset at entry r - 1 (r = 1 .. max rank + 1).
    // Entries past each list's length are 0.
    int n_int = 0, n_ranked = 0, max_rank = 0;
    int before_int = 0, lower_rank = 0, same_rank_before = 0, off = 0;
    for (int i = 0; i < N; ++i) {
      const int ri = rank[i];
      if (nch[i] > 0) {
        ++n_int;
        if (i < j) ++before_int;
      }
      if (i >= 1 && ri >= 1) {
        ++n_ranked;
        max_rank = max(max_rank, ri);
        if (ri < rank[j]) ++lower_rank;
        if (ri == rank[j] && i < j) ++same_rank_before;
        if (ri < j + 1) ++off;
      }
    }
    if (nch[j] > 0) tables[kTabInternal * kMaxNodes + before_int] = j;
    if (j >= n_int) tables[kTabInternal * kMaxNodes + j] = 0;
    if (j >= 1 && rank[j] >= 1) tables[kTabRanked * kMaxNodes + lower_rank + same_rank_before] = j;
    if (j >= n_ranked) tables[kTabRanked * kMaxNodes + j] = 0;
    tables[kTabRankOff * kMaxNodes + j] = j <= max_rank ? off : 0;
  }
}

template <int NMAX>
__global__ __launch_bounds__(kThreads) void k_tree_setup(TreeArgsN<NMAX> tree, int N,
                                                        int* __restrict__ tables) {
  tree_setup_block<NMAX>(tree, N, tables);
}

// ---------------------------------------------------------------------------
// Shared pieces
// ---------------------------------------------------------------------------

// Float64 row statistic of one chunk of a row: a reference m (a logit) and
// S = sum over the chunk of e^{(x - m)/T}, every term a float64 exp.  The
// rows of nodes with children (both of their rows) carry this statistic,
// so that the tests, the masses and the draws there use the distributions
// softmax(z/T) to float64 precision, as the oracle does; a leaf's target
// row keeps the float32 statistic (only its reference is used: its bonus
// draw normalises its own weights).
struct TreeStat64 {
  double m, s;
};


// (m, s) <- the pair's merge at the larger reference; exp2_256(0) = 1
// exactly, so the side that holds it keeps its sum.
__device__ __forceinline__ void ms64_merge(float& m, double& s, float m2, double s2, double c1,
                                           const double* tab) {
  if (m2 == -INFINITY) return;
  if (m == -INFINITY) {
    m = m2;
    s = s2;
    return;
  }
  if (m == m2) {  // the usual case: both sides kept the row's first reference
    s += s2;
    return;
  }
  const float mn = fmaxf(m, m2);
  s = s * exp2_256(((double)m - (double)mn) * c1, tab) +
      s2 * exp2_256(((double)m2 - (double)mn) * c1, tab);
  m = mn;
}

// Row statistics of target row u and draft row u of request b.  Nodes with
// children (`internal`): the float64 statistics k_tree_stats stored at
// slots b*2N + u and b*2N + N + u (tree_xchunks(V) chunks each), merged in
// chunk order (plain sums when the chunks share their reference, as they
// do unless a row's values exceed its first element by far).  A leaf: the
// reference of its target row's float32 statistic, with S = 1 (its weights
// are normalised by their own total).
struct RowPair {
  float mp, mq;
  double sp, sq;
};
__device__ __forceinline__ RowPair node_rows(const TreeStat64* xs, const uint64_t* part, int b,
                                             int N, int u, int V, int C1, float c, double c1,
                                             const double* tab, bool internal) {
  RowPair r;
  r.mp = r.mq = -INFINITY;
  r.sp = r.sq = 0.0;
  const long base = (long)b * 2 * N;
  if (internal) {
    const int Cx = tree_xchunks(V);
    const TreeStat64* xa = xs + (base + u) * Cx;
    const TreeStat64* xd = xs + (base + N + u) * Cx;
    constexpr int kBatch = 8;  // loads requested together
    for (int c0 = 0; c0 < Cx; c0 += kBatch) {
      TreeStat64 a[kBatch], d[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        const int ch = min(c0 + i, Cx - 1);
        a[i] = xa[ch];
        d[i] = xd[ch];
      }
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        if (c0 + i < Cx) {
          ms64_merge(r.mp, r.sp, (float)a[i].m, a[i].s, c1, tab);
          ms64_merge(r.mq, r.sq, (float)d[i].m, d[i].s, c1, tab);
        }
      }
    }
  } else {
    float mq;
    double sq;
    merge_two_rows(part, (base + u) * C1, (base + N + u) * C1, false, C1, c, r.mp, r.sp, mq, sq);
    r.sp = 1.0;
  }
  return r;
}

// Term coefficients: p_j = 2^(t/256) / S with t = z c1 - fl(m c1),
// c1 = 256 / (T ln 2), i.e. e^{(z - m)/T} / S.  Probability rows are used
// as given.
struct TermCoef {
  double c1, c0p, c0q, ip, iq;
};
template <int KIND>
__device__ __forceinline__ TermCoef term_coef(const RowPair& r, double c1) {
  TermCoef k;
  if (KIND == 0) {
    k.c1 = c1;
    k.c0p = -((double)r.mp * c1);
    k.c0q = -((double)r.mq * c1);
    k.ip = 1.0 / r.sp;
    k.iq = 1.0 / r.sq;
  } else {
    k.c1 = k.c0p = k.c0q = 0.0;
    k.ip = k.iq = 1.0;
  }
  return k;
}
template <int KIND>
__device__ __forceinline__ double tterm(float z, double c1, double c0, double inv,
                                        const double* tab) {
  return KIND == 0 ? exp2_256(fma((double)z, c1, c0), tab) * inv : (double)z;
}
// tterm for terms that are only summed (the residual masses).
template <int KIND>
__device__ __forceinline__ double tterm_sum(float z, double c1, double c0, double inv,
                                            const double* tab) {
  return KIND == 0 ? exp2_256_sum(fma((double)z, c1, c0), tab) * inv : (double)z;
}

// One chunk of kDrawChunk elements by one wave: lane l holds the running
// sums (inclusive) of the weights w_j = max(0, p_j - C q_j) (p_j when !use_q)
// of its kSegPerThread consecutive elements, offset by the total of the
// lower lanes (a fixed-order scan), so run[e] is the chunk's running sum up
// to that element.  Returns the chunk total (lane 63's last running sum) in
// every lane.  Every caller of one chunk gets bit-identical sums.
template <int DT, int NE, int KIND>
__device__ __forceinline__ double chunk_scan(const void* prow, const void* qrow, int V, long chunk,
                                             double C, bool use_q, const TermCoef& k,
                                             const double* tab, double (&run)[kSegPerThread],
                                             double& base) {
  const int lane = threadIdx.x & 63;
  const long j0 = chunk * kDrawChunk + (long)lane * kSegPerThread;
  constexpr uint32_t fill = run_fill<DT, KIND>();
  RunWords<DT> rp, rq;
  load_run_words<DT, NE>(prow, j0, V, fill, rp);
  if (use_q) load_run_words<DT, NE>(qrow, j0, V, fill, rq);
  double acc = 0.0;
#pragma unroll
  for (int e = 0; e < kSegPerThread; ++e) {
    const double a = tterm<KIND>(run_elem<DT>(rp, e), k.c1, k.c0p, k.ip, tab);
    double w = a;
    if (use_q) w = fmax(0.0, a - C * tterm<KIND>(run_elem<DT>(rq, e), k.c1, k.c0q, k.iq, tab));
    acc += w;
    run[e] = acc;
  }
  const double excl = wave_exclusive_scan_d(acc);
#pragma unroll
  for (int e = 0; e < kSegPerThread; ++e) run[e] += excl;
  base = excl;
  return __shfl(excl + acc, 63, 64);
}

// The totals chunk_scan returns for one chunk at two factors, C = cf (with
// q when use_f) and C = cp (with q when use_p), from one evaluation of the
// chunk's terms: the same sums in the same order, so each total is
// bit-identical to chunk_scan's at that factor.
template <int DT, int NE, int KIND>
__device__ __forceinline__ void chunk_totals2(const void* prow, const void* qrow, int V,
                                              long chunk, double cf, bool use_f, double cp,
                                              bool use_p, const TermCoef& k, const double* tab,
                                              double& tf, double& tp) {
  const int lane = threadIdx.x & 63;
  const long j0 = chunk * kDrawChunk + (long)lane * kSegPerThread;
  constexpr uint32_t fill = run_fill<DT, KIND>();
  RunWords<DT> rp, rq;
  load_run_words<DT, NE>(prow, j0, V, fill, rp);
  load_run_words<DT, NE>(qrow, j0, V, fill, rq);
  double af = 0.0, ap = 0.0;
#pragma unroll
  for (int e = 0; e < kSegPerThread; ++e) {
    const double a = tterm<KIND>(run_elem<DT>(rp, e), k.c1, k.c0p, k.ip, tab);
    const double q = tterm<KIND>(run_elem<DT>(rq, e), k.c1, k.c0q, k.iq, tab);
    af += use_f ? fmax(0.0, a - cf * q) : a;
    ap += use_p ? fmax(0.0, a - cp * q) : a;
  }
  const double ef = wave_exclusive_scan_d(af), ep = wave_exclusive_scan_d(ap);
  tf = __shfl(ef + af, 63, 64);
  tp = __shfl(ep + ap, 63, 64);
}

// Sum of n chunk partials in a fixed order (lane l: entries l, l+64, ...,
// then a symmetric butterfly), the same value in every lane.
__device__ __forceinline__ double wave_sum_fixed(const double* p, long n, long stride = 1) {
  const int lane = threadIdx.x & 63;
  double s = 0.0;
  for (long i = lane; i < n; i += 64) s += p[i * stride];
  return wave_sum_d(s);
}

// (C, M) after rejecting the children of u of ranks 0 .. r-1, from the
// mass rounds' partials (mpart row of child j = masses at its parent for
// the test of j).  Wave-uniform.
__device__ __forceinline__ void residual_state(const int* tables, const double* mpart, int b,
                                               int N, int Cm, int u, int r, double& C,
                                               double& M) {
  C = 0.0;
  M = 1.0;
  constexpr int kFast = 8;  // ranks whose partials are loaded together
  if (N <= kWaveSize && Cm <= kWaveSize && r <= kFast) {
    // Small trees: the children of u from one load of the parent table
    // (lane l: node l; a child's rank is its position among the set bits),
    // then every needed rank's partials in one round trip, summed as
    // wave_sum_fixed sums them (lane l holds entry l, then the butterfly):
    // the same numbers as the loop below.
    const int lane = threadIdx.x & 63;
    const int pl = lane < N ? tree_tab(tables, kTabParent)[lane] : -1;
    uint64_t kids = __ballot(lane > 0 && pl == u);
    int js[kFast];
#pragma unroll
    for (int i = 0; i <= kFast; ++i) {  // js[i - 1]: the child of rank i
      const int jj = kids ? __builtin_ctzll(kids) : -1;
      if (kids) kids &= kids - 1;
      if (i >= 1) js[i - 1] = jj;
    }
    double v[kFast];
#pragma unroll
    for (int i = 0; i < kFast; ++i) {
      const int jj = js[i] >= 0 ? js[i] : 0;
      const double x = mpart[((long)b * N + jj) * Cm + min(lane, Cm - 1)];
      v[i] = lane < Cm ? x : 0.0;
    }
#pragma unroll
    for (int i = 0; i < kFast; ++i) {
      if (i >= r || js[i] < 0) break;
      const double cn = C + M;
      const double F = wave_sum_d(v[i]);
      if (F > 0.0) {
        C = cn;
        M = F;
      }
    }
    return;
  }
  int j = tree_tab(tables, kTabFirst)[u];
  for (int i = 0; i < r && j >= 0; ++i) {
    // state for child rank i + 1 from child rank i's rejection
    j = tree_tab(tables, kTabNext)[j];
    if (j < 0) break;
    const double cn = C + M;
    const double F = wave_sum_fixed(mpart + ((long)b * N + j) * Cm, Cm);
    if (F > 0.0) {
      C = cn;
      M = F;
    }
  }
}

// ---------------------------------------------------------------------------
// Kernels
// ---------------------------------------------------------------------------

// Float64 statistic of this thread's groups g0 + tid, g0 + tid + NT, ...
// below g1 (16-byte words of NE elements; NE = 1: elements), relative to
// the reference m0 on entry (the row's first element, the same for every
// chunk of the row, so that the chunks' sums add without rescaling; -inf
// when that element is not finite).  The reference moves up (rescaling the
// sum) only when an element exceeds it by more than kRefSlack in the scaled
// exponent, so every term and the sum stay far below overflow, and a first
// finite element sets it when there is none.
constexpr double kRefSlack = 256.0 * 400.0;  // terms below 2^400
constexpr int kStatU = 8;  // words per thread requested together

// Words g, g + NT, ... (kStatU of them) of a row; a word at or past g1 is
// not loaded (its offset is past the row's buffer) and reads as 0.
__device__ __forceinline__ void stats64_load(const RowBuf& buf, long g, long g1,
                                             u32x4 (&w)[kStatU]) {
#pragma unroll
  for (int u = 0; u < kStatU; ++u) {
    const long gu = g + (long)u * kThreads;
    w[u] = buf.load_nt(gu < g1 ? static_cast<uint32_t>(gu) * 16u : 0xfffffff0u, 0);
  }
}

// With 16-byte words (NE > 1) the caller has already requested the first
// kStatU words (w0, from stats64_load at g0 + tid), so that their latency
// overlaps its set-up.
template <int DT, int NE>
__device__ __forceinline__ void stats64_thread(const void* rp, uint32_t row_bytes, long g0,
                                               long g1, double c1, const double* tab, float& m,
                                               double& s, const u32x4 (&w0)[kStatU]) {
  s = 0.0;
  // With no reference yet (m = -inf) every element seen is -inf: its term,
  // clamped, is 0 at any mc.
  double mc = m == -INFINITY ? 0.0 : -((double)m * c1);
  const double lim = kRefSlack / c1;  // in logit units
  float mlim = (float)((double)m + lim);
  auto fold = [&](const float (&x)[NE]) {
    float bm = x[0];
#pragma unroll
    for (int e = 1; e < NE; ++e) bm = fmaxf(bm, x[e]);
    if (bm > mlim) {  // rare: a first finite element, or far above
      if (m != -INFINITY) s *= exp2_256(((double)m - (double)bm) * c1, tab);
      m = bm;
      mc = -((double)m * c1);
      mlim = (float)((double)m + lim);
    }
#pragma unroll
    for (int e = 0; e < NE; ++e) s += exp2_256_sum(fma((double)x[e], c1, mc), tab);
  };
  if constexpr (NE == 1) {
    for (long g = g0 + threadIdx.x; g < g1; g += kThreads) {
      const float x[1] = {load_elem<DT>(rp, g)};
      fold(x);
    }
  } else {
    auto fold_words = [&](const u32x4 (&w)[kStatU], long g) {
#pragma unroll
      for (int u = 0; u < kStatU; ++u) {
        if (g + (long)u * kThreads < g1) {
          float x[NE];
          unpack16<DT>(w[u], x);
          fold(x);
        }
      }
    };
    fold_words(w0, g0 + threadIdx.x);
    const RowBuf buf(rp, row_bytes);
    for (long g = g0 + threadIdx.x + (long)kStatU * kThreads; g < g1;
         g += (long)kStatU * kThreads) {
      u32x4 w[kStatU];
      stats64_load(buf, g, g1, w);
      fold_words(w, g);
    }
  }
}

// Work-group merge of the threads' float64 statistics; the result is valid
// in thread 0.
__device__ __forceinline__ void block_reduce_ms64(float& m, double& s, double c1,
                                                  const double* tab) {
  __shared__ float sm[kWaves];
  __shared__ double ss[kWaves];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float m2 = shfl_xor_f(m, o);
    const double s2 = shfl_xor_d(s, o);
    ms64_merge(m, s, m2, s2, c1, tab);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) {
    sm[wave] = m;
    ss[wave] = s;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    m = sm[0];
    s = ss[0];
    for (int w = 1; w < kWaves; ++w) ms64_merge(m, s, sm[w], ss[w], c1, tab);
  }
}

// Float64 row statistics of the rows of the nodes with children -- per
// request the target rows, then the draft rows, of nodes internal[0 ..
// n_int-1] -- in chunks of kTreeStatChunk elements (xstat).  SETUP (trees
// of up to kSmallTree nodes): the nodes with a child come in the argument
// `internal`, and work-group 0 also writes the tree tables for the launches
// after this one (no launch of its own); otherwise they come from the
// tables k_tree_setup wrote.
template <int DT, int NE, bool SETUP>
__global__ __launch_bounds__(kThreads) void k_tree_stats(
    const void* __restrict__ target, const void* __restrict__ draft, int N, int n_int, int V,
    double c1, TreeArgsN<kSmallTree> tree, TreeArgsN<kSmallTree> internal,
    int* __restrict__ tables, TreeStat64* __restrict__ xstat) {
  __shared__ double tab[256];
  if constexpr (SETUP) {
    if (blockIdx.x == 0) tree_setup_block<kSmallTree>(tree, N, tables);
  }
  if (n_int == 0) return;  // a launch for the tables alone
  const int Cx = tree_xchunks(V);
  const long eb = Elems<DT>::kBytes;
  const long idx = blockIdx.x;
  {
    const int chunk = static_cast<int>(idx % Cx);
    const int j = static_cast<int>((idx / Cx) % (2 * n_int));
    const int b = static_cast<int>(idx / Cx / (2 * n_int));
    const int jj = j < n_int ? j : j - n_int;
    const int node = SETUP ? internal.parent[jj] : tree_tab(tables, kTabInternal)[jj];
    const bool is_draft = j >= n_int;
    const void* rp = static_cast<const char*>(is_draft ? draft : target) +
                     ((long)b * N + node) * V * eb;
    const int slot = is_draft ? N + node : node;
    const long n_groups = V / NE;
    const long gpc = (n_groups + Cx - 1) / Cx;
    const long g0 = (long)chunk * gpc;
    const long g1 = min(g0 + gpc, n_groups);
    const uint32_t row_bytes = static_cast<uint32_t>((long)V * eb);
    u32x4 w0[kStatU];
    if constexpr (NE > 1) stats64_load(RowBuf(rp, row_bytes), g0 + threadIdx.x, g1, w0);
    const float z0 = load_elem<DT>(rp, 0);
    tab[threadIdx.x] = kExp2Frac256[threadIdx.x];
    __syncthreads();
    float m = z0 > -INFINITY && z0 < INFINITY ? z0 : -INFINITY;
    double s;
    stats64_thread<DT, NE>(rp, row_bytes, g0, g1, c1, tab, m, s, w0);
    block_reduce_ms64(m, s, c1, tab);
    if (threadIdx.x == 0) xstat[((long)b * 2 * N + slot) * Cx + chunk] = TreeStat64{m, s};
  }
}

// The float32 statistic (reference, sum) of one chunk of C1 of the target
// row of a leaf, the node where request b's walk stopped: the leaf's bonus
// draw normalises its own weights, so only the reference is used.  One
// work-group per (request, chunk); a request whose walk stopped at a node
// with children (cf > 0: its rows have float64 statistics) has nothing to
// do.  Only the stop leaf's row is read, one row per request.
template <int DT, int NE>
__global__ __launch_bounds__(kThreads) void k_tree_leaf(const void* __restrict__ target, int N,
                                                        int V, int C1, float c,
                                                        const TreeDraw* __restrict__ tstate,
                                                        uint64_t* __restrict__ part) {
  const int chunk = static_cast<int>(blockIdx.x % C1);
  const int b = static_cast<int>(blockIdx.x / C1);
  const TreeDraw st = tstate[b];
  if (st.cf > 0.0) return;  // work-group-uniform
  const int node = st.node;
  const long eb = Elems<DT>::kBytes;
  const void* rp = static_cast<const char*>(target) + ((long)b * N + node) * V * eb;
  const long n_groups = V / NE;
  const long gpc = (n_groups + C1 - 1) / C1;
  const long g0 = (long)chunk * gpc;
  const long g1 = min(g0 + gpc, n_groups);
  float m = -INFINITY, mc = -INFINITY;
  double s = 0.0;
  if constexpr (NE == 1)
    stats_sweep_scalar<DT>(rp, g0, g1, c, m, mc, s);
  else
    stats_sweep<DT, kThreads>(rp, static_cast<uint32_t>((long)V * eb), g0, g1, c, m, mc, s,
                              threadIdx.x);
  block_reduce_ms(m, s, c);
  if (threadIdx.x == 0) part[((long)b * 2 * N + node) * C1 + chunk] = pack2(m, (float)s);
}

// Work-groups of the draw cover kTreeChunksPerGroup consecutive chunks of
// the stop node's row pair.
constexpr int kTreeChunksPerWave = 2;
constexpr int kTreeChunksPerGroup = kWaves * kTreeChunksPerWave;

// Mass round r: unit = a child j of rank r (its parent u has more than r
// children); one work-group per (request, unit, chunk of kTreeMassChunk
// elements) sums max(0, p_u - C_r q_u) over its chunk.  Every word of the
// chunk is requested before any is used; the work-group's sum is taken in
// a fixed order (lanes, then waves), so the partials are reproducible.
template <int DT, int NE, int KIND>
__global__ __launch_bounds__(kThreads) void k_tree_mass(
    const void* __restrict__ target, const void* __restrict__ draft, int N, int V, int Cm,
    double c1, int r, int n_units, const int* __restrict__ tables,
    const TreeStat64* __restrict__ xstat, double* __restrict__ mpart) {
  __shared__ double tab[256];
  __shared__ RowPair s_rows;
  __shared__ double s_C;
  __shared__ double s_red[kWaves];
  const long idx = blockIdx.x;
  const int chunk = static_cast<int>(idx % Cm);
  const int unit = static_cast<int>((idx / Cm) % n_units);
  const int b = static_cast<int>(idx / Cm / n_units);
  const int j = tree_tab(tables, kTabRanked)[tree_tab(tables, kTabRankOff)[r - 1] + unit];
  const int u = tree_tab(tables, kTabParent)[j];
  const long eb = Elems<DT>::kBytes;
  const void* prow = static_cast<const char*>(target) + ((long)b * N + u) * V * eb;
  const void* qrow = static_cast<const char*>(draft) + ((long)b * N + u) * V * eb;
  const long e0 = (long)chunk * kTreeMassChunk;
  const long e1 = min(e0 + (long)kTreeMassChunk, (long)V);
  // With 16-byte words the chunk's words are requested first: they do not
  // depend on the residual state the first wave works out below.  A word
  // past the chunk is not loaded (its offset is past the row's buffer).
  constexpr int W = NE > 1 ? kTreeMassChunk / (kThreads * NE) : 1;  // words per thread and row
  static_assert(NE == 1 || kTreeMassChunk % (kThreads * NE) == 0, "whole words per thread");
  const long g0 = e0 / NE + threadIdx.x, g1 = e1 / NE;
  u32x4 wp[W], wq[W];
  if constexpr (NE > 1) {
    const uint32_t row_bytes = static_cast<uint32_t>((long)V * eb);
    const RowBuf bp(prow, row_bytes), bq(qrow, row_bytes);
#pragma unroll
    for (int i = 0; i < W; ++i) {
      const long g = g0 + (long)i * kThreads;
      const uint32_t off = g < g1 ? static_cast<uint32_t>(g) * 16u : 0xfffffff0u;
      wp[i] = bp.load_nt(off, 0);
      wq[i] = bq.load_nt(off, 0);
    }
  }
  if (KIND == 0) tab[threadIdx.x] = kExp2Frac256[threadIdx.x];
  __syncthreads();
  if (threadIdx.x < kWaveSize) {
    double C, M;
    residual_state(tables, mpart, b, N, Cm, u, r - 1, C, M);
    if (threadIdx.x == 0) {
      s_C = C + M;
      if (KIND == 0) s_rows = node_rows(xstat, nullptr, b, N, u, V, 0, 0.f, c1, tab, true);
    }
  }
  __syncthreads();
  const double C = s_C;
  RowPair rows{};
  if (KIND == 0) rows = s_rows;
  const TermCoef k = term_coef<KIND>(rows, c1);
  double acc = 0.0;
  if constexpr (NE == 1) {
    for (long e = e0 + threadIdx.x; e < e1; e += kThreads) {
      const double a = tterm_sum<KIND>(load_elem<DT>(prow, e), k.c1, k.c0p, k.ip, tab);
      acc += fmax(0.0, a - C * tterm_sum<KIND>(load_elem<DT>(qrow, e), k.c1, k.c0q, k.iq, tab));
    }
  } else {
#pragma unroll
    for (int i = 0; i < W; ++i) {
      if (g0 + (long)i * kThreads < g1) {
        float xp[NE], xq[NE];
        unpack16<DT>(wp[i], xp);
        unpack16<DT>(wq[i], xq);
#pragma unroll
        for (int e = 0; e < NE; ++e) {
          const double a = tterm_sum<KIND>(xp[e], k.c1, k.c0p, k.ip, tab);
          acc += fmax(0.0, a - C * tterm_sum<KIND>(xq[e], k.c1, k.c0q, k.iq, tab));
        }
      }
    }
  }
  acc = wave_sum_d(acc);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) s_red[wave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = s_red[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) t += s_red[w];
    mpart[((long)b * N + j) * Cm + chunk] = t;
  }
}

// Dynamic shared memory of k_tree_walk: the exp table, then three int
// tables of N entries and two per wave.
inline size_t tree_walk_lds(int N) { return 256 * sizeof(double) + (3 + 2 * kWaves) * (size_t)N * 4; }

// The walk: one wave per request.  The tree tables come into shared memory
// once per work-group and the request's node tokens once per wave; at each
// node the children's tokens, values and uniforms are fetched by their own
// lanes together, and the tests then run in child order.  Work-groups from
// n_walk on instead compute the leaves' row statistics (logits), which only
// the draw after this launch reads: streaming work beside the walk's
// latency-bound waves.
// Mass partials per node that the walk of a small tree keeps in registers.
constexpr int kWalkLanePartials = 16;

// Lane l's value of v in every lane (l wave-uniform).
__device__ __forceinline__ double lane_value_d(double v, int l) {
  const uint64_t bits = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<int>(bits), l);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<int>(bits >> 32), l);
  return __builtin_bit_cast(double, (static_cast<uint64_t>(hi) << 32) | lo);
}

template <int DT, int NE, int KIND>
__global__ __launch_bounds__(kThreads) void k_tree_walk(
    const void* __restrict__ target, const void* __restrict__ draft, int B, int N, int V, int Cm,
    int D, double c1, const int32_t* __restrict__ node_tokens,
    const float* __restrict__ uniforms, uint64_t seed, uint64_t ctr0,
    const int* __restrict__ tables, const TreeStat64* __restrict__ xstat,
    const double* __restrict__ mpart, TreeDraw* __restrict__ tstate,
    int32_t* __restrict__ accepted_len, int32_t* __restrict__ out_tokens,
    int32_t* __restrict__ out_path) {
  extern __shared__ __align__(16) unsigned char walk_lds[];
  double* tab = reinterpret_cast<double*>(walk_lds);
  int* s_nchild = reinterpret_cast<int*>(tab + 256);
  int* s_first = s_nchild + N;
  int* s_next = s_first + N;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int* tok = s_next + N + wave * N;
  int* path = s_next + N + (kWaves + wave) * N;
  const int b = static_cast<int>(blockIdx.x) * kWaves + wave;
  if (KIND == 0) tab[threadIdx.x] = kExp2Frac256[threadIdx.x];
  for (int j = threadIdx.x; j < N; j += kThreads) {
    s_nchild[j] = tree_tab(tables, kTabNChild)[j];
    s_first[j] = tree_tab(tables, kTabFirst)[j];
    s_next[j] = tree_tab(tables, kTabNext)[j];
  }
  if (b < B)
    for (int j = lane; j < N; j += kWaveSize) tok[j] = node_tokens[(long)b * N + j];
  __syncthreads();
  if (b >= B) return;  // wave-uniform
  const long eb = Elems<DT>::kBytes;
  int cur = 0, depth = 0;
  double cf = 0.0, cp = 0.0;
  if (lane == 0) path[0] = 0;
  if (N <= kWaveSize && Cm <= kWalkLanePartials) {
    // Small trees: lane j holds everything node j's test needs, requested
    // together before the walk: its parent, token, uniform, the values of
    // its token in its parent's rows, and F_j, the sum of its mass partials
    // in the order wave_sum_fixed adds them (a wave holding them in lanes
    // 0 .. Cm-1 and zeros above, halves added at distances 32, 16, .., 1;
    // the zeros add exactly).  The walk itself then only moves registers.
    const bool is_node = lane >= 1 && lane < N;
    const int pj = is_node ? tree_tab(tables, kTabParent)[lane] : -1;
    const int x = is_node ? tok[lane] : -1;
    const bool valid = is_node && x >= 0 && x < V;
    const double uj = is_node ? (double)get_uniform(uniforms, seed, ctr0, b, lane, 0, N - 1) : 0.0;
    double f[kWalkLanePartials];
    const double* mp = mpart + ((long)b * N + (is_node ? lane : 0)) * Cm;
#pragma unroll
    for (int i = 0; i < kWalkLanePartials; ++i) f[i] = i < Cm ? mp[i] : 0.0;
#pragma unroll
    for (int o = kWalkLanePartials / 2; o >= 1; o >>= 1)
#pragma unroll
      for (int i = 0; i < o; ++i) f[i] += f[i + o];
    double px = 0.0, qx = 0.0;
    if (is_node) {
      RowPair rows{};
      if (KIND == 0) rows = node_rows(xstat, nullptr, b, N, pj, V, 0, 0.f, c1, tab, true);
      const TermCoef k = term_coef<KIND>(rows, c1);
      const long ro = ((long)b * N + pj) * V * eb;
      const int xs = valid ? x : 0;
      px = tterm<KIND>(load_elem<DT>(static_cast<const char*>(target) + ro, xs), k.c1, k.c0p,
                       k.ip, tab);
      qx = tterm<KIND>(load_elem<DT>(static_cast<const char*>(draft) + ro, xs), k.c1, k.c0q,
                       k.iq, tab);
    }
    for (;;) {
      uint64_t kids = __ballot(pj == cur);  // children of cur, in index order
      if (kids == 0) break;                 // a leaf: the bonus draw from its target row
      double C = 0.0, M = 1.0;
      int acc = -1;
      for (bool first = true; kids != 0; first = false) {
        const int ji = __builtin_ctzll(kids);
        kids &= kids - 1;
        if (!first) {
          const double cn = C + M;
          const double F = lane_value_d(f[0], ji);
          if (F > 0.0) {
            C = cn;
            M = F;
          }
        }
        const double pxi = lane_value_d(px, ji), qxi = lane_value_d(qx, ji);
        const double ui = lane_value_d(uj, ji);
        if (__builtin_amdgcn_readlane((int)valid, ji) &&
            ui * qxi * M < fmax(0.0, pxi - C * qxi)) {
          acc = ji;
          break;
        }
      }
      if (acc < 0) {  // every child rejected: draw from the residual
        cf = C + M;
        cp = C;
        break;
      }
      cur = acc;
      ++depth;
      if (lane == 0) path[depth] = cur;
    }
  } else
  for (;;) {
    const int m = s_nchild[cur];
    if (m == 0) break;  // a leaf: the bonus draw from its target row
    RowPair rows{};
    // every lane merges the chunk statistics itself (uniform loads, one
    // round trip; the same numbers as in the other kernels)
    if (KIND == 0) rows = node_rows(xstat, nullptr, b, N, cur, V, 0, 0.f, c1, tab, true);
    const TermCoef k = term_coef<KIND>(rows, c1);
    const char* prow = static_cast<const char*>(target) + ((long)b * N + cur) * V * eb;
    const char* qrow = static_cast<const char*>(draft) + ((long)b * N + cur) * V * eb;
    double C = 0.0, M = 1.0;
    int acc = -1;
    int i0 = 0;
    for (int j0 = s_first[cur]; j0 >= 0;) {  // children in tiles of 64, in order
      // lane i: child i0 + i (its node, token, values at the token, uniform)
      const int n_here = min(kWaveSize, m - i0);
      int j = j0;
      for (int s = 0; s < lane && s < n_here - 1; ++s) j = s_next[j];
      double px = 0.0, qx = 0.0, uu = 0.0;
      bool valid = false;
      if (lane < n_here) {
        const int x = tok[j];
        valid = x >= 0 && x < V;
        const int xs = valid ? x : 0;
        px = tterm<KIND>(load_elem<DT>(prow, xs), k.c1, k.c0p, k.ip, tab);
        qx = tterm<KIND>(load_elem<DT>(qrow, xs), k.c1, k.c0q, k.iq, tab);
        uu = (double)get_uniform(uniforms, seed, ctr0, b, j, 0, N - 1);
      }
      for (int i = 0; i < n_here; ++i) {  // wave-uniform
        const int ji = __shfl(j, i, kWaveSize);
        if (i0 + i > 0) {
          const double cn = C + M;
          const double F = wave_sum_fixed(mpart + ((long)b * N + ji) * Cm, Cm);
          if (F > 0.0) {
            C = cn;
            M = F;
          }
        }
        const double pxi = __shfl(px, i, kWaveSize), qxi = __shfl(qx, i, kWaveSize);
        const double ui = __shfl(uu, i, kWaveSize);
        if (__shfl((int)valid, i, kWaveSize) && ui * qxi * M < fmax(0.0, pxi - C * qxi)) {
          acc = ji;
          break;
        }
      }
      if (acc >= 0) break;
      i0 += n_here;
      if (i0 >= m) break;
      j0 = s_next[__shfl(j, kWaveSize - 1, kWaveSize)];  // after the tile's last child
    }
    if (acc < 0) {  // every child rejected: draw from the residual
      cf = C + M;
      cp = C;
      break;
    }
    cur = acc;
    ++depth;
    if (lane == 0) path[depth] = cur;
  }
  wave_lds_sync();
  // Outputs: the accepted path's tokens then -1 (the final token comes from
  // k_tree_draw), the path, the draw state.
  for (int d = lane; d <= D; d += kWaveSize) {
    const int node = d <= depth ? path[d] : -1;
    if (d >= 1 && d <= depth) out_tokens[(long)b * (D + 1) + d - 1] = tok[node];
    if (d > depth) out_tokens[(long)b * (D + 1) + d] = -1;
    if (out_path != nullptr) out_path[(long)b * (D + 1) + d] = node;
  }
  if (lane == 0) {
    accepted_len[b] = depth;
    TreeDraw st;
    st.node = cur;
    st.depth = depth;
    st.cf = cf;
    st.cp = cp;
    tstate[b] = st;
  }
}

// The draw of request b by one wave, from the chunk totals dp (entry 0 at
// cf, entry 1 at cp, as k_tree_draw stored them in this launch: coherent
// loads): t = min{ j : P(c) + run_c(j) > u * total }, P(c) the running total
// of the chunks before chunk c in chunk order.
template <int DT, int NE, int KIND>
__device__ __forceinline__ void tree_pick_wave(
    const void* __restrict__ target, const void* __restrict__ draft, int b, int N, int V, int C1,
    int C2, int D, float c, double c1, const float* __restrict__ uniforms, uint64_t seed,
    uint64_t ctr0, const TreeDraw& st, const uint64_t* __restrict__ part,
    const TreeStat64* __restrict__ xstat, const double* __restrict__ dp, const double* tab,
    int32_t* __restrict__ out_tokens) {
  const int lane = threadIdx.x & 63;
  // The chunk totals of the first kPickTiles tiles of 64 chunks (both
  // entries) come into registers in one round trip, together with the row
  // statistics' loads; tiles past them (rows beyond kPickTiles * 64
  // chunks) are loaded as the scans reach them.
  constexpr int kPickTiles = 8;
  double r0[kPickTiles], r1[kPickTiles];
#pragma unroll
  for (int t = 0; t < kPickTiles; ++t) {
    const int ch = t * kWaveSize + lane;
    const long cc = min(ch, C2 - 1);  // unconditional loads
    const double a0 = ld_dev_d(&dp[cc * 2]), a1 = ld_dev_d(&dp[cc * 2 + 1]);
    r0[t] = ch < C2 ? a0 : 0.0;
    r1[t] = ch < C2 ? a1 : 0.0;
  }
  RowPair rows{};
  if (KIND == 0) rows = node_rows(xstat, part, b, N, st.node, V, C1, c, c1, tab, st.cf > 0.0);
  const int n_tiles = (C2 + kWaveSize - 1) / kWaveSize;
  auto entry = [&](int t, int w) {  // chunk t * 64 + lane's total, entry w
    double v = 0.0;
#pragma unroll
    for (int i = 0; i < kPickTiles; ++i)
      if (i == t) v = w ? r1[i] : r0[i];
    if (t >= kPickTiles) {
      const int ch = t * kWaveSize + lane;
      v = ch < C2 ? ld_dev_d(&dp[(long)ch * 2 + w]) : 0.0;
    }
    return v;
  };
  int which = 0;
  double C = st.cf;
  bool use_q = st.cf > 0.0;
  if (use_q) {  // empty residual: the weights before the last rejection
    double any = 0.0;
    for (int t = 0; t < n_tiles; ++t) any += entry(t, 0);
    if (!(wave_sum_d(any) > 0.0)) {
      which = 1;
      C = st.cp;
      use_q = st.cp > 0.0;
    }
  }
  // Running chunk totals in chunk order: tiles of 64 chunks, lane l on
  // chunk base + l, a wave scan per tile.  The grand total and the search
  // below run the same scans, so they see the same prefixes.
  const double u = (double)get_uniform(uniforms, seed, ctr0, b, st.node, 1, N - 1);
  auto tile = [&](int t, double running, double& v, double& excl) {
    v = entry(t, which);
    const double inc = wave_inclusive_scan_d(v);
    excl = running + (inc - v);
    return running + __shfl(inc, 63, 64);  // running total after the tile
  };
  double total = 0.0;
  for (int t = 0; t < n_tiles; ++t) {  // wave-uniform
    double v, excl;
    total = tile(t, total, v, excl);
  }
  int tok = -1;
  if (total > 0.0) {
    const double thr = u * total;
    // The first chunk whose running total exceeds thr, and the total of
    // the chunks before it (past the end, a last-bit difference: the last).
    int sel = C2 - 1;
    double P = 0.0, running = 0.0;
    for (int t = 0; t < n_tiles; ++t) {  // wave-uniform
      const int base = t * kWaveSize;
      double v, excl;
      const double after = tile(t, running, v, excl);
      const uint64_t mh = __ballot(base + lane < C2 && excl + v > thr);
      if (mh != 0) {
        const int f = __builtin_ctzll(mh);
        sel = base + f;
        P = __shfl(excl, f, 64);
        break;
      }
      if (base + kWaveSize >= C2) {
        P = __shfl(excl, C2 - 1 - base, 64);
        break;
      }
      running = after;
    }
    const TermCoef k = term_coef<KIND>(rows, c1);
    const long eb = Elems<DT>::kBytes;
    const void* prow = static_cast<const char*>(target) + ((long)b * N + st.node) * V * eb;
    const void* qrow = static_cast<const char*>(draft) + ((long)b * N + st.node) * V * eb;
    double run[kSegPerThread], base;
    chunk_scan<DT, NE, KIND>(prow, qrow, V, sel, C, use_q, k, tab, run, base);
    int hit = INT_MAX, lastpos = -1;
    const long j0 = (long)sel * kDrawChunk + (long)lane * kSegPerThread;
#pragma unroll
    for (int e = 0; e < kSegPerThread; ++e) {
      const long j = j0 + e;
      if (j < V) {
        if (run[e] > (e == 0 ? base : run[e - 1])) lastpos = static_cast<int>(j);
        if (hit == INT_MAX && P + run[e] > thr) hit = static_cast<int>(j);
      }
    }
    const uint64_t mh = __ballot(hit != INT_MAX);
    if (mh != 0) {
      tok = __shfl(hit, __builtin_ctzll(mh), 64);
    } else {
      // u * total rounded up to total (no chunk's running total exceeds
      // it): the last positive-weight element of the last chunk
      const uint64_t ml = __ballot(lastpos >= 0);
      tok = ml ? __shfl(lastpos, 63 - __builtin_clzll(ml), 64) : -1;
    }
  }
  if (lane == 0) out_tokens[(long)b * (D + 1) + st.depth] = tok;
}

// Draw weights of the stop node: chunk totals at cf (entry 0) and, after a
// rejection, at cp (entry 1, used only if cf's weights have no mass); the
// request's last work-group (completion ticket) then draws the token on one
// wave.
template <int DT, int NE, int KIND>
__global__ __launch_bounds__(kThreads) void k_tree_draw(
    const void* __restrict__ target, const void* __restrict__ draft, int N, int V, int C1, int C2,
    int D, float c, double c1, const float* __restrict__ uniforms, uint64_t seed, uint64_t ctr0,
    const TreeDraw* __restrict__ tstate, const uint64_t* __restrict__ part,
    const TreeStat64* __restrict__ xstat, double* __restrict__ dpart,
    unsigned* __restrict__ counters, int32_t* __restrict__ out_tokens) {
  __shared__ double tab[256];
  __shared__ RowPair s_rows;
  const int G = (C2 + kTreeChunksPerGroup - 1) / kTreeChunksPerGroup;
  const int g = static_cast<int>(blockIdx.x % G);
  const int b = static_cast<int>(blockIdx.x / G);
  const TreeDraw st = tstate[b];
  const bool use_q = st.cf > 0.0;
  if (KIND == 0) {
    tab[threadIdx.x] = kExp2Frac256[threadIdx.x];
    __syncthreads();
    if (threadIdx.x == 0) s_rows = node_rows(xstat, part, b, N, st.node, V, C1, c, c1, tab, use_q);
  }
  __syncthreads();
  RowPair rows{};
  if (KIND == 0) rows = s_rows;
  const TermCoef k = term_coef<KIND>(rows, c1);
  const long eb = Elems<DT>::kBytes;
  const void* prow = static_cast<const char*>(target) + ((long)b * N + st.node) * V * eb;
  const void* qrow = static_cast<const char*>(draft) + ((long)b * N + st.node) * V * eb;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  double* dp = dpart + (long)b * C2 * 2;
  for (int t = 0; t < kTreeChunksPerWave; ++t) {
    const long ch = (long)g * kTreeChunksPerGroup + wave * kTreeChunksPerWave + t;
    if (ch >= C2) break;  // wave-uniform
    double tf, tp = 0.0;
    if (use_q) {
      chunk_totals2<DT, NE, KIND>(prow, qrow, V, ch, st.cf, true, st.cp, st.cp > 0.0, k, tab, tf,
                                  tp);
    } else {
      double run[kSegPerThread], base;
      tf = chunk_scan<DT, NE, KIND>(prow, qrow, V, ch, st.cf, false, k, tab, run, base);
    }
    if (lane == 0) {
      st_dev_d(&dp[ch * 2], tf);
      st_dev_d(&dp[ch * 2 + 1], tp);
    }
  }
  wait_stores();  // every wave's totals complete before the ticket below
  __syncthreads();
  if (!block_arrive(&counters[(long)b * kCountersPerReq + 1], (unsigned)G)) return;
  if (wave != 0) return;
  // The last work-group of request b: it decides when the request ends
  // while the others stream, so it issues first.
  __builtin_amdgcn_s_setprio(3);
  tree_pick_wave<DT, NE, KIND>(target, draft, b, N, V, C1, C2, D, c, c1, uniforms, seed, ctr0,
                               st, part, xstat, dp, tab, out_tokens);
}

// ---------------------------------------------------------------------------
// Host launcher
// ---------------------------------------------------------------------------

static bool tree_rows_aligned(const void* p, int V, int dtype) {
  const long eb = dtype == 1 ? 2 : 4;
  return (reinterpret_cast<uintptr_t>(p) % 16 == 0) && (((long)V * eb) % 16 == 0) &&
         (long)V * eb < (1L << 31);
}

template <int DT, int NE, int KIND>
static hipError_t launch_tree_sample_t(const void* target, const void* draft, int B, int N, int V,
                                       const TreeArgs& tree, const TreeShape& shape,
                                       const int32_t* node_tokens, const float* uniforms,
                                       uint64_t seed, uint64_t ctr0, float temperature,
                                       int32_t* accepted_len, int32_t* out_tokens,
                                       int32_t* out_path, char* w, const WsLayout& L,
                                       hipStream_t s) {
  const int C1 = (V + kRowChunkElems - 1) / kRowChunkElems;
  const int C2 = res_chunks(V);
  const float c = KIND == 0 ? 1.4426950408889634f / temperature : 1.f;
  // 256 / (T ln 2) in float64 (the float64 terms' scale, as the oracle's T)
  const double c1 = KIND == 0 ? (1.0 / (double)temperature) * kInvLn2x256 : 0.0;
  auto* xstat = reinterpret_cast<TreeStat64*>(w + L.xstat);
  auto* tables = reinterpret_cast<int*>(w + L.tree);
  auto* part = reinterpret_cast<uint64_t*>(w + L.part1);
  auto* mpart = reinterpret_cast<double*>(w + L.part3);
  auto* dpart = reinterpret_cast<double*>(w + L.part2);
  auto* tstate = reinterpret_cast<TreeDraw*>(w + L.tstate);
  static_assert(sizeof(TreeDraw) <= kTreeDrawBytes, "draw state fits its region");
  static_assert(sizeof(TreeStat64) == kTreeStatBytes, "float64 statistic fits its region");
  hipError_t e = hipSuccess;
  // Small trees: small argument blocks (launches with a 2 KiB one start
  // much later), and with logits the tables come from the row-statistics
  // launch (its first work-group), not a launch of their own.
  const bool small = N <= kSmallTree;
  TreeArgsN<kSmallTree> small_tree{}, internal{};
  if (small) {
    for (int j = 0; j < N; ++j) small_tree.parent[j] = tree.parent[j];
    int ni = 0;
    for (int j = 0; j < N; ++j)
      if (shape.has_child[j]) internal.parent[ni++] = (int16_t)j;
  }
  if (!small)
    e = launch_timed(kProfTreeWalk, &k_tree_setup<kMaxNodes>, dim3(1), dim3(kThreads), 0, s,
                     tree, N, tables);
  else if (KIND != 0)
    e = launch_timed(kProfTreeWalk, &k_tree_setup<kSmallTree>, dim3(1), dim3(kThreads), 0, s,
                     small_tree, N, tables);
  if (e != hipSuccess) return e;
  if (KIND == 0) {
    const long nA = std::max(1L, (long)B * 2 * shape.n_internal * tree_xchunks(V));
    if (small)
      e = launch_timed(kProfTreeStats, &k_tree_stats<DT, NE, true>, dim3((unsigned)nA),
                       dim3(kThreads), 0, s, target, draft, N, shape.n_internal, V, c1,
                       small_tree, internal, tables, xstat);
    else
      e = launch_timed(kProfTreeStats, &k_tree_stats<DT, NE, false>, dim3((unsigned)nA),
                       dim3(kThreads), 0, s, target, draft, N, shape.n_internal, V, c1,
                       small_tree, internal, tables, xstat);
    if (e != hipSuccess) return e;
  }
  const int Cm = tree_mchunks(V);
  for (int r = 1; r <= shape.max_rank; ++r) {
    const int n_units = shape.rank_count[r];
    if (n_units == 0) continue;
    e = launch_timed(kProfTreeMass, &k_tree_mass<DT, NE, KIND>,
                     dim3((unsigned)((long)B * n_units * Cm)), dim3(kThreads), 0, s, target,
                     draft, N, V, Cm, c1, r, n_units, (const int*)tables,
                     (const TreeStat64*)xstat, mpart);
    if (e != hipSuccess) return e;
  }
  const int G = (C2 + kTreeChunksPerGroup - 1) / kTreeChunksPerGroup;
  const int wgs = (B + kWaves - 1) / kWaves;
  e = launch_timed(kProfTreeWalk, &k_tree_walk<DT, NE, KIND>, dim3((unsigned)wgs),
                   dim3(kThreads), tree_walk_lds(N), s, target, draft, B, N, V, Cm, shape.depth,
                   c1, node_tokens, uniforms, seed, ctr0, (const int*)tables,
                   (const TreeStat64*)xstat, (const double*)mpart, tstate, accepted_len,
                   out_tokens, out_path);
  if (e != hipSuccess) return e;
  if (KIND == 0) {  // the stop leaves' row statistics (logits)
    e = launch_timed(kProfTreeLeaf, &k_tree_leaf<DT, NE>, dim3((unsigned)((long)B * C1)),
                     dim3(kThreads), 0, s, target, N, V, C1, c, (const TreeDraw*)tstate, part);
    if (e != hipSuccess) return e;
  }
  return launch_timed(kProfTreeDraw, &k_tree_draw<DT, NE, KIND>, dim3((unsigned)((long)B * G)),
                      dim3(kThreads), 0, s, target, draft, N, V, C1, C2, shape.depth, c, c1,
                      uniforms, seed, ctr0, (const TreeDraw*)tstate, (const uint64_t*)part,
                      (const TreeStat64*)xstat, dpart, reinterpret_cast<unsigned*>(w + L.count),
                      out_tokens);
}

hipError_t launch_tree_sample(const void* target, const void* draft, int dtype, int kind, int B,
                              int N, int V, const TreeArgs& tree, const TreeShape& shape,
                              const int32_t* node_tokens, const float* uniforms, uint64_t seed,
                              uint64_t counter0, float temperature, int32_t* accepted_len,
                              int32_t* out_tokens, int32_t* out_path, void* ws,
                              const WsLayout& L, hipStream_t s) {
  char* w = static_cast<char*>(ws);
  const bool vec = tree_rows_aligned(target, V, dtype) && tree_rows_aligned(draft, V, dtype);
  if (kind == 1)
    return vec ? launch_tree_sample_t<0, 4, 1>(target, draft, B, N, V, tree, shape, node_tokens,
                                               uniforms, seed, counter0, temperature,
                                               accepted_len, out_tokens, out_path, w, L, s)
               : launch_tree_sample_t<0, 1, 1>(target, draft, B, N, V, tree, shape, node_tokens,
                                               uniforms, seed, counter0, temperature,
                                               accepted_len, out_tokens, out_path, w, L, s);
  if (dtype == 1)
    return vec ? launch_tree_sample_t<1, 8, 0>(target, draft, B, N, V, tree, shape, node_tokens,
                                               uniforms, seed, counter0, temperature,
                                               accepted_len, out_tokens, out_path, w, L, s)
               : launch_tree_sample_t<1, 1, 0>(target, draft, B, N, V, tree, shape, node_tokens,
                                               uniforms, seed, counter0, temperature,
                                               accepted_len, out_tokens, out_path, w, L, s);
  return vec ? launch_tree_sample_t<0, 4, 0>(target, draft, B, N, V, tree, shape, node_tokens,
                                             uniforms, seed, counter0, temperature, accepted_len,
                                             out_tokens, out_path, w, L, s)
             : launch_tree_sample_t<0, 1, 0>(target, draft, B, N, V, tree, shape, node_tokens,
                                             uniforms, seed, counter0, temperature, accepted_len,
                                             out_tokens, out_path, w, L, s);
}

}  // namespace specv
