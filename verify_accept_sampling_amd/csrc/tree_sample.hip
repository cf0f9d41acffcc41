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
//   k_tree_setup     one work-group: child lists, ranks, depths, the list of
//                    nodes with children, and the children of rank >= 1 by
//                    rank, from the parent array, into the workspace;
//   k_tree_stats     (logits) float32 row statistic of every target row and
//                    of the draft rows of nodes with children;
//   k_tree_mass      one launch per round: per (request, child of rank i,
//                    chunk) the chunk's sum of max(0, p - C_i q) at its
//                    parent;
//   k_tree_walk      one wave per request: the tests, the accepted path, the
//                    outputs but the final token, and the draw state;
//   k_tree_draw_part per (request, chunk) the chunk's draw-weight total;
//   k_tree_pick      one wave per request: chunk by running total, then the
//                    element, by the same per-chunk scan as k_tree_draw_part.
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

template <int NMAX>
__global__ __launch_bounds__(kThreads) void k_tree_setup(TreeArgsN<NMAX> tree, int N,
                                                        int* __restrict__ tables) {
  __shared__ int nchild[NMAX], first[NMAX], next[NMAX], rank[NMAX], depth[NMAX];
  __shared__ int internal[NMAX], ranked[NMAX], rank_off[NMAX], fill[NMAX];
  for (int j = threadIdx.x; j < NMAX; j += kThreads) {
    nchild[j] = 0;
    first[j] = next[j] = -1;
    rank[j] = depth[j] = 0;
    internal[j] = ranked[j] = rank_off[j] = fill[j] = 0;
  }
  __syncthreads();
  if (threadIdx.x == 0) {  // O(N), sequential: N <= NMAX
    // From the last node down, so each child list is ascending.
    for (int j = N - 1; j >= 1; --j) {
      const int u = tree.parent[j];
      next[j] = first[u];
      first[u] = j;
      ++nchild[u];
    }
    int max_rank = 0, n_int = 0;
    for (int u = 0; u < N; ++u) {  // parents precede their children
      int r = 0;
      for (int j = first[u]; j >= 0; j = next[j]) {
        rank[j] = r++;
        depth[j] = depth[u] + 1;
      }
      if (r > 0) internal[n_int++] = u;
      if (r - 1 > max_rank) max_rank = r - 1;
    }
    // Children of rank >= 1 grouped by rank (counting sort), ascending
    // index within a rank.
    for (int j = 1; j < N; ++j)
      if (rank[j] >= 1) ++fill[rank[j]];
    int pos = 0;
    for (int r = 1; r <= max_rank; ++r) {
      rank_off[r - 1] = pos;
      pos += fill[r];
      fill[r] = rank_off[r - 1];
    }
    rank_off[max_rank] = pos;
    for (int j = 1; j < N; ++j)
      if (rank[j] >= 1) ranked[fill[rank[j]]++] = j;
  }
  __syncthreads();
  for (int j = threadIdx.x; j < N; j += kThreads) {
    tables[kTabParent * kMaxNodes + j] = j == 0 ? -1 : tree.parent[j];
    tables[kTabNChild * kMaxNodes + j] = nchild[j];
    tables[kTabFirst * kMaxNodes + j] = first[j];
    tables[kTabNext * kMaxNodes + j] = next[j];
    tables[kTabRank * kMaxNodes + j] = rank[j];
    tables[kTabDepth * kMaxNodes + j] = depth[j];
    tables[kTabInternal * kMaxNodes + j] = internal[j];
    tables[kTabRanked * kMaxNodes + j] = ranked[j];
    tables[kTabRankOff * kMaxNodes + j] = rank_off[j];
  }
}

// ---------------------------------------------------------------------------
// Shared pieces
// ---------------------------------------------------------------------------

// Row statistics (reference M, sum S) of target row u and draft row u of
// request b, whose chunk partials k_tree_stats stored at rows b*2N + u and
// b*2N + N + u.
struct RowPair {
  float mp, mq;
  double sp, sq;
};
__device__ __forceinline__ RowPair tree_rows(const uint64_t* part, int b, int N, int u, int C1,
                                             float c, bool with_q) {
  RowPair r;
  const long base = (long)b * 2 * N;
  merge_two_rows(part, (base + u) * C1, (base + N + u) * C1, with_q, C1, c, r.mp, r.sp, r.mq,
                 r.sq);
  return r;
}

// Normalised-term coefficients: p_j = 2^(t/256) / S with
// t = z * 256 c - 256 fl32(M c), i.e. 2^(z c - fl32(M c)) / S, the
// distribution the float32 row statistic describes.  Probability rows are
// used as given.
struct TermCoef {
  double c1, c0p, c0q, ip, iq;
};
template <int KIND>
__device__ __forceinline__ TermCoef term_coef(const RowPair& r, float c) {
  TermCoef k;
  if (KIND == 0) {
    k.c1 = 256.0 * (double)c;
    k.c0p = -256.0 * (double)mul_rn(r.mp, c);
    k.c0q = -256.0 * (double)mul_rn(r.mq, c);
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
                                               int N, int C2, int u, int r, double& C,
                                               double& M) {
  C = 0.0;
  M = 1.0;
  int j = tree_tab(tables, kTabFirst)[u];
  for (int i = 0; i < r && j >= 0; ++i) {
    // state for child rank i + 1 from child rank i's rejection
    j = tree_tab(tables, kTabNext)[j];
    if (j < 0) break;
    const double cn = C + M;
    const double F = wave_sum_fixed(mpart + ((long)b * N + j) * C2, C2);
    if (F > 0.0) {
      C = cn;
      M = F;
    }
  }
}

// ---------------------------------------------------------------------------
// Kernels
// ---------------------------------------------------------------------------

// Row statistic of one chunk of one row: rows 0 .. N-1 of a request are
// the target rows, rows N .. N + n_int - 1 the draft rows of the nodes with
// children.
template <int DT, int NE>
__global__ __launch_bounds__(kThreads) void k_tree_stats(
    const void* __restrict__ target, const void* __restrict__ draft, int N, int n_int, int V,
    int C1, float c, const int* __restrict__ tables, uint64_t* __restrict__ part) {
  const long idx = blockIdx.x;
  const int chunk = static_cast<int>(idx % C1);
  const int rr = static_cast<int>((idx / C1) % (N + n_int));
  const int b = static_cast<int>(idx / C1 / (N + n_int));
  const long eb = Elems<DT>::kBytes;
  int node, slot;
  const void* rp;
  if (rr < N) {
    node = rr;
    slot = rr;
    rp = static_cast<const char*>(target) + ((long)b * N + node) * V * eb;
  } else {
    node = tree_tab(tables, kTabInternal)[rr - N];
    slot = N + node;
    rp = static_cast<const char*>(draft) + ((long)b * N + node) * V * eb;
  }
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
  if (threadIdx.x == 0) part[((long)b * 2 * N + slot) * C1 + chunk] = pack2(m, (float)s);
}

// Work-groups cover kTreeChunksPerGroup consecutive chunks of one row pair.
constexpr int kTreeChunksPerWave = 2;
constexpr int kTreeChunksPerGroup = kWaves * kTreeChunksPerWave;

// Mass round r: unit = a child j of rank r (its parent u has more than r
// children); the chunk sums of max(0, p_u - C_r q_u).
template <int DT, int NE, int KIND>
__global__ __launch_bounds__(kThreads) void k_tree_mass(
    const void* __restrict__ target, const void* __restrict__ draft, int N, int V, int C1,
    int C2, float c, int r, int n_units, const int* __restrict__ tables,
    const uint64_t* __restrict__ part, double* __restrict__ mpart) {
  __shared__ double tab[256];
  __shared__ RowPair s_rows;
  __shared__ double s_C;
  const int G = (C2 + kTreeChunksPerGroup - 1) / kTreeChunksPerGroup;
  const long idx = blockIdx.x;
  const int g = static_cast<int>(idx % G);
  const int unit = static_cast<int>((idx / G) % n_units);
  const int b = static_cast<int>(idx / G / n_units);
  const int j = tree_tab(tables, kTabRanked)[tree_tab(tables, kTabRankOff)[r - 1] + unit];
  const int u = tree_tab(tables, kTabParent)[j];
  if (KIND == 0) tab[threadIdx.x] = kExp2Frac256[threadIdx.x];
  if (threadIdx.x < kWaveSize) {
    double C, M;
    residual_state(tables, mpart, b, N, C2, u, r - 1, C, M);
    if (threadIdx.x == 0) {
      s_C = C + M;
      if (KIND == 0) s_rows = tree_rows(part, b, N, u, C1, c, true);
    }
  }
  __syncthreads();
  const double C = s_C;
  RowPair rows{};
  if (KIND == 0) rows = s_rows;
  const TermCoef k = term_coef<KIND>(rows, c);
  const long eb = Elems<DT>::kBytes;
  const void* prow = static_cast<const char*>(target) + ((long)b * N + u) * V * eb;
  const void* qrow = static_cast<const char*>(draft) + ((long)b * N + u) * V * eb;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  double* out = mpart + ((long)b * N + j) * C2;
  for (int t = 0; t < kTreeChunksPerWave; ++t) {
    const long ch = (long)g * kTreeChunksPerGroup + wave * kTreeChunksPerWave + t;
    if (ch >= C2) break;  // wave-uniform
    double run[kSegPerThread], base;
    const double tot = chunk_scan<DT, NE, KIND>(prow, qrow, V, ch, C, true, k, tab, run, base);
    if (lane == 0) out[ch] = tot;
  }
}

// The walk: one wave per request.
template <int DT, int KIND>
__global__ __launch_bounds__(kThreads) void k_tree_walk(
    const void* __restrict__ target, const void* __restrict__ draft, int B, int N, int V, int C1,
    int C2, int D, float c, const int32_t* __restrict__ node_tokens,
    const float* __restrict__ uniforms, uint64_t seed, uint64_t ctr0,
    const int* __restrict__ tables, const uint64_t* __restrict__ part,
    const double* __restrict__ mpart, TreeDraw* __restrict__ tstate,
    int32_t* __restrict__ accepted_len, int32_t* __restrict__ out_tokens,
    int32_t* __restrict__ out_path) {
  __shared__ double tab[256];
  __shared__ int s_path[kWaves][kMaxNodes];
  if (KIND == 0) tab[threadIdx.x] = kExp2Frac256[threadIdx.x];
  __syncthreads();
  const int b = static_cast<int>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
  if (b >= B) return;  // wave-uniform
  const int lane = threadIdx.x & 63;
  const long eb = Elems<DT>::kBytes;
  const int* nchild = tree_tab(tables, kTabNChild);
  const int* first = tree_tab(tables, kTabFirst);
  const int* next = tree_tab(tables, kTabNext);
  int* path = s_path[threadIdx.x >> 6];
  int cur = 0, depth = 0;
  double cf = 0.0, cp = 0.0;
  if (lane == 0) path[0] = 0;
  for (;;) {
    const int m = nchild[cur];
    if (m == 0) break;  // a leaf: the bonus draw from its target row
    RowPair rows{};
    if (KIND == 0) rows = tree_rows(part, b, N, cur, C1, c, true);
    const TermCoef k = term_coef<KIND>(rows, c);
    const char* prow = static_cast<const char*>(target) + ((long)b * N + cur) * V * eb;
    const char* qrow = static_cast<const char*>(draft) + ((long)b * N + cur) * V * eb;
    double C = 0.0, M = 1.0;
    int acc = -1;
    int i = 0;
    for (int j = first[cur]; j >= 0; j = next[j], ++i) {
      if (i > 0) {
        const double cn = C + M;
        const double F = wave_sum_fixed(mpart + ((long)b * N + j) * C2, C2);
        if (F > 0.0) {
          C = cn;
          M = F;
        }
      }
      const int x = node_tokens[(long)b * N + j];
      bool accept = false;
      if (x >= 0 && x < V) {
        const double px = tterm<KIND>(load_elem<DT>(prow, x), k.c1, k.c0p, k.ip, tab);
        const double qx = tterm<KIND>(load_elem<DT>(qrow, x), k.c1, k.c0q, k.iq, tab);
        const double u = (double)get_uniform(uniforms, seed, ctr0, b, j, 0, N - 1);
        accept = u * qx * M < fmax(0.0, px - C * qx);
      }
      if (accept) {
        acc = j;
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
  wave_lds_sync();
  // Outputs: the accepted path's tokens then -1 (the final token comes from
  // k_tree_pick), the path, the draw state.
  for (int d = lane; d <= D; d += kWaveSize) {
    const int node = d <= depth ? path[d] : -1;
    if (d >= 1 && d <= depth)
      out_tokens[(long)b * (D + 1) + d - 1] = node_tokens[(long)b * N + node];
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

// Draw weights of the stop node: chunk totals at cf (entry 0) and, after a
// rejection, at cp (entry 1, used only if cf's weights have no mass).
template <int DT, int NE, int KIND>
__global__ __launch_bounds__(kThreads) void k_tree_draw_part(
    const void* __restrict__ target, const void* __restrict__ draft, int N, int V, int C1, int C2,
    float c, const TreeDraw* __restrict__ tstate, const uint64_t* __restrict__ part,
    double* __restrict__ dpart) {
  __shared__ double tab[256];
  __shared__ RowPair s_rows;
  const int G = (C2 + kTreeChunksPerGroup - 1) / kTreeChunksPerGroup;
  const int g = static_cast<int>(blockIdx.x % G);
  const int b = static_cast<int>(blockIdx.x / G);
  const TreeDraw st = tstate[b];
  const bool use_q = st.cf > 0.0;
  if (KIND == 0) {
    tab[threadIdx.x] = kExp2Frac256[threadIdx.x];
    if (threadIdx.x == 0) s_rows = tree_rows(part, b, N, st.node, C1, c, use_q);
  }
  __syncthreads();
  RowPair rows{};
  if (KIND == 0) rows = s_rows;
  const TermCoef k = term_coef<KIND>(rows, c);
  const long eb = Elems<DT>::kBytes;
  const void* prow = static_cast<const char*>(target) + ((long)b * N + st.node) * V * eb;
  const void* qrow = static_cast<const char*>(draft) + ((long)b * N + st.node) * V * eb;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int t = 0; t < kTreeChunksPerWave; ++t) {
    const long ch = (long)g * kTreeChunksPerGroup + wave * kTreeChunksPerWave + t;
    if (ch >= C2) break;  // wave-uniform
    double run[kSegPerThread], base;
    const double tf =
        chunk_scan<DT, NE, KIND>(prow, qrow, V, ch, st.cf, use_q, k, tab, run, base);
    double tp = 0.0;
    if (use_q)
      tp = chunk_scan<DT, NE, KIND>(prow, qrow, V, ch, st.cp, st.cp > 0.0, k, tab, run, base);
    if (lane == 0) {
      dpart[((long)b * C2 + ch) * 2] = tf;
      dpart[((long)b * C2 + ch) * 2 + 1] = tp;
    }
  }
}

// The draw: t = min{ j : P(c) + run_c(j) > u * total }, P(c) the running
// total of the chunks before chunk c in chunk order.
template <int DT, int NE, int KIND>
__global__ __launch_bounds__(kThreads) void k_tree_pick(
    const void* __restrict__ target, const void* __restrict__ draft, int B, int N, int V, int C1,
    int C2, int D, float c, const float* __restrict__ uniforms, uint64_t seed, uint64_t ctr0,
    const TreeDraw* __restrict__ tstate, const uint64_t* __restrict__ part,
    const double* __restrict__ dpart, int32_t* __restrict__ out_tokens) {
  __shared__ double tab[256];
  if (KIND == 0) tab[threadIdx.x] = kExp2Frac256[threadIdx.x];
  __syncthreads();
  const int b = static_cast<int>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
  if (b >= B) return;  // wave-uniform
  const int lane = threadIdx.x & 63;
  const TreeDraw st = tstate[b];
  const double* dp = dpart + (long)b * C2 * 2;
  int which = 0;
  double C = st.cf;
  bool use_q = st.cf > 0.0;
  if (use_q && !(wave_sum_fixed(dp, C2, 2) > 0.0)) {  // empty residual: the weights before it
    which = 1;
    C = st.cp;
    use_q = st.cp > 0.0;
  }
  // Running chunk totals, in chunk order, on lane 0 (the prefix the chunk
  // scan's sums are added to; one order everywhere).
  const double u = (double)get_uniform(uniforms, seed, ctr0, b, st.node, 1, N - 1);
  double total = 0.0;
  if (lane == 0)
    for (int ch = 0; ch < C2; ++ch) total += dp[(long)ch * 2 + which];
  total = __shfl(total, 0, 64);
  int tok = -1;
  if (total > 0.0) {
    const double thr = u * total;
    int sel = C2 - 1;
    double P = 0.0;
    if (lane == 0) {
      double run = 0.0;
      for (int ch = 0; ch < C2; ++ch) {
        const double nx = run + dp[(long)ch * 2 + which];
        if (nx > thr) {
          sel = ch;
          break;
        }
        run = nx;
      }
      P = run;
    }
    sel = __shfl(sel, 0, 64);
    P = __shfl(P, 0, 64);
    RowPair rows{};
    if (KIND == 0) rows = tree_rows(part, b, N, st.node, C1, c, use_q);
    const TermCoef k = term_coef<KIND>(rows, c);
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
  auto* tables = reinterpret_cast<int*>(w + L.tree);
  auto* part = reinterpret_cast<uint64_t*>(w + L.part1);
  auto* mpart = reinterpret_cast<double*>(w + L.part3);
  auto* dpart = reinterpret_cast<double*>(w + L.part2);
  auto* tstate = reinterpret_cast<TreeDraw*>(w + L.tstate);
  static_assert(sizeof(TreeDraw) <= kTreeDrawBytes, "draw state fits its region");
  hipError_t e;
  if (N <= kSmallTree) {
    // a small argument block: launches with a 2 KiB one start much later
    TreeArgsN<kSmallTree> small;
    for (int j = 0; j < kSmallTree; ++j) small.parent[j] = j < N ? tree.parent[j] : 0;
    e = launch_timed(kProfTreeWalk, &k_tree_setup<kSmallTree>, dim3(1), dim3(kThreads), 0, s,
                     small, N, tables);
  } else {
    e = launch_timed(kProfTreeWalk, &k_tree_setup<kMaxNodes>, dim3(1), dim3(kThreads), 0, s,
                     tree, N, tables);
  }
  if (e != hipSuccess) return e;
  if (KIND == 0) {
    const long blocks = (long)B * (N + shape.n_internal) * C1;
    e = launch_timed(kProfTreeStats, &k_tree_stats<DT, NE>, dim3((unsigned)blocks),
                     dim3(kThreads), 0, s, target, draft, N, shape.n_internal, V, C1, c,
                     (const int*)tables, part);
    if (e != hipSuccess) return e;
  }
  const int G = (C2 + kTreeChunksPerGroup - 1) / kTreeChunksPerGroup;
  for (int r = 1; r <= shape.max_rank; ++r) {
    const int n_units = shape.rank_count[r];
    if (n_units == 0) continue;
    e = launch_timed(kProfTreeMass, &k_tree_mass<DT, NE, KIND>,
                     dim3((unsigned)((long)B * n_units * G)), dim3(kThreads), 0, s, target,
                     draft, N, V, C1, C2, c, r, n_units, (const int*)tables,
                     (const uint64_t*)part, mpart);
    if (e != hipSuccess) return e;
  }
  const unsigned wgs = (unsigned)((B + kWaves - 1) / kWaves);
  e = launch_timed(kProfTreeWalk, &k_tree_walk<DT, KIND>, dim3(wgs), dim3(kThreads), 0, s,
                   target, draft, B, N, V, C1, C2, shape.depth, c, node_tokens, uniforms, seed,
                   ctr0, (const int*)tables, (const uint64_t*)part, (const double*)mpart, tstate,
                   accepted_len, out_tokens, out_path);
  if (e != hipSuccess) return e;
  e = launch_timed(kProfTreeDraw, &k_tree_draw_part<DT, NE, KIND>, dim3((unsigned)((long)B * G)),
                   dim3(kThreads), 0, s, target, draft, N, V, C1, C2, c,
                   (const TreeDraw*)tstate, (const uint64_t*)part, dpart);
  if (e != hipSuccess) return e;
  return launch_timed(kProfTreeDraw, &k_tree_pick<DT, NE, KIND>, dim3(wgs), dim3(kThreads), 0, s,
                      target, draft, B, N, V, C1, C2, shape.depth, c, uniforms, seed, ctr0,
                      (const TreeDraw*)tstate, (const uint64_t*)part, (const double*)dpart,
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
