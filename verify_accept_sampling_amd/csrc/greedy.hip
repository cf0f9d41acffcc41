// Greedy chain and greedy tree verification for gfx950, one launch per call.
//
// Work-group (chunk, row) streams one chunk of one logit row with 16-byte
// non-temporal loads and reduces it to (max value, lowest index), publishes
// that partial and takes its request's completion ticket.  The last
// work-group of a request merges the partials of the request's rows and
// applies the greedy rule:
//   chain: the first draft token that differs from the target argmax ends
//          the accepted prefix and the argmax there is emitted
//          ("EAGLE-3 speculative decoding review", greedy bullets of the
//          section on whether a small draft hurts quality);
//   tree:  a node is accepted when its parent is and its token equals the
//          parent's argmax; the deepest accepted node (lowest index on ties)
//          ends the path and its argmax is emitted (same page, section on the
//          full inference loop, "Strict Acceptance").
#include <algorithm>
#include <climits>

#include "device_common.h"

namespace specv {


// Fold one group of NE elements (group index gi) into the running argmax;
// a strict '>' keeps the lowest index because groups arrive in ascending
// order within a thread.
template <int NE>
__device__ __forceinline__ void argmax_update(float& bv, int& bi, const float (&x)[NE], long gi) {
  float lm = x[0];
#pragma unroll
  for (int e = 1; e < NE; ++e) lm = fmaxf(lm, x[e]);
  if (lm > bv) {
    int first = NE - 1;
#pragma unroll
    for (int e = NE - 1; e >= 0; --e)
      if (x[e] == lm) first = e;
    bv = lm;
    bi = static_cast<int>(gi * NE + first);
  }
}

// Argmax of this thread's groups in [g0, g1) (ascending, so a strict '>'
// keeps the lowest index).  NE = elements per load.  Scalar loads (NE = 1,
// rows that are not 16-byte aligned).
template <int DT, int NE>
__device__ __forceinline__ void argmax_sweep(const void* row, long g0, long g1, float& bv,
                                             int& bi) {
  bv = -INFINITY;
  bi = INT_MAX;
  for (long g = g0 + threadIdx.x; g < g1; g += kThreads) {
    float x[NE];
    load_group<DT, NE, true>(row, g * NE, x);
    argmax_update<NE>(bv, bi, x, g);
  }
}

// Fold kArgmaxBatch words (groups g, g + NT, ...) into the running argmax.
constexpr int kArgmaxBatch = 4;
template <int DT, int NT>
__device__ __forceinline__ void argmax_words(float& bv, int& bi, const u32x4 (&w)[kArgmaxBatch],
                                             long g) {
  constexpr int NE = Elems<DT>::kVec;
#pragma unroll
  for (int u = 0; u < kArgmaxBatch; ++u) {
    float x[NE];
    unpack16<DT>(w[u], x);
    argmax_update<NE>(bv, bi, x, g + (long)u * NT);
  }
}

// 16-byte form over a row of row_bytes bytes: buffer loads (base and size
// in SGPRs, one 32-bit lane offset) in two word buffers used in turn, so the
// next batch is in flight while the current one is folded in.
template <int DT, int NT>
__device__ __forceinline__ void argmax_sweep_buf(const void* row, uint32_t row_bytes, long g0,
                                                 long g1, float& bv, int& bi) {
  constexpr int NE = Elems<DT>::kVec;
  constexpr uint32_t kStep = NT * kArgmaxBatch * 16u;
  bv = -INFINITY;
  bi = INT_MAX;
  const RowBuf buf(row, row_bytes);
  long g = g0 + threadIdx.x;
  uint32_t off = static_cast<uint32_t>(g) * 16u;
  const long span = (long)(kArgmaxBatch - 1) * NT;
  if (g + span < g1) {
    u32x4 wa[kArgmaxBatch], wb[kArgmaxBatch];
#pragma unroll
    for (int u = 0; u < kArgmaxBatch; ++u) wa[u] = buf.load_nt(off, u * NT * 16u);
    for (;;) {
      const long ga = g;
      g += (long)NT * kArgmaxBatch;
      off += kStep;
      if (!(g + span < g1)) {
        argmax_words<DT, NT>(bv, bi, wa, ga);
        break;
      }
#pragma unroll
      for (int u = 0; u < kArgmaxBatch; ++u) wb[u] = buf.load_nt(off, u * NT * 16u);
      __builtin_amdgcn_sched_barrier(0);
      argmax_words<DT, NT>(bv, bi, wa, ga);
      const long gb = g;
      g += (long)NT * kArgmaxBatch;
      off += kStep;
      if (!(g + span < g1)) {
        argmax_words<DT, NT>(bv, bi, wb, gb);
        break;
      }
#pragma unroll
      for (int u = 0; u < kArgmaxBatch; ++u) wa[u] = buf.load_nt(off, u * NT * 16u);
      __builtin_amdgcn_sched_barrier(0);
      argmax_words<DT, NT>(bv, bi, wb, gb);
    }
  }
  for (; g < g1; g += NT, off += NT * 16u) {
    float x[NE];
    unpack16<DT>(buf.load_nt(off, 0), x);
    argmax_update<NE>(bv, bi, x, g);
  }
}

// Stream this work-group's (chunk, row), publish its (value, index) partial
// and take the request's ticket.  Returns true in the request's last
// work-group.
template <int DT, int NE>
__device__ __forceinline__ bool argmax_chunk(const void* target, int n_pos, int V, int C1,
                                            uint64_t* part, unsigned* counters, int& b) {
  const int chunk = blockIdx.x % C1;
  const long row = blockIdx.x / C1;
  b = static_cast<int>(row / n_pos);
  const long n_groups = V / NE;
  const long gpc = (n_groups + C1 - 1) / C1;
  const long g0 = (long)chunk * gpc;
  const long g1 = min(g0 + gpc, n_groups);
  const void* rp = reinterpret_cast<const char*>(target) + row * (long)V * Elems<DT>::kBytes;
  float bv;
  int bi;
  if constexpr (NE == 1)
    argmax_sweep<DT, NE>(rp, g0, g1, bv, bi);
  else
    argmax_sweep_buf<DT, kThreads>(rp, static_cast<uint32_t>((long)V * Elems<DT>::kBytes), g0,
                                   g1, bv, bi);
  block_reduce_am(bv, bi);
  if (threadIdx.x == 0) st_dev(&part[row * C1 + chunk], pack2(bv, __int_as_float(bi)));
  return block_arrive(&counters[(long)b * kCountersPerReq + 0], (unsigned)(n_pos * C1));
}

// Merge every row's chunk partials of request b into amax[0..n_pos-1]
// (shared memory), one thread per row.  All-(-inf) rows resolve to index 0.
__device__ __forceinline__ void merge_argmax_rows(const uint64_t* part, int b, int n_pos, int C1,
                                                  int* amax) {
  for (int j = threadIdx.x; j < n_pos; j += kThreads) {
    const long row = (long)b * n_pos + j;
    float v = -INFINITY;
    int i = INT_MAX;
    for (int c = 0; c < C1; ++c) {
      const uint64_t p = ld_dev(&part[row * C1 + c]);
      am_merge(v, i, unpack_lo(p), __float_as_int(unpack_hi(p)));
    }
    amax[j] = (i == INT_MAX) ? 0 : i;
  }
  __syncthreads();
}

template <int DT, int NE>
__global__ __launch_bounds__(kThreads) void k_greedy_chain(
    const void* __restrict__ target, int k, int V, int C1,
    const int32_t* __restrict__ draft_tokens, int32_t* __restrict__ accepted_len,
    int32_t* __restrict__ out_tokens, uint64_t* __restrict__ part,
    unsigned* __restrict__ counters) {
  const int n_pos = k + 1;
  // Thread i < k loads draft token i of this work-group's request now; only
  // the request's last work-group uses it, by then long arrived, so its
  // finish waits on one round trip (the partials) instead of two.
  const int b0 = static_cast<int>(blockIdx.x / C1 / n_pos);
  const int my_tok = (int)threadIdx.x < k ? draft_tokens[(long)b0 * k + threadIdx.x] : -1;
  int b;
  if (!argmax_chunk<DT, NE>(target, n_pos, V, C1, part, counters, b)) return;
  if (n_pos <= kWaveSize) {
    // One wave finishes, lane j on position j, with no work-group barrier.
    if (threadIdx.x >= kWaveSize) return;
    const int lane = threadIdx.x;
    int am = 0;
    if (lane < n_pos) {
      const long row = (long)b * n_pos + lane;
      float v = -INFINITY;
      int i = INT_MAX;
      for (int c = 0; c < C1; ++c) {
        const uint64_t p = ld_dev(&part[row * C1 + c]);
        am_merge(v, i, unpack_lo(p), __float_as_int(unpack_hi(p)));
      }
      am = (i == INT_MAX) ? 0 : i;  // all-(-inf) rows resolve to index 0
    }
    const uint64_t mm = __ballot(lane < k && my_tok != am);
    const int n = mm != 0 ? __builtin_ctzll(mm) : k;
    if (lane < n_pos) out_tokens[(long)b * n_pos + lane] = lane < n ? my_tok : lane == n ? am : -1;
    if (lane == 0) accepted_len[b] = n;
    return;
  }
  __shared__ int amax[kMaxK + 1];
  merge_argmax_rows(part, b, n_pos, C1, amax);
  int first = k;
  for (int i = threadIdx.x; i < k; i += kThreads)
    if (draft_tokens[(long)b * k + i] != amax[i]) first = min(first, i);
  const int n = block_min_i(first);
  for (int i = threadIdx.x; i <= k; i += kThreads) {
    int t = -1;
    if (i < n) t = draft_tokens[(long)b * k + i];
    else if (i == n) t = amax[n];
    out_tokens[(long)b * n_pos + i] = t;
  }
  if (threadIdx.x == 0) accepted_len[b] = n;
}

// Small chains (up to 64 positions, every row of a request within
// kSmallChainElems elements in all): one work-group per request of one wave
// per row (at most kSmallChainWaves; wave w takes rows w, w + waves, ...),
// lanes striding each row; the row argmaxes meet in shared memory and wave
// 0 applies the greedy rule.  No partials and no ticket: one round trip of
// row loads instead of three dependent ones.
constexpr long kSmallChainElems = 16384;
constexpr int kSmallChainWaves = 16;
template <int DT, int NE>
__global__ __launch_bounds__(kSmallChainWaves * kWaveSize) void k_greedy_chain_small(
    const void* __restrict__ target, int k, int V, const int32_t* __restrict__ draft_tokens,
    int32_t* __restrict__ accepted_len, int32_t* __restrict__ out_tokens) {
  __shared__ int amax[kWaveSize];
  const int n_pos = k + 1;
  const int b = static_cast<int>(blockIdx.x);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int waves = static_cast<int>(blockDim.x >> 6);
  const int my_tok = wave == 0 && lane < k ? draft_tokens[(long)b * k + lane] : -1;
  const long n_groups = V / NE;
  for (int j = wave; j < n_pos; j += waves) {
    const void* rp = reinterpret_cast<const char*>(target) +
                     ((long)b * n_pos + j) * (long)V * Elems<DT>::kBytes;
    float bv = -INFINITY;
    int bi = INT_MAX;
#pragma unroll 4
    for (long g = lane; g < n_groups; g += kWaveSize) {  // ascending per lane
      float x[NE];
      load_group<DT, NE, true>(rp, g * NE, x);
      argmax_update<NE>(bv, bi, x, g);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) am_merge(bv, bi, shfl_xor_f(bv, o), shfl_xor_i(bi, o));
    if (lane == 0) amax[j] = bi == INT_MAX ? 0 : bi;  // all-(-inf) rows resolve to index 0
  }
  __syncthreads();
  if (wave != 0) return;
  const int am = lane < n_pos ? amax[lane] : 0;
  const uint64_t mm = __ballot(lane < k && my_tok != am);
  const int n = mm != 0 ? __builtin_ctzll(mm) : k;
  if (lane < n_pos) out_tokens[(long)b * n_pos + lane] = lane < n ? my_tok : lane == n ? am : -1;
  if (lane == 0) accepted_len[b] = n;
}

template <int DT, int NE, int NMAX>
__global__ __launch_bounds__(kThreads) void k_tree_greedy(
    const void* __restrict__ target, int n_nodes, int V, int C1, TreeArgsN<NMAX> tree, int D,
    const int32_t* __restrict__ node_tokens, int32_t* __restrict__ accepted_len,
    int32_t* __restrict__ out_tokens, int32_t* __restrict__ out_path,
    uint64_t* __restrict__ part, unsigned* __restrict__ counters) {
  int b;
  if (!argmax_chunk<DT, NE>(target, n_nodes, V, C1, part, counters, b)) return;
  __shared__ int amax[NMAX];
  __shared__ int tok[NMAX];
  __shared__ int16_t par[NMAX];
  __shared__ int path[NMAX];
  __shared__ int s_len, s_best;
  for (int j = threadIdx.x; j < n_nodes; j += kThreads) {
    tok[j] = node_tokens[(long)b * n_nodes + j];
    par[j] = tree.parent[j];
  }
  merge_argmax_rows(part, b, n_nodes, C1, amax);  // ends with a barrier
  // Node j is accepted when every node on its path below the root matches
  // its parent's argmax.  Each thread walks up from its own nodes (stopping
  // at the first mismatch), so the whole tree is settled in about its depth
  // of steps; the deepest accepted node wins, the lowest index among equals
  // (key: depth, then -index; the root alone is depth 0).
  int key = 0xFFFF;  // the root: depth 0, index 0
  for (int j = threadIdx.x + 1; j < n_nodes; j += kThreads) {
    int x = j, d = 0;
    bool ok = true;
    while (x != 0 && ok) {
      const int pa = par[x];
      ok = tok[x] == amax[pa];
      x = pa;
      ++d;
    }
    if (ok) key = max(key, d << 16 | (0xFFFF - j));
  }
  key = -block_min_i(-key);  // the largest key, in every thread
  if (threadIdx.x == 0) {
    const int best = 0xFFFF - (key & 0xFFFF);
    const int len = key >> 16;
    int node = best;
    for (int d = len; d >= 0; --d) {
      path[d] = node;
      node = par[node];
    }
    s_best = best;
    s_len = len;
  }
  __syncthreads();
  const int best = s_best;
  const int len = s_len;
  for (int d = threadIdx.x; d <= D; d += kThreads) {
    int t = -1, p = -1;
    if (d < len) t = tok[path[d + 1]];
    else if (d == len) t = amax[best];
    if (d <= len) p = path[d];
    out_tokens[(long)b * (D + 1) + d] = t;
    if (out_path) out_path[(long)b * (D + 1) + d] = p;
  }
  if (threadIdx.x == 0) accepted_len[b] = len;
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------

// Chunks per row: at most as many as keep every (row, chunk) work-group
// within one round of resident work-groups (a second, partial round streams
// at low concurrency while the rest of the chip idles) divided by `share`,
// with chunks of at least 16K elements.  Measured on MI355X at B=64, 9 rows,
// V=128256 (three chunks: 27.0 us, two: 27.6, four: 28.4; share 1) and at
// B=16, 61 tree rows (one chunk: 51.5 us, two: 53.7; share 2).
static int row_chunks(int per_cu, long rows, int V, int share) {
  int dev = 0, cus = 1;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 1;
  const long by_slots = (long)max(per_cu, 1) * cus / max(rows * share, 1L);
  const long by_size = ((long)V + kMinChunkElems - 1) / kMinChunkElems;
  return (int)max(1L, min(by_slots, by_size));
}

// Resident work-groups per compute unit of a kernel (queried once).
template <typename K>
static int groups_per_cu(K kernel) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(kernel),
                                                   kThreads, 0) != hipSuccess || n <= 0)
    n = 1;
  return n;
}

// 16-byte loads need every row to start on a 16-byte boundary; the buffer
// loads of the sweep address rows below 2 GiB.
static bool rows_aligned(const void* p, int V, int dtype) {
  const long eb = dtype == 1 ? 2 : 4;
  return (reinterpret_cast<uintptr_t>(p) % 16 == 0) && (((long)V * eb) % 16 == 0) &&
         (long)V * eb < (1L << 31);
}

// Kernel instantiation for the logit type and row alignment.
template <template <int, int> class Pick>
static auto pick_kernel(int dtype, bool vec) {
  if (dtype == 1) return vec ? Pick<1, 8>::fn() : Pick<1, 1>::fn();
  return vec ? Pick<0, 4>::fn() : Pick<0, 1>::fn();
}
template <template <int, int> class Pick>
static int pick_per_cu(int dtype, bool vec) {
  if (dtype == 1) return vec ? Pick<1, 8>::per_cu() : Pick<1, 1>::per_cu();
  return vec ? Pick<0, 4>::per_cu() : Pick<0, 1>::per_cu();
}

template <int DT, int NE>
struct ChainKernel {
  static auto fn() { return &k_greedy_chain<DT, NE>; }
  static int per_cu() {
    static const int n = groups_per_cu(fn());
    return n;
  }
};
template <int DT, int NE>
struct SmallChainKernel {
  static auto fn() { return &k_greedy_chain_small<DT, NE>; }
  static int per_cu() { return 1; }
};
template <int DT, int NE>
struct SmallTreeKernel {
  static auto fn() { return &k_tree_greedy<DT, NE, kSmallTree>; }
  static int per_cu() {
    static const int n = groups_per_cu(fn());
    return n;
  }
};
template <int DT, int NE>
struct TreeKernel {
  static auto fn() { return &k_tree_greedy<DT, NE, kMaxNodes>; }
  static int per_cu() {
    static const int n = groups_per_cu(fn());
    return n;
  }
};

hipError_t launch_greedy_chain(const void* target, int dtype, int B, int k, int V,
                               const int32_t* draft_tokens, int32_t* accepted_len,
                               int32_t* out_tokens, void* ws, const WsLayout& L,
                               hipStream_t s) {
  const bool vec = rows_aligned(target, V, dtype);
  if (k + 1 <= kWaveSize && (long)V * (k + 1) <= kSmallChainElems)
    return launch_timed(kProfRowPass, pick_kernel<SmallChainKernel>(dtype, vec), dim3(B),
                        dim3(kWaveSize * std::min(k + 1, kSmallChainWaves)), 0, s, target, k, V,
                        draft_tokens, accepted_len, out_tokens);
  const auto kern = pick_kernel<ChainKernel>(dtype, vec);
  const int C1 = row_chunks(pick_per_cu<ChainKernel>(dtype, vec), (long)B * (k + 1), V, 1);
  char* w = static_cast<char*>(ws);
  auto* part = reinterpret_cast<uint64_t*>(w + L.part1);
  auto* cnt = reinterpret_cast<unsigned*>(w + L.count);
  const dim3 grid((unsigned)((long)B * (k + 1) * C1)), block(kThreads);
  return launch_timed(kProfRowPass, kern, grid, block, 0, s, target, k, V, C1, draft_tokens,
                      accepted_len, out_tokens, part, cnt);
}

hipError_t launch_tree_greedy(const void* target, int dtype, int B, int n_nodes, int V,
                              const TreeArgs& tree, int depth, const int32_t* node_tokens,
                              int32_t* accepted_len, int32_t* out_tokens, int32_t* out_path,
                              void* ws, const WsLayout& L, hipStream_t s) {
  const bool vec = rows_aligned(target, V, dtype);
  char* w = static_cast<char*>(ws);
  auto* part = reinterpret_cast<uint64_t*>(w + L.part1);
  auto* cnt = reinterpret_cast<unsigned*>(w + L.count);
  if (n_nodes <= kSmallTree) {
    // A 2 KiB argument block made each launch ~20 us slower on the device
    // at 61 nodes than this 256-byte one.
    TreeArgsN<kSmallTree> small;
    for (int j = 0; j < kSmallTree; ++j) small.parent[j] = j < n_nodes ? tree.parent[j] : 0;
    const auto kern = pick_kernel<SmallTreeKernel>(dtype, vec);
    const int C1 =
        row_chunks(pick_per_cu<SmallTreeKernel>(dtype, vec), (long)B * n_nodes, V, 2);
    const dim3 grid((unsigned)((long)B * n_nodes * C1)), block(kThreads);
    return launch_timed(kProfRowPass, kern, grid, block, 0, s, target, n_nodes, V, C1, small,
                        depth, node_tokens, accepted_len, out_tokens, out_path, part, cnt);
  }
  const auto kern = pick_kernel<TreeKernel>(dtype, vec);
  const int C1 = row_chunks(pick_per_cu<TreeKernel>(dtype, vec), (long)B * n_nodes, V, 2);
  const dim3 grid((unsigned)((long)B * n_nodes * C1)), block(kThreads);
  return launch_timed(kProfRowPass, kern, grid, block, 0, s, target, n_nodes, V, C1, tree, depth,
                      node_tokens, accepted_len, out_tokens, out_path, part, cnt);
}

}  // namespace specv
