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
#include <climits>

#include "device_common.h"

namespace specv {

// Groups in flight per thread in the streaming loop.
constexpr int kUnrollArgmax = kRowUnroll;

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
// keeps the lowest index).  NE = elements per load.
template <int DT, int NE>
__device__ __forceinline__ void argmax_sweep(const void* row, long g0, long g1, float& bv,
                                             int& bi) {
  bv = -INFINITY;
  bi = INT_MAX;
  long g = g0 + threadIdx.x;
  // Main loop: kUnrollArgmax loads issued back to back, no bounds branch.
  for (; g + (long)(kUnrollArgmax - 1) * kThreads < g1; g += (long)kThreads * kUnrollArgmax) {
    float x[kUnrollArgmax][NE];
#pragma unroll
    for (int u = 0; u < kUnrollArgmax; ++u)
      load_group<DT, NE, true>(row, (g + (long)u * kThreads) * NE, x[u]);
#pragma unroll
    for (int u = 0; u < kUnrollArgmax; ++u) argmax_update<NE>(bv, bi, x[u], g + (long)u * kThreads);
  }
  for (; g < g1; g += kThreads) {
    float x[NE];
    load_group<DT, NE, true>(row, g * NE, x);
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
  argmax_sweep<DT, NE>(rp, g0, g1, bv, bi);
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
  int b;
  if (!argmax_chunk<DT, NE>(target, n_pos, V, C1, part, counters, b)) return;
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

template <int DT, int NE>
__global__ __launch_bounds__(kThreads) void k_tree_greedy(
    const void* __restrict__ target, int n_nodes, int V, int C1, TreeArgs tree, int D,
    const int32_t* __restrict__ node_tokens, int32_t* __restrict__ accepted_len,
    int32_t* __restrict__ out_tokens, int32_t* __restrict__ out_path,
    uint64_t* __restrict__ part, unsigned* __restrict__ counters) {
  int b;
  if (!argmax_chunk<DT, NE>(target, n_nodes, V, C1, part, counters, b)) return;
  __shared__ int amax[kMaxNodes];
  __shared__ int tok[kMaxNodes];
  __shared__ int path[kMaxNodes];
  __shared__ int16_t dep[kMaxNodes];
  __shared__ int s_best;
  for (int j = threadIdx.x; j < n_nodes; j += kThreads) tok[j] = node_tokens[(long)b * n_nodes + j];
  merge_argmax_rows(part, b, n_nodes, C1, amax);
  if (threadIdx.x == 0) {
    // parent[j] < j, so one ascending pass settles every node's depth and
    // acceptance.  The accepted flags use path[] as scratch before the path
    // is written.
    path[0] = 1;
    dep[0] = 0;
    int best = 0;
    for (int j = 1; j < n_nodes; ++j) {
      const int pa = tree.parent[j];
      dep[j] = static_cast<int16_t>(dep[pa] + 1);
      const int ok = path[pa] && (tok[j] == amax[pa]);
      path[j] = ok;
      if (ok && dep[j] > dep[best]) best = j;
    }
    s_best = best;
  }
  __syncthreads();
  const int best = s_best;
  const int len = dep[best];
  __syncthreads();
  if (threadIdx.x == 0) {
    int node = best;
    for (int d = len; d >= 0; --d) {
      path[d] = node;
      node = tree.parent[node];
    }
  }
  __syncthreads();
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

static int row_chunks(int V) { return (V + kRowChunkElems - 1) / kRowChunkElems; }

// 16-byte loads need every row to start on a 16-byte boundary.
static bool rows_aligned(const void* p, int V, int dtype) {
  const int eb = dtype == 1 ? 2 : 4;
  return (reinterpret_cast<uintptr_t>(p) % 16 == 0) && (((long)V * eb) % 16 == 0);
}

// Kernel instantiation for the logit type and row alignment.
template <template <int, int> class Pick>
static auto pick_kernel(int dtype, bool vec) {
  if (dtype == 1) return vec ? Pick<1, 8>::fn() : Pick<1, 1>::fn();
  return vec ? Pick<0, 4>::fn() : Pick<0, 1>::fn();
}

template <int DT, int NE>
struct ChainKernel {
  static auto fn() { return &k_greedy_chain<DT, NE>; }
};
template <int DT, int NE>
struct TreeKernel {
  static auto fn() { return &k_tree_greedy<DT, NE>; }
};

hipError_t launch_greedy_chain(const void* target, int dtype, int B, int k, int V,
                               const int32_t* draft_tokens, int32_t* accepted_len,
                               int32_t* out_tokens, void* ws, const WsLayout& L,
                               hipStream_t s) {
  const int C1 = row_chunks(V);
  char* w = static_cast<char*>(ws);
  auto* part = reinterpret_cast<uint64_t*>(w + L.part1);
  auto* cnt = reinterpret_cast<unsigned*>(w + L.count);
  const dim3 grid((unsigned)((long)B * (k + 1) * C1)), block(kThreads);
  const auto kern = pick_kernel<ChainKernel>(dtype, rows_aligned(target, V, dtype));
  return launch_timed(kProfRowPass, kern, grid, block, 0, s, target, k, V, C1, draft_tokens,
                      accepted_len, out_tokens, part, cnt);
}

hipError_t launch_tree_greedy(const void* target, int dtype, int B, int n_nodes, int V,
                              const TreeArgs& tree, int depth, const int32_t* node_tokens,
                              int32_t* accepted_len, int32_t* out_tokens, int32_t* out_path,
                              void* ws, const WsLayout& L, hipStream_t s) {
  const int C1 = row_chunks(V);
  char* w = static_cast<char*>(ws);
  auto* part = reinterpret_cast<uint64_t*>(w + L.part1);
  auto* cnt = reinterpret_cast<unsigned*>(w + L.count);
  const dim3 grid((unsigned)((long)B * n_nodes * C1)), block(kThreads);
  const auto kern = pick_kernel<TreeKernel>(dtype, rows_aligned(target, V, dtype));
  return launch_timed(kProfRowPass, kern, grid, block, 0, s, target, n_nodes, V, C1, tree, depth,
                      node_tokens, accepted_len, out_tokens, out_path, part, cnt);
}

}  // namespace specv
