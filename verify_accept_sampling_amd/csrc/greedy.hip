// Greedy chain and greedy tree verification for gfx950.
//
// One launch per call.  Work-group (chunk, row) streams one chunk of one
// logit row with 16-byte loads and reduces it to (max value, lowest index).
// The last work-group to finish a request (ticket counter) merges the chunk
// partials of that request's rows and applies the greedy rule:
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

struct ArgmaxPart {
  float v;
  int i;
};

// Unroll depth of the streaming loops: groups in flight per thread.
constexpr int kUnrollArgmax = 4;

// Argmax of row elements [chunk range) for this thread (ascending order, so
// a strict '>' keeps the lowest index).  NE = elements per load.
template <int DT, int NE>
__device__ __forceinline__ void argmax_sweep(const void* row, long n_groups, long g0, long g1,
                                             float& bv, int& bi) {
  bv = -INFINITY;
  bi = INT_MAX;
  for (long g = g0 + threadIdx.x; g < g1; g += (long)kThreads * kUnrollArgmax) {
    float x[kUnrollArgmax][NE];
#pragma unroll
    for (int u = 0; u < kUnrollArgmax; ++u) {
      const long gg = g + (long)u * kThreads;
      if (gg < g1) {
        load_group<DT, NE>(row, gg * NE, x[u]);
      } else {
#pragma unroll
        for (int e = 0; e < NE; ++e) x[u][e] = -INFINITY;
      }
    }
#pragma unroll
    for (int u = 0; u < kUnrollArgmax; ++u) {
      float lm = x[u][0];
#pragma unroll
      for (int e = 1; e < NE; ++e) lm = fmaxf(lm, x[u][e]);
      if (lm > bv) {
        int first = NE - 1;
#pragma unroll
        for (int e = NE - 1; e >= 0; --e)
          if (x[u][e] == lm) first = e;
        bv = lm;
        bi = static_cast<int>((g + (long)u * kThreads) * NE + first);
      }
    }
  }
  (void)n_groups;
}

// Stream the (chunk, row) of this work-group and publish its partial.
// Returns the request index of the row.
template <int DT, int NE>
__device__ __forceinline__ int argmax_chunk(const void* target, int n_pos, int V, int C1,
                                            ArgmaxPart* part) {
  const int blk = blockIdx.x;
  const int chunk = blk % C1;
  const long row = blk / C1;
  const long n_groups = V / NE;
  const long gpc = (n_groups + C1 - 1) / C1;
  const long g0 = (long)chunk * gpc;
  const long g1 = min(g0 + gpc, n_groups);
  const void* rp = reinterpret_cast<const char*>(target) + row * (long)V * Elems<DT>::kBytes;
  float bv;
  int bi;
  argmax_sweep<DT, NE>(rp, n_groups, g0, g1, bv, bi);
  block_reduce_am(bv, bi);
  if (threadIdx.x == 0) part[row * C1 + chunk] = ArgmaxPart{bv, bi};
  return static_cast<int>(row / n_pos);
}

// In the last work-group of request b: merge every row's chunk partials into
// amax[0..n_pos-1] (shared memory).  All-(-inf) rows resolve to index 0.
__device__ __forceinline__ void merge_argmax_rows(const ArgmaxPart* part, int b, int n_pos,
                                                  int C1, int* amax) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int j = wave; j < n_pos; j += kWaves) {
    const long row = (long)b * n_pos + j;
    float v = -INFINITY;
    int i = INT_MAX;
    for (int c = lane; c < C1; c += 64) {
      const ArgmaxPart p = part[row * C1 + c];
      am_merge(v, i, p.v, p.i);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float v2 = shfl_xor_f(v, o);
      const int i2 = shfl_xor_i(i, o);
      am_merge(v, i, v2, i2);
    }
    if (lane == 0) amax[j] = (i == INT_MAX) ? 0 : i;
  }
  __syncthreads();
}

template <int DT, int NE>
__global__ __launch_bounds__(kThreads) void k_greedy_chain(
    const void* __restrict__ target, int k, int V, int C1,
    const int32_t* __restrict__ draft_tokens, int32_t* __restrict__ accepted_len,
    int32_t* __restrict__ out_tokens, ArgmaxPart* __restrict__ part,
    unsigned* __restrict__ counters) {
  const int n_pos = k + 1;
  const int b = argmax_chunk<DT, NE>(target, n_pos, V, C1, part);
  if (!last_block_ticket(&counters[(long)b * kCountersPerReq + 0], (unsigned)(n_pos * C1)))
    return;
  __shared__ int amax[kMaxK + 1];
  merge_argmax_rows(part, b, n_pos, C1, amax);
  // first mismatch: minimum over positions that differ
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
    ArgmaxPart* __restrict__ part, unsigned* __restrict__ counters) {
  const int b = argmax_chunk<DT, NE>(target, n_nodes, V, C1, part);
  if (!last_block_ticket(&counters[(long)b * kCountersPerReq + 0], (unsigned)(n_nodes * C1)))
    return;
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

hipError_t launch_greedy_chain(const void* target, int dtype, int B, int k, int V,
                               const int32_t* draft_tokens, int32_t* accepted_len,
                               int32_t* out_tokens, void* ws, const WsLayout& L,
                               hipStream_t s) {
  const int C1 = row_chunks(V);
  char* w = static_cast<char*>(ws);
  auto* part = reinterpret_cast<ArgmaxPart*>(w + L.part1);
  auto* cnt = reinterpret_cast<unsigned*>(w + L.count);
  const dim3 grid((unsigned)((long)B * (k + 1) * C1)), block(kThreads);
  const bool vec = rows_aligned(target, V, dtype);
  if (dtype == 1) {
    if (vec)
      hipLaunchKernelGGL((k_greedy_chain<1, 8>), grid, block, 0, s, target, k, V, C1,
                         draft_tokens, accepted_len, out_tokens, part, cnt);
    else
      hipLaunchKernelGGL((k_greedy_chain<1, 1>), grid, block, 0, s, target, k, V, C1,
                         draft_tokens, accepted_len, out_tokens, part, cnt);
  } else {
    if (vec)
      hipLaunchKernelGGL((k_greedy_chain<0, 4>), grid, block, 0, s, target, k, V, C1,
                         draft_tokens, accepted_len, out_tokens, part, cnt);
    else
      hipLaunchKernelGGL((k_greedy_chain<0, 1>), grid, block, 0, s, target, k, V, C1,
                         draft_tokens, accepted_len, out_tokens, part, cnt);
  }
  return hipGetLastError();
}

hipError_t launch_tree_greedy(const void* target, int dtype, int B, int n_nodes, int V,
                              const TreeArgs& tree, int depth, const int32_t* node_tokens,
                              int32_t* accepted_len, int32_t* out_tokens, int32_t* out_path,
                              void* ws, const WsLayout& L, hipStream_t s) {
  const int C1 = row_chunks(V);
  char* w = static_cast<char*>(ws);
  auto* part = reinterpret_cast<ArgmaxPart*>(w + L.part1);
  auto* cnt = reinterpret_cast<unsigned*>(w + L.count);
  const dim3 grid((unsigned)((long)B * n_nodes * C1)), block(kThreads);
  const bool vec = rows_aligned(target, V, dtype);
  if (dtype == 1) {
    if (vec)
      hipLaunchKernelGGL((k_tree_greedy<1, 8>), grid, block, 0, s, target, n_nodes, V, C1,
                         tree, depth, node_tokens, accepted_len, out_tokens, out_path, part,
                         cnt);
    else
      hipLaunchKernelGGL((k_tree_greedy<1, 1>), grid, block, 0, s, target, n_nodes, V, C1,
                         tree, depth, node_tokens, accepted_len, out_tokens, out_path, part,
                         cnt);
  } else {
    if (vec)
      hipLaunchKernelGGL((k_tree_greedy<0, 4>), grid, block, 0, s, target, n_nodes, V, C1,
                         tree, depth, node_tokens, accepted_len, out_tokens, out_path, part,
                         cnt);
    else
      hipLaunchKernelGGL((k_tree_greedy<0, 1>), grid, block, 0, s, target, n_nodes, V, C1,
                         tree, depth, node_tokens, accepted_len, out_tokens, out_path, part,
                         cnt);
  }
  return hipGetLastError();
}

}  // namespace specv
