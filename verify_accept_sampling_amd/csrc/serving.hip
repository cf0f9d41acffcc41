// Rejected-draft masks for KV-cache trimming after a verification step.
// The target's forward pass wrote a KV entry for every drafted token; only
// the entries on the accepted prefix (chain) or the accepted root-to-node
// path (tree) stay, and the rest are dropped before drafting resumes from
// the confirmed prefix (EAGLE-3 review, section on the full inference loop,
// step 5 "KV cache update").  A serving engine marks those tokens with a
// rejected-token mask and points their slot-mapping entries at a padding
// slot so that their KV never lands in the cache ("[vLLM] EAGLE" code walk,
// sections on rejected-token handling and on slot mapping / KV-cache
// management).
#include "device_common.h"

namespace specv {

// One work-group per request b, n_ent entries per request.
//   path == nullptr (chain): entry i is rejected iff i >= accepted_len[b].
//   path != nullptr (tree):  entry j (node j) is rejected iff j > 0 and j is
//     not among path[b, 0 .. path_len-1]; entries outside [0, n_ent) (the
//     -1 padding after the path's end) mark nothing.
// rejected[b, j] = 0 or 1; where slots is given, slots[b, j] = pad_slot for
// every rejected entry and is left as it is elsewhere.
__global__ __launch_bounds__(kThreads) void k_rejected_mask(
    const int32_t* __restrict__ accepted_len, const int32_t* __restrict__ path, int path_len,
    int n_ent, uint8_t* __restrict__ rejected, int64_t* __restrict__ slots, int64_t pad_slot) {
  const long b = blockIdx.x;
  __shared__ uint8_t on_path[kMaxNodes];
  int n = 0;
  if (path != nullptr) {  // grid-uniform
    for (int j = threadIdx.x; j < n_ent; j += kThreads) on_path[j] = 0;
    __syncthreads();
    for (int d = threadIdx.x; d < path_len; d += kThreads) {
      const int v = path[b * path_len + d];
      if (v >= 0 && v < n_ent) on_path[v] = 1;
    }
    __syncthreads();
  } else {
    n = accepted_len[b];
  }
  for (int j = threadIdx.x; j < n_ent; j += kThreads) {
    const bool r = path != nullptr ? (j > 0 && on_path[j] == 0) : j >= n;
    rejected[b * n_ent + j] = r ? 1 : 0;
    if (slots != nullptr && r) slots[b * n_ent + j] = pad_slot;
  }
}

hipError_t launch_rejected_mask(const int32_t* accepted_len, const int32_t* path, int path_len,
                                int B, int n_ent, uint8_t* rejected, int64_t* slots,
                                int64_t pad_slot, hipStream_t s) {
  return launch_timed(kProfServing, &k_rejected_mask, dim3((unsigned)B), dim3(kThreads), 0, s,
                      accepted_len, path, path_len, n_ent, rejected, slots, pad_slot);
}

}  // namespace specv
