// C ABI of the verifier: argument validation, workspace layout and dispatch
// to the gfx950 kernels.  Nothing is enqueued unless every check passes.
#include <cmath>
#include <cstring>

#include <atomic>
#include <map>
#include <random>
#include <vector>

#include "../../include/spec_verify.h"
#include "internal.h"

using namespace specv;

namespace {

bool valid_dtype(int dt) { return dt == SPEC_F32 || dt == SPEC_BF16; }

// Largest number of threads a one-dimensional grid may hold.
constexpr long kMaxGridThreads = 0xFFFFFFFFL;

int check_workspace(void* ws, size_t ws_bytes, int B, int n_pos, int V, WsLayout* L) {
  *L = ws_layout(B, n_pos, V);
  if (ws == nullptr || ws_bytes < L->total) return SPEC_EWORKSPACE;
  return SPEC_OK;
}

int check_grid(long blocks) {
  return (blocks * kThreads <= kMaxGridThreads) ? SPEC_OK : SPEC_EINVAL;
}

long row_chunks_for(int V) { return (V + kRowChunkElems - 1) / kRowChunkElems; }

// Most chunks per row the greedy kernels use.
long greedy_chunks_max(int V) { return (V + kMinChunkElems - 1) / kMinChunkElems; }

int tree_depth_checked(const int32_t* parent, int n_nodes) {
  if (parent == nullptr || n_nodes < 1 || n_nodes > kMaxNodes) return SPEC_EINVAL;
  if (parent[0] != -1) return SPEC_ETREE;
  int depth[kMaxNodes];
  depth[0] = 0;
  int D = 0;
  for (int j = 1; j < n_nodes; ++j) {
    const int p = parent[j];
    if (p < 0 || p >= j) return SPEC_ETREE;
    depth[j] = depth[p] + 1;
    if (depth[j] > D) D = depth[j];
  }
  return D;
}

}  // namespace

namespace specv {
uint64_t next_call_tag() {
  static const uint64_t process_bits = [] {
    std::random_device rd;
    return (uint64_t)(rd() & 0xffffu);
  }();
  static std::atomic<uint64_t> calls{0};
  const uint64_t n = calls.fetch_add(1, std::memory_order_relaxed) + 1;
  return (0xC3ull << 56) | (process_bits << 40) | (n & ((1ull << 40) - 1));
}
}  // namespace specv

extern "C" {

const char* spec_strerror(int code) {
  switch (code) {
    case SPEC_OK: return "ok";
    case SPEC_EINVAL: return "invalid argument (null pointer, size or scalar out of range)";
    case SPEC_EDTYPE: return "unsupported dtype / kind combination";
    case SPEC_EWORKSPACE: return "workspace missing or smaller than spec_workspace_bytes()";
    case SPEC_EHIP: return "HIP launch failed";
    case SPEC_ETREE: return "parent array is not a tree with parent[0] = -1 and parent[j] < j";
    case SPEC_ESCRATCH:
      return "shape needs more scratch than the no-alloc entry point's static array "
             "(SPEC_NOALLOC_SCRATCH_BYTES); use spec_verify_sample with a workspace";
    default: return "unknown error code";
  }
}

size_t spec_workspace_bytes(int B, int n_pos, int V) {
  if (B < 0 || B > kMaxB || n_pos < 1 || n_pos > kMaxNodes || V < 1 || V > kMaxV) return 0;
  return ws_layout(B, n_pos, V).total;
}

int spec_fill_uniforms(uint64_t seed, uint64_t counter0, int64_t n, float* out, void* stream) {
  if (n < 0) return SPEC_EINVAL;
  if (n == 0) return SPEC_OK;
  if (out == nullptr) return SPEC_EINVAL;
  if (launch_fill_uniforms(seed, counter0, n, out, static_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return SPEC_EHIP;
  return SPEC_OK;
}

int spec_tree_depth(const int32_t* parent_host, int n_nodes) {
  return tree_depth_checked(parent_host, n_nodes);
}

int spec_verify_greedy(const void* target, int dtype, int B, int k, int V,
                       const int32_t* draft_tokens, int32_t* accepted_len, int32_t* out_tokens,
                       void* ws, size_t ws_bytes, void* stream) {
  if (!valid_dtype(dtype)) return SPEC_EDTYPE;
  if (B < 0 || B > kMaxB || k < 0 || k > kMaxK || V < 1 || V > kMaxV) return SPEC_EINVAL;
  if (B == 0) return SPEC_OK;
  if (target == nullptr || accepted_len == nullptr || out_tokens == nullptr) return SPEC_EINVAL;
  if (k > 0 && draft_tokens == nullptr) return SPEC_EINVAL;
  if (check_grid((long)B * (k + 1) * greedy_chunks_max(V)) != SPEC_OK) return SPEC_EINVAL;
  WsLayout L;
  if (int rc = check_workspace(ws, ws_bytes, B, k + 1, V, &L)) return rc;
  if (launch_greedy_chain(target, dtype, B, k, V, draft_tokens, accepted_len, out_tokens, ws, L,
                          static_cast<hipStream_t>(stream)) != hipSuccess)
    return SPEC_EHIP;
  return SPEC_OK;
}

}  // extern "C"

namespace {

// Checks shared by both sampling entry points; on success *mode and *L are
// filled in for the launch.
int check_sample(const void* target, const void* draft, int dtype, int kind, int B, int k,
                 int V, const int32_t* draft_tokens, float temperature, int flags,
                 int32_t* accepted_len, int32_t* out_tokens, void* stream, SampleMode* mode,
                 WsLayout* L) {
  if (!valid_dtype(dtype) || (kind != SPEC_LOGITS && kind != SPEC_PROBS)) return SPEC_EDTYPE;
  if ((flags & ~(0xF | SPEC_FLAG_TEST_GIVE_UP)) != 0 || (flags & 0xF) > SPEC_SCHED_EARLY_EXIT)
    return SPEC_EINVAL;
  if (kind == SPEC_PROBS && dtype != SPEC_F32) return SPEC_EDTYPE;
  if (B < 0 || B > kMaxB || k < 0 || k > kMaxK || V < 1 || V > kMaxV) return SPEC_EINVAL;
  if (kind == SPEC_LOGITS) {
    if (!(temperature > 0.f) || !std::isfinite(temperature)) return SPEC_EINVAL;
    const float c = 1.4426950408889634f / temperature;
    if (!std::isfinite(c) || !std::isfinite(1.0 / (double)temperature)) return SPEC_EINVAL;
  } else if (temperature != 1.f) {
    return SPEC_EINVAL;
  }
  if (B == 0) return SPEC_OK;
  if (target == nullptr || accepted_len == nullptr || out_tokens == nullptr) return SPEC_EINVAL;
  if (k > 0 && (draft == nullptr || draft_tokens == nullptr)) return SPEC_EINVAL;
  const long C2 = (V + kDrawChunk - 1) / kDrawChunk;
  const long draws = (long)B * specv::draw_groups(res_chunks(V), 1);
  const long finalizers = ((long)B + kWaves - 1) / kWaves;
  if (check_grid((long)B * (2L * k + 1) * row_chunks_for(V) + finalizers + draws) != SPEC_OK)
    return SPEC_EINVAL;
  if (check_grid((long)B * C2) != SPEC_OK) return SPEC_EINVAL;
  *L = ws_layout(B, k + 1, V);
  mode->sched = flags & 0xF;
  mode->test_give_up = (flags & SPEC_FLAG_TEST_GIVE_UP) != 0;
  mode->capturing = false;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(static_cast<hipStream_t>(stream), &cs) == hipSuccess)
    mode->capturing = cs == hipStreamCaptureStatusActive;
  else
    (void)hipGetLastError();  // not capturing; leave no error for the launch check
  return SPEC_OK;
}

}  // namespace

extern "C" {

int spec_verify_sample(const void* target, const void* draft, int dtype, int kind, int B, int k,
                       int V, const int32_t* draft_tokens, const float* uniforms, uint64_t seed,
                       uint64_t counter0, float temperature, int flags, int32_t* accepted_len,
                       int32_t* out_tokens, float* probe, void* ws, size_t ws_bytes,
                       void* stream) {
  SampleMode mode;
  WsLayout L;
  if (int rc = check_sample(target, draft, dtype, kind, B, k, V, draft_tokens, temperature,
                            flags, accepted_len, out_tokens, stream, &mode, &L))
    return rc;
  if (B == 0) return SPEC_OK;
  if (ws == nullptr || ws_bytes < L.total) return SPEC_EWORKSPACE;
  if (launch_sample(target, draft, dtype, kind, B, k, V, draft_tokens, uniforms, seed, counter0,
                    temperature, mode, accepted_len, out_tokens, probe, ws, L,
                    static_cast<hipStream_t>(stream)) != hipSuccess)
    return SPEC_EHIP;
  return SPEC_OK;
}

int spec_verify_sample_noalloc(const void* target, const void* draft, int dtype, int kind,
                               int B, int k, int V, const int32_t* draft_tokens,
                               const float* uniforms, uint64_t seed, uint64_t counter0,
                               float temperature, int flags, int32_t* accepted_len,
                               int32_t* out_tokens, float* probe, void* stream) {
  SampleMode mode;
  WsLayout L;
  if (int rc = check_sample(target, draft, dtype, kind, B, k, V, draft_tokens, temperature,
                            flags, accepted_len, out_tokens, stream, &mode, &L))
    return rc;
  if (B == 0) return SPEC_OK;
  if (L.total > kNoAllocScratchBytes) return SPEC_ESCRATCH;
  const auto s = static_cast<hipStream_t>(stream);
  int dev = -1, sdev = -1;
  if (hipGetDevice(&dev) != hipSuccess || hipStreamGetDevice(s, &sdev) != hipSuccess)
    return SPEC_EHIP;
  if (sdev != dev) return SPEC_EINVAL;
  void* scratch_ptr = nullptr;
  if (noalloc_scratch(dev, &scratch_ptr) != hipSuccess) return SPEC_EHIP;
  if (launch_clear_requests(scratch_ptr, B, s) != hipSuccess) return SPEC_EHIP;
  if (launch_sample(target, draft, dtype, kind, B, k, V, draft_tokens, uniforms, seed, counter0,
                    temperature, mode, accepted_len, out_tokens, probe, scratch_ptr, L, s) !=
      hipSuccess)
    return SPEC_EHIP;
  return SPEC_OK;
}

int spec_workspace_status(const void* ws, size_t ws_bytes, uint32_t* status_host, void* stream) {
  if (ws == nullptr || status_host == nullptr) return SPEC_EINVAL;
  if (ws_bytes < kCounterRegionBytes) return SPEC_EWORKSPACE;
  const auto s = static_cast<hipStream_t>(stream);
  uint32_t v = 0;
  if (hipMemcpyAsync(&v, static_cast<const char*>(ws) + SPEC_WORKSPACE_STATUS_OFFSET,
                     sizeof(v), hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return SPEC_EHIP;
  *status_host = v;
  return SPEC_OK;
}

int spec_workspace_reset(void* ws, size_t ws_bytes, void* stream) {
  if (ws == nullptr) return SPEC_EINVAL;
  if (ws_bytes < kCounterRegionBytes) return SPEC_EWORKSPACE;
  if (launch_reset_counters(ws, static_cast<hipStream_t>(stream)) != hipSuccess) return SPEC_EHIP;
  return SPEC_OK;
}

int spec_verify_tree_greedy(const void* target, int dtype, int B, int n_nodes, int V,
                            const int32_t* parent_host, const int32_t* node_tokens,
                            int32_t* accepted_len, int32_t* out_tokens, int32_t* out_path,
                            void* ws, size_t ws_bytes, void* stream) {
  if (!valid_dtype(dtype)) return SPEC_EDTYPE;
  if (B < 0 || B > kMaxB || n_nodes < 1 || n_nodes > kMaxNodes || V < 1 || V > kMaxV)
    return SPEC_EINVAL;
  const int D = tree_depth_checked(parent_host, n_nodes);
  if (D < 0) return D;
  if (B == 0) return SPEC_OK;
  if (target == nullptr || node_tokens == nullptr || accepted_len == nullptr ||
      out_tokens == nullptr)
    return SPEC_EINVAL;
  if (check_grid((long)B * n_nodes * greedy_chunks_max(V)) != SPEC_OK) return SPEC_EINVAL;
  WsLayout L;
  if (int rc = check_workspace(ws, ws_bytes, B, n_nodes, V, &L)) return rc;
  TreeArgs tree;
  std::memset(&tree, 0, sizeof(tree));
  for (int j = 0; j < n_nodes; ++j) tree.parent[j] = static_cast<int16_t>(parent_host[j]);
  if (launch_tree_greedy(target, dtype, B, n_nodes, V, tree, D, node_tokens, accepted_len,
                         out_tokens, out_path, ws, L, static_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return SPEC_EHIP;
  return SPEC_OK;
}

int spec_verify_tree_sample(const void* target, const void* draft, int dtype, int kind, int B,
                            int n_nodes, int V, const int32_t* parent_host,
                            const int32_t* node_tokens, const float* uniforms, uint64_t seed,
                            uint64_t counter0, float temperature, int32_t* accepted_len,
                            int32_t* out_tokens, int32_t* out_path, void* ws, size_t ws_bytes,
                            void* stream) {
  if (!valid_dtype(dtype) || (kind != SPEC_LOGITS && kind != SPEC_PROBS)) return SPEC_EDTYPE;
  if (kind == SPEC_PROBS && dtype != SPEC_F32) return SPEC_EDTYPE;
  if (B < 0 || B > kMaxB || n_nodes < 1 || n_nodes > kMaxNodes || V < 1 || V > kMaxV)
    return SPEC_EINVAL;
  if (kind == SPEC_LOGITS) {
    if (!(temperature > 0.f) || !std::isfinite(temperature)) return SPEC_EINVAL;
    const float c = 1.4426950408889634f / temperature;
    if (!std::isfinite(c)) return SPEC_EINVAL;
  } else if (temperature != 1.f) {
    return SPEC_EINVAL;
  }
  const int D = tree_depth_checked(parent_host, n_nodes);
  if (D < 0) return D;
  if (B == 0) return SPEC_OK;
  if (target == nullptr || accepted_len == nullptr || out_tokens == nullptr) return SPEC_EINVAL;
  if (n_nodes > 1 && (draft == nullptr || node_tokens == nullptr)) return SPEC_EINVAL;
  // The same shape k_tree_setup derives on the device.
  static thread_local TreeShape shape;
  shape = TreeShape();
  shape.depth = D;
  {
    std::vector<int> nchild(n_nodes, 0);
    for (int j = 1; j < n_nodes; ++j) {
      const int r = nchild[parent_host[j]]++;
      if (r >= 1) ++shape.rank_count[r];
      if (r > shape.max_rank) shape.max_rank = r;
    }
    for (int u = 0; u < n_nodes; ++u) {
      shape.has_child[u] = nchild[u] > 0;
      shape.n_internal += nchild[u] > 0;
    }
  }
  const long C2 = (V + kDrawChunk - 1) / kDrawChunk;
  if (check_grid((long)B * (2L * shape.n_internal * tree_xchunks(V) +
                            (long)n_nodes * row_chunks_for(V))) != SPEC_OK ||
      check_grid((long)B * n_nodes * C2) != SPEC_OK)
    return SPEC_EINVAL;
  WsLayout L;
  if (int rc = check_workspace(ws, ws_bytes, B, n_nodes, V, &L)) return rc;
  TreeArgs tree;
  std::memset(&tree, 0, sizeof(tree));
  for (int j = 0; j < n_nodes; ++j) tree.parent[j] = static_cast<int16_t>(parent_host[j]);
  if (launch_tree_sample(target, draft, dtype, kind, B, n_nodes, V, tree, shape, node_tokens,
                         uniforms, seed, counter0, temperature, accepted_len, out_tokens,
                         out_path, ws, L, static_cast<hipStream_t>(stream)) != hipSuccess)
    return SPEC_EHIP;
  return SPEC_OK;
}

int spec_rejected_mask(const int32_t* accepted_len, int B, int k, uint8_t* rejected,
                       int64_t* slot_mapping, int64_t pad_slot, void* stream) {
  if (B < 0 || B > kMaxB || k < 0 || k > kMaxK) return SPEC_EINVAL;
  if (B == 0 || k == 0) return SPEC_OK;
  if (accepted_len == nullptr || rejected == nullptr) return SPEC_EINVAL;
  if (launch_rejected_mask(accepted_len, nullptr, 0, B, k, rejected, slot_mapping, pad_slot,
                           static_cast<hipStream_t>(stream)) != hipSuccess)
    return SPEC_EHIP;
  return SPEC_OK;
}

int spec_tree_rejected_mask(const int32_t* out_path, int B, int n_nodes, int depth,
                            uint8_t* rejected, int64_t* slot_mapping, int64_t pad_slot,
                            void* stream) {
  if (B < 0 || B > kMaxB || n_nodes < 1 || n_nodes > kMaxNodes || depth < 0 ||
      depth >= n_nodes)
    return SPEC_EINVAL;
  if (B == 0) return SPEC_OK;
  if (out_path == nullptr || rejected == nullptr) return SPEC_EINVAL;
  if (launch_rejected_mask(nullptr, out_path, depth + 1, B, n_nodes, rejected, slot_mapping,
                           pad_slot, static_cast<hipStream_t>(stream)) != hipSuccess)
    return SPEC_EHIP;
  return SPEC_OK;
}

int spec_tree_from_choices(const int32_t* choices_host, const int32_t* lengths_host,
                           int n_choices, int width, int32_t* parent_host) {
  if (n_choices < 0 || n_choices + 1 > kMaxNodes || width < 1 || parent_host == nullptr)
    return SPEC_EINVAL;
  if (n_choices > 0 && (choices_host == nullptr || lengths_host == nullptr)) return SPEC_EINVAL;
  // Node j + 1 is choice j; a choice's parent is the node whose choice is
  // the same sequence without its last entry (the root for one entry).
  std::map<std::vector<int32_t>, int> node_of;
  node_of[{}] = 0;
  parent_host[0] = -1;
  for (int j = 0; j < n_choices; ++j) {
    const int len = lengths_host[j];
    if (len < 1 || len > width) return SPEC_EINVAL;
    const int32_t* c = choices_host + (long)j * width;
    std::vector<int32_t> seq(c, c + len);
    for (int32_t v : seq)
      if (v < 0) return SPEC_ETREE;
    const auto up = node_of.find(std::vector<int32_t>(seq.begin(), seq.end() - 1));
    if (up == node_of.end()) return SPEC_ETREE;  // parent missing or listed later
    if (!node_of.emplace(std::move(seq), j + 1).second) return SPEC_ETREE;  // listed twice
    parent_host[j + 1] = up->second;
  }
  return n_choices + 1;
}

}  // extern "C"
