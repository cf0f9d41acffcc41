// Internal declarations shared by the host entry points (api.cpp) and the
// kernel translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace specv {

// Block shape of every kernel: 256 threads = 4 waves of 64 lanes.
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

// Elements per work-group chunk of the pass over every row.
constexpr int kRowChunkElems = 16384;
// Smallest chunk the workspace is sized for (leaves room to retune).
constexpr int kRowChunkElemsMin = 2048;
// Elements per work-group chunk of the float64 residual / bonus pass:
// 256 threads x 16 consecutive elements.
constexpr int kSegPerThread = 16;
constexpr int kResChunkElems = kThreads * kSegPerThread;

constexpr int kMaxK = 1023;
constexpr int kMaxNodes = 1024;
constexpr int kMaxV = 1 << 30;

// Per-request state handed from one kernel of a call to the next.
struct ReqState {
  int n;        // accepted length (first rejection or k)
  int mode;     // kModeResidual or kModeBonus
  float mp;     // max logit of the target row drawn from (offset for exp)
  float mq;     // max logit of the draft row (residual mode)
  double sp;    // float64 normaliser sum exp((z - mp) / T) of the target row
  double sq;    // float64 normaliser of the draft row
  double pad[2];
};
constexpr int kModeResidual = 0;
constexpr int kModeBonus = 1;

// Counters per request: [0] row pass, [1] normaliser pass, [2] draw pass.
constexpr int kCountersPerReq = 4;

// Workspace layout.  The ticket counters sit at a fixed place (the first
// kMaxB * kCountersPerReq words) whatever the call's shape, so a workspace
// reused across shapes never reads another call's partial results as a
// counter; every call leaves the counters it used at zero.
constexpr int kMaxB = 65536;

struct WsLayout {
  size_t count;  // uint32 [kMaxB * kCountersPerReq], always at offset 0
  size_t part1;  // float2 [rows * chunks]: (max, sum) or (value, index)
  size_t state;  // ReqState [B]
  size_t part2;  // double2 [B * res_chunks]
  size_t total;
};

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

inline int row_chunks_max(int V) {
  return (V + kRowChunkElemsMin - 1) / kRowChunkElemsMin;
}
inline int res_chunks(int V) { return (V + kResChunkElems - 1) / kResChunkElems; }

inline WsLayout ws_layout(int B, int n_pos, int V) {
  WsLayout L;
  size_t rows = (size_t)B * (size_t)n_pos * 2;
  size_t off = 0;
  L.count = off;
  off = align_up(off + (size_t)kMaxB * kCountersPerReq * 4, 256);
  L.part1 = off;
  off = align_up(off + rows * (size_t)row_chunks_max(V) * 8, 256);
  L.state = off;
  off = align_up(off + (size_t)B * sizeof(ReqState), 256);
  L.part2 = off;
  off = align_up(off + (size_t)B * (size_t)res_chunks(V) * 16, 256);
  L.total = off;
  return L;
}

// Tree description passed by value in the kernel arguments (2 KiB).
struct TreeArgs {
  int16_t parent[kMaxNodes];
};

// Launch wrappers (defined in the .hip files).  Each returns a hipError_t.
hipError_t launch_fill_uniforms(uint64_t seed, uint64_t counter0, int64_t n,
                                float* out, hipStream_t s);

hipError_t launch_greedy_chain(const void* target, int dtype, int B, int k, int V,
                               const int32_t* draft_tokens, int32_t* accepted_len,
                               int32_t* out_tokens, void* ws, const WsLayout& L,
                               hipStream_t s);

hipError_t launch_tree_greedy(const void* target, int dtype, int B, int n_nodes,
                              int V, const TreeArgs& tree, int depth,
                              const int32_t* node_tokens, int32_t* accepted_len,
                              int32_t* out_tokens, int32_t* out_path, void* ws,
                              const WsLayout& L, hipStream_t s);

hipError_t launch_sample(const void* target, const void* draft, int dtype, int kind,
                         int B, int k, int V, const int32_t* draft_tokens,
                         const float* uniforms, uint64_t seed, uint64_t counter0,
                         float temperature, int32_t* accepted_len,
                         int32_t* out_tokens, float* probe, void* ws,
                         const WsLayout& L, hipStream_t s);

}  // namespace specv
