// Internal declarations shared by the host entry points (api.cpp) and the
// kernel translation units.  Not part of the public ABI.
#pragma once

#include <atomic>

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/spec_verify.h"

namespace specv {

// Block shape of every kernel: 256 threads = 4 waves of 64 lanes.
constexpr int kThreads = 256;
constexpr int kWaveSize = 64;
constexpr int kWaves = kThreads / kWaveSize;

// Elements per work-group chunk of the pass over every row (tunable at
// build time).
#ifndef SPEC_ROW_CHUNK
#define SPEC_ROW_CHUNK 65536
#endif
constexpr int kRowChunkElems = SPEC_ROW_CHUNK;
// 16-byte loads in flight per thread in the argmax sweep.
#ifndef SPEC_ROW_UNROLL
#define SPEC_ROW_UNROLL 8
#endif
constexpr int kRowUnroll = SPEC_ROW_UNROLL;
// 16-byte loads per thread per batch in the row-statistics sweep, which
// keeps two batches in flight (the next one loads while the current one is
// folded in).  4 keeps the kernel near 64 VGPRs, i.e. 7 waves per SIMD; 8
// needs about 100 VGPRs (4 waves) and is slower.
#ifndef SPEC_STATS_UNROLL
#define SPEC_STATS_UNROLL 4
#endif
// Smallest chunk the workspace is sized for (leaves room to retune).
constexpr int kRowChunkElemsMin = 2048;
// Smallest row chunk the greedy kernels split rows into.
constexpr int kMinChunkElems = 16384;
static_assert(kMinChunkElems >= kRowChunkElemsMin, "partials are sized for chunks of at least this");
// Float64 residual / bonus pass: the row is cut into chunks of
// kDrawChunk elements, one wave per chunk (64 lanes x kSegPerThread
// consecutive elements); a work-group of kThreads/64 waves handles kDrawChunksPerWave
// consecutive chunks per wave.
#ifndef SPEC_DRAW_SEG
#define SPEC_DRAW_SEG 8
#endif
constexpr int kSegPerThread = SPEC_DRAW_SEG;
constexpr int kDrawChunk = 64 * kSegPerThread;
#ifndef SPEC_DRAW_CHUNKS_PER_WAVE
#define SPEC_DRAW_CHUNKS_PER_WAVE 3
#endif
constexpr int kDrawChunksPerWave = SPEC_DRAW_CHUNKS_PER_WAVE;
constexpr int kDrawChunksPerGroup = kWaves * kDrawChunksPerWave;
// Draw work-groups per request when each takes nb batches of
// kDrawChunksPerGroup chunks.
__host__ __device__ inline int draw_groups(int C2, int nb) {
  const int per = kDrawChunksPerGroup * nb;
  return (C2 + per - 1) / per;
}
// Elements per thread when a whole work-group searches one chunk.
constexpr int kSearchPerThread = kDrawChunk / kThreads;

constexpr int kMaxK = 1023;
constexpr int kMaxNodes = 1024;
constexpr int kMaxV = 1 << 30;
constexpr int kMaxB = 65536;

// Per-request state handed from the row pass to the draw pass.
struct ReqState {
  int n;         // accepted length (first rejection or k)
  int mode;      // kModeResidual or kModeBonus
  float mp;      // max logit of the target row drawn from (offset for exp)
  float mq;      // max logit of the draft row (residual mode)
  double rho32;  // S_p / S_q of the rejected rows from the float32 statistics
};
constexpr int kModeResidual = 0;
constexpr int kModeBonus = 1;

// Chunk partial of the float64 draw pass.
// Elements in the kink band of max(0, a - rho b) are kept out of w and dq
// (their sign may differ between rho32 and the exact rho) and recorded, up
// to kKinkSlots of them, as (a, b) pairs; a chunk with more is recomputed.
constexpr int kKinkSlots = 2;
struct DrawPart {
  double sp;    // sum of e^{(z - mp)/T} (probabilities: sum of p) over the chunk
  double sq;    // sum of e^{(y - mq)/T} over the chunk (residual mode)
  double w;     // sum of the draw weights at rho32, kink-band elements excluded
  double dq;    // d w / d rho at rho32: minus the sum of e^{(y-mq)/T} where the weight is positive
  double nk;    // number of kink-band elements (more than kKinkSlots: recompute)
  double ka[kKinkSlots];  // their target terms a
  double kb[kKinkSlots];  // and draft terms b
  double pad;
};
static_assert(sizeof(DrawPart) == 80, "DrawPart layout");

// Per-request 32-bit words of the counter region: [0] row-pass completion
// ticket, [1] draw completion ticket, [2] the verdict word of the one-launch
// kernel's early acceptance tests, [3] unused, [4..7] its ready slot, two
// 64-bit words that carry a request's packed draw state.  The one-launch
// words of position j belong to request j with its two bytes swapped.
// Every per-request word is back to 0 when a call completes.  The last 256
// bytes hold the workspace status word (sticky bits, SPEC_STATUS_*) and the
// 64-bit call epoch of graph-captured one-launch calls.
constexpr int kCountersPerReq = 8;
constexpr int kVerdictWord = 2;
constexpr int kReadySlotWord = 4;
constexpr size_t kCounterRegionBytes = (size_t)kMaxB * kCountersPerReq * 4 + 256;
static_assert(kCounterRegionBytes == SPEC_WORKSPACE_COUNTER_BYTES, "counter region");
constexpr size_t kPerRequestWords = (size_t)kMaxB * kCountersPerReq;
constexpr size_t kStatusWord = kPerRequestWords;     // uint32 index
constexpr size_t kEpochWord = kPerRequestWords + 2;  // uint32 index of a uint64
static_assert(kEpochWord % 2 == 0, "epoch word is 8-byte aligned");
static_assert(SPEC_WORKSPACE_STATUS_OFFSET == kStatusWord * 4, "status word offset");

// Workspace layout.  The counter region (kCounterRegionBytes) sits at a
// fixed place whatever the call's shape; it must be zero before the first
// call, and every call leaves it zero (tickets reset by their last taker,
// ready slots cleared by the request's draw).  The completion tags of the
// one-launch row pass hold the tag of the call that wrote them; every call
// has a tag of its own, so a tag left by an earlier call (or any other
// content) is never taken for a current one.  The other regions are written
// before they are read within each call.
// Tree-sampling regions: the tree tables (nine int32 tables of kMaxNodes),
// the per-request draw state and the float64 row statistics.
constexpr size_t kTreeTableBytes = 10 * (size_t)kMaxNodes * 4;
constexpr size_t kTreeDrawBytes = 32;
constexpr size_t kTreeStatBytes = 16;  // float64 row statistic of one row chunk
// Tree rows that carry the float64 statistic are cut into chunks of this
// many elements (one work-group each: float64 terms are ALU work).
// Measured at B=16, 61 nodes, V=128256: 16384-, 32768- and 65536-element
// chunks 212.0, 208.0 and 208.5 us per call (fewer chunks are fewer
// statistics for every later kernel to merge; the largest leave the
// statistics launch a ragged last round).
constexpr int kTreeStatChunk = 32768;
__host__ __device__ inline int tree_xchunks(int V) {
  return (V + kTreeStatChunk - 1) / kTreeStatChunk;
}
// Tree sampling's residual masses: one partial per chunk of this many
// elements of a row pair (at most res_chunks(V) per row: they fit part3).
constexpr int kTreeMassChunk = 8192;
__host__ __device__ inline int tree_mchunks(int V) {
  return (V + kTreeMassChunk - 1) / kTreeMassChunk;
}

struct WsLayout {
  size_t count;  // counter region, always at offset 0
  size_t part1;  // uint64 [rows * row_chunks]: packed (max, sum) or (value, index)
  size_t flag;   // uint64 [rows * row_chunks]: completion tags of the one-launch row pass
  size_t zrow;   // float [rows]: each row's logit at its draft token
  size_t state;  // ReqState [B]
  size_t part2;  // DrawPart [B * res_chunks]
  size_t part3;  // double [B * n_pos * res_chunks]: tree sampling's residual masses
  size_t tree;   // tree tables (kTreeTableBytes)
  size_t tstate; // tree sampling's draw state, kTreeDrawBytes per request
  size_t xstat;  // tree sampling's float64 row statistics, [rows * row_chunks]
  size_t total;
};

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

inline int row_chunks_max(int V) {
  return (V + kRowChunkElemsMin - 1) / kRowChunkElemsMin;
}
inline int res_chunks(int V) { return (V + kDrawChunk - 1) / kDrawChunk; }

inline WsLayout ws_layout(int B, int n_pos, int V) {
  WsLayout L;
  const size_t rows = (size_t)B * (size_t)n_pos * 2;
  size_t off = 0;
  L.count = off;
  off = align_up(off + kCounterRegionBytes, 256);
  L.part1 = off;
  off = align_up(off + rows * (size_t)row_chunks_max(V) * 8, 256);
  L.flag = off;
  off = align_up(off + rows * (size_t)row_chunks_max(V) * 8, 256);
  L.zrow = off;
  off = align_up(off + rows * 4, 256);
  L.state = off;
  off = align_up(off + (size_t)B * sizeof(ReqState), 256);
  L.part2 = off;
  off = align_up(off + (size_t)B * (size_t)res_chunks(V) * sizeof(DrawPart), 256);
  L.part3 = off;
  off = align_up(off + (size_t)B * (size_t)n_pos * (size_t)res_chunks(V) * 8, 256);
  L.tree = off;
  off = align_up(off + kTreeTableBytes, 256);
  L.tstate = off;
  off = align_up(off + (size_t)B * kTreeDrawBytes, 256);
  L.xstat = off;
  off = align_up(off + rows * (size_t)tree_xchunks(V) * kTreeStatBytes, 256);
  L.total = off;
  return L;
}

// Tree description passed by value in the kernel arguments: a small form
// for trees of up to kSmallTree nodes (the kernel-argument block stays
// small), and the full one.
constexpr int kSmallTree = 128;
template <int N>
struct TreeArgsN {
  int16_t parent[N];
};
using TreeArgs = TreeArgsN<kMaxNodes>;

// Kernel kinds for the optional event timing (same values as the public
// SPEC_KERNEL_* constants).
constexpr int kProfRowPass = 0;   // row statistics / argmax sweep + per-request finish
constexpr int kProfDraw = 1;      // float64 residual / bonus pass + inverse-CDF draw
constexpr int kProfUniforms = 2;  // spec_fill_uniforms
constexpr int kProfFused = 3;     // one-launch sampling verification (row pass + draw)
constexpr int kProfServing = 4;   // rejected-draft masks
constexpr int kProfTreeStats = 5; // tree sampling: row statistics
constexpr int kProfTreeMass = 6;  // tree sampling: residual-mass rounds
constexpr int kProfTreeWalk = 7;  // tree sampling: table setup and the walk
constexpr int kProfTreeDraw = 8;  // tree sampling: draw weights and the pick
constexpr int kProfTreeLeaf = 9;  // tree sampling: the stop leaves' row statistics
constexpr int kProfKinds = 10;
// While timing is enabled, prof_begin hands out a start/stop event pair that
// the launch itself stamps (hipExtLaunchKernel records them from the
// kernel's dispatch, so the interval is the kernel alone); otherwise both
// events are null and the launch is an ordinary one.
struct ProfEvents {
  hipEvent_t start = nullptr, stop = nullptr;
  int slot = -1;
};
ProfEvents prof_begin(int kind);
void prof_end(const ProfEvents& ev, hipError_t launch_status);

// Launch `kernel` with `shmem` bytes of dynamic shared memory on stream s,
// timed as `kind`.
template <typename... KArgs, typename... Args>
hipError_t launch_timed(int kind, void (*kernel)(KArgs...), dim3 grid, dim3 block,
                        uint32_t shmem, hipStream_t s, Args... args) {
  const ProfEvents ev = prof_begin(kind);
  hipExtLaunchKernelGGL(kernel, grid, block, shmem, s, ev.start, ev.stop, 0, args...);
  const hipError_t e = hipGetLastError();
  prof_end(ev, e);
  return e;
}

// Completion tag of one call (tags that work-groups store to say a partial
// is complete): a marker byte, 16 bits drawn once per process and a 40-bit
// call counter, so no two calls of a process share a tag, and neither
// zero-filled memory nor any value the workspace holds otherwise (floats,
// doubles, counts) looks like one.
uint64_t next_call_tag();

// Launch wrappers (defined in the .hip files).  Each returns a hipError_t.
hipError_t launch_fill_uniforms(uint64_t seed, uint64_t counter0, int64_t n,
                                float* out, hipStream_t s);

hipError_t launch_rejected_mask(const int32_t* accepted_len, const int32_t* path, int path_len,
                                int B, int n_ent, uint8_t* rejected, int64_t* slots,
                                int64_t pad_slot, hipStream_t s);

hipError_t launch_greedy_chain(const void* target, int dtype, int B, int k, int V,
                               const int32_t* draft_tokens, int32_t* accepted_len,
                               int32_t* out_tokens, void* ws, const WsLayout& L,
                               hipStream_t s);

hipError_t launch_tree_greedy(const void* target, int dtype, int B, int n_nodes,
                              int V, const TreeArgs& tree, int depth,
                              const int32_t* node_tokens, int32_t* accepted_len,
                              int32_t* out_tokens, int32_t* out_path, void* ws,
                              const WsLayout& L, hipStream_t s);

// Host-side shape of a tree, the same as the tables k_tree_setup writes:
// depth, nodes with a child, the highest sibling rank, how many children
// have each rank, and which nodes have a child.
struct TreeShape {
  int depth = 0;
  int n_internal = 0;
  int max_rank = 0;
  int rank_count[kMaxNodes] = {0};
  bool has_child[kMaxNodes] = {false};
};

hipError_t launch_tree_sample(const void* target, const void* draft, int dtype, int kind, int B,
                              int N, int V, const TreeArgs& tree, const TreeShape& shape,
                              const int32_t* node_tokens, const float* uniforms, uint64_t seed,
                              uint64_t counter0, float temperature, int32_t* accepted_len,
                              int32_t* out_tokens, int32_t* out_path, void* ws,
                              const WsLayout& L, hipStream_t s);

// How one sampling call is run (from the call's flags and its stream).
struct SampleMode {
  int sched;       // a SPEC_SCHED_* value (AUTO is resolved at the launch, from the shape)
  bool capturing;  // the stream is being captured into a graph
  bool test_give_up;  // SPEC_FLAG_TEST_GIVE_UP
};

// Compute units of the current device (cached per device).
int device_cus();

// Sampling verification on float32 probability rows (probs.hip); vec: rows
// 16-byte aligned and shorter than 2 GiB.
hipError_t launch_probs(const void* target, const void* draft, int B, int k, int V,
                        const int32_t* draft_tokens, const float* uniforms, uint64_t seed,
                        uint64_t ctr0, int32_t* accepted_len, int32_t* out_tokens, float* probe,
                        bool vec, void* ws, const WsLayout& L, hipStream_t s);

hipError_t launch_sample(const void* target, const void* draft, int dtype, int kind,
                         int B, int k, int V, const int32_t* draft_tokens,
                         const float* uniforms, uint64_t seed, uint64_t counter0,
                         float temperature, const SampleMode& mode, int32_t* accepted_len,
                         int32_t* out_tokens, float* probe, void* ws,
                         const WsLayout& L, hipStream_t s);

// Zeroes the counter region of a workspace except its call epoch.
hipError_t launch_reset_counters(void* ws, hipStream_t s);

// Device address of the no-alloc scratch array on `device`, which must be
// the current device (looked up once per device, then cached).
constexpr size_t kNoAllocScratchBytes = SPEC_NOALLOC_SCRATCH_BYTES;
hipError_t noalloc_scratch(int device, void** ptr);
// Zeroes the counter words of requests 0..B-1 and the status word of a
// workspace (the call epoch is kept).
hipError_t launch_clear_requests(void* ws, int B, hipStream_t s);

}  // namespace specv
