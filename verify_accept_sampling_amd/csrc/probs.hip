// Sampling chain verification on probability rows for gfx950: the target
// and draft distributions p_i, q_i are given as float32 rows.  The rule is
// the sampling chain's ("EAGLE-3 speculative decoding review", equations
// A(x) and p_residual in the section on whether a small draft hurts quality;
// the serving chapter's acceptance-rule section): accept draft x_i while
// u_i q_i(x_i) < p_i(x_i), stop at the first rejection n and draw from
// max(0, p_n - q_n) normalised (from p_n when that residual is empty), or
// from p_k when every draft passes.
//
// Two launches:
//   1. k_probs_rows, work-group (request b, group g), 4 waves.  Every
//      work-group runs the request's acceptance tests itself (k gathers and
//      comparisons, exact in float64 for float32 inputs), so it knows the
//      stop position n without waiting for anyone; group 0 also writes the
//      accepted prefix, the probe values and n.  Wave w then sums its m
//      consecutive chunks (kPChunk elements each) of the rows drawn from --
//      target and draft row n after a rejection, target row k at the bonus
//      -- into S_p = sum p and W = sum max(0, p - q), in float64, one record
//      per chunk.  16-byte loads each cover 1 KB of a row, and each chunk is
//      read as two halves in two register buffers used in turn.
//   2. k_probs_pick, one work-group per request: the grand total, the chunk
//      where the running total first exceeds u times it, and that chunk
//      element by element.
// The terms are the given values, so a chunk costs a few float64
// operations per element and the row pass is bound by HBM.  One wave
// reduction per 2048 elements keeps the cross-lane traffic off the
// streaming path (per 256 elements, the shuffles alone cost about a tenth
// of the run).  The draw is a launch of its own because, as the tail of
// each request's last row work-group (by completion ticket), its three
// dependent round trips (ticket, chunk sums, chunk elements) held a
// work-group slot each and the last request's came after all streaming:
// 89-90 us against 84 us for the two launches at B = 512, V = 128256.
#include <algorithm>
#include <atomic>
#include <climits>

#include "sample_device.h"

namespace specv {
namespace {

#ifndef SPEC_PROBS_ROUNDS_X2
#define SPEC_PROBS_ROUNDS_X2 5
#endif
constexpr long kProbsRoundsX2 = SPEC_PROBS_ROUNDS_X2;  // rounds of resident work-groups, x2
constexpr int kPChunk = 2048;                          // elements per chunk (one wave)
constexpr int kPLoads = kPChunk / (kWaveSize * 4);     // 16-byte loads per lane and row
constexpr int kPSearch = kPChunk / kThreads;           // elements per thread in the search
static_assert(kPLoads == 8 && kPSearch == 8, "chunk shape");

// Sums of one chunk: S_p and W.
struct ProbsPart {
  double sp;  // sum of p over the chunk
  double w;   // sum of max(0, p - q) over the chunk (0 at the bonus)
};

int probs_chunks(int V) { return (V + kPChunk - 1) / kPChunk; }

// Acceptance tests on probability rows: u * q(x) < p(x), exact in float64
// for float32 inputs.  Every thread returns n; with `write` the accepted
// prefix and the probe values are stored, except probe[b, n, 2], which the
// request's finishing work-group owns.
__device__ int accept_scan_probs(const float* target, const float* draft, int b, int k, int V,
                                 const int32_t* draft_tokens, const float* uniforms,
                                 uint64_t seed, uint64_t ctr0, bool write,
                                 int32_t* accepted_len, int32_t* out_tokens, float* probe) {
  // k <= 1023, so each thread handles at most 4 positions.
  float pv[4] = {0.f, 0.f, 0.f, 0.f}, qv[4] = {0.f, 0.f, 0.f, 0.f};
  int first = k;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int i = threadIdx.x + s * kThreads;
    if (i >= k) break;
    const int x = draft_tokens[(long)b * k + i];
    bool accept = false;
    if (x >= 0 && x < V) {
      pv[s] = target[((long)b * (k + 1) + i) * V + x];
      qv[s] = draft[((long)b * k + i) * V + x];
      const float u = get_uniform(uniforms, seed, ctr0, b, i, 0, k);
      accept = (double)u * (double)qv[s] < (double)pv[s];
    }
    if (!accept) first = min(first, i);
  }
  const int n = block_min_i(first);
  if (write) {
    if (probe) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int i = threadIdx.x + s * kThreads;
        if (i > k) break;
        float* pr = probe + ((long)b * (k + 1) + i) * 4;
        pr[0] = i < k ? pv[s] : 0.f;
        pr[1] = i < k ? qv[s] : 0.f;
        if (i != n) pr[2] = 0.f;
        pr[3] = 0.f;
      }
    }
    for (int i = threadIdx.x; i <= k; i += kThreads) {
      if (i < n) out_tokens[(long)b * (k + 1) + i] = draft_tokens[(long)b * k + i];
      else if (i > n) out_tokens[(long)b * (k + 1) + i] = -1;
    }
    if (threadIdx.x == 0) accepted_len[b] = n;
  }
  return n;
}

// The draw weight of one element pair: max(0, p - q), 0 for NaN.
__device__ __forceinline__ double resid_weight(double p, double q) {
  const double d = p - q;
  return d > 0.0 ? d : 0.0;
}

// Sums of chunks c0 .. c0 + m - 1 (all below C), one record per chunk:
// S_p and W summed over the wave (lanes 0-31 store S_p, lanes 32-63 W).
// NE = 4: rows 16-byte aligned and shorter than 2 GiB; each chunk is read
// as two halves of 4 loads per lane and row into two register buffers, the
// second half's loads issued before the first half is summed.  NE = 1:
// element loads.
template <int NE, bool RESID>
__device__ __forceinline__ void wave_chunks(const float* prow, const float* qrow, int V, int c0,
                                            int m, ProbsPart* __restrict__ rp) {
  const int lane = threadIdx.x & 63;
  double sa = 0.0, w = 0.0;
  auto finish = [&](int c) {
    // One exchange per level: the halves swap their other sum, then each
    // half reduces its own.
    const bool h = (lane & 32) != 0;
    double r = h ? w : sa;
    r += shfl_xor_d(h ? sa : w, 32);
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) r += shfl_xor_d(r, o);
    if (lane == 0) rp[c].sp = r;
    if (lane == 32) rp[c].w = r;
    sa = w = 0.0;
  };
  if constexpr (NE == 4) {
    constexpr int kH = kPLoads / 2;  // loads per lane and row in half a chunk
    const RowBuf bp(prow, (uint32_t)V * 4u), bq(qrow, (uint32_t)V * 4u);
    const uint32_t off0 = (uint32_t)c0 * (uint32_t)(kPChunk * 4) + (uint32_t)lane * 16u;
    u32x4 pa[kH], qa[kH], pb[kH], qb[kH];
    auto load = [&](u32x4 (&p)[kH], u32x4 (&q)[kH], int half) {
      const uint32_t off = off0 + (uint32_t)half * (uint32_t)(kPChunk * 2);
#pragma unroll
      for (int j = 0; j < kH; ++j) p[j] = bp.load_nt(off + (uint32_t)j * 1024u, 0);
      if constexpr (RESID) {
#pragma unroll
        for (int j = 0; j < kH; ++j) q[j] = bq.load_nt(off + (uint32_t)j * 1024u, 0);
      }
    };
    auto fold = [&](const u32x4 (&p)[kH], const u32x4 (&q)[kH]) {
#pragma unroll
      for (int j = 0; j < kH; ++j) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const double a = (double)__uint_as_float(p[j][e]);
          sa += a;
          if constexpr (RESID) w += resid_weight(a, (double)__uint_as_float(q[j][e]));
        }
      }
    };
    // Every load is unconditional (the last chunk is peeled), so the
    // buffers need no register copies, which would wait for loads in flight.
    load(pa, qa, 0);
#pragma unroll 1
    for (int i = 0; i + 1 < m; ++i) {  // wave-uniform
      load(pb, qb, 2 * i + 1);
      fold(pa, qa);
      load(pa, qa, 2 * i + 2);
      fold(pb, qb);
      finish(c0 + i);
    }
    load(pb, qb, 2 * m - 1);
    fold(pa, qa);
    fold(pb, qb);
    finish(c0 + m - 1);
  } else {
    for (int i = 0; i < m; ++i) {
      const long j0 = (long)(c0 + i) * kPChunk + lane;
#pragma unroll 8
      for (int j = 0; j < kPChunk / kWaveSize; ++j) {
        const long e = j0 + (long)j * kWaveSize;
        if (e < V) {
          const double a = (double)prow[e];
          sa += a;
          if constexpr (RESID) w += resid_weight(a, (double)qrow[e]);
        }
      }
      finish(c0 + i);
    }
  }
}

// Pass over the rows drawn from: work-group (request b, group g).
template <int NE>
__global__ __launch_bounds__(kThreads) void k_probs_rows(
    const float* __restrict__ target, const float* __restrict__ draft, int k, int V, int C,
    int G, int m, const int32_t* __restrict__ draft_tokens, const float* __restrict__ uniforms,
    uint64_t seed, uint64_t ctr0, int32_t* __restrict__ accepted_len,
    int32_t* __restrict__ out_tokens, float* __restrict__ probe, ProbsPart* __restrict__ part,
    int32_t* __restrict__ stop) {
  const int b = static_cast<int>(blockIdx.x / G), g = static_cast<int>(blockIdx.x % G);
  const int n = accept_scan_probs(target, draft, b, k, V, draft_tokens, uniforms, seed, ctr0,
                                  g == 0, accepted_len, out_tokens, probe);
  if (g == 0 && threadIdx.x == 0) stop[b] = n;
  const bool resid = n < k;
  const float* prow = target + ((long)b * (k + 1) + n) * V;
  const float* qrow = resid ? draft + ((long)b * k + n) * V : prow;
  const int wave = threadIdx.x >> 6;
  ProbsPart* rp = part + (long)b * C;
  // This wave's chunks: m consecutive ones (fewer at the end of the row).
  const int c0 = (g * kWaves + wave) * m;
  const int mc = min(m, C - c0);
  if (mc > 0) {  // wave-uniform
    if (resid) wave_chunks<NE, true>(prow, qrow, V, c0, mc, rp);
    else wave_chunks<NE, false>(prow, qrow, V, c0, mc, rp);
  }
}

// The draw of request b = blockIdx.x from the chunk sums: grand total,
// chunk, element.
template <int NE>
__global__ __launch_bounds__(kThreads) void k_probs_pick(
    const float* __restrict__ target, const float* __restrict__ draft, int k, int V, int C,
    const float* __restrict__ uniforms, uint64_t seed, uint64_t ctr0,
    int32_t* __restrict__ out_tokens, float* __restrict__ probe,
    const ProbsPart* __restrict__ part, const int32_t* __restrict__ stop) {
  const int b = static_cast<int>(blockIdx.x);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const ProbsPart* rp = part + (long)b * C;
  const int n = stop[b];  // loaded together with the chunk sums below
  const bool resid = n < k;
  const float* prow = target + ((long)b * (k + 1) + n) * V;
  const float* qrow = resid ? draft + ((long)b * k + n) * V : prow;
  // Each wave finds the chunk by itself (the same loads and the same
  // arithmetic in every wave, so the same result), without a barrier.
  // Grand totals: lane l sums chunks l, l + 64, ...
  double tw = 0.0, tp = 0.0;
  for (int cc = lane; cc < C; cc += kWaveSize) {
    tw += rp[cc].w;
    tp += rp[cc].sp;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    tw += shfl_xor_d(tw, o);
    tp += shfl_xor_d(tp, o);
  }
  // Weights drawn from: the residual, or the target when the residual is
  // empty (or at the bonus position).
  const bool use_w = resid && tw > 0.0;
  const double grand = use_w ? tw : tp;
  const float u = get_uniform(uniforms, seed, ctr0, b, n, 1, k);
  const double thr = (double)u * grand;
  // The chunk where the running total first exceeds thr, and the total of
  // the chunks before it; past the end (a last-bit difference) the last
  // chunk.  Tiles of 64 chunks, one per lane, in order.
  int cs = C - 1;
  double P = 0.0, running = 0.0;
  for (int base = 0; base < C; base += kWaveSize) {  // wave-uniform
    const int cc = base + lane;
    const double v = cc < C ? (use_w ? rp[cc].w : rp[cc].sp) : 0.0;
    const double inc = wave_inclusive_scan_d(v);
    const double excl = running + (inc - v);
    const uint64_t mh = __ballot(cc < C && excl + v > thr);
    if (mh != 0) {
      const int f = __builtin_ctzll(mh);
      cs = base + f;
      P = __shfl(excl, f, kWaveSize);
      break;
    }
    if (base + kWaveSize >= C) {  // past the end: the last chunk
      P = __shfl(excl, C - 1 - base, kWaveSize);
      break;
    }
    running += __shfl(inc, kWaveSize - 1, kWaveSize);
  }
  // Search chunk cs: wave w takes its quarter, lane l the kPSearch
  // consecutive elements from cs * kPChunk + kPChunk / 4 * w + kPSearch l,
  // so the running sum in element order is the sum of the earlier waves'
  // totals, the lane's exclusive prefix and its own running sum.  The loads
  // are unconditional (past the row's end: out of the buffer's range, or
  // clamped), so all are in flight together.
  const long j0 = (long)cs * kPChunk + (long)threadIdx.x * kPSearch;
  const int rem = (int)min((long)kPSearch, (long)V - j0);  // valid elements of this lane
  float pv[kPSearch], qv[kPSearch];
  if constexpr (NE == 4) {
    const RowBuf bp(prow, (uint32_t)V * 4u), bq(qrow, (uint32_t)V * 4u);
    const uint32_t off = (uint32_t)j0 * 4u;
#pragma unroll
    for (int h = 0; h < kPSearch / 4; ++h) {
      const u32x4 wp = bp.load_nt(off + 16u * h, 0), wq = bq.load_nt(off + 16u * h, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pv[4 * h + e] = __uint_as_float(wp[e]);
        qv[4 * h + e] = __uint_as_float(wq[e]);
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < kPSearch; ++e) {
      const long j = min(j0 + e, (long)V - 1);
      pv[e] = prow[j];
      qv[e] = qrow[j];
    }
  }
  // Elements past the row's end weigh 0; drawing from p (bonus, or an empty
  // residual), q is taken as 0 and the clamp at 0 is skipped.
  double w[kPSearch];
  double lsum = 0.0;
#pragma unroll
  for (int e = 0; e < kPSearch; ++e) {
    const float pe = e < rem ? pv[e] : 0.f, qe = (e < rem && use_w) ? qv[e] : 0.f;
    const double d = (double)pe - (double)qe;
    w[e] = (d > 0.0 || !use_w) ? d : 0.0;
    lsum += w[e];
  }
  const double inc = wave_inclusive_scan_d(lsum);
  __shared__ double s_wsum[kWaves];
  __shared__ int s_tok[kWaves], s_last[kWaves];
  if (lane == kWaveSize - 1) s_wsum[wave] = inc;
  __syncthreads();
  double before = 0.0;  // the earlier waves' totals, in order
  for (int v = 0; v < wave; ++v) before += s_wsum[v];
  const double excl = before + (inc - lsum);
  int tok = INT_MAX, lastpos = -1;
  double run = 0.0;
#pragma unroll
  for (int e = 0; e < kPSearch; ++e) {
    run += w[e];
    if (e < rem) {
      if (w[e] > 0.0) lastpos = e;
      if (tok == INT_MAX && P + (excl + run) > thr) tok = e;
    }
  }
  // Element indices grow with the lane: the wave's first hit is in its
  // lowest hitting lane, its last positive weight in its highest one.
  const uint64_t mt = __ballot(tok != INT_MAX), ml = __ballot(lastpos >= 0);
  const int jt = static_cast<int>(j0);  // below 2^31: V <= 2^30
  if (mt != 0) {
    const int f = __builtin_ctzll(mt);
    const int t = __shfl(tok, f, kWaveSize) + __shfl(jt, f, kWaveSize);
    if (lane == 0) s_tok[wave] = t;
  } else if (lane == 0) {
    s_tok[wave] = INT_MAX;
  }
  if (ml != 0) {
    const int f = 63 - __builtin_clzll(ml);
    const int t = __shfl(lastpos, f, kWaveSize) + __shfl(jt, f, kWaveSize);
    if (lane == 0) s_last[wave] = t;
  } else if (lane == 0) {
    s_last[wave] = -1;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int t = -1;
    for (int v = kWaves - 1; v >= 0; --v) {  // the first hit; else the last positive weight
      if (s_tok[v] != INT_MAX) t = s_tok[v];
    }
    if (t < 0) {
      for (int v = 0; v < kWaves; ++v) t = max(t, s_last[v]);
    }
    if (!(grand > 0.0)) t = -1;  // rows without mass (invalid input)
    out_tokens[(long)b * (k + 1) + n] = t;
    // Mass of the distribution drawn from: W after a rejection (0 when the
    // residual is empty), S_p at the bonus.
    if (probe)
      probe[((long)b * (k + 1) + n) * 4 + 2] = (float)(use_w ? grand : (resid ? 0.0 : grand));
  }
}

template <int NE>
hipError_t launch_probs_t(const float* target, const float* draft, int B, int k, int V,
                          const int32_t* draft_tokens, const float* uniforms, uint64_t seed,
                          uint64_t ctr0, int32_t* accepted_len, int32_t* out_tokens, float* probe,
                          char* w, const WsLayout& L, hipStream_t s) {
  const int C = probs_chunks(V);
  // Work-groups of m chunks per wave, sized for about two and a half rounds
  // of resident work-groups (fewer acceptance scans per byte than one chunk
  // per wave: 8192 such work-groups took 146 us at B = 512, V = 128256;
  // 1.5 to 6 rounds were within 1.5 us of each other).
  static std::atomic<int> per_cu_cached{0};
  int per_cu = per_cu_cached.load(std::memory_order_relaxed);
  if (per_cu <= 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void*>(&k_probs_rows<NE>), kThreads, 0) !=
            hipSuccess ||
        per_cu <= 0)
      per_cu = 1;
    per_cu_cached.store(per_cu, std::memory_order_relaxed);
  }
  const long slots = (long)device_cus() * per_cu;
  const int g1 = (C + kWaves - 1) / kWaves;  // work-groups at one chunk per wave
  const int want = (int)std::max(
      1L, std::min((long)g1, (kProbsRoundsX2 * slots + 2L * B - 1) / (2L * B)));
  const int m = (g1 + want - 1) / want;
  const int G = (C + kWaves * m - 1) / (kWaves * m);
  auto* part = reinterpret_cast<ProbsPart*>(w + L.part2);
  auto* stop = reinterpret_cast<int32_t*>(w + L.state);
  const hipError_t e = launch_timed(kProfRowPass, &k_probs_rows<NE>,
                                    dim3((unsigned)((long)B * G)), dim3(kThreads), 0, s, target,
                                    draft, k, V, C, G, m, draft_tokens, uniforms, seed, ctr0,
                                    accepted_len, out_tokens, probe, part, stop);
  if (e != hipSuccess) return e;
  return launch_timed(kProfDraw, &k_probs_pick<NE>, dim3((unsigned)B), dim3(kThreads), 0, s,
                      target, draft, k, V, C, uniforms, seed, ctr0, out_tokens, probe,
                      (const ProbsPart*)part, (const int32_t*)stop);
}

}  // namespace

// The chunk sums fit in the workspace's draw-record region, which is sized
// for the logits draw's finer chunks and larger records.
static_assert(sizeof(ProbsPart) <= sizeof(DrawPart) && kPChunk >= kDrawChunk,
              "probability-row sums fit the draw-record region");

hipError_t launch_probs(const void* target, const void* draft, int B, int k, int V,
                        const int32_t* draft_tokens, const float* uniforms, uint64_t seed,
                        uint64_t ctr0, int32_t* accepted_len, int32_t* out_tokens, float* probe,
                        bool vec, void* ws, const WsLayout& L, hipStream_t s) {
  const auto* t = static_cast<const float*>(target);
  const auto* d = static_cast<const float*>(draft);
  char* w = static_cast<char*>(ws);
  if (vec)
    return launch_probs_t<4>(t, d, B, k, V, draft_tokens, uniforms, seed, ctr0, accepted_len,
                             out_tokens, probe, w, L, s);
  return launch_probs_t<1>(t, d, B, k, V, draft_tokens, uniforms, seed, ctr0, accepted_len,
                           out_tokens, probe, w, L, s);
}

}  // namespace specv
