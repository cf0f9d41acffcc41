// Sampling chain verification for gfx950: the min(1, p/q) rule with
// residual resampling ("EAGLE-3 speculative decoding review", equations
// A(x) and p_residual in the section on whether a small draft hurts quality;
// the serving chapter's acceptance-rule section), stopping at the first
// rejection and drawing a bonus token when every draft passes (EAGLE-3
// review "Speculative Decoding" step 3; serving chapter "how it works").
//
// Logits path, three launches on the caller's stream:
//   1. k_row_stats: work-group (chunk, row) streams one chunk of one of the
//      request's 2k+1 rows (k+1 target, k draft) with 16-byte loads and
//      reduces it to (max, sum 2^((x - max) c)), c = log2(e)/T, in float32.
//      The request's last work-group merges the chunk partials in float64,
//      evaluates every acceptance ratio p_i(x_i)/q_i(x_i) from the gathered
//      logits, finds the first rejection n and writes the accepted prefix.
//   2. k_res_norm: only for requests that rejected; recomputes the float64
//      normalisers of target row n and draft row n.
//   3. k_res_draw: float64 weights of the row drawn from (residual
//      max(0, p_n - q_n), or p_k for the bonus), one inclusive scan per
//      chunk, and in the request's last work-group the cross-chunk prefix and
//      the inverse-CDF search inside the chunk that holds the draw.
// Probabilities path (rows already normalised): a gather-only acceptance
// kernel replaces launches 1-2.
#include <climits>

#include "device_common.h"

namespace specv {

struct MSPart {
  float m;
  float s;
};

constexpr int kUnrollStats = 4;

// ---------------------------------------------------------------------------
// 1. Row statistics
// ---------------------------------------------------------------------------

template <int NE>
__device__ __forceinline__ void ms_update(float& m, float& s, const float (&x)[NE], float c) {
  float lm = x[0];
#pragma unroll
  for (int e = 1; e < NE; ++e) lm = fmaxf(lm, x[e]);
  const float mn = fmaxf(m, lm);
  const float base = (mn == -INFINITY) ? 0.f : mn;
  float acc = s * __builtin_amdgcn_exp2f((m - base) * c);
#pragma unroll
  for (int e = 0; e < NE; ++e) acc += __builtin_amdgcn_exp2f((x[e] - base) * c);
  s = acc;
  m = mn;
}

// Row r of request b: r <= k is target row r, r > k is draft row r-k-1.
template <int DT>
__device__ __forceinline__ const void* stat_row(const void* target, const void* draft, int b,
                                                int r, int k, int V) {
  const long eb = Elems<DT>::kBytes;
  if (r <= k)
    return reinterpret_cast<const char*>(target) + ((long)b * (k + 1) + r) * V * eb;
  return reinterpret_cast<const char*>(draft) + ((long)b * k + (r - k - 1)) * V * eb;
}

template <int DT, int NE>
__global__ __launch_bounds__(kThreads) void k_row_stats(
    const void* __restrict__ target, const void* __restrict__ draft, int k, int V, int C1,
    float c, double inv_t, const int32_t* __restrict__ draft_tokens,
    const float* __restrict__ uniforms, uint64_t seed, uint64_t ctr0,
    int32_t* __restrict__ accepted_len, int32_t* __restrict__ out_tokens,
    float* __restrict__ probe, MSPart* __restrict__ part, ReqState* __restrict__ state,
    unsigned* __restrict__ counters) {
  const int R = 2 * k + 1;
  const int blk = blockIdx.x;
  const int chunk = blk % C1;
  const long rowid = blk / C1;
  const int b = static_cast<int>(rowid / R);
  const int r = static_cast<int>(rowid % R);
  {
    const void* rp = stat_row<DT>(target, draft, b, r, k, V);
    const long n_groups = V / NE;
    const long gpc = (n_groups + C1 - 1) / C1;
    const long g0 = (long)chunk * gpc;
    const long g1 = min(g0 + gpc, n_groups);
    float m = -INFINITY, s = 0.f;
    for (long g = g0 + threadIdx.x; g < g1; g += (long)kThreads * kUnrollStats) {
      float x[kUnrollStats][NE];
#pragma unroll
      for (int u = 0; u < kUnrollStats; ++u) {
        const long gg = g + (long)u * kThreads;
        if (gg < g1) {
          load_group<DT, NE>(rp, gg * NE, x[u]);
        } else {
#pragma unroll
          for (int e = 0; e < NE; ++e) x[u][e] = -INFINITY;
        }
      }
#pragma unroll
      for (int u = 0; u < kUnrollStats; ++u) ms_update<NE>(m, s, x[u], c);
    }
    block_reduce_ms(m, s, c);
    if (threadIdx.x == 0) part[rowid * C1 + chunk] = MSPart{m, s};
  }
  if (!last_block_ticket(&counters[(long)b * kCountersPerReq + 0], (unsigned)(R * C1))) return;

  // ---- last work-group of request b: merge, accept scan, emit prefix ----
  // One wave per draft position: merge the chunk partials of target row i
  // and draft row i (float64 sums), then test draft token i.
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int first = k;
  for (int i = wave; i < k; i += kWaves) {
    float mrow[2];
    double l2s[2];
#pragma unroll
    for (int side = 0; side < 2; ++side) {
      const long base_idx = ((long)b * R + (side == 0 ? i : k + 1 + i)) * C1;
      float M = -INFINITY;
      for (int cc = lane; cc < C1; cc += 64) M = fmaxf(M, part[base_idx + cc].m);
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, shfl_xor_f(M, o));
      const float mb = (M == -INFINITY) ? 0.f : M;
      double S = 0.0;
      for (int cc = lane; cc < C1; cc += 64) {
        const MSPart pp = part[base_idx + cc];
        S += (double)pp.s * exp2((double)((pp.m - mb) * c));
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) S += shfl_xor_d(S, o);
      mrow[side] = M;
      l2s[side] = log2(S);
    }
    if (lane == 0) {
      const int x = draft_tokens[(long)b * k + i];
      float pv = 0.f, qv = 0.f;
      bool accept = false;
      if (x >= 0 && x < V) {
        const float zp = load_elem<DT>(stat_row<DT>(target, draft, b, i, k, V), x);
        const float zq = load_elem<DT>(stat_row<DT>(target, draft, b, k + 1 + i, k, V), x);
        // log2 p_i(x) and log2 q_i(x) from the row statistics
        const double lp = (double)((zp - mrow[0]) * c) - l2s[0];
        const double lq = (double)((zq - mrow[1]) * c) - l2s[1];
        const double ratio = exp2(lp - lq);
        const float u = get_uniform(uniforms, seed, ctr0, b, i, 0, k);
        accept = (double)u < ratio;
        pv = (float)exp2(lp);
        qv = (float)exp2(lq);
      }
      if (!accept) first = min(first, i);
      if (probe) {
        float* pr = probe + ((long)b * (k + 1) + i) * 4;
        pr[0] = pv; pr[1] = qv; pr[2] = 0.f; pr[3] = 0.f;
      }
    }
  }
  const int n = block_min_i(first);
  if (probe && threadIdx.x == 0) {
    float* pr = probe + ((long)b * (k + 1) + k) * 4;
    pr[0] = 0.f; pr[1] = 0.f; pr[2] = 0.f; pr[3] = 0.f;
  }
  for (int i = threadIdx.x; i <= k; i += kThreads) {
    if (i < n) out_tokens[(long)b * (k + 1) + i] = draft_tokens[(long)b * k + i];
    else if (i > n) out_tokens[(long)b * (k + 1) + i] = -1;
  }
  // Maxima of the rows the draw uses: target row n and (rejection) draft row n.
  if (wave == 0) {
    float mrow[2] = {0.f, 0.f};
#pragma unroll
    for (int side = 0; side < 2; ++side) {
      if (side == 1 && n == k) break;
      const long base_idx = ((long)b * R + (side == 0 ? n : k + 1 + n)) * C1;
      float M = -INFINITY;
      for (int cc = lane; cc < C1; cc += 64) M = fmaxf(M, part[base_idx + cc].m);
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, shfl_xor_f(M, o));
      mrow[side] = M;
    }
    if (lane == 0) {
      accepted_len[b] = n;
      ReqState st;
      st.n = n;
      st.mode = n < k ? kModeResidual : kModeBonus;
      st.mp = mrow[0];
      st.mq = mrow[1];
      st.sp = 0.0;
      st.sq = 0.0;
      st.pad[0] = st.pad[1] = 0.0;
      state[b] = st;
    }
  }
  (void)inv_t;
}

// Probabilities path: rows are given distributions; the acceptance test
// u * q(x) < p(x) is exact in float64 for float32 inputs.
__global__ __launch_bounds__(kThreads) void k_accept_probs(
    const float* __restrict__ target, const float* __restrict__ draft, int k, int V,
    const int32_t* __restrict__ draft_tokens, const float* __restrict__ uniforms, uint64_t seed,
    uint64_t ctr0, int32_t* __restrict__ accepted_len, int32_t* __restrict__ out_tokens,
    float* __restrict__ probe, ReqState* __restrict__ state) {
  const int b = blockIdx.x;
  int first = k;
  for (int i = threadIdx.x; i < k; i += kThreads) {
    const int x = draft_tokens[(long)b * k + i];
    float pv = 0.f, qv = 0.f;
    bool accept = false;
    if (x >= 0 && x < V) {
      pv = target[((long)b * (k + 1) + i) * V + x];
      qv = draft[((long)b * k + i) * V + x];
      const float u = get_uniform(uniforms, seed, ctr0, b, i, 0, k);
      accept = (double)u * (double)qv < (double)pv;
    }
    if (!accept) first = min(first, i);
    if (probe) {
      float* pr = probe + ((long)b * (k + 1) + i) * 4;
      pr[0] = pv; pr[1] = qv; pr[2] = 0.f; pr[3] = 0.f;
    }
  }
  const int n = block_min_i(first);
  if (probe && threadIdx.x == 0) {
    float* pr = probe + ((long)b * (k + 1) + k) * 4;
    pr[0] = 0.f; pr[1] = 0.f; pr[2] = 0.f; pr[3] = 0.f;
  }
  for (int i = threadIdx.x; i <= k; i += kThreads) {
    if (i < n) out_tokens[(long)b * (k + 1) + i] = draft_tokens[(long)b * k + i];
    else if (i > n) out_tokens[(long)b * (k + 1) + i] = -1;
  }
  if (threadIdx.x == 0) {
    accepted_len[b] = n;
    ReqState st;
    st.n = n;
    st.mode = n < k ? kModeResidual : kModeBonus;
    st.mp = 0.f; st.mq = 0.f; st.sp = 0.0; st.sq = 0.0;
    st.pad[0] = st.pad[1] = 0.0;
    state[b] = st;
  }
}

// ---------------------------------------------------------------------------
// 2. Float64 normalisers of the rejected target / draft rows
// ---------------------------------------------------------------------------

// Load this thread's 16-element segment [j0, j0 + 16) of a row as floats;
// elements at or beyond V read as -inf (logits) / 0 (probabilities) via
// `fill`.
template <int DT, int NE>
__device__ __forceinline__ void load_segment(const void* row, long j0, int V, float fill,
                                             float (&x)[kSegPerThread]) {
#pragma unroll
  for (int g = 0; g < kSegPerThread / NE; ++g) {
    const long e0 = j0 + (long)g * NE;
    float t[NE];
    if (e0 + NE <= V) {
      load_group<DT, NE>(row, e0, t);
    } else {
#pragma unroll
      for (int e = 0; e < NE; ++e) t[e] = (e0 + e < V) ? load_elem<DT>(row, e0 + e) : fill;
    }
#pragma unroll
    for (int e = 0; e < NE; ++e) x[g * NE + e] = t[e];
  }
}

template <int DT, int NE>
__global__ __launch_bounds__(kThreads) void k_res_norm(
    const void* __restrict__ target, const void* __restrict__ draft, int k, int V, int C2,
    double inv_t, ReqState* __restrict__ state, double2* __restrict__ part2,
    unsigned* __restrict__ counters) {
  const int b = blockIdx.x / C2;
  const int chunk = blockIdx.x % C2;
  const ReqState st = state[b];
  if (st.mode != kModeResidual) return;  // uniform over the request's work-groups
  const int n = st.n;
  const long eb = Elems<DT>::kBytes;
  const void* prow = reinterpret_cast<const char*>(target) + ((long)b * (k + 1) + n) * V * eb;
  const void* qrow = reinterpret_cast<const char*>(draft) + ((long)b * k + n) * V * eb;
  const long j0 = (long)chunk * kResChunkElems + (long)threadIdx.x * kSegPerThread;
  float zp[kSegPerThread], zq[kSegPerThread];
  load_segment<DT, NE>(prow, j0, V, -INFINITY, zp);
  load_segment<DT, NE>(qrow, j0, V, -INFINITY, zq);
  const double mp = st.mp, mq = st.mq;
  double sp = 0.0, sq = 0.0;
#pragma unroll
  for (int e = 0; e < kSegPerThread; ++e) {
    sp += exp(((double)zp[e] - mp) * inv_t);
    sq += exp(((double)zq[e] - mq) * inv_t);
  }
  sp = block_sum_d(sp);
  sq = block_sum_d(sq);
  if (threadIdx.x == 0) part2[(long)b * C2 + chunk] = make_double2(sp, sq);
  if (!last_block_ticket(&counters[(long)b * kCountersPerReq + 1], (unsigned)C2)) return;
  if (threadIdx.x == 0) {
    double tp = 0.0, tq = 0.0;
    for (int cc = 0; cc < C2; ++cc) {
      const double2 v = part2[(long)b * C2 + cc];
      tp += v.x;
      tq += v.y;
    }
    state[b].sp = tp;
    state[b].sq = tq;
  }
}

// ---------------------------------------------------------------------------
// 3. Float64 residual / bonus weights, scan and inverse-CDF draw
// ---------------------------------------------------------------------------

enum WeightMode { kWResidual = 0, kWBonusOrP = 1 };

struct ChunkResult {
  double total;  // chunk total (value of the chunk's last running sum)
  int token;     // first element whose running sum exceeds thr, or INT_MAX
};

// Weights of one chunk for this work-group, their running sums, the chunk
// total, and (search) the first element j with P + running_sum_j > thr.
// Every chunk total and every searched running sum comes from this one
// function, so the pass that finds the chunk and the pass that searches it
// evaluate identical operations.
template <int DT, int NE, int KIND>
__device__ __attribute__((noinline)) ChunkResult chunk_pass(
    const void* prow, const void* qrow, int V, int chunk, int wmode, double mp, double mq,
    double inv_t, double rho, bool search, double P, double thr) {
  const long j0 = (long)chunk * kResChunkElems + (long)threadIdx.x * kSegPerThread;
  const float fill = KIND == 0 ? -INFINITY : 0.f;
  float zp[kSegPerThread], zq[kSegPerThread];
  load_segment<DT, NE>(prow, j0, V, fill, zp);
  if (wmode == kWResidual) load_segment<DT, NE>(qrow, j0, V, fill, zq);
  double w[kSegPerThread];
#pragma unroll
  for (int e = 0; e < kSegPerThread; ++e) {
    double we;
    if (KIND == 0) {
      const double ep = exp(((double)zp[e] - mp) * inv_t);
      if (wmode == kWResidual) {
        const double eq = exp(((double)zq[e] - mq) * inv_t);
        we = fmax(0.0, ep - rho * eq);
      } else {
        we = ep;
      }
    } else {
      we = (wmode == kWResidual) ? fmax(0.0, (double)zp[e] - (double)zq[e]) : (double)zp[e];
    }
    w[e] = we;
  }
  double tsum = 0.0;
#pragma unroll
  for (int e = 0; e < kSegPerThread; ++e) tsum += w[e];
  const double excl = block_exclusive_scan_d(tsum);
  // The chunk total is the running sum at the chunk's last element inside
  // the row, so the element that made the chunk qualify also qualifies here.
  const long j_last = min((long)(chunk + 1) * kResChunkElems, (long)V) - 1;
  __shared__ double s_total;
  int tok = INT_MAX;
  double run = 0.0;
#pragma unroll
  for (int e = 0; e < kSegPerThread; ++e) {
    run += w[e];
    const double local = excl + run;
    if (j0 + e == j_last) s_total = local;
    if (search && tok == INT_MAX && j0 + e <= j_last && P + local > thr)
      tok = static_cast<int>(j0 + e);
  }
  __syncthreads();
  ChunkResult res;
  res.total = s_total;
  res.token = search ? block_min_i(tok) : INT_MAX;
  return res;
}

template <int DT, int NE, int KIND>
__global__ __launch_bounds__(kThreads) void k_res_draw(
    const void* __restrict__ target, const void* __restrict__ draft, int k, int V, int C2,
    double inv_t, const float* __restrict__ uniforms, uint64_t seed, uint64_t ctr0,
    int32_t* __restrict__ out_tokens, float* __restrict__ probe,
    const ReqState* __restrict__ state, double2* __restrict__ part2,
    unsigned* __restrict__ counters) {
  const int b = blockIdx.x / C2;
  const int own = blockIdx.x % C2;
  const ReqState st = state[b];
  const int n = st.n;
  const long eb = Elems<DT>::kBytes;
  const void* prow = reinterpret_cast<const char*>(target) + ((long)b * (k + 1) + n) * V * eb;
  const void* qrow = st.mode == kModeResidual
                         ? reinterpret_cast<const char*>(draft) + ((long)b * k + n) * V * eb
                         : nullptr;
  const double rho = (KIND == 0 && st.mode == kModeResidual) ? st.sp / st.sq : 0.0;
  int wmode = st.mode == kModeResidual ? kWResidual : kWBonusOrP;
  const double2* pc = part2 + (long)b * C2;
  double2* pw = part2 + (long)b * C2;

  // Phases: 0 = own chunk total; 1 = fallback totals (zero residual);
  // 2 = search.  One call site of chunk_pass serves all of them.
  int phase = 0;
  int chunk = own;
  double P = 0.0, thr = 0.0, mass = 0.0;
  __shared__ int s_chunk;
  __shared__ double s_P, s_thr, s_mass;
  __shared__ int s_phase;
  for (;;) {
    const ChunkResult cr = chunk_pass<DT, NE, KIND>(prow, qrow, V, chunk, wmode, st.mp, st.mq,
                                                    inv_t, rho, phase == 2, P, thr);
    if (phase == 2) {
      if (threadIdx.x == 0) {
        const int t = (cr.token == INT_MAX) ? -1 : cr.token;
        out_tokens[(long)b * (k + 1) + n] = t;
        if (probe) probe[((long)b * (k + 1) + n) * 4 + 2] = (float)mass;
      }
      return;
    }
    if (phase == 0) {
      if (threadIdx.x == 0) pw[own].x = cr.total;
      if (!last_block_ticket(&counters[(long)b * kCountersPerReq + 2], (unsigned)C2)) return;
    } else {
      if (threadIdx.x == 0) pw[chunk].y = cr.total;
      __syncthreads();
      if (chunk + 1 < C2) {
        ++chunk;
        continue;
      }
    }
    // Cross-chunk prefix (sequential, float64) and the chunk holding the draw.
    if (threadIdx.x == 0) {
      const float u = get_uniform(uniforms, seed, ctr0, b, n, 1, k);
      double tot = 0.0;
      for (int cc = 0; cc < C2; ++cc) tot += (phase == 0) ? pc[cc].x : pc[cc].y;
      int next_phase = 2, cs = C2 - 1;
      double Pc = 0.0, th = (double)u * tot;
      if (phase == 0 && !(tot > 0.0)) {
        next_phase = 1;  // zero residual: draw from p_n instead
      } else {
        double run = 0.0;
        for (int cc = 0; cc < C2; ++cc) {
          const double wc = (phase == 0) ? pc[cc].x : pc[cc].y;
          if (run + wc > th) { cs = cc; break; }
          run += wc;
        }
        Pc = run;
      }
      if (phase == 0) {
        if (KIND == 0) s_mass = (st.mode == kModeResidual) ? tot / st.sp : 1.0;
        else s_mass = tot;
      }
      s_phase = next_phase;
      s_chunk = cs;
      s_P = Pc;
      s_thr = th;
    }
    __syncthreads();
    if (phase == 0) mass = s_mass;
    phase = s_phase;
    if (phase == 1) {
      wmode = kWBonusOrP;
      chunk = 0;
    } else {
      chunk = s_chunk;
      P = s_P;
      thr = s_thr;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Host launcher
// ---------------------------------------------------------------------------

static int row_chunks(int V) { return (V + kRowChunkElems - 1) / kRowChunkElems; }

static bool rows_aligned(const void* p, int V, int dtype) {
  const int eb = dtype == 1 ? 2 : 4;
  return (reinterpret_cast<uintptr_t>(p) % 16 == 0) && (((long)V * eb) % 16 == 0);
}

template <int DT, int NE>
static void launch_logits(const void* target, const void* draft, int B, int k, int V,
                          const int32_t* draft_tokens, const float* uniforms, uint64_t seed,
                          uint64_t ctr0, float temperature, int32_t* accepted_len,
                          int32_t* out_tokens, float* probe, char* w, const WsLayout& L,
                          hipStream_t s) {
  const int C1 = row_chunks(V);
  const int C2 = res_chunks(V);
  const float c = 1.4426950408889634f / temperature;
  const double inv_t = 1.0 / (double)temperature;
  auto* part = reinterpret_cast<MSPart*>(w + L.part1);
  auto* st = reinterpret_cast<ReqState*>(w + L.state);
  auto* p2 = reinterpret_cast<double2*>(w + L.part2);
  auto* cnt = reinterpret_cast<unsigned*>(w + L.count);
  const long R = 2L * k + 1;
  hipLaunchKernelGGL((k_row_stats<DT, NE>), dim3((unsigned)(B * R * C1)), dim3(kThreads), 0, s,
                     target, draft, k, V, C1, c, inv_t, draft_tokens, uniforms, seed, ctr0,
                     accepted_len, out_tokens, probe, part, st, cnt);
  if (k > 0)
    hipLaunchKernelGGL((k_res_norm<DT, NE>), dim3((unsigned)(B * C2)), dim3(kThreads), 0, s,
                       target, draft, k, V, C2, inv_t, st, p2, cnt);
  hipLaunchKernelGGL((k_res_draw<DT, NE, 0>), dim3((unsigned)(B * C2)), dim3(kThreads), 0, s,
                     target, draft, k, V, C2, inv_t, uniforms, seed, ctr0, out_tokens, probe,
                     st, p2, cnt);
}

hipError_t launch_sample(const void* target, const void* draft, int dtype, int kind, int B,
                         int k, int V, const int32_t* draft_tokens, const float* uniforms,
                         uint64_t seed, uint64_t counter0, float temperature,
                         int32_t* accepted_len, int32_t* out_tokens, float* probe, void* ws,
                         const WsLayout& L, hipStream_t s) {
  char* w = static_cast<char*>(ws);
  const bool vec = rows_aligned(target, V, dtype) && (k == 0 || rows_aligned(draft, V, dtype));
  if (kind == 1) {
    auto* st = reinterpret_cast<ReqState*>(w + L.state);
    auto* p2 = reinterpret_cast<double2*>(w + L.part2);
    auto* cnt = reinterpret_cast<unsigned*>(w + L.count);
    const int C2 = res_chunks(V);
    hipLaunchKernelGGL(k_accept_probs, dim3((unsigned)B), dim3(kThreads), 0, s,
                       static_cast<const float*>(target), static_cast<const float*>(draft), k, V,
                       draft_tokens, uniforms, seed, counter0, accepted_len, out_tokens, probe,
                       st);
    if (vec)
      hipLaunchKernelGGL((k_res_draw<0, 4, 1>), dim3((unsigned)(B * C2)), dim3(kThreads), 0, s,
                         target, draft, k, V, C2, 1.0, uniforms, seed, counter0, out_tokens,
                         probe, st, p2, cnt);
    else
      hipLaunchKernelGGL((k_res_draw<0, 1, 1>), dim3((unsigned)(B * C2)), dim3(kThreads), 0, s,
                         target, draft, k, V, C2, 1.0, uniforms, seed, counter0, out_tokens,
                         probe, st, p2, cnt);
    return hipGetLastError();
  }
  if (dtype == 1) {
    if (vec)
      launch_logits<1, 8>(target, draft, B, k, V, draft_tokens, uniforms, seed, counter0,
                          temperature, accepted_len, out_tokens, probe, w, L, s);
    else
      launch_logits<1, 1>(target, draft, B, k, V, draft_tokens, uniforms, seed, counter0,
                          temperature, accepted_len, out_tokens, probe, w, L, s);
  } else {
    if (vec)
      launch_logits<0, 4>(target, draft, B, k, V, draft_tokens, uniforms, seed, counter0,
                          temperature, accepted_len, out_tokens, probe, w, L, s);
    else
      launch_logits<0, 1>(target, draft, B, k, V, draft_tokens, uniforms, seed, counter0,
                          temperature, accepted_len, out_tokens, probe, w, L, s);
  }
  return hipGetLastError();
}

}  // namespace specv
