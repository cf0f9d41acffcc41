// Sampling chain verification for gfx950: the min(1, p/q) rule with
// residual resampling ("EAGLE-3 speculative decoding review", equations
// A(x) and p_residual in the section on whether a small draft hurts quality;
// the serving chapter's acceptance-rule section), stopping at the first
// rejection and drawing a bonus token when every draft passes (EAGLE-3
// review "Speculative Decoding" step 3; serving chapter "how it works").
//
// Logits path, two launches on the caller's stream:
//   1. k_row_stats: work-group (chunk, row) streams one chunk of one of the
//      request's 2k+1 rows (k+1 target, k draft) with 16-byte non-temporal
//      loads and reduces it to (max, sum 2^((x - max) c)), c = log2(e)/T, in
//      float32; it publishes the pair and takes the request's ticket.  The
//      request's last work-group merges the pairs (float64), evaluates every
//      acceptance ratio p_i(x_i)/q_i(x_i) from the gathered logits, finds the
//      first rejection n and writes the accepted prefix and the request state.
//   2. k_draw: work-group (request, chunk) over the row(s) the final token is
//      drawn from -- target and draft row n after a rejection, target row k
//      for the bonus -- in float64: the normaliser partials S_p, S_q and the
//      draw weights, evaluated at the float32 estimate rho32 of S_p/S_q with
//      their derivative in rho.  The request's last work-group forms the
//      float64 rho, moves every chunk total to it (linear in rho unless an
//      element sits at the kink of max(0, .), in which case the chunk is
//      recomputed), locates the chunk holding the inverse-CDF point and
//      searches it with the exact weights.
// Probabilities path (rows given as distributions): k_draw alone, each
// work-group first repeating the (gather-only) acceptance tests.
#include <climits>

#include "device_common.h"
#include "device_math.h"

namespace specv {

constexpr int kUnrollStats = kRowUnroll;

// An element whose two terms differ by less than this fraction (relative to
// rho32 e^{(y-mq)/T}) may change sides of max(0, .) between rho32 and the
// float64 rho; its chunk is then recomputed exactly.  rho32 is within about
// 1e-6 of rho.
constexpr double kKinkBand = 1e-5;

// Row r of request b: r <= k is target row r, r > k is draft row r-k-1.
template <int DT>
__device__ __forceinline__ const void* stat_row(const void* target, const void* draft, int b,
                                                int r, int k, int V) {
  const long eb = Elems<DT>::kBytes;
  if (r <= k)
    return reinterpret_cast<const char*>(target) + ((long)b * (k + 1) + r) * V * eb;
  return reinterpret_cast<const char*>(draft) + ((long)b * k + (r - k - 1)) * V * eb;
}

// ---------------------------------------------------------------------------
// 1. Row statistics and acceptance
// ---------------------------------------------------------------------------

// Streaming softmax statistic of a chunk: running maximum m and
// s = sum 2^(x c - mc) with mc = fl32(m c), the rounded product (each
// element costs one fused multiply-add; merges recompute mc from m, so its
// rounding cancels exactly).  Each group of NE terms is added in float32
// and the group sums in float64: a float32 running sum near 1 would absorb
// the many terms far below its last bit.
template <int NE>
__device__ __forceinline__ void ms_update(float& m, float& mc, double& s, const float (&x)[NE],
                                          float c) {
  float lm = x[0];
#pragma unroll
  for (int e = 1; e < NE; ++e) lm = fmaxf(lm, x[e]);
  if (lm > m) {  // rare after the first groups
    const float mcn = mul_rn(lm, c);
    s = (m == -INFINITY) ? 0.0 : s * (double)__builtin_amdgcn_exp2f(mc - mcn);
    m = lm;
    mc = mcn;
  }
  if (m == -INFINITY) return;  // only -inf so far
  float g = 0.f;
#pragma unroll
  for (int e = 0; e < NE; ++e) g += __builtin_amdgcn_exp2f(fmaf(x[e], c, -mc));
  s += (double)g;
}

// Merged maximum M and normaliser S = sum 2^(x c - fl32(M c)) (float64) of
// one row from its chunk partials, by one thread: each partial is loaded
// once and folded in.
__device__ __forceinline__ void merge_row_thread(const uint64_t* part, long base_idx, int C1,
                                                 float c, float& M, double& S) {
  M = -INFINITY;
  S = 0.0;
  for (int cc = 0; cc < C1; ++cc) {
    const uint64_t pp = ld_dev(&part[base_idx + cc]);
    const float m2 = unpack_lo(pp);
    const double s2 = (double)unpack_hi(pp);
    if (m2 == -INFINITY) continue;
    if (M == -INFINITY) {
      M = m2;
      S = s2;
      continue;
    }
    const float mn = fmaxf(M, m2);
    const double mcn = (double)mul_rn(mn, c);
    S = S * exp2((double)mul_rn(M, c) - mcn) + s2 * exp2((double)mul_rn(m2, c) - mcn);
    M = mn;
  }
}

template <int DT, int NE>
__global__ __launch_bounds__(kThreads) void k_row_stats(
    const void* __restrict__ target, const void* __restrict__ draft, int k, int V, int C1,
    float c, const int32_t* __restrict__ draft_tokens, const float* __restrict__ uniforms,
    uint64_t seed, uint64_t ctr0, int32_t* __restrict__ accepted_len,
    int32_t* __restrict__ out_tokens, float* __restrict__ probe, uint64_t* __restrict__ part,
    ReqState* __restrict__ state, unsigned* __restrict__ counters) {
  const int R = 2 * k + 1;
  const int chunk = blockIdx.x % C1;
  const long rowid = blockIdx.x / C1;
  const int b = static_cast<int>(rowid / R);
  const int r = static_cast<int>(rowid % R);
  {
    const void* rp = stat_row<DT>(target, draft, b, r, k, V);
    const long n_groups = V / NE;
    const long gpc = (n_groups + C1 - 1) / C1;
    const long g0 = (long)chunk * gpc;
    const long g1 = min(g0 + gpc, n_groups);
    float m = -INFINITY, mc = -INFINITY;
    double s = 0.0;
    long g = g0 + threadIdx.x;
    // Main loop: kUnrollStats loads issued back to back, no bounds branch.
    for (; g + (long)(kUnrollStats - 1) * kThreads < g1; g += (long)kThreads * kUnrollStats) {
      float x[kUnrollStats][NE];
#pragma unroll
      for (int u = 0; u < kUnrollStats; ++u)
        load_group<DT, NE, true>(rp, (g + (long)u * kThreads) * NE, x[u]);
#pragma unroll
      for (int u = 0; u < kUnrollStats; ++u) ms_update<NE>(m, mc, s, x[u], c);
    }
    for (; g < g1; g += kThreads) {
      float x[NE];
      load_group<DT, NE, true>(rp, g * NE, x);
      ms_update<NE>(m, mc, s, x, c);
    }
    block_reduce_ms(m, s, c);
    if (threadIdx.x == 0) st_dev(&part[rowid * C1 + chunk], pack2(m, (float)s));
  }
  if (!block_arrive(&counters[(long)b * kCountersPerReq + 0], (unsigned)(R * C1))) return;

  // ---- last work-group of request b: acceptance tests ----
  // Every row of the request is merged by its own thread (one round of
  // coherent loads) while the logits at the draft tokens are gathered; then
  // thread i tests draft i.
  __shared__ float s_m[2 * kMaxK + 1];
  __shared__ double s_s[2 * kMaxK + 1];
  for (int rr = threadIdx.x; rr < R; rr += kThreads) {
    float M;
    double S;
    merge_row_thread(part, ((long)b * R + rr) * C1, C1, c, M, S);
    s_m[rr] = M;
    s_s[rr] = S;
  }
  __syncthreads();
  int first = k;
  for (int i = threadIdx.x; i < k; i += kThreads) {
    const int x = draft_tokens[(long)b * k + i];
    float pv = 0.f, qv = 0.f;
    bool accept = false;
    if (x >= 0 && x < V) {
      const float zp = load_elem<DT>(stat_row<DT>(target, draft, b, i, k, V), x);
      const float zq = load_elem<DT>(stat_row<DT>(target, draft, b, k + 1 + i, k, V), x);
      // log2 p_i(x) and log2 q_i(x) from the row statistics
      const double lp = ((double)zp * c - (double)mul_rn(s_m[i], c)) - log2(s_s[i]);
      const double lq =
          ((double)zq * c - (double)mul_rn(s_m[k + 1 + i], c)) - log2(s_s[k + 1 + i]);
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
  const int n = block_min_i(first);
  for (int i = threadIdx.x; i <= k; i += kThreads) {
    if (i < n) out_tokens[(long)b * (k + 1) + i] = draft_tokens[(long)b * k + i];
    else if (i > n) out_tokens[(long)b * (k + 1) + i] = -1;
  }
  // State for the draw: maxima of target row n and (rejection) draft row n,
  // and the float32-based normaliser ratio of that pair.
  if (threadIdx.x == 0) {
    const float mp = s_m[n];
    const float mq = n < k ? s_m[k + 1 + n] : 0.f;
    // S relative to 2^(m c) instead of 2^fl32(m c): ratio of the pair.
    const double sp = s_s[n] * exp2((double)mul_rn(mp, c) - (double)mp * c);
    const double sq =
        n < k ? s_s[k + 1 + n] * exp2((double)mul_rn(mq, c) - (double)mq * c) : 1.0;
    accepted_len[b] = n;
    state[b] = ReqState{n, n < k ? kModeResidual : kModeBonus, mp, mq, sp / sq};
    if (probe) {
      float* pr = probe + ((long)b * (k + 1) + k) * 4;
      pr[0] = 0.f; pr[1] = 0.f; pr[2] = 0.f; pr[3] = 0.f;
    }
  }
}

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

// ---------------------------------------------------------------------------
// 2. Float64 draw pass
// ---------------------------------------------------------------------------

// NN consecutive elements from j0 as floats (NN a multiple of NE); elements
// at or beyond V read as `fill`.
template <int DT, int NE, int NN>
__device__ __forceinline__ void load_run(const void* row, long j0, int V, float fill,
                                         float (&x)[NN]) {
  static_assert(NN % NE == 0, "run length must be a multiple of the load width");
#pragma unroll
  for (int g = 0; g < NN / NE; ++g) {
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

// Float64 term of one element.  KIND 0 (logits): e^{(z - m)/T}, evaluated as
// 2^(t/64) with t = z c1 + c0, c1 = 64/(T ln 2), c0 = -m c1; KIND 1
// (probabilities): the value itself.
template <int KIND>
__device__ __forceinline__ double draw_term(float z, double c1, double c0, const double* tab) {
  return KIND == 0 ? exp2_64(fma((double)z, c1, c0), tab) : (double)z;
}

// Sums of one chunk by one wave (lane l covers the 16 elements from
// chunk * kDrawChunk + 16 l), reduced across the wave (valid in every lane):
//   v[0] = sum a, v[1] = sum b (a, b the target and draft terms),
//   v[2] = sum of the draw weights at rho32 (max(0, a - rho32 b), or a for
//          the bonus), v[3] = their derivative in rho (minus the sum of b
//          where the weight is positive), v[4] = 1 if an element lies within
//          the kink band of max(0, .).
template <int DT, int NE, int KIND>
__device__ __forceinline__ void wave_chunk_sums(const void* prow, const void* qrow, int V,
                                                int chunk, bool resid, double c1, double c0p,
                                                double c0q, double rho32, const double* tab,
                                                double (&v)[5]) {
  const int lane = threadIdx.x & 63;
  const long j0 = (long)chunk * kDrawChunk + (long)lane * kSegPerThread;
  const float fill = KIND == 0 ? -INFINITY : 0.f;
  float zp[kSegPerThread], zq[kSegPerThread];
  load_run<DT, NE, kSegPerThread>(prow, j0, V, fill, zp);
  if (resid) load_run<DT, NE, kSegPerThread>(qrow, j0, V, fill, zq);
#pragma unroll
  for (int q = 0; q < 5; ++q) v[q] = 0.0;
#pragma unroll
  for (int e = 0; e < kSegPerThread; ++e) {
    const double a = draw_term<KIND>(zp[e], c1, c0p, tab);
    v[0] += a;
    if (resid) {
      const double bq = draw_term<KIND>(zq[e], c1, c0q, tab);
      v[1] += bq;
      const double d = a - rho32 * bq;
      if (d > 0.0) {
        v[2] += d;
        v[3] -= bq;
      }
      if (KIND == 0 && bq > 0.0 && fabs(d) <= kKinkBand * rho32 * bq) v[4] = 1.0;
    } else {
      v[2] += a;
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
#pragma unroll
    for (int q = 0; q < 5; ++q) v[q] += shfl_xor_d(v[q], o);
  }
}

// kSearchPerThread consecutive elements of a chunk for this thread of a
// whole work-group: [chunk * kDrawChunk + kSearchPerThread t, ...).
template <int DT, int KIND>
__device__ __forceinline__ void search_terms(const void* prow, const void* qrow, int V, int chunk,
                                             bool resid, double c1, double c0p, double c0q,
                                             double rho, const double* tab,
                                             double (&w)[kSearchPerThread], long& j0) {
  j0 = (long)chunk * kDrawChunk + (long)threadIdx.x * kSearchPerThread;
  const float fill = KIND == 0 ? -INFINITY : 0.f;
  float zp[kSearchPerThread], zq[kSearchPerThread];
#pragma unroll
  for (int e = 0; e < kSearchPerThread; ++e) {
    zp[e] = (j0 + e < V) ? load_elem<DT>(prow, j0 + e) : fill;
    zq[e] = (resid && j0 + e < V) ? load_elem<DT>(qrow, j0 + e) : fill;
  }
  // Runs once per request on a cold instruction cache: rolled.
#pragma unroll 1
  for (int e = 0; e < kSearchPerThread; ++e) {
    const double a = draw_term<KIND>(zp[e], c1, c0p, tab);
    w[e] = resid ? fmax(0.0, a - rho * draw_term<KIND>(zq[e], c1, c0q, tab)) : a;
  }
}

// Exact chunk total with the float64 rho (for chunks flagged at the kink).
template <int DT, int KIND>
__device__ double chunk_total_exact(const void* prow, const void* qrow, int V, int chunk,
                                    double c1, double c0p, double c0q, double rho,
                                    const double* tab) {
  double w[kSearchPerThread];
  long j0;
  search_terms<DT, KIND>(prow, qrow, V, chunk, true, c1, c0p, c0q, rho, tab, w, j0);
  double t = 0.0;
#pragma unroll
  for (int e = 0; e < kSearchPerThread; ++e) t += w[e];
  return block_sum_d(t);
}

// Search one chunk with the exact weights.  Returns the first element whose
// running sum, added to the prefix P of the earlier chunks, exceeds thr,
// falling back to the chunk's last positive-weight element (reachable only
// through a last-bit difference between the chunk total used to locate it
// and the sums here).
template <int DT, int KIND>
__device__ int search_chunk(const void* prow, const void* qrow, int V, int chunk, bool resid,
                            double c1, double c0p, double c0q, double rho, double P, double thr,
                            const double* tab) {
  double w[kSearchPerThread];
  long j0;
  search_terms<DT, KIND>(prow, qrow, V, chunk, resid, c1, c0p, c0q, rho, tab, w, j0);
  double tsum = 0.0;
#pragma unroll
  for (int e = 0; e < kSearchPerThread; ++e) tsum += w[e];
  const double excl = block_exclusive_scan_d(tsum);
  int tok = INT_MAX, lastpos = -1;
  double run = 0.0;
#pragma unroll
  for (int e = 0; e < kSearchPerThread; ++e) {
    run += w[e];
    if (j0 + e < V) {
      if (w[e] > 0.0) lastpos = static_cast<int>(j0 + e);
      if (tok == INT_MAX && P + (excl + run) > thr) tok = static_cast<int>(j0 + e);
    }
  }
  tok = block_min_i(tok);
  lastpos = -block_min_i(-lastpos);
  return tok == INT_MAX ? lastpos : tok;
}

// Wait until this wave's earlier stores have completed.
__device__ __forceinline__ void wait_stores() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

template <int DT, int NE, int KIND>
__global__ __launch_bounds__(kThreads) void k_draw(
    const void* __restrict__ target, const void* __restrict__ draft, int k, int V, int C2,
    double inv_t, const int32_t* __restrict__ draft_tokens, const float* __restrict__ uniforms,
    uint64_t seed, uint64_t ctr0, int32_t* __restrict__ accepted_len,
    int32_t* __restrict__ out_tokens, float* __restrict__ probe,
    const ReqState* __restrict__ state, DrawPart* __restrict__ part,
    unsigned* __restrict__ counters) {
  const int G2 = (C2 + kDrawChunksPerGroup - 1) / kDrawChunksPerGroup;
  const int b = blockIdx.x / G2;
  const int grp = blockIdx.x % G2;
  __shared__ double tab[64];
  if (KIND == 0 && threadIdx.x < 64) tab[threadIdx.x] = kExp2Frac64[threadIdx.x];
  int n;
  double mp = 0.0, mq = 0.0, rho32 = 1.0;
  if (KIND == 0) {
    const ReqState st = state[b];
    n = st.n;
    mp = st.mp;
    mq = st.mq;
    rho32 = st.rho32;
  } else {
    n = accept_scan_probs(static_cast<const float*>(target), static_cast<const float*>(draft), b,
                          k, V, draft_tokens, uniforms, seed, ctr0, grp == 0, accepted_len,
                          out_tokens, probe);
  }
  __syncthreads();
  const bool resid = n < k;
  const double c1 = inv_t * kInvLn2x64, c0p = -mp * c1, c0q = -mq * c1;
  const long eb_bytes = Elems<DT>::kBytes;
  const void* prow =
      reinterpret_cast<const char*>(target) + ((long)b * (k + 1) + n) * V * eb_bytes;
  const void* qrow =
      resid ? reinterpret_cast<const char*>(draft) + ((long)b * k + n) * V * eb_bytes : nullptr;

  // ---- this work-group's chunks, one wave per chunk ----
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int i = 0; i < kDrawChunksPerWave; ++i) {
    const int cc = grp * kDrawChunksPerGroup + wave * kDrawChunksPerWave + i;
    if (cc >= C2) break;  // wave-uniform
    double v[5];
    wave_chunk_sums<DT, NE, KIND>(prow, qrow, V, cc, resid, c1, c0p, c0q, rho32, tab, v);
    if (lane == 0) {
      DrawPart* p = &part[(long)b * C2 + cc];
      st_dev_d(&p->sp, v[0]);
      st_dev_d(&p->sq, v[1]);
      st_dev_d(&p->w, v[2]);
      st_dev_d(&p->dq, v[3]);
      st_dev_d(&p->flag, v[4]);
    }
  }
  wait_stores();  // every wave's partials complete before the ticket below
  __syncthreads();
  if (!block_arrive(&counters[(long)b * kCountersPerReq + 1], (unsigned)G2)) return;

  // ---- last work-group of request b: exact rho, chunk totals, draw ----
  DrawPart* rp = part + (long)b * C2;
  __shared__ double s_rho, s_sp;
  {
    double v[5] = {0.0, 0.0, 0.0, 0.0, 0.0};
    for (int cc = threadIdx.x; cc < C2; cc += kThreads) {
      v[0] += ld_dev_d(&rp[cc].sp);
      v[1] += ld_dev_d(&rp[cc].sq);
    }
    block_sum_d5(v);
    if (threadIdx.x == 0) {
      s_sp = v[0];
      s_rho = (KIND == 0 && resid) ? v[0] / v[1] : 1.0;
    }
  }
  __syncthreads();
  const double rho = s_rho, sp_tot = s_sp;
  // Chunk totals at the exact rho: linear correction, or recomputation for
  // the (rare) chunks with an element at the kink.  Written back in place,
  // one chunk per thread.
  if (KIND == 0 && resid) {
    __shared__ int s_kink[kThreads];
    for (int base = 0; base < C2; base += kThreads) {
      const int cc = base + threadIdx.x;
      int kink = 0;
      if (cc < C2) {
        kink = ld_dev_d(&rp[cc].flag) > 0.0;
        if (!kink)
          st_dev_d(&rp[cc].w,
                   fmax(0.0, ld_dev_d(&rp[cc].w) + (rho - rho32) * ld_dev_d(&rp[cc].dq)));
      }
      s_kink[threadIdx.x] = kink;
      if (__syncthreads_count(kink) > 0) {
        for (int j = 0; j < kThreads && base + j < C2; ++j) {
          if (!s_kink[j]) continue;  // block-uniform
          const double wt =
              chunk_total_exact<DT, KIND>(prow, qrow, V, base + j, c1, c0p, c0q, rho, tab);
          if (threadIdx.x == 0) st_dev_d(&rp[base + j].w, fmax(0.0, wt));
        }
      }
      __syncthreads();
    }
  }
  // Prefix of the chunk totals (residual weights, or the target terms when
  // the residual is empty) by a tiled work-group scan: first the total, then
  // the chunk holding u * total.
  const float u = get_uniform(uniforms, seed, ctr0, b, n, 1, k);
  int mode = resid ? 0 : 1;  // 0: residual weights, 1: target terms
  double grand = 0.0;
  for (int pass = 0; pass < 2; ++pass) {
    double running = 0.0;
    for (int base = 0; base < C2; base += kThreads) {
      const int cc = base + threadIdx.x;
      const double wc = cc < C2 ? (mode == 0 ? ld_dev_d(&rp[cc].w) : ld_dev_d(&rp[cc].sp)) : 0.0;
      running += block_sum_d(wc);
    }
    grand = running;
    if (!(grand > 0.0) && mode == 0) mode = 1;  // zero residual: draw from p_n
    else break;
  }
  const double thr = (double)u * grand;
  __shared__ double s_P;
  __shared__ int s_cs;
  if (threadIdx.x == 0) { s_cs = C2 - 1; s_P = 0.0; }
  {
    double running = 0.0;
    int found = 0;
    for (int base = 0; base < C2 && !found; base += kThreads) {
      const int cc = base + threadIdx.x;
      const double wc = cc < C2 ? (mode == 0 ? ld_dev_d(&rp[cc].w) : ld_dev_d(&rp[cc].sp)) : 0.0;
      const double excl = running + block_exclusive_scan_d(wc);
      const int hit = (cc < C2 && excl + wc > thr) ? cc : INT_MAX;
      const int first_hit = block_min_i(hit);
      if (first_hit != INT_MAX) {
        if (cc == first_hit) { s_cs = cc; s_P = excl; }
        found = 1;
      } else if (cc == C2 - 1) {
        s_P = excl;  // no hit (last-bit case): search the last chunk from its prefix
      }
      running += block_sum_d(wc);
    }
    __syncthreads();
  }
  int t = search_chunk<DT, KIND>(prow, qrow, V, s_cs, mode == 0, c1, c0p, c0q, rho, s_P, thr,
                                 tab);
  if (threadIdx.x == 0) {
    if (!(grand > 0.0)) t = -1;  // rows without mass (invalid input)
    out_tokens[(long)b * (k + 1) + n] = t;
    if (probe) {
      // Mass of the distribution drawn from, in probability units.
      double mass;
      if (KIND == 0) mass = resid ? (mode == 0 ? grand / sp_tot : 0.0) : 1.0;
      else mass = mode == 0 ? grand : (resid ? 0.0 : grand);
      probe[((long)b * (k + 1) + n) * 4 + 2] = (float)mass;
    }
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
static hipError_t launch_logits(const void* target, const void* draft, int B, int k, int V,
                          const int32_t* draft_tokens, const float* uniforms, uint64_t seed,
                          uint64_t ctr0, float temperature, int32_t* accepted_len,
                          int32_t* out_tokens, float* probe, char* w, const WsLayout& L,
                          hipStream_t s) {
  const int C1 = row_chunks(V);
  const int C2 = res_chunks(V);
  const float c = 1.4426950408889634f / temperature;
  const double inv_t = 1.0 / (double)temperature;
  auto* p1 = reinterpret_cast<uint64_t*>(w + L.part1);
  auto* st = reinterpret_cast<ReqState*>(w + L.state);
  auto* p2 = reinterpret_cast<DrawPart*>(w + L.part2);
  auto* cnt = reinterpret_cast<unsigned*>(w + L.count);
  const long R = 2L * k + 1;
  hipError_t e = launch_timed(kProfRowPass, &k_row_stats<DT, NE>,
                             dim3((unsigned)(B * R * C1)), dim3(kThreads), s, target, draft, k,
                             V, C1, c, draft_tokens, uniforms, seed, ctr0, accepted_len,
                             out_tokens, probe, p1, st, cnt);
  if (e != hipSuccess) return e;
  const int G2 = (C2 + kDrawChunksPerGroup - 1) / kDrawChunksPerGroup;
  return launch_timed(kProfDraw, &k_draw<DT, NE, 0>, dim3((unsigned)(B * G2)), dim3(kThreads), s,
                      target, draft, k, V, C2, inv_t, draft_tokens, uniforms, seed, ctr0,
                      accepted_len, out_tokens, probe, (const ReqState*)st, p2, cnt);
}

template <int NE>
static hipError_t launch_probs(const void* target, const void* draft, int B, int k, int V,
                         const int32_t* draft_tokens, const float* uniforms, uint64_t seed,
                         uint64_t ctr0, int32_t* accepted_len, int32_t* out_tokens,
                         float* probe, char* w, const WsLayout& L, hipStream_t s) {
  const int C2 = res_chunks(V);
  auto* st = reinterpret_cast<ReqState*>(w + L.state);
  auto* p2 = reinterpret_cast<DrawPart*>(w + L.part2);
  auto* cnt = reinterpret_cast<unsigned*>(w + L.count);
  const int G2 = (C2 + kDrawChunksPerGroup - 1) / kDrawChunksPerGroup;
  return launch_timed(kProfDraw, &k_draw<0, NE, 1>, dim3((unsigned)(B * G2)), dim3(kThreads), s,
                      target, draft, k, V, C2, 1.0, draft_tokens, uniforms, seed, ctr0,
                      accepted_len, out_tokens, probe, (const ReqState*)st, p2, cnt);
}

hipError_t launch_sample(const void* target, const void* draft, int dtype, int kind, int B,
                         int k, int V, const int32_t* draft_tokens, const float* uniforms,
                         uint64_t seed, uint64_t counter0, float temperature,
                         int32_t* accepted_len, int32_t* out_tokens, float* probe, void* ws,
                         const WsLayout& L, hipStream_t s) {
  char* w = static_cast<char*>(ws);
  const bool vec = rows_aligned(target, V, dtype) && (k == 0 || rows_aligned(draft, V, dtype));
  if (kind == 1) {
    if (vec)
      return launch_probs<4>(target, draft, B, k, V, draft_tokens, uniforms, seed, counter0,
                      accepted_len, out_tokens, probe, w, L, s);
    else
      return launch_probs<1>(target, draft, B, k, V, draft_tokens, uniforms, seed, counter0,
                      accepted_len, out_tokens, probe, w, L, s);
  } else if (dtype == 1) {
    if (vec)
      return launch_logits<1, 8>(target, draft, B, k, V, draft_tokens, uniforms, seed, counter0,
                          temperature, accepted_len, out_tokens, probe, w, L, s);
    else
      return launch_logits<1, 1>(target, draft, B, k, V, draft_tokens, uniforms, seed, counter0,
                          temperature, accepted_len, out_tokens, probe, w, L, s);
  } else {
    if (vec)
      return launch_logits<0, 4>(target, draft, B, k, V, draft_tokens, uniforms, seed, counter0,
                          temperature, accepted_len, out_tokens, probe, w, L, s);
    else
      return launch_logits<0, 1>(target, draft, B, k, V, draft_tokens, uniforms, seed, counter0,
                          temperature, accepted_len, out_tokens, probe, w, L, s);
  }
}

}  // namespace specv
