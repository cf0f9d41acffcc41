// Sampling chain verification for gfx950: the min(1, p/q) rule with
// residual resampling ("EAGLE-3 speculative decoding review", equations
// A(x) and p_residual in the section on whether a small draft hurts quality;
// the serving chapter's acceptance-rule section), stopping at the first
// rejection and drawing a bonus token when every draft passes (EAGLE-3
// review "Speculative Decoding" step 3; serving chapter "how it works").
//
// Logits path.  Three kinds of work-group:
//   1. row pass: work-group (chunk, row) streams one chunk of one of the
//      request's 2k+1 rows (k+1 target, k draft) with 16-byte non-temporal
//      loads and reduces it to (max, sum 2^((x - max) c)), c = log2(e)/T, in
//      float32, publishing the pair (and, in the chunk holding the row's
//      draft token, the logit there).
//   2. acceptance tests, one wave per request: merge the pairs (float64),
//      evaluate each acceptance ratio p_i(x_i)/q_i(x_i) from the gathered
//      logits, find the first rejection n, write the accepted prefix and the
//      draw state.
//   3. draw: work-group (request, chunk group) over the row(s) the final
//      token is drawn from -- target and draft row n after a rejection,
//      target row k for the bonus -- in float64: the normaliser partials
//      S_p, S_q and the draw weights, evaluated at the float32 estimate rho32
//      of S_p/S_q with their derivative in rho.  The request's last
//      work-group forms the float64 rho, moves every chunk total to it
//      (linear in rho unless an element sits at the kink of max(0, .), in
//      which case the chunk is recomputed), locates the chunk holding the
//      inverse-CDF point and searches it with the exact weights.
// By default all run in one launch (k_sample_one): rows in position order,
// so that most requests are decided by their early positions while the
// rows of later ones stream (the grid order and its waits are described at
// the kernel).  The two-launch form (k_row_stats, then k_draw) computes the
// same thing, with the acceptance tests in the request's last row-pass
// work-group (by ticket).
// Rows given as probabilities have a kernel of their own (probs.hip).
#include <algorithm>
#include <atomic>
#include <mutex>

#include "sample_device.h"

#ifndef SPEC_GATE_GBPS
#define SPEC_GATE_GBPS 3300
#endif

namespace specv {

// Early-exit schedule: the rows of early positions after position 0 first
// wait about as long as position 0's rows take to stream at this rate (GB/s),
// so that position 0 has the memory system to itself and most requests are
// decided before those rows start (a row of a decided request then stops
// after its first batch).  Measured at B = 64, k = 8, V = 128256 bf16 (mean
// accepted 0.57): no wait 55.2 us; 2300, 2700, 3000, 3300, 3600, 4000 GB/s
// 55.9, 54.1, 53.1, 53.0, 53.4, 55.5 us.  Waiting instead for each request's
// position-0 outcome (polling a progress word the finalizer publishes) gave
// 54.3-54.7 us: the polls and the extra stores cost more than they save.
// Workloads whose requests mostly accept position 0 gain nothing from the
// wait and lose part of the memory system to it for its duration.
constexpr long kGateGBps = SPEC_GATE_GBPS;

// Statistic of chunk `chunk` (of C1) of row r of request b: the sweep, the
// block reduction, and thread 0's coherent stores of the (reference, sum)
// pair and, in the chunk holding the row's draft token, of the logit there.
// Every thread returns.  WATCH: the sweep stops early once the request's
// ready slot (`watch`) shows it stopped before this row's position; then
// nothing is stored.  Returns, in thread 0, whether the pair was stored.
template <int DT, int NE, bool WATCH = false>
__device__ __forceinline__ bool row_chunk_stat(int b, int r, int chunk,
                                               const void* __restrict__ target,
                                               const void* __restrict__ draft, int k, int V,
                                               int C1, float c,
                                               const int32_t* __restrict__ draft_tokens,
                                               uint64_t* __restrict__ part,
                                               float* __restrict__ zrow,
                                               const uint64_t* watch = nullptr,
                                               bool precheck = false) {
  const int R = 2 * k + 1;
  const long rowid = (long)b * R + r;
  const void* rp = stat_row<DT>(target, draft, b, r, k, V);
  // The draft token this row is tested at (target row i and draft row i
  // share x_i; the bonus row k has none), loaded now and used after the
  // sweep.
  const int tpos = r < k ? r : (r > k ? r - k - 1 : -1);
  int x = -1;
  if (threadIdx.x == 0 && tpos >= 0) x = draft_tokens[(long)b * k + tpos];
  const long n_groups = V / NE;
  const long gpc = (n_groups + C1 - 1) / C1;
  const long g0 = (long)chunk * gpc;
  const long g1 = min(g0 + gpc, n_groups);
  float m = -INFINITY, mc = -INFINITY;
  double s = 0.0;
  if constexpr (NE == 1)
    stats_sweep_scalar<DT>(rp, g0, g1, c, m, mc, s);
  else
    stats_sweep<DT, kThreads, WATCH>(rp, static_cast<uint32_t>((long)V * Elems<DT>::kBytes), g0,
                                     g1, c, m, mc, s, threadIdx.x, watch,
                                     r <= k ? r : r - k - 1, precheck);
  // The chunk that holds the token also publishes the logit there.
  const bool own = x >= 0 && x < V && (long)x >= g0 * NE && (long)x < g1 * NE;
  float zx = 0.f;
  if (own) zx = load_elem<DT>(rp, x);
  block_reduce_ms(m, s, c);
  // m = +inf: a wave stopped early (inputs are finite or -inf)
  const bool store = !WATCH || m != INFINITY;
  if (threadIdx.x == 0 && store) {
    st_dev(&part[rowid * C1 + chunk], pack2(m, (float)s));
    if (own) st_dev_f(&zrow[rowid], zx);
  }
  return store;
}

// Position i of request b, by one lane, from the published row statistics:
// the token, the two token logits and the chunk partials of target row i
// and draft row i are loaded in one round and the rows merged.  With
// e_p = z c - fl(M_p c) (z the target logit at x_i) and e_q likewise,
// p_i(x_i) / q_i(x_i) = 2^(e_p - e_q) S_q / S_p, one exp2.  Position k, the
// bonus row, has no test: it reports acceptance.  mp, mq and rho are the
// draw state if the request stops here (target row k for the bonus).
struct PosResult {
  bool accept;
  float pv, qv;  // p_i(x_i), q_i(x_i) when asked for, else 0
  float mp, mq;  // references of the rows drawn from
  double rho;    // S_p / S_q of those rows from the float32 statistics
};
__device__ __forceinline__ PosResult test_position(
    int b, int i, int k, int V, int C1, float c, const int32_t* __restrict__ draft_tokens,
    const float* __restrict__ uniforms, uint64_t seed, uint64_t ctr0,
    const uint64_t* __restrict__ part, const float* __restrict__ zrow, bool want_probe) {
  const int R = 2 * k + 1;
  const bool draft_pos = i < k;
  int x = -1;
  float zp = 0.f, zq = 0.f;
  if (draft_pos) {
    x = draft_tokens[(long)b * k + i];
    zp = ld_dev_f(&zrow[(long)b * R + i]);
    zq = ld_dev_f(&zrow[(long)b * R + k + 1 + i]);
  }
  float Mp, Mq;
  double Sp, Sq;
  merge_two_rows(part, ((long)b * R + i) * C1, ((long)b * R + k + 1 + i) * C1, draft_pos, C1, c,
                 Mp, Sp, Mq, Sq);
  PosResult res{true, 0.f, 0.f, Mp, 0.f, 1.0};
  if (!draft_pos) return res;
  res.accept = false;
  if (x >= 0 && x < V) {
    const double ep = (double)zp * c - (double)mul_rn(Mp, c);
    const double eq = (double)zq * c - (double)mul_rn(Mq, c);
    const double ratio = exp2(ep - eq) * (Sq / Sp);
    const float u = get_uniform(uniforms, seed, ctr0, b, i, 0, k);
    res.accept = (double)u < ratio;
    if (want_probe) {
      res.pv = (float)(exp2(ep) / Sp);
      res.qv = (float)(exp2(eq) / Sq);
    }
  }
  if (!res.accept) {
    // S_p / S_q with both sums taken relative to 2^(M c) instead of
    // 2^fl32(M c), rounded to float: it travels packed in the one-launch
    // kernel's ready slot, and both forms use the same value.
    res.mq = Mq;
    res.rho = (double)(float)(Sp / Sq *
                              exp2(((double)mul_rn(Mp, c) - (double)Mp * c) -
                                   ((double)mul_rn(Mq, c) - (double)Mq * c)));
  }
  return res;
}

// probe[b, i, 0, 1, 3] of a tested position (i < k): p, q and 0.
__device__ __forceinline__ void write_probe_position(float* probe, int b, int i, int k,
                                                     const PosResult& r) {
  float* pr = probe + ((long)b * (k + 1) + i) * 4;
  pr[0] = r.pv;
  pr[1] = r.qv;
  pr[3] = 0.f;
}

// Outputs of the acceptance tests once n is known, by one wave of the
// request's last draw work-group (the one work-group that writes them):
// accepted_len[b], the accepted prefix, the -1 padding, probe[b, i, 2] = 0
// for i != n (probe[b, n, 2] is written with the drawn token) and the other
// probe entries of the bonus row k.
__device__ __forceinline__ void write_accept_outputs(int b, int k, int n,
                                                     const int32_t* __restrict__ draft_tokens,
                                                     int32_t* __restrict__ accepted_len,
                                                     int32_t* __restrict__ out_tokens,
                                                     float* __restrict__ probe) {
  const int lane = threadIdx.x & 63;
  for (int i = lane; i <= k; i += kWaveSize) {
    if (i < n) out_tokens[(long)b * (k + 1) + i] = draft_tokens[(long)b * k + i];
    else if (i > n) out_tokens[(long)b * (k + 1) + i] = -1;
    if (probe && i != n) probe[((long)b * (k + 1) + i) * 4 + 2] = 0.f;
  }
  if (lane == 0) {
    accepted_len[b] = n;
    if (probe) {
      float* pr = probe + ((long)b * (k + 1) + k) * 4;
      pr[0] = 0.f;
      pr[1] = 0.f;
      pr[3] = 0.f;
    }
  }
}

// Acceptance tests of request b by one wave once every row is complete.
// Lane i handles position i (and i + 64, ...); each lane keeps the draw
// state of its first rejected position (or of the bonus row), and after the
// wave minimum the owner of the first rejection supplies it.  Returns the
// state in every lane and stores the probe values p_i(x_i), q_i(x_i) of the
// tested positions (the request's draw writes the other outputs).
__device__ __forceinline__ ReqState finalize_request(
    int b, int k, int V, int C1, float c, const int32_t* __restrict__ draft_tokens,
    const float* __restrict__ uniforms, uint64_t seed, uint64_t ctr0,
    const uint64_t* __restrict__ part, const float* __restrict__ zrow,
    float* __restrict__ probe) {
  const int lane = threadIdx.x & 63;
  const bool want_probe = probe != nullptr;
  int first = k;
  float cand_mp = 0.f, cand_mq = 0.f;  // draw state of this lane's hand-over row
  double cand_rho = 1.0;
  for (int i = lane; i <= k; i += kWaveSize) {
    const PosResult r = test_position(b, i, k, V, C1, c, draft_tokens, uniforms, seed, ctr0, part,
                                      zrow, want_probe);
    if (first == k && (!r.accept || i == k)) {
      if (!r.accept) first = i;
      cand_mp = r.mp;
      cand_mq = r.mq;
      cand_rho = r.rho;
    }
    if (want_probe && i < k) write_probe_position(probe, b, i, k, r);
  }
  const int n = wave_min_i(first);
  const int owner = n & (kWaveSize - 1);  // the lane that handled position n
  ReqState st;
  st.n = n;
  st.mode = n < k ? kModeResidual : kModeBonus;
  st.mp = __shfl(cand_mp, owner, 64);
  st.mq = __shfl(cand_mq, owner, 64);
  st.rho32 = __shfl(cand_rho, owner, 64);
  return st;
}

// Whether every chunk of the rows of position i of request b (target row i,
// and draft row i for i < k) carries this call's completion tag.
__device__ __forceinline__ bool position_complete(const uint64_t* __restrict__ flags, int b, int i,
                                                  int k, int C1, uint64_t tag) {
  const long R = 2L * k + 1;
  const long tr = ((long)b * R + i) * C1;
  const long dr = ((long)b * R + k + 1 + i) * C1;
  bool have = true;
  for (int ch = 0; ch < C1; ++ch) {
    have &= ld_dev(&flags[tr + ch]) == tag;
    if (i < k) have &= ld_dev(&flags[dr + ch]) == tag;
  }
  return have;
}

// Acceptance tests of request b by one wave while the rows still stream
// (one-launch kernel, rows in position order), from position `base` (every
// earlier one tested and accepted) up to, not including, `limit`.  Each round
// takes the positions whose rows are complete, tests that prefix, and stops
// at the first rejection, or after the bonus row k; rows past that point are
// never waited for.  kDecided: `st` holds the state.  kDeferred: every
// position below `limit` was accepted and position k lies beyond it.
// kTimedOut: the wait bound was reached.  `tested` is the number of
// positions tested (whose probe values were written, with a probe).
enum { kDecided = 0, kDeferred = 1, kTimedOut = 2 };
__device__ __forceinline__ int finalize_progressive(
    int b, int k, int V, int C1, float c, int base, int limit,
    const int32_t* __restrict__ draft_tokens, const float* __restrict__ uniforms, uint64_t seed,
    uint64_t ctr0, const uint64_t* __restrict__ part, const float* __restrict__ zrow,
    const uint64_t* __restrict__ flags, uint64_t tag, float* __restrict__ probe, ReqState& st,
    int& tested, long spin_limit) {
  const int lane = threadIdx.x & 63;
  const bool want_probe = probe != nullptr;
  const int end = min(limit, k + 1);
  tested = base;
  for (long spin = 0; spin < spin_limit; ++spin) {
    if (base >= end) return kDeferred;
    const int i = base + lane;
    const bool have = i < end && position_complete(flags, b, i, k, C1, tag);
    const uint64_t hm = __ballot(have);
    const int m = ~hm == 0 ? kWaveSize : __builtin_ctzll(~hm);  // complete prefix
    if (m == 0) {
      if (spin < 4) __builtin_amdgcn_s_sleep(2);
      else __builtin_amdgcn_s_sleep(32);
      continue;
    }
    PosResult r{true, 0.f, 0.f, 0.f, 0.f, 1.0};
    if (lane < m)
      r = test_position(b, i, k, V, C1, c, draft_tokens, uniforms, seed, ctr0, part, zrow,
                        want_probe);
    if (want_probe && lane < m && i < k) write_probe_position(probe, b, i, k, r);
    tested = base + m;
    const uint64_t rm = __ballot(lane < m && !r.accept);
    if (rm != 0 || base + m > k) {
      const int owner = rm != 0 ? __builtin_ctzll(rm) : k - base;
      const int n = base + owner;
      st.n = n;
      st.mode = n < k ? kModeResidual : kModeBonus;
      st.mp = __shfl(r.mp, owner, 64);
      st.mq = __shfl(r.mq, owner, 64);
      st.rho32 = __shfl(r.rho, owner, 64);
      return kDecided;
    }
    base += m;
  }
  return kTimedOut;
}

// Publishes a decided state in request b's ready slot (lane 0 of the
// deciding wave).
__device__ __forceinline__ void publish_state(unsigned* counters, int b, const ReqState& st) {
  uint64_t w0, w1;
  pack_state(st, w0, w1);
  uint64_t* slot = ready_slot(counters, b);
  st_dev(&slot[0], w0);
  st_dev(&slot[1], w1);
}

// Verdict word of request b's early acceptance tests (one-launch kernel):
// 0 until they end; then kVerdictDecided | tested << 2 (the state is in the
// ready slot, `tested` positions have probe values), kVerdictDeferred |
// next << 2 (positions from `next` on remain to be tested) or
// kVerdictFailed (the wait for the rows gave up).  The request's first draw
// work-group reads it and resets it.
constexpr unsigned kVerdictDecided = 1, kVerdictDeferred = 2, kVerdictFailed = 3;
__device__ __forceinline__ unsigned* verdict_word(unsigned* counters, int b) {
  return &counters[handover_pos(b) + kVerdictWord];
}

// Early acceptance tests of request b, by one wave of a finalizer
// work-group, over the positions whose rows precede the finalizers in the
// grid (`limit` of them).
__device__ __forceinline__ void early_finalize(
    int b, int k, int V, int C1, float c, int limit, const int32_t* __restrict__ draft_tokens,
    const float* __restrict__ uniforms, uint64_t seed, uint64_t ctr0,
    const uint64_t* __restrict__ part, const float* __restrict__ zrow,
    const uint64_t* __restrict__ flags, uint64_t tag, float* __restrict__ probe,
    unsigned* __restrict__ counters, long spin_limit) {
  // This wave decides when the request's draw can start: it issues first.
  __builtin_amdgcn_s_setprio(3);
  ReqState st;
  int tested = 0;
  const int res = finalize_progressive(b, k, V, C1, c, 0, limit, draft_tokens, uniforms, seed,
                                       ctr0, part, zrow, flags, tag, probe, st, tested,
                                       spin_limit);
  if ((threadIdx.x & 63) != 0) return;
  unsigned verdict;
  if (res == kDecided) {
    publish_state(counters, b, st);
    verdict = kVerdictDecided | (unsigned)tested << 2;
  } else if (res == kDeferred) {
    verdict = kVerdictDeferred | (unsigned)tested << 2;
  } else {  // the rows never appeared: the request fails loudly
    note_give_up(counters);
    verdict = kVerdictFailed;
  }
  __hip_atomic_store(verdict_word(counters, b), verdict, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

// One thread waits until the verdict word is set, returns it and resets it.
// 0 if the bound (`spin_limit` polls) is reached.
__device__ __forceinline__ unsigned take_verdict(unsigned* word, long spin_limit) {
  for (long spin = 0; spin < spin_limit; ++spin) {
    const unsigned v = __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (v != 0) {
      __hip_atomic_store(word, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return v;
    }
    if (spin < 4) __builtin_amdgcn_s_sleep(2);
    else __builtin_amdgcn_s_sleep(32);
  }
  return 0;
}

// Probe values of the positions from `from` on that the progressive tests
// did not reach (they follow the first rejection), by one wave, each once
// its rows are complete.
__device__ __forceinline__ void probe_remaining(
    int b, int k, int V, int C1, float c, int from, const int32_t* __restrict__ draft_tokens,
    const float* __restrict__ uniforms, uint64_t seed, uint64_t ctr0,
    const uint64_t* __restrict__ part, const float* __restrict__ zrow,
    const uint64_t* __restrict__ flags, uint64_t tag, float* __restrict__ probe,
    unsigned* __restrict__ counters, long spin_limit) {
  const int lane = threadIdx.x & 63;
  for (int base = from; base < k; base += kWaveSize) {
    const int i = base + lane;
    bool done = i >= k;
    for (long spin = 0; spin < spin_limit; ++spin) {
      if (!done && position_complete(flags, b, i, k, C1, tag)) {
        const PosResult r = test_position(b, i, k, V, C1, c, draft_tokens, uniforms, seed, ctr0,
                                          part, zrow, true);
        write_probe_position(probe, b, i, k, r);
        done = true;
      }
      if (__ballot(!done) == 0) break;
      __builtin_amdgcn_s_sleep(32);
    }
    if (__ballot(!done) != 0) {  // these rows never appeared: the call fails loudly
      if (lane == 0) note_give_up(counters);
      return;
    }
  }
}

// Row-pass grid of the one-launch kernel, in position order: for each
// position i = 0..k-1 every request's target row i and draft row i (C1
// chunks each), then every request's bonus row k.  Requests are decided by
// the rows of the positions up to their first rejection, so most are
// decided early in the pass and their draws overlap the rest of it.
__device__ __forceinline__ void position_major_row(long bid, int B, int k, int C1, int& b,
                                                   int& r, int& chunk) {
  const long per_pos = (long)B * 2 * C1;
  if (bid < (long)k * per_pos) {
    const int pos = static_cast<int>(bid / per_pos);
    const long rem = bid % per_pos;
    b = static_cast<int>(rem / (2 * C1));
    const int rem2 = static_cast<int>(rem % (2 * C1));
    r = rem2 < C1 ? pos : k + 1 + pos;
    chunk = rem2 % C1;
  } else {
    const long rem = bid - (long)k * per_pos;
    b = static_cast<int>(rem / C1);
    r = k;
    chunk = static_cast<int>(rem % C1);
  }
}

// Row pass of one work-group: block `bid` of the row-pass grid.
// Two-launch form (rows in request order): the request's last work-group
// (by ticket) runs the acceptance tests on one wave and stores the draw
// state.  One-launch kernel (rows in position order): the work-group tags
// its chunk complete once its pair is published, and the request's first
// draw work-group takes it from there.
// `withhold` (test only): the work-group of request 0, target row 0, chunk 0
// publishes its pair but never its completion tag.
template <int DT, int NE, bool EXIT = false>
__device__ __forceinline__ void row_block(
    long bid, bool one_launch, bool late, int B, const void* __restrict__ target,
    const void* __restrict__ draft, int k, int V, int C1, float c,
    const int32_t* __restrict__ draft_tokens, const float* __restrict__ uniforms, uint64_t seed,
    uint64_t ctr0, float* __restrict__ probe, uint64_t* __restrict__ part,
    float* __restrict__ zrow, uint64_t* __restrict__ flags, uint64_t tag,
    ReqState* __restrict__ state, unsigned* __restrict__ counters, bool withhold = false,
    int gate_ticks = 0) {
  const int R = 2 * k + 1;
  int b, r, chunk;
  if (one_launch) {
    position_major_row(bid, B, k, C1, b, r, chunk);
  } else {
    chunk = static_cast<int>(bid % C1);
    b = static_cast<int>(bid / C1 / R);
    r = static_cast<int>(bid / C1 % R);
  }
  if (EXIT && one_launch && !late && r != 0 && r != k + 1) {  // work-group-uniform
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    while (__builtin_amdgcn_s_memrealtime() - t0 < (uint64_t)gate_ticks)
      __builtin_amdgcn_s_sleep(8);
  }
  // Early exit: rows after position 0 stop once the request is decided
  // before their position (no probe values are asked for then).  Rows after
  // the early positions (`late`) look before their second batch: most of
  // their requests are decided by the time they start.
  const bool stored =
      EXIT && (r <= k ? r : r - k - 1) > 0
          ? row_chunk_stat<DT, NE, true>(b, r, chunk, target, draft, k, V, C1, c, draft_tokens,
                                         part, zrow, ready_slot(counters, b),
                                         late || gate_ticks > 0)
          : row_chunk_stat<DT, NE>(b, r, chunk, target, draft, k, V, C1, c, draft_tokens, part,
                                   zrow);
  if (one_launch) {
    // The tag follows the pair (and logit) once they are complete.
    if (threadIdx.x == 0 && stored && !(withhold && b == 0 && r == 0 && chunk == 0)) {
      wait_stores();  // the thread that stored them
      st_dev(&flags[((long)b * R + r) * C1 + chunk], tag);
    }
    return;
  }
  if (threadIdx.x >= kWaveSize) return;  // wave 0 finishes the work-group
  if (!wave_arrive(&counters[(long)b * kCountersPerReq + 0], (unsigned)(R * C1))) return;
  // ---- last work-group of request b, one wave: acceptance tests ----
  // The other waves of this compute unit stream rows; this one decides when
  // the request's draw can start: it issues first.
  __builtin_amdgcn_s_setprio(3);
  const ReqState st = finalize_request(b, k, V, C1, c, draft_tokens, uniforms, seed, ctr0, part,
                                       zrow, probe);
  if ((threadIdx.x & 63) == 0) st_dev_state(&state[b], st);
}

// How a draw work-group learns its request's state.
enum {
  kStateStored = 0,  // from the state array, written by an earlier launch
  kStateSlot = 1,    // one-launch hand-over: verdict word, then the ready slot
};

// Row-pass outputs the request's first draw work-group reads.
struct RowPass {
  const uint64_t* part;   // (reference, sum) pairs, C1 per row
  const float* zrow;      // each row's logit at its draft token
  const uint64_t* flags;  // completion tag of each row chunk
  uint64_t tag;           // this call's completion tag
  int C1;                 // chunks per row
  float c;                // log2(e) / T
};

// Draw of one work-group: chunk group grp of request b.  With kStateSlot,
// work-group 0 of the request takes the verdict of the request's early
// acceptance tests; if they left positions untested it tests those on one
// wave as their rows complete and publishes the packed state in the
// request's ready slot.  The request's other draw work-groups wait for the
// ready slot.  Every draw work-group takes the request's draw ticket, and
// the last one writes the request's outputs and clears the ready slot.  A wait that gives up sets the workspace status;
// the request's work-groups then skip their sums, and the last one writes
// accepted_len = -1 and out_tokens all -1, as it does whenever the status
// word is set.
template <int DT, int NE, int HOW>
__device__ __forceinline__ void draw_block(
    int b, int grp, int nb, const void* __restrict__ target, const void* __restrict__ draft,
    int k, int V, int C2, double inv_t, const int32_t* __restrict__ draft_tokens,
    const float* __restrict__ uniforms, uint64_t seed, uint64_t ctr0,
    int32_t* __restrict__ accepted_len, int32_t* __restrict__ out_tokens,
    float* __restrict__ probe, const ReqState* __restrict__ state, const RowPass& rows,
    DrawPart* __restrict__ part, unsigned* __restrict__ counters, long spin_limit) {
  const int G2 = draw_groups(C2, nb);
  __shared__ double tab[256];
  static_assert(kThreads == 256, "one table entry per thread");
  // The exp table's load is issued now and stored to shared memory after
  // the wait below, so the load and the first poll share one round trip.
  const double tv = kExp2Frac256[threadIdx.x];
  int n = 0;
  bool ok = true;  // this work-group holds the request's state
  double mp = 0.0, mq = 0.0, rho32 = 1.0;
  {
    ReqState st;
    if constexpr (HOW != kStateStored) {
      __shared__ int s_ok;
      __shared__ uint64_t s_w[2];
      if (grp == 0) {  // work-group-uniform
        // The request's early acceptance tests either decided it or left
        // the positions from some point on to this work-group.
        if (threadIdx.x < kWaveSize) {
          unsigned v = 0;
          if (threadIdx.x == 0) v = take_verdict(verdict_word(counters, b), spin_limit);
          v = __shfl(v, 0, 64);
          int tested = (int)(v >> 2);
          // gave_up: this wave's own wait gave up (a failed verdict was
          // already noted by its finalizer)
          bool gave_up = v == 0;
          bool failed = gave_up || (v & 3) == kVerdictFailed;
          bool mine_ready = false;
          ReqState mine;
          if ((v & 3) == kVerdictDeferred) {
            __builtin_amdgcn_s_setprio(3);
            const int res = finalize_progressive(
                b, k, V, rows.C1, rows.c, tested, INT_MAX, draft_tokens, uniforms, seed, ctr0,
                rows.part, rows.zrow, rows.flags, rows.tag, probe, mine, tested, spin_limit);
            __builtin_amdgcn_s_setprio(0);
            if (res == kDecided) {
              if (threadIdx.x == 0) publish_state(counters, b, mine);
              mine_ready = true;
            } else {
              failed = gave_up = true;
            }
          }
          if (!failed && probe)  // positions after the first rejection, as their rows complete
            probe_remaining(b, k, V, rows.C1, rows.c, tested, draft_tokens, uniforms, seed, ctr0,
                            rows.part, rows.zrow, rows.flags, rows.tag, probe, counters,
                            spin_limit);
          if (threadIdx.x == 0) {
            uint64_t w0 = 0, w1 = 0;
            int good = 1;
            if (failed) {
              // Tell the request's other draw work-groups not to wait.
              if (gave_up) note_give_up(counters);
              uint64_t* slot = ready_slot(counters, b);
              st_dev(&slot[0], kSlotFailed);
              st_dev(&slot[1], kSlotFailed);
              good = 0;
            } else if (mine_ready) {
              pack_state(mine, w0, w1);
            } else if (!wait_slot(ready_slot(counters, b), w0, w1, spin_limit)) {
              note_give_up(counters);
              good = 0;
            } else if (w0 == kSlotFailed) {
              good = 0;
            }
            s_w[0] = w0;
            s_w[1] = w1;
            s_ok = good;
          }
        }
      } else if (threadIdx.x == 0) {
        uint64_t w0 = 0, w1 = 0;
        int good = 1;
        if (!wait_slot(ready_slot(counters, b), w0, w1, spin_limit)) {
          note_give_up(counters);
          good = 0;
        } else if (w0 == kSlotFailed) {
          good = 0;
        }
        s_ok = good;
        s_w[0] = w0;
        s_w[1] = w1;
      }
      __syncthreads();
      ok = s_ok != 0;
      if (ok) st = unpack_state(s_w[0], s_w[1], k);
    } else {
      st = ld_dev_state(&state[b]);
    }
    if (ok) {
      n = min(max(st.n, 0), k);  // always a valid row index
      mp = st.mp;
      mq = st.mq;
      rho32 = st.rho32;
    }
  }
  tab[threadIdx.x] = tv;
  __syncthreads();
  const bool resid = n < k;
  const double c1 = inv_t * kInvLn2x256, c0p = -mp * c1, c0q = -mq * c1;
  const long eb_bytes = Elems<DT>::kBytes;
  const void* prow =
      reinterpret_cast<const char*>(target) + ((long)b * (k + 1) + n) * V * eb_bytes;
  const void* qrow =
      resid ? reinterpret_cast<const char*>(draft) + ((long)b * k + n) * V * eb_bytes : nullptr;

  // ---- this work-group's chunks: nb * kDrawChunksPerWave consecutive
  // chunks per wave ----
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (ok) {
    const int per_wave = nb * kDrawChunksPerWave;
    const int first = grp * nb * kDrawChunksPerGroup + wave * per_wave;
    DrawPart* pb = part + (long)b * C2;
    if (first < C2) {  // wave-uniform
      if (resid)
        wave_draw_chunks<DT, NE, 0, true>(prow, qrow, V, C2, first, per_wave, c1, c0p, c0q,
                                             rho32, tab, pb);
      else
        wave_draw_chunks<DT, NE, 0, false>(prow, qrow, V, C2, first, per_wave, c1, c0p, c0q,
                                              rho32, tab, pb);
    }
  }
  wait_stores();  // every wave's partials complete before the ticket below
  __syncthreads();
  if (!block_arrive(&counters[(long)b * kCountersPerReq + 1], (unsigned)G2)) return;

  // ---- last work-group of request b: exact rho, chunk totals, draw ----
  // Every other wave on this compute unit is bulk work of other requests,
  // while this one decides when its request ends: it issues first.
  __builtin_amdgcn_s_setprio(3);
  // A failed request (this work-group has no state), or any give-up recorded
  // in the workspace (sticky until it is reset): -1 outputs instead of a
  // draw.  Every draw work-group of the request has passed its wait (each
  // took the ticket after it), so the ready slot goes back to 0 for the next
  // call either way.
  auto fail_outputs = [&]() {
    if (wave == 0) {
      for (int i = lane; i <= k; i += kWaveSize) out_tokens[(long)b * (k + 1) + i] = -1;
      if (lane == 0) {
        accepted_len[b] = -1;
        uint64_t* slot = ready_slot(counters, b);
        st_dev(&slot[0], (uint64_t)0);
        st_dev(&slot[1], (uint64_t)0);
      }
    }
  };
  unsigned status_v = 0;  // loaded now, used at the end: off the tail's critical path
  if constexpr (HOW != kStateStored) {
    if (!ok) {  // block-uniform
      fail_outputs();
      return;
    }
    status_v = ld_dev_u32(status_word(counters));
  }
  // Thread t owns chunk base + t of each tile of kThreads chunks.  With one
  // tile (V up to kThreads * kDrawChunk) the partials are loaded once and
  // every step below works on registers; with more tiles the corrected
  // totals are written back and reloaded by the same thread.
  DrawPart* rp = part + (long)b * C2;
  const int n_tiles = (C2 + kThreads - 1) / kThreads;
  double csp = 0.0, csq = 0.0, cw = 0.0, cdq = 0.0, cnk = 0.0;
  double cka[kKinkSlots], ckb[kKinkSlots];
  auto load_chunk = [&](int cc) {
    csp = csq = cw = cdq = cnk = 0.0;
    for (int j = 0; j < kKinkSlots; ++j) cka[j] = ckb[j] = 0.0;
    if (cc < C2) {
      csp = ld_dev_d(&rp[cc].sp);
      csq = ld_dev_d(&rp[cc].sq);
      cw = ld_dev_d(&rp[cc].w);
      cdq = ld_dev_d(&rp[cc].dq);
      cnk = ld_dev_d(&rp[cc].nk);
      for (int j = 0; j < kKinkSlots; ++j) {
        cka[j] = ld_dev_d(&rp[cc].ka[j]);
        ckb[j] = ld_dev_d(&rp[cc].kb[j]);
      }
    }
  };
  const bool resid_w = resid;  // weights move with rho
  __shared__ int s_cs;      // chunk holding the threshold
  __shared__ double s_P;    // weight of the chunks before it
  if (threadIdx.x == 0) s_cs = INT_MAX;  // ordered by the reduction's barriers
  // S_p, S_q and the number of chunks with more kink-band elements than
  // recorded, in one reduction.
  double sums[3] = {0.0, 0.0, 0.0};
  for (int base = 0; base < C2; base += kThreads) {
    load_chunk(base + threadIdx.x);
    sums[0] += csp;
    sums[1] += csq;
    sums[2] += cnk > (double)kKinkSlots ? 1.0 : 0.0;
  }
  block_sum_dn<3>(sums);
  const double sp_tot = sums[0];
  const double rho = resid_w ? sums[0] / sums[1] : 1.0;
  // The weights were summed at rho32 with the elements within kKinkBand of
  // the kink left out; moving them linearly to rho is exact only while no
  // other element changes sides, i.e. while rho stays well inside that band
  // around rho32.  Otherwise (far-off float32 statistics: extreme
  // temperatures or logit ranges) every chunk is recomputed exactly.
  const bool drift = resid_w && !(fabs(rho - rho32) <= 0.5 * kKinkBand * rho32);
  const bool any_redo = resid_w && (sums[2] > 0.0 || drift);  // block-uniform
  // Chunk totals of the draw weights at the exact rho: the linear part moved
  // to rho, plus the exact weights of the recorded kink-band elements; a
  // chunk with more of them than recorded is recomputed (one wave each).
  double acc_w = 0.0, acc_p = 0.0;  // this thread's share of the totals
  for (int base = 0; base < C2; base += kThreads) {
    const int cc = base + threadIdx.x;
    if (n_tiles > 1) load_chunk(cc);
    const bool redo = resid_w && cc < C2 && (drift || cnk > (double)kKinkSlots);
    if (resid_w && !redo) {
      cw = fmax(0.0, cw + (rho - rho32) * cdq);
      for (int j = 0; j < kKinkSlots; ++j)
        if ((double)j < cnk) cw += fmax(0.0, cka[j] - rho * ckb[j]);
    }
    if (any_redo) {
      __shared__ int s_list[kThreads];
      __shared__ int s_nr;
      __shared__ double s_wx[kThreads];
      if (threadIdx.x == 0) s_nr = 0;
      __syncthreads();
      if (redo) s_list[atomicAdd(&s_nr, 1)] = threadIdx.x;
      __syncthreads();
      const int nr = s_nr;
      for (int idx = wave; idx < nr; idx += kWaves) {  // wave-uniform
        const int t2 = s_list[idx];
        const double wx =
            wave_chunk_w_exact<DT, 0>(prow, qrow, V, base + t2, c1, c0p, c0q, rho, tab);
        if (lane == 0) s_wx[t2] = wx;
      }
      __syncthreads();
      if (redo) cw = fmax(0.0, s_wx[threadIdx.x]);
    }
    if (n_tiles > 1) {
      if (cc < C2) st_dev_d(&rp[cc].w, cw);
      wait_stores();  // reloaded by this same thread below
    }
    acc_w += cw;
    acc_p += csp;
  }
  // Weights drawn from: the residual, or the target terms when the
  // residual is empty (or at the bonus position).  Locate the chunk where
  // the running total first exceeds u times the grand total; past the end
  // (a last-bit difference) the last chunk is searched.
  const float u = get_uniform(uniforms, seed, ctr0, b, n, 1, k);
  bool use_w;
  double grand;
  if (n_tiles == 1) {
    // One scan gives every chunk's prefix and both totals.
    const double v2[2] = {cw, csp};
    double ex[2], tot[2];
    block_exclusive_scan_total_dn<2>(v2, ex, tot);
    use_w = resid && tot[0] > 0.0;
    grand = use_w ? tot[0] : tot[1];
    const double thr = (double)u * grand;
    const int cc = threadIdx.x;
    const double val = use_w ? cw : csp, excl = use_w ? ex[0] : ex[1];
    const uint64_t mh = __ballot(cc < C2 && excl + val > thr);
    if (mh != 0 && lane == __builtin_ctzll(mh)) atomicMin(&s_cs, cc);  // the wave's first
    __syncthreads();
    if (cc == (s_cs == INT_MAX ? C2 - 1 : s_cs)) s_P = excl;
  } else {
    double tot[2] = {acc_w, acc_p};
    block_sum_dn<2>(tot);
    use_w = resid && tot[0] > 0.0;
    grand = use_w ? tot[0] : tot[1];
    const double thr = (double)u * grand;
    double running = 0.0;
    for (int base = 0; base < C2; base += kThreads) {
      const int cc = base + threadIdx.x;
      load_chunk(cc);  // totals as written back above
      const double v1[1] = {use_w ? cw : csp};
      double ex[1], ts[1];
      block_exclusive_scan_total_dn<1>(v1, ex, ts);
      const double excl = running + ex[0];
      const uint64_t mh = __ballot(cc < C2 && excl + v1[0] > thr);
      if (mh != 0 && lane == __builtin_ctzll(mh)) atomicMin(&s_cs, cc);
      __syncthreads();
      const int hit = s_cs;
      if (hit != INT_MAX || base + kThreads >= C2) {  // block-uniform
        if (cc == (hit == INT_MAX ? C2 - 1 : hit)) s_P = excl;
        break;
      }
      running += ts[0];
    }
  }
  const double thr = (double)u * grand;
  const int cs = s_cs == INT_MAX ? C2 - 1 : s_cs;
  const int mode = use_w ? 0 : 1;
  // s_P is stored by one thread above; the search reads it after a barrier.
  int t = search_chunk<DT, 0>(prow, qrow, V, cs, mode == 0, c1, c0p, c0q, rho, s_P, thr, tab);
  if (status_v != 0) {  // block-uniform
    fail_outputs();
    return;
  }
  if (wave == 0)  // the acceptance tests' outputs: this work-group's alone
    write_accept_outputs(b, k, n, draft_tokens, accepted_len, out_tokens, probe);
  if (threadIdx.x == 0) {
    if (!(grand > 0.0)) t = -1;  // rows without mass (invalid input)
    out_tokens[(long)b * (k + 1) + n] = t;
    if (probe) {
      // Mass of the distribution drawn from, in probability units.
      const double mass = resid ? (mode == 0 ? grand / sp_tot : 0.0) : 1.0;
      probe[((long)b * (k + 1) + n) * 4 + 2] = (float)mass;
    }
    if constexpr (HOW != kStateStored) {
      uint64_t* slot = ready_slot(counters, b);
      st_dev(&slot[0], (uint64_t)0);
      st_dev(&slot[1], (uint64_t)0);
    }
  }
}

// Two-launch path: the row pass, then the draw.
template <int DT, int NE>
__global__ __launch_bounds__(kThreads) void k_row_stats(
    const void* __restrict__ target, const void* __restrict__ draft, int k, int V, int C1,
    float c, const int32_t* __restrict__ draft_tokens, const float* __restrict__ uniforms,
    uint64_t seed, uint64_t ctr0, float* __restrict__ probe, uint64_t* __restrict__ part,
    float* __restrict__ zrow, ReqState* __restrict__ state, unsigned* __restrict__ counters) {
  row_block<DT, NE>(blockIdx.x, false, false, 0, target, draft, k, V, C1, c, draft_tokens,
                    uniforms, seed, ctr0, probe, part, zrow, nullptr, 0, state, counters);
}

template <int DT, int NE>
__global__ __launch_bounds__(kThreads) void k_draw(
    const void* __restrict__ target, const void* __restrict__ draft, int k, int V, int C2, int nb,
    double inv_t, const int32_t* __restrict__ draft_tokens, const float* __restrict__ uniforms,
    uint64_t seed, uint64_t ctr0, int32_t* __restrict__ accepted_len,
    int32_t* __restrict__ out_tokens, float* __restrict__ probe,
    const ReqState* __restrict__ state, DrawPart* __restrict__ part,
    unsigned* __restrict__ counters) {
  const int G2 = draw_groups(C2, nb);
  const RowPass none{nullptr, nullptr, nullptr, 0, 0, 0.f};
  draw_block<DT, NE, kStateStored>(static_cast<int>(blockIdx.x / G2),
                                         static_cast<int>(blockIdx.x % G2), nb, target, draft, k, V,
                                         C2, inv_t, draft_tokens, uniforms, seed, ctr0,
                                         accepted_len, out_tokens, probe, state, none, part,
                                         counters, kSpinLimit);
}

// One-launch path.  Grid, in dispatch order:
//   1. the row-pass work-groups of positions 0 .. E-1 of every request, in
//      position order (E: as many positions as the first round of resident
//      work-groups streams);
//   2. the finalizer work-groups, one request per wave, which test each
//      request's early positions as their rows complete;
//   3. for each request b in turn but the last n_tail: the row-pass
//      work-groups of b's positions E .. k, then b's draw work-groups;
//   4. the draw work-groups of the last n_tail requests, then their rows of
//      positions E .. k.
// Most requests stop at one of their early positions, so their states are
// ready about when the first round of row-pass work-groups ends, and their
// draws run while the rows of later positions and requests stream; the
// grid ends with rows that no draw waits for (4.).  A request the
// finalizers leave undecided is finished by its first draw work-group from
// its remaining rows.  Work-groups are dispatched in index order.  Every
// wait in 1.-3. is for work earlier in the grid (a finalizer for early
// rows, a first draw work-group for its finalizer and its request's rows,
// the other draw work-groups for the request's state); in 4. a draw
// work-group may wait for rows after it, but those draw work-groups are at
// most half of the resident ones, so the other half keep taking the rows
// and every wait ends.  EXIT: row-pass work-groups after position 0 stop
// once their request is decided before their position.
// tag: this call's completion tag, or 0 to derive it from the workspace's
// call epoch (graph-captured calls; k_advance_epoch follows the kernel).
// spin_limit: polls before a bounded wait gives up.  withhold: test only
// (row_block).
template <int DT, int NE, bool EXIT>
__global__ __launch_bounds__(kThreads) void k_sample_one(
    const void* __restrict__ target, const void* __restrict__ draft, int B, int k, int V, int C1,
    int C2, float c, double inv_t, const int32_t* __restrict__ draft_tokens,
    const float* __restrict__ uniforms, uint64_t seed, uint64_t ctr0,
    int32_t* __restrict__ accepted_len, int32_t* __restrict__ out_tokens,
    float* __restrict__ probe, uint64_t* __restrict__ part1, float* __restrict__ zrow,
    uint64_t* __restrict__ flags, uint64_t tag, ReqState* __restrict__ state,
    DrawPart* __restrict__ part2, unsigned* __restrict__ counters, int E, long n_early_rows,
    int n_fin, long spin_limit, int withhold, int n_tail, int gate_ticks) {
  const long bid = blockIdx.x;
  if (tag == 0) tag = epoch_tag(ld_dev(epoch_word(counters)));
  const int G2 = draw_groups(C2, 1);
  long row = -1;  // row-pass index in position order
  bool late = false;
  long draw = -1;
  if (bid < n_early_rows) {
    row = bid;
  } else if (bid < n_early_rows + n_fin) {
    const int b = static_cast<int>((bid - n_early_rows) * kWaves + (threadIdx.x >> 6));
    if (b < B)
      early_finalize(b, k, V, C1, c, E, draft_tokens, uniforms, seed, ctr0, part1, zrow, flags,
                     tag, probe, counters, spin_limit);
    return;
  } else {
    // Request b's rows of positions E .. k (target and draft row of each
    // position, then the bonus row), then its draw work-groups; for the last
    // n_tail requests, all their draw work-groups first, then all their
    // later rows, so that the grid ends with rows nobody waits for.
    const long L = E > k ? 0 : (2L * (k - E) + 1) * C1;
    const long j = bid - n_early_rows - n_fin;
    const int Bh = B - n_tail;
    int b;
    long o;
    if (j < (long)Bh * (L + G2)) {
      b = static_cast<int>(j / (L + G2));
      o = j % (L + G2);
    } else {
      const long j2 = j - (long)Bh * (L + G2);
      if (j2 < (long)n_tail * G2) {
        b = Bh + static_cast<int>(j2 / G2);
        o = L + j2 % G2;
      } else {
        const long j3 = j2 - (long)n_tail * G2;
        b = Bh + static_cast<int>(j3 / (L > 0 ? L : 1));
        o = j3 % (L > 0 ? L : 1);
      }
    }
    if (o >= L) {
      draw = (long)b * G2 + (o - L);
    } else {
      const long per_pos = (long)B * 2 * C1;
      const int pos = E + static_cast<int>(o / (2 * C1));
      const long w = o % (2 * C1);
      row = pos < k ? (long)pos * per_pos + (long)b * 2 * C1 + w
                    : (long)k * per_pos + (long)b * C1 + w;
      late = true;
    }
  }
  if (row >= 0) {
    row_block<DT, NE, EXIT>(row, true, late, B, target, draft, k, V, C1, c, draft_tokens,
                            uniforms, seed, ctr0, probe, part1, zrow, flags, tag, state,
                            counters, withhold != 0, gate_ticks);
  } else {
    const RowPass rows{part1, zrow, flags, tag, C1, c};
    draw_block<DT, NE, kStateSlot>(static_cast<int>(draw / G2), static_cast<int>(draw % G2),
                                      1, target, draft, k, V, C2, inv_t, draft_tokens, uniforms,
                                      seed, ctr0, accepted_len, out_tokens, probe, state, rows,
                                      part2, counters, spin_limit);
  }
}

// Graph-captured one-launch calls: the next call epoch, after the kernel.
__global__ void k_advance_epoch(unsigned* __restrict__ counters) {
  if (threadIdx.x == 0) {
    uint64_t* e = epoch_word(counters);
    st_dev(e, ld_dev(e) + 1);
  }
}

// spec_workspace_reset: every word of the counter region but the epoch.
__global__ __launch_bounds__(kThreads) void k_reset_counters(unsigned* __restrict__ counters) {
  const long n = (long)(kCounterRegionBytes / 4);
  for (long i = (long)blockIdx.x * kThreads + threadIdx.x; i < n; i += (long)gridDim.x * kThreads)
    if (i != (long)kEpochWord && i != (long)kEpochWord + 1) counters[i] = 0u;
}

hipError_t launch_reset_counters(void* ws, hipStream_t s) {
  hipLaunchKernelGGL(k_reset_counters, dim3(256), dim3(kThreads), 0, s,
                     static_cast<unsigned*>(ws));
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Scratch of the no-alloc entry point
// ---------------------------------------------------------------------------
//
// A file-scope device array: each GPU the library runs on holds its own
// copy, at its own address, until the process ends.  In host code the name
// is a stand-in, not a device address, so host code only ever uses the
// address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

hipError_t noalloc_scratch(int device, void** ptr) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[device] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr || reinterpret_cast<uintptr_t>(p) % 256 != 0) return hipErrorInvalidSymbol;
    g_scratch_ptr[device] = p;
  }
  *ptr = g_scratch_ptr[device];
  return hipSuccess;
}

// The words a call over requests 0..B-1 uses: each request's own eight
// (tickets) and the eight at its hand-over position (verdict, ready slot),
// plus the status word.  A kernel, not a memset, so the clear can sit in a
// captured graph.
__global__ __launch_bounds__(kThreads) void k_clear_requests(unsigned* __restrict__ counters,
                                                             int B) {
  const long i = (long)blockIdx.x * kThreads + threadIdx.x;
  if (i < (long)B * kCountersPerReq) {
    const int b = static_cast<int>(i / kCountersPerReq);
    const int j = static_cast<int>(i % kCountersPerReq);
    counters[(long)b * kCountersPerReq + j] = 0u;
    counters[handover_pos(b) + j] = 0u;
  }
  if (i == 0) counters[kStatusWord] = 0u;
}

hipError_t launch_clear_requests(void* ws, int B, hipStream_t s) {
  const long n = std::max(1L, (long)B * kCountersPerReq);
  hipLaunchKernelGGL(k_clear_requests, dim3((unsigned)((n + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, s, static_cast<unsigned*>(ws), B);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Host launcher
// ---------------------------------------------------------------------------

static int row_chunks(int V) { return (V + kRowChunkElems - 1) / kRowChunkElems; }


// Work-groups of the one-launch kernel resident per compute unit; the
// first round of row-pass work-groups (compute units x this) sets how many
// positions are early.  Measured at B = 64, k = 8, V = 128256 bf16: six per
// unit needs the kernel held to 80 VGPRs, which spills, and is slower.
#ifndef SPEC_ONE_LAUNCH_GROUPS_PER_CU
#define SPEC_ONE_LAUNCH_GROUPS_PER_CU 5
#endif
constexpr int kOneLaunchGroupsPerCU = SPEC_ONE_LAUNCH_GROUPS_PER_CU;

// Requests at the end of the one-launch grid whose draws precede their
// later rows (at most this many), and the share of resident work-groups
// their draws may take (1 / kTailDrawSlotFraction).  Measured at B = 64,
// k = 8, V = 128256 bf16 (one-launch kernel): 0, 4, 8, 15, 20, 30 such
// requests gave 63.8, 63.6, 62.9, 62.1, 61.7 and 61.4 us; 45 and 64 (more
// than half the resident work-groups) 63.5 and 65.5 us.
#ifndef SPEC_TAIL_REQUESTS
#define SPEC_TAIL_REQUESTS 65536
#endif
constexpr int kTailRequests = SPEC_TAIL_REQUESTS;
#ifndef SPEC_TAIL_DRAW_SLOT_FRACTION
#define SPEC_TAIL_DRAW_SLOT_FRACTION 2
#endif
constexpr long kTailDrawSlotFraction = SPEC_TAIL_DRAW_SLOT_FRACTION;

// Compute units of the current device.
int device_cus() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cached[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        v <= 0)
      return 256;
    cached[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

// Shared memory per compute unit of the current device.
static int device_lds_per_cu() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int v = cached[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) !=
        hipSuccess)
      return 0;
    cached[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

// Dynamic shared memory for the one-launch kernel: at least `need`, and
// with the kernel's static shared memory more than 1/(groups + 1) of a
// compute unit's (plus allocation granularity), so that at most
// kOneLaunchGroupsPerCU work-groups are resident per unit.
template <int DT, int NE>
static uint32_t one_launch_lds(uint32_t need) {
  static std::atomic<int> static_lds{-1};
  int sl = static_lds.load(std::memory_order_relaxed);
  if (sl < 0) {
    hipFuncAttributes fa;
    if (hipFuncGetAttributes(&fa, reinterpret_cast<const void*>(&k_sample_one<DT, NE, false>)) !=
        hipSuccess)
      return need;
    sl = static_cast<int>(fa.sharedSizeBytes);
    static_lds.store(sl, std::memory_order_relaxed);
  }
  const int lds_cu = device_lds_per_cu();
  if (lds_cu <= 0) return need;
  const long pad = (long)lds_cu / (kOneLaunchGroupsPerCU + 1) + 1024 - sl;
  return pad > (long)need ? static_cast<uint32_t>(pad) : need;
}

// 16-byte loads need every row to start on a 16-byte boundary; the buffer
// loads of the row-statistics sweep address rows below 2 GiB.
static bool rows_aligned(const void* p, int V, int dtype) {
  const long eb = dtype == 1 ? 2 : 4;
  return (reinterpret_cast<uintptr_t>(p) % 16 == 0) && (((long)V * eb) % 16 == 0) &&
         (long)V * eb < (1L << 31);
}

template <int DT, int NE>
static hipError_t launch_logits(const void* target, const void* draft, int B, int k, int V,
                          const int32_t* draft_tokens, const float* uniforms, uint64_t seed,
                          uint64_t ctr0, float temperature, const SampleMode& mode,
                          int32_t* accepted_len, int32_t* out_tokens, float* probe, char* w,
                          const WsLayout& L, hipStream_t s) {
  const int C1 = row_chunks(V);
  const int C2 = res_chunks(V);
  const float c = 1.4426950408889634f / temperature;
  const double inv_t = 1.0 / (double)temperature;
  auto* p1 = reinterpret_cast<uint64_t*>(w + L.part1);
  auto* st = reinterpret_cast<ReqState*>(w + L.state);
  auto* p2 = reinterpret_cast<DrawPart*>(w + L.part2);
  auto* cnt = reinterpret_cast<unsigned*>(w + L.count);
  const long R = 2L * k + 1;
  auto* zr = reinterpret_cast<float*>(w + L.zrow);
  const long n_row = (long)B * R * C1;
  const long slots = (long)device_cus() * kOneLaunchGroupsPerCU;
  // AUTO: early exit when the row pass takes more than one round of
  // resident work-groups (then rows started after the first decisions can
  // be skipped); with fewer rows every row is in flight from the start and
  // the one-launch schedule is faster (B = 8, k = 4, V = 32000 bf16: 22.1
  // us against 24.0 us with early exit); with at most a third of a round of
  // rows, the two launches (row pass, then draw) are faster still: their
  // draw work-groups start on known verdicts instead of waiting in the grid
  // (per call: B = 8, k = 4, V = 32000: 19.8 against 20.7 us; B = 8, k = 8,
  // V = 128256: 26.3 against 28.2; 816 rows, B = 24, k = 8, V = 128256:
  // 46.0 against 42.3).
  const int sched = mode.sched != SPEC_SCHED_AUTO ? mode.sched
                    : n_row > slots              ? SPEC_SCHED_EARLY_EXIT
                    : n_row * 3 > slots          ? SPEC_SCHED_ONE_LAUNCH
                                                 : SPEC_SCHED_TWO_LAUNCH;
  if (sched != SPEC_SCHED_TWO_LAUNCH) {
    auto* fl = reinterpret_cast<uint64_t*>(w + L.flag);
    // Early positions: as many as the first round of resident work-groups
    // streams (at least one).
    const long per_pos = (long)B * 2 * C1;
    // Early exit needs no probe values beyond each request's stop.
    const bool exit_early = sched == SPEC_SCHED_EARLY_EXIT && probe == nullptr;
    // Measured at B = 64, k = 8, V = 128256 bf16 with early exit: E = 2, 3,
    // 4, 5 (this rule), 6, 7, 9 gave 63.2, 59.9, 57.4, 55.4, 56.9, 60.8 and
    // 65.8 us; row chunks of 32K or 16K elements instead of 64K (so that the
    // first round holds fewer positions) gave 65.4 and 87.2 us.
    const int E = (int)std::max(1L, std::min((long)k + 1, slots / per_pos));
    const long n_early_rows = E > k ? n_row : (long)E * per_pos;
    const int n_fin = (B + kWaves - 1) / kWaves;
    const int G2 = draw_groups(C2, 1);
    // The last n_tail requests' draw work-groups precede their later rows.
    // Such a draw work-group may wait for rows after it in the grid (a
    // request its finalizer left undecided), so their number stays within
    // 1 / kTailDrawSlotFraction of the resident work-groups: the rest keep
    // taking those rows, and every wait ends.
    const int n_tail =
        E > k ? 0
              : (int)std::min((long)std::min(B, kTailRequests),
                              slots / kTailDrawSlotFraction / std::max(1, G2));
    // A captured launch is replayed as it is recorded, so its tag comes from
    // the workspace's call epoch, advanced by a kernel after it.
    const uint64_t tag = mode.capturing ? 0 : next_call_tag();
    const long spin = mode.test_give_up ? 256 : kSpinLimit;
    // The early-exit gate in ticks of the 100 MHz clock (at most 1 ms).
    const long pos0_bytes = (long)B * 2 * V * (DT == 1 ? 2 : 4);
    const int gate_ticks = exit_early ? (int)std::min(100000L, pos0_bytes / 10 / kGateGBps) : 0;
    const hipError_t e = launch_timed(
        kProfFused, exit_early ? &k_sample_one<DT, NE, true> : &k_sample_one<DT, NE, false>,
        dim3((unsigned)(n_row + n_fin + (long)B * G2)), dim3(kThreads), one_launch_lds<DT, NE>(0),
        s, target, draft, B, k, V, C1, C2, c, inv_t, draft_tokens, uniforms, seed, ctr0,
        accepted_len, out_tokens, probe, p1, zr, fl, tag, st, p2, cnt, E, n_early_rows, n_fin,
        spin, mode.test_give_up ? 1 : 0, n_tail, gate_ticks);
    if (e != hipSuccess || !mode.capturing) return e;
    hipLaunchKernelGGL(k_advance_epoch, dim3(1), dim3(kWaveSize), 0, s, cnt);
    return hipGetLastError();
  }
  hipError_t e = launch_timed(kProfRowPass, &k_row_stats<DT, NE>, dim3((unsigned)n_row),
                             dim3(kThreads), 0, s, target, draft, k, V, C1, c, draft_tokens,
                             uniforms, seed, ctr0, probe, p1, zr, st, cnt);
  if (e != hipSuccess) return e;
  const int G2 = draw_groups(C2, 1);
  return launch_timed(kProfDraw, &k_draw<DT, NE>, dim3((unsigned)(B * G2)), dim3(kThreads), 0, s,
                      target, draft, k, V, C2, 1, inv_t, draft_tokens, uniforms, seed, ctr0,
                      accepted_len, out_tokens, probe, (const ReqState*)st, p2, cnt);
}

hipError_t launch_sample(const void* target, const void* draft, int dtype, int kind, int B,
                         int k, int V, const int32_t* draft_tokens, const float* uniforms,
                         uint64_t seed, uint64_t counter0, float temperature,
                         const SampleMode& mode, int32_t* accepted_len, int32_t* out_tokens,
                         float* probe, void* ws, const WsLayout& L, hipStream_t s) {
  char* w = static_cast<char*>(ws);
  const bool vec = rows_aligned(target, V, dtype) && (k == 0 || rows_aligned(draft, V, dtype));
  if (kind == 1) {
    return launch_probs(target, draft, B, k, V, draft_tokens, uniforms, seed, counter0,
                        accepted_len, out_tokens, probe, vec, ws, L, s);
  } else if (dtype == 1) {
    if (vec)
      return launch_logits<1, 8>(target, draft, B, k, V, draft_tokens, uniforms, seed, counter0,
                          temperature, mode, accepted_len, out_tokens, probe, w, L, s);
    else
      return launch_logits<1, 1>(target, draft, B, k, V, draft_tokens, uniforms, seed, counter0,
                          temperature, mode, accepted_len, out_tokens, probe, w, L, s);
  } else {
    if (vec)
      return launch_logits<0, 4>(target, draft, B, k, V, draft_tokens, uniforms, seed, counter0,
                          temperature, mode, accepted_len, out_tokens, probe, w, L, s);
    else
      return launch_logits<0, 1>(target, draft, B, k, V, draft_tokens, uniforms, seed, counter0,
                          temperature, mode, accepted_len, out_tokens, probe, w, L, s);
  }
}

}  // namespace specv
