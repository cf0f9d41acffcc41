// Device routines of the sampling verification kernels: the float32 row
// statistic and its sweep, the float64 draw terms and chunk sums, the chunk
// search of the inverse-CDF draw, and the coherent state and ready slots
// the one-launch kernel passes between work-groups.
#pragma once

#include <climits>

#include "device_common.h"
#include "device_math.h"

namespace specv {

constexpr int kUnrollStats = SPEC_STATS_UNROLL;


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

// Streaming softmax statistic of a chunk: a reference value m (an element
// of the chunk) and s = sum 2^(x c - mc) with mc = fl32(m c), the rounded
// product; merges recompute mc from m, so its rounding cancels exactly.
// Any reference gives the same statistic, since log p(x) = x c - mc -
// log2 s; the reference only has to keep the terms finite.  So m is not
// the running maximum: it is updated only when a batch's sum reaches
// kBatchLimit (every term of the batch is then below 2^64) and on the first
// batch that holds a finite value.  Each element costs one fused
// multiply-add, one exp2 and one add.  Terms are added pairwise within a
// batch in float32; batch sums are accumulated in float64, because a
// float32 running sum would absorb the many terms far below its last bit.
constexpr float kBatchLimit = 0x1p64f;

template <int N>
__device__ __forceinline__ float batch_sum(const float* x, float c, float mc) {
  float t[N];
#pragma unroll
  for (int e = 0; e < N; ++e) t[e] = __builtin_amdgcn_exp2f(fmaf(x[e], c, -mc));
#pragma unroll
  for (int w = 1; w < N; w *= 2)
#pragma unroll
    for (int e = 0; e + w < N; e += 2 * w) t[e] += t[e + w];
  return t[0];
}

// Sum of one group's terms, moving the reference first when the group holds
// a value far above it (or the first finite value).
template <int N>
__device__ __forceinline__ float group_sum(float& m, float& mc, double& s, const float* x,
                                           float c) {
  float g = batch_sum<N>(x, c, mc);
  if (!(g < kBatchLimit)) {  // rare: no reference yet, or far above it
    float lm = x[0];
#pragma unroll
    for (int e = 1; e < N; ++e) lm = fmaxf(lm, x[e]);
    if (lm > m) {
      const float mcn = mul_rn(lm, c);
      s = (m == -INFINITY) ? 0.0 : s * (double)__builtin_amdgcn_exp2f(mc - mcn);
      m = lm;
      mc = mcn;
    }
    g = (m == -INFINITY) ? 0.f : batch_sum<N>(x, c, mc);
  }
  return g;
}

// Sum of the terms 2^(x c - mc) of U words, pairwise in float32.  Every
// term is below 2^64 exactly when the sum is (all terms are >= 0), so
// `ok` records whether the reference was good enough for this batch.
template <int DT, int U>
__device__ __forceinline__ float batch_terms(const u32x4 (&w)[U], float c, float mc, bool& ok) {
  constexpr int NE = Elems<DT>::kVec;
  float gs[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float x[NE];
    unpack16<DT>(w[u], x);
    gs[u] = batch_sum<NE>(x, c, mc);
  }
#pragma unroll
  for (int w2 = 1; w2 < U; w2 *= 2)
#pragma unroll
    for (int e = 0; e + w2 < U; e += 2 * w2) gs[e] += gs[e + w2];
  ok = ok && gs[0] < kBatchLimit;  // false for inf / NaN too
  return gs[0];
}

// Largest element of U words.
template <int DT, int U>
__device__ __forceinline__ float batch_max(const u32x4 (&w)[U]) {
  constexpr int NE = Elems<DT>::kVec;
  float lm = -INFINITY;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float x[NE];
    unpack16<DT>(w[u], x);
#pragma unroll
    for (int e = 0; e < NE; ++e) lm = fmaxf(lm, x[e]);
  }
  return lm;
}

// Fold a batch of U words, kUnrollStats at a time: a scheduling barrier
// between the parts keeps the compiler from unpacking the whole batch at
// once.  No branch: a batch whose sum is not below kBatchLimit (a value far
// above the reference, or no finite reference yet) only clears `ok`, and
// the caller recomputes the statistic.
template <int DT, int U>
__device__ __forceinline__ void stat_batch(double& s, const u32x4 (&w)[U], float c, float mc,
                                           bool& ok) {
  if constexpr (U <= kUnrollStats) {
    s += (double)batch_terms<DT, U>(w, c, mc, ok);
  } else {
    static_assert(U % kUnrollStats == 0, "batch of whole parts");
#pragma unroll
    for (int p = 0; p < U / kUnrollStats; ++p) {
      s += (double)batch_terms<DT, kUnrollStats>(
          *reinterpret_cast<const u32x4(*)[kUnrollStats]>(&w[p * kUnrollStats]), c, mc, ok);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// Bit pattern of a 16-byte word of -inf elements (terms of 0).
template <int DT>
__device__ __forceinline__ u32x4 neg_inf_word() {
  const uint32_t v = DT == 1 ? 0xff80ff80u : 0xff800000u;
  return u32x4{v, v, v, v};
}

// Groups (16-byte words) [g0, g1) of one row shared by NT threads.  Batch i
// gives this thread (index tid) the groups g0 + i NT U + u NT + tid, u < U.
// The batch count is uniform, so the loop is too; the last batch may be
// partial: its groups at or past g1 count as -inf (loads past the row's end
// read zeros and never reach memory).  Software pipelined over two word
// buffers used in turn: the next batch's U loads are issued before the
// current batch is folded in, so every wave keeps loads in flight while it
// computes.
// The reference m is the largest element of the thread's first batch, and
// every later batch is summed against it without a branch.  If a batch sum
// reaches kBatchLimit (an element more than 64/c above m, or nothing finite
// in the first batch), the thread's statistic is recomputed after the loop
// from memory with the lazy reference of group_sum: rare, and kept out of
// the streaming loop, whose speed it would otherwise cost.
template <int DT, int NT, bool WATCH = false, int U = kUnrollStats>
__device__ __forceinline__ void stats_sweep(const void* rp, uint32_t row_bytes, long g0, long g1,
                                            float c, float& m, float& mc, double& s, int tid,
                                            const uint64_t* watch = nullptr, int pos = 0,
                                            bool precheck = false) {
  constexpr int NE = Elems<DT>::kVec;
  constexpr uint32_t kStep = NT * U * 16u;
  const RowBuf buf(rp, row_bytes);
  const uint32_t off0 = static_cast<uint32_t>(g0 + tid) * 16u;
  const long n = g1 - g0;
  const int nb = static_cast<int>((n + (long)NT * U - 1) / ((long)NT * U));  // uniform
  const bool partial = n % ((long)NT * U) != 0;  // the last batch is partial
  // WATCH: the request's ready slot is read once per pair of batches; each
  // read is used after the next batch's sums, whose data it precedes, so it
  // never stalls the stream.  Once it shows the request stopped before
  // position `pos`, this row decides nothing and the wave stops, marking its
  // partial with m = +inf.  With `precheck` the first read is also used
  // before the second batch is issued (one round trip without a second batch
  // in flight, for rows whose request is likely decided already).
  uint64_t wv = 0;
  if constexpr (WATCH) wv = ld_dev(watch);
  auto stopped = [&]() { return wv != 0 && (int)(uint32_t)wv - 1 < pos; };
  auto load = [&](u32x4 (&w)[U], int i) {
#pragma unroll
    for (int u = 0; u < U; ++u) w[u] = buf.load_nt(off0 + (uint32_t)i * kStep, u * NT * 16u);
  };
  // Groups of batch i at or past g1 (only in a partial last batch) become -inf.
  auto mask = [&](u32x4 (&w)[U], int i) {
    if (partial && i == nb - 1) {  // uniform
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (g0 + (long)i * NT * U + (long)u * NT + tid >= g1) w[u] = neg_inf_word<DT>();
    }
  };
  bool ok = true;
  double acc = 0.0;
  float lmc = -INFINITY;
  if (nb > 0) {
    // Two word buffers used in turn (no register copies, which would wait
    // for the loads in flight).
    u32x4 wa[U], wb[U];
    load(wa, 0);
    if constexpr (WATCH) {
      if (precheck) {  // wave-uniform
        if (stopped()) {
          m = INFINITY;
          s = 0.0;
          return;
        }
        wv = ld_dev(watch);
      }
    }
    if (nb > 1) load(wb, 1);
    __builtin_amdgcn_sched_barrier(0);
    mask(wa, 0);
    const float lm = batch_max<DT, U>(wa);
    lmc = mul_rn(lm, c);
    stat_batch<DT, U>(acc, wa, c, lmc, ok);
    if (lm == -INFINITY) ok = false;  // nothing finite yet: recompute
    if (!ok) lmc = -INFINITY;
    m = lm;
    int i = 2;
    for (; i < nb; i += 2) {
      load(wa, i);
      __builtin_amdgcn_sched_barrier(0);
      mask(wb, i - 1);
      stat_batch<DT, U>(acc, wb, c, lmc, ok);
      if constexpr (WATCH) {
        if (stopped()) {  // wave-uniform: one address
          m = INFINITY;
          s = 0.0;
          return;
        }
        wv = ld_dev(watch);
      }
      if (i + 1 < nb) load(wb, i + 1);
      __builtin_amdgcn_sched_barrier(0);
      mask(wa, i);
      stat_batch<DT, U>(acc, wa, c, lmc, ok);
    }
    if (i == nb) {  // batch nb - 1 is in wb
      mask(wb, nb - 1);
      stat_batch<DT, U>(acc, wb, c, lmc, ok);
    }
  }
  if (__ballot(!ok) != 0) {  // rare: recompute this thread's groups from memory
    if (!ok) {
      float rm = -INFINITY, rmc = -INFINITY;
      double rs = 0.0;
      for (long g = g0 + tid; g < g1; g += NT) {
        float x[NE];
        unpack16<DT>(buf.load_nt(static_cast<uint32_t>(g) * 16u, 0), x);
        const float gsum = group_sum<NE>(rm, rmc, rs, x, c);  // may rescale rs first
        rs += (double)gsum;
      }
      m = rm;
      lmc = rmc;
      acc = rs;
    }
  }
  // Fold into the caller's (m, mc, s) (empty on entry).
  mc = lmc;
  s = acc;
}

// Scalar form for rows that are not 16-byte aligned: elements [e0, e1).
template <int DT>
__device__ __forceinline__ void stats_sweep_scalar(const void* rp, long e0, long e1, float c,
                                                   float& m, float& mc, double& s) {
  for (long e = e0 + threadIdx.x; e < e1; e += kThreads) {
    const float x = load_elem<DT>(rp, e);
    const float gsum = group_sum<1>(m, mc, s, &x, c);  // may rescale s first
    s += (double)gsum;
  }
}

// Fold one chunk partial (reference m2, sum s2 relative to 2^fl32(m2 c))
// into the row's running (M, S), S = sum 2^(x c - fl32(M c)) in float64.
__device__ __forceinline__ void fold_partial(float& M, double& S, uint64_t pp, float c) {
  const float m2 = unpack_lo(pp);
  const double s2 = (double)unpack_hi(pp);
  if (m2 == -INFINITY) return;
  if (M == -INFINITY) {
    M = m2;
    S = s2;
    return;
  }
  // One scale factor: the side with the smaller reference moves to the
  // larger one (the other factor is 2^0 = 1).
  const bool up = m2 > M;
  const float mn = up ? m2 : M, mo = up ? M : m2;
  const double e = exp2((double)mul_rn(mo, c) - (double)mul_rn(mn, c));
  S = up ? S * e + s2 : S + s2 * e;
  M = mn;
}

// (M, S) of two rows of one request (the second only when has_b) from their
// chunk partials, by one thread: up to four partials of each row are loaded
// before any is folded in, so the loads of both rows are in flight together.
__device__ __forceinline__ void merge_two_rows(const uint64_t* part, long base_a, long base_b,
                                               bool has_b, int C1, float c, float& Ma,
                                               double& Sa, float& Mb, double& Sb) {
  Ma = Mb = -INFINITY;
  Sa = Sb = 0.0;
  for (int c0 = 0; c0 < C1; c0 += 4) {
    uint64_t pa[4], pb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      pa[j] = pb[j] = 0;
      if (c0 + j < C1) {
        pa[j] = ld_dev(&part[base_a + c0 + j]);
        if (has_b) pb[j] = ld_dev(&part[base_b + c0 + j]);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (c0 + j < C1) {
        fold_partial(Ma, Sa, pa[j], c);
        if (has_b) fold_partial(Mb, Sb, pb[j], c);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 2. Float64 draw pass
// ---------------------------------------------------------------------------

// Float64 term of one element.  KIND 0 (logits): e^{(z - m)/T}, evaluated as
// 2^(t/256) with t = z c1 + c0, c1 = 256/(T ln 2), c0 = -m c1; KIND 1
// (probabilities): the value itself.
template <int KIND>
__device__ __forceinline__ double draw_term(float z, double c1, double c0, const double* tab) {
  return KIND == 0 ? exp2_256(fma((double)z, c1, c0), tab) : (double)z;
}

// One lane's run of kSegPerThread consecutive elements of one row, kept as
// the raw words loaded (two bfloat16 or one float32 per word) until used.
template <int DT>
struct RunWords {
  static constexpr int kWords = kSegPerThread * Elems<DT>::kBytes / 4;
  uint32_t w[kWords];
};

// Loads the run at element j0; elements at or beyond V read as `fill`
// (raw bits of the element type).  With 16-byte groups (NE > 1) the row
// length is a multiple of NE, so each group is wholly inside or wholly past
// the end; a group past the end loads the row's first group instead and
// keeps the fill, so the loads are unconditional.
template <int DT, int NE>
__device__ __forceinline__ void load_run_words(const void* row, long j0, int V, uint32_t fill,
                                               RunWords<DT>& r) {
  constexpr int kPerWord = 4 / Elems<DT>::kBytes;
  if constexpr (NE > 1) {
    static_assert(NE == Elems<DT>::kVec, "vector group must be 16 bytes");
    static_assert(kSegPerThread % NE == 0, "run length must be a multiple of the load width");
    const uint32_t fw = DT == 1 ? (fill | (fill << 16)) : fill;
#pragma unroll
    for (int g = 0; g < kSegPerThread / NE; ++g) {
      const long e0 = j0 + (long)g * NE;
      const bool ok = e0 < V;
      const u32x4 w = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(row) +
                                                      (ok ? e0 : 0) * Elems<DT>::kBytes);
      r.w[g * 4 + 0] = ok ? w.x : fw;
      r.w[g * 4 + 1] = ok ? w.y : fw;
      r.w[g * 4 + 2] = ok ? w.z : fw;
      r.w[g * 4 + 3] = ok ? w.w : fw;
    }
  } else {
#pragma unroll
    for (int q = 0; q < RunWords<DT>::kWords; ++q) r.w[q] = 0;
#pragma unroll
    for (int e = 0; e < kSegPerThread; ++e) {
      uint32_t bits = fill;
      if (j0 + e < V) {
        if constexpr (DT == 1) bits = reinterpret_cast<const uint16_t*>(row)[j0 + e];
        else bits = reinterpret_cast<const uint32_t*>(row)[j0 + e];
      }
      r.w[e / kPerWord] |= bits << (32 / kPerWord * (e % kPerWord));
    }
  }
}

template <int DT>
__device__ __forceinline__ float run_elem(const RunWords<DT>& r, int e) {
  if constexpr (DT == 1) return (e & 1) ? bf16_hi(r.w[e >> 1]) : bf16_lo(r.w[e >> 1]);
  else return __uint_as_float(r.w[e]);
}

// Raw bits read for elements past the end of a row: -inf logits (weight 0)
// or probability 0.
template <int DT, int KIND>
__host__ __device__ constexpr uint32_t run_fill() {
  if constexpr (KIND == 1) return 0u;
  else return DT == 1 ? 0xff80u : 0xff800000u;
}

// Sums of one chunk by one wave (lane l covers the kSegPerThread elements
// from chunk * kDrawChunk + kSegPerThread l, given as runs rp, rq of the
// target and draft rows), reduced across the wave (valid in every lane):
//   v[0] = sum a, v[1] = sum b (a, b the target and draft terms),
//   v[2] = sum of the draw weights at rho32 (max(0, a - rho32 b), or a for
//          the bonus), v[3] = their derivative in rho (minus the sum of b
//          where the weight is positive), v[4] = the number of elements in
//          the kink band of max(0, .), which are left out of v[2] and v[3];
//   ka, kb = (a, b) of the first kKinkSlots of them, in element order
//          within each lane position (valid when v[4] is at most
//          kKinkSlots; then they are uniform across the wave).
// RESID: the residual draw (false: the bonus draw, from the target terms).
// The loop has no branches: kink-band membership is kept as one wave mask
// per element position, and the rare kink elements are reloaded and
// evaluated after it.
template <int DT, int KIND, bool RESID>
__device__ __forceinline__ void wave_chunk_sums(const RunWords<DT>& rp, const RunWords<DT>& rq,
                                                const void* prow, const void* qrow, int chunk,
                                                double c1, double c0p, double c0q, double rho32,
                                                const double* tab, double& red, double& nkd,
                                                double (&ka)[kKinkSlots],
                                                double (&kb)[kKinkSlots]) {
  double sa = 0.0, sb = 0.0, sw = 0.0, sq = 0.0;
  uint64_t km[kSegPerThread];
  const double bandr = kKinkBand * rho32;
#pragma unroll
  for (int e = 0; e < kSegPerThread; ++e) {
    const double a = draw_term<KIND>(run_elem<DT>(rp, e), c1, c0p, tab);
    sa += a;
    km[e] = 0;
    if constexpr (RESID) {
      const double bq = draw_term<KIND>(run_elem<DT>(rq, e), c1, c0q, tab);
      const double d = fma(-rho32, bq, a);
      bool kink = false;
      if constexpr (KIND == 0) {
        kink = fabs(d) < bandr * bq;  // false when bq = 0
        km[e] = __ballot(kink);
      }
      const bool pos = d > 0.0 && !kink;
      sw += pos ? d : 0.0;
      // S_q and dw/drho only move the weights to the exact rho of logits;
      // probability rows are drawn from as given (rho = 1).
      if constexpr (KIND == 0) {
        sb += bq;
        sq += pos ? bq : 0.0;
      }
    }
  }
  // Record fields 0-3 (S_p, S_q, w, dw/drho) summed over the wave; lane
  // group q (lanes 16q .. 16q+15) ends with field q in `red`.
  const int lane = threadIdx.x & 63;
  if constexpr (RESID && KIND == 1) {
    // S_p and w only (S_q and dw/drho stay 0): lanes 0-31 end with S_p,
    // lanes 32-63 with w.
    const bool h = (lane & 32) != 0;
    double r = h ? sw : sa;
    r += shfl_xor_d(h ? sa : sw, 32);
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) r += shfl_xor_d(r, o);
    red = (lane & 16) ? 0.0 : r;
  } else if constexpr (RESID) {
    // Transposed reduction: each exchange also halves the values a lane
    // carries (4 -> 2 -> 1), then one value per lane group finishes: 7
    // exchanges instead of 24.
    const bool h = (lane & 32) != 0, g = (lane & 16) != 0;
    double k0 = h ? sw : sa, k1 = h ? -sq : sb;
    k0 += shfl_xor_d(h ? sa : sw, 32);
    k1 += shfl_xor_d(h ? sb : -sq, 32);
    red = g ? k1 : k0;
    red += shfl_xor_d(g ? k0 : k1, 16);
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) red += shfl_xor_d(red, o);
  } else {
    // bonus: S_p alone (S_q = 0, w = S_p, dw/drho = -0)
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) sa += shfl_xor_d(sa, o);
    const int q = lane >> 4;
    red = (q & 1) ? (q == 1 ? 0.0 : -0.0) : sa;
  }
  nkd = 0.0;
#pragma unroll
  for (int j = 0; j < kKinkSlots; ++j) ka[j] = kb[j] = 0.0;
  if constexpr (KIND == 0 && RESID) {
    static_assert(kKinkSlots == 2, "two recorded kink elements");
    int nk = 0;
#pragma unroll
    for (int e = 0; e < kSegPerThread; ++e) nk += __popcll(km[e]);
    nkd = (double)nk;
    if (nk > 0 && nk <= kKinkSlots) {  // wave-uniform, rare
      int kj0 = -1, kj1 = -1;          // element offsets within the chunk
#pragma unroll
      for (int e = 0; e < kSegPerThread; ++e) {
        uint64_t m = km[e];
        while (m) {
          const int off = __builtin_ctzll(m) * kSegPerThread + e;
          m &= m - 1;
          if (kj0 < 0) kj0 = off;
          else if (kj1 < 0) kj1 = off;
        }
      }
      const long base = (long)chunk * kDrawChunk;
      ka[0] = draw_term<KIND>(load_elem<DT>(prow, base + kj0), c1, c0p, tab);
      kb[0] = draw_term<KIND>(load_elem<DT>(qrow, base + kj0), c1, c0q, tab);
      if (kj1 >= 0) {
        ka[1] = draw_term<KIND>(load_elem<DT>(prow, base + kj1), c1, c0p, tab);
        kb[1] = draw_term<KIND>(load_elem<DT>(qrow, base + kj1), c1, c0q, tab);
      }
    }
  }
}

// This wave's chunks first .. first + count - 1 of the draw (those below
// C2; count is a multiple of kDrawChunksPerWave), with a ring of
// kDrawChunksPerWave run buffers: the first kDrawChunksPerWave chunks' runs
// are loaded up front, and once a chunk is summed its buffer is refilled
// with the chunk kDrawChunksPerWave ahead, so every chunk's sums wait only
// for its own loads and a wave with many chunks keeps its loads in flight
// while it sums.  Every block of the ring but the last refills
// unconditionally (a chunk index past the end loads the last chunk again),
// so the number of loads in flight, and each wait, is fixed.  Lanes 0-8
// publish each chunk's record (one coalesced coherent store).
template <int DT, int NE, int KIND, bool RESID>
__device__ __forceinline__ void wave_draw_chunks(const void* prow, const void* qrow, int V, int C2,
                                                 int first, int count, double c1, double c0p,
                                                 double c0q, double rho32, const double* tab,
                                                 DrawPart* __restrict__ part) {
  constexpr int P = kDrawChunksPerWave;
  const int lane = threadIdx.x & 63;
  constexpr uint32_t fill = run_fill<DT, KIND>();
  RunWords<DT> rp[P], rq[P];
  auto load = [&](int i, int cc) {
    const long j0 = (long)min(cc, C2 - 1) * kDrawChunk + (long)lane * kSegPerThread;
    load_run_words<DT, NE>(prow, j0, V, fill, rp[i]);
    if constexpr (RESID) load_run_words<DT, NE>(qrow, j0, V, fill, rq[i]);
  };
  auto sum_store = [&](int i, int cc) {
    double red, nkd, ka[kKinkSlots], kb[kKinkSlots];
    wave_chunk_sums<DT, KIND, RESID>(rp[i], rq[i], prow, qrow, cc, c1, c0p, c0q, rho32, tab,
                                     red, nkd, ka, kb);
    // One coalesced store of the record: fields 0-3 from lanes 0, 16, 32
    // and 48 (their groups' sums), fields 4-8 (kink count and recorded kink
    // terms, the same in every lane) from lanes 4-8.
    static_assert(sizeof(DrawPart) == 10 * sizeof(double) && kKinkSlots == 2,
                  "DrawPart fields");
    int field = -1;
    double f = red;
    if ((lane & 15) == 0) {
      field = lane >> 4;
    } else if (lane >= 4 && lane <= 8) {
      field = lane;
      f = lane == 4 ? nkd : lane == 5 ? ka[0] : lane == 6 ? ka[1] : lane == 7 ? kb[0] : kb[1];
    }
    if (field >= 0) st_dev_d(reinterpret_cast<double*>(&part[cc]) + field, f);
  };
  const int blocks = count / P;
#pragma unroll
  for (int i = 0; i < P; ++i) load(i, first + i);
  for (int blk = 0; blk + 1 < blocks; ++blk) {
#pragma unroll
    for (int i = 0; i < P; ++i) {
      const int cc = first + blk * P + i;
      if (cc < C2) sum_store(i, cc);  // wave-uniform
      load(i, cc + P);
    }
  }
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const int cc = first + (blocks - 1) * P + i;
    if (cc < C2) sum_store(i, cc);  // wave-uniform
  }
}

// Draw-weight total of one chunk at the exact rho, by one wave, one element
// at a time per lane (rolled: few registers; for chunks with too many
// kink-band elements, which are rare).
template <int DT, int KIND>
__device__ double wave_chunk_w_exact(const void* prow, const void* qrow, int V, int chunk,
                                     double c1, double c0p, double c0q, double rho,
                                     const double* tab) {
  const int lane = threadIdx.x & 63;
  const long j0 = (long)chunk * kDrawChunk + (long)lane * kSegPerThread;
  double w = 0.0;
#pragma unroll 1
  for (int e = 0; e < kSegPerThread; ++e) {
    if (j0 + e >= V) break;
    const double a = draw_term<KIND>(load_elem<DT>(prow, j0 + e), c1, c0p, tab);
    const double bq = draw_term<KIND>(load_elem<DT>(qrow, j0 + e), c1, c0q, tab);
    w += fmax(0.0, a - rho * bq);
  }
  return wave_sum_d(w);
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
  // Unconditional loads (index clamped, then replaced by the fill), so they
  // are all in flight together instead of one round trip each.
  const void* qsrc = resid ? qrow : prow;
#pragma unroll
  for (int e = 0; e < kSearchPerThread; ++e) {
    const long j = min(j0 + e, (long)V - 1);
    zp[e] = load_elem<DT>(prow, j);
    zq[e] = load_elem<DT>(qsrc, j);
  }
#pragma unroll
  for (int e = 0; e < kSearchPerThread; ++e) {
    if (!(j0 + e < V)) zp[e] = fill;
    if (!(resid && j0 + e < V)) zq[e] = fill;
  }
  // Runs once per request on a cold instruction cache: rolled.
#pragma unroll 1
  for (int e = 0; e < kSearchPerThread; ++e) {
    const double a = draw_term<KIND>(zp[e], c1, c0p, tab);
    w[e] = resid ? fmax(0.0, a - rho * draw_term<KIND>(zq[e], c1, c0q, tab)) : a;
  }
}

// Search one chunk with the exact weights.  Returns the first element whose
// running sum, added to the prefix P of the earlier chunks, exceeds thr,
// falling back to the chunk's last positive-weight element (reachable only
// through a last-bit difference between the chunk total used to locate it
// and the sums here).
template <int DT, int KIND>
__device__ int search_chunk(const void* prow, const void* qrow, int V, int chunk, bool resid,
                            double c1, double c0p, double c0q, double rho, const double& P,
                            double thr, const double* tab) {
  __shared__ int s_tok, s_last;
  if (threadIdx.x == 0) {
    s_tok = INT_MAX;
    s_last = -1;
  }
  double w[kSearchPerThread];
  long j0;
  search_terms<DT, KIND>(prow, qrow, V, chunk, resid, c1, c0p, c0q, rho, tab, w, j0);
  double tsum = 0.0;
#pragma unroll
  for (int e = 0; e < kSearchPerThread; ++e) tsum += w[e];
  // The scan's barriers order the initialisation above and the caller's
  // store of P before the reads below.
  const double excl = block_exclusive_scan_d(tsum);
  const double P0 = P;
  int tok = INT_MAX, lastpos = -1;
  double run = 0.0;
#pragma unroll
  for (int e = 0; e < kSearchPerThread; ++e) {
    run += w[e];
    if (j0 + e < V) {
      if (w[e] > 0.0) lastpos = static_cast<int>(j0 + e);
      if (tok == INT_MAX && P0 + (excl + run) > thr) tok = static_cast<int>(j0 + e);
    }
  }
  // Element indices grow with the lane: the wave's first hit is in its
  // lowest hitting lane, its last positive weight in its highest lane.
  const int lane = threadIdx.x & 63;
  const uint64_t mt = __ballot(tok != INT_MAX), ml = __ballot(lastpos >= 0);
  if (mt != 0 && lane == __builtin_ctzll(mt)) atomicMin(&s_tok, tok);
  if (ml != 0 && lane == 63 - __builtin_clzll(ml)) atomicMax(&s_last, lastpos);
  __syncthreads();
  return s_tok == INT_MAX ? s_last : s_tok;
}

// Counter-region position of request b's ready slot: that of request j,
// j = b with its two bytes swapped, so the slots of up to 256 consecutive
// requests are 8 KB apart: many work-groups waiting on neighbouring
// requests then poll different memory channels instead of one.
__device__ __forceinline__ long handover_pos(int b) {
  static_assert(kMaxB == 65536, "two-byte request index");
  return (long)((b & 255) << 8 | (b >> 8 & 255)) * kCountersPerReq;
}
// Ready slot: two 64-bit words that hold the request's packed draw state
// once its acceptance tests are done, both zero otherwise (the request's
// draw clears them).
__device__ __forceinline__ uint64_t* ready_slot(unsigned* counters, int b) {
  return reinterpret_cast<uint64_t*>(&counters[handover_pos(b) + kReadySlotWord]);
}

// Packed draw state: word 0 = (n + 1, mp), word 1 = (mq, rho32 as float with
// the sign bit set).  Neither word of a published state is zero, so a reader
// that sees both nonzero has the whole state whatever order the two stores
// arrive in.  rho32 only places the kink band (relative width 1e-5) and the
// linear correction's base point, so float precision suffices.
__device__ __forceinline__ void pack_state(const ReqState& st, uint64_t& w0, uint64_t& w1) {
  w0 = (uint64_t)(uint32_t)(st.n + 1) | ((uint64_t)__float_as_uint(st.mp) << 32);
  w1 = (uint64_t)__float_as_uint(st.mq) |
       ((uint64_t)(__float_as_uint((float)st.rho32) | 0x80000000u) << 32);
}
__device__ __forceinline__ ReqState unpack_state(uint64_t w0, uint64_t w1, int k) {
  ReqState st;
  st.n = (int)(uint32_t)w0 - 1;
  st.mode = st.n < k ? kModeResidual : kModeBonus;
  st.mp = __uint_as_float((uint32_t)(w0 >> 32));
  st.mq = __uint_as_float((uint32_t)w1);
  st.rho32 = (double)__uint_as_float((uint32_t)(w1 >> 32) & 0x7fffffffu);
  return st;
}

// ReqState through coherent 64-bit words (read by other work-groups).
__device__ __forceinline__ void st_dev_state(ReqState* p, const ReqState& v) {
  static_assert(sizeof(ReqState) == 24, "ReqState layout");
  const uint64_t* w = reinterpret_cast<const uint64_t*>(&v);
  uint64_t* d = reinterpret_cast<uint64_t*>(p);
  st_dev(&d[0], w[0]);
  st_dev(&d[1], w[1]);
  st_dev(&d[2], w[2]);
}
__device__ __forceinline__ ReqState ld_dev_state(const ReqState* p) {
  ReqState v;
  uint64_t* w = reinterpret_cast<uint64_t*>(&v);
  const uint64_t* s = reinterpret_cast<const uint64_t*>(p);
  w[0] = ld_dev(&s[0]);
  w[1] = ld_dev(&s[1]);
  w[2] = ld_dev(&s[2]);
  return v;
}


// Ready-slot value of a request whose acceptance tests gave up: both words
// all ones (a published state never has 0xffffffff as its low word, n + 1).
constexpr uint64_t kSlotFailed = ~0ull;

// Workspace status word (sticky SPEC_STATUS_* bits) and the call epoch of
// graph-captured calls, in the counter region's reserved tail.
__device__ __forceinline__ unsigned* status_word(unsigned* counters) {
  return &counters[kStatusWord];
}
__device__ __forceinline__ uint64_t* epoch_word(unsigned* counters) {
  return reinterpret_cast<uint64_t*>(&counters[kEpochWord]);
}
// Completion tag of a graph-captured call from the workspace's call epoch:
// a marker byte other than that of the host's per-call tags, so no tag of
// one kind equals one of the other.
__device__ __forceinline__ uint64_t epoch_tag(uint64_t epoch) {
  return (0xC4ull << 56) | (epoch & ((1ull << 56) - 1));
}
// A bounded wait gave up: set the sticky status bit, and wait until the
// atomic has completed, so that whatever this thread publishes next (a
// failed verdict or slot, a ticket) is seen only after it.
__device__ __forceinline__ void note_give_up(unsigned* counters) {
  __hip_atomic_fetch_or(status_word(counters), (unsigned)SPEC_STATUS_WAIT_GAVE_UP,
                        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  wait_stores();
}

// One thread waits until both words of a ready slot are set and returns
// them.  False if the bound (`spin` polls) is reached.
__device__ __forceinline__ bool wait_slot(const uint64_t* slot, uint64_t& w0, uint64_t& w1,
                                          long spin_limit) {
  for (long spin = 0; spin < spin_limit; ++spin) {
    w0 = ld_dev(&slot[0]);
    w1 = ld_dev(&slot[1]);
    if (w0 != 0 && w1 != 0) return true;
    // A few quick polls, then about 2000 cycles between polls.
    if (spin < 4) __builtin_amdgcn_s_sleep(2);
    else __builtin_amdgcn_s_sleep(32);
  }
  return false;
}


}  // namespace specv
