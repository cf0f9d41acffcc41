/*
 * spec_verify.h — C ABI of the batched speculative-decoding verifier for
 * AMD MI355X (gfx950).
 *
 * The operation is the verification step of speculative decoding as the
 * pages define it:
 *   - "EAGLE-3 speculative decoding review" (6unoyunr.github.io), section
 *     "Speculative Decoding" (the draft / verify / accept-or-reject cycle),
 *     the section asking whether a small draft hurts quality (greedy rule,
 *     acceptance probability A(x) = min(1, p(x)/q(x)), residual
 *     p_residual = norm(max(0, p - q))), and the section on the full EAGLE-3
 *     inference loop (tree verification, strict acceptance);
 *   - the speculative-decoding chapter of an LLM-serving book
 *     (froggydisk.github.io), sections on how it works and on the acceptance
 *     rule that preserves the output distribution.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers are DEVICE pointers unless the parameter name ends in _host.
 *  - Tensors are dense, row-major, the vocabulary axis V contiguous.  bf16
 *    tensors hold IEEE bfloat16 bit patterns.
 *  - All buffers are owned by the caller.  The library never allocates,
 *    frees or synchronises inside a call; kernels are enqueued on `stream`
 *    (a hipStream_t passed as void*; NULL = the default stream) and the
 *    outputs are valid once that stream has been synchronised.
 *  - `ws` is a caller-owned device workspace of at least
 *    spec_workspace_bytes(B, n_pos, V) bytes.  It must be zero-filled before
 *    its first use.  Its first SPEC_WORKSPACE_COUNTER_BYTES bytes are the
 *    counter region: per-request completion counters, verdict words and
 *    ready slots at fixed places, which every completed call leaves zero
 *    again, so one workspace serves calls of any shape without clearing it;
 *    then a status word (SPEC_STATUS_*, sticky) and the call epoch of
 *    graph-captured calls.  The caller must not write to the counter region
 *    other than through spec_workspace_reset.  The rest is scratch that
 *    each call writes before reading.  Calls that share a workspace must be
 *    ordered on one stream.
 *  - Return value: SPEC_OK, or a negative code.  Any code other than
 *    SPEC_EHIP means the arguments were rejected on the host and nothing was
 *    enqueued.  SPEC_EHIP reports a failed HIP launch.
 *  - Device-side failure: the one-launch sampling kernels hand results
 *    between work-groups through bounded waits.  A wait that gives up (it
 *    never does while every work-group of the launch gets to run) sets
 *    SPEC_STATUS_WAIT_GAVE_UP in the workspace status word and the request
 *    it concerns gets accepted_len = -1 and out_tokens all -1.  The bit
 *    stays set: until spec_workspace_reset, every one-launch sampling call on
 *    that workspace writes those -1 outputs for every request.  Read it with
 *    spec_workspace_status.
 *  - Inputs must be finite except that -inf marks a masked token.  Every
 *    row must hold at least one finite value.
 *  - A draft or node token outside [0, V) is a rejection (sampling) or a
 *    mismatch (greedy); it is never used as an index.
 *  - Sizes: 0 <= B <= 65536, 0 <= k <= 1023, 1 <= V <= 2^30, 1 <= n_nodes <= 1024.
 *    B == 0 is a no-op that returns SPEC_OK.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes at the start of every workspace that must be zero before the first
 * call (the counter region); each completed call leaves its per-request
 * words zero. */
#define SPEC_WORKSPACE_COUNTER_BYTES (2097152 + 256)

/* Element type of logit / probability tensors. */
enum { SPEC_F32 = 0, SPEC_BF16 = 1 };

/* What the sampling rows hold.
 * SPEC_LOGITS: raw logits; p = softmax(target / T), q = softmax(draft / T).
 * SPEC_PROBS:  float32 probabilities used as given (T must be 1). */
enum { SPEC_LOGITS = 0, SPEC_PROBS = 1 };

enum {
  SPEC_OK = 0,
  SPEC_EINVAL = -1,     /* null pointer, size or scalar out of range */
  SPEC_EDTYPE = -2,     /* unsupported dtype / kind combination */
  SPEC_EWORKSPACE = -3, /* workspace null or smaller than required */
  SPEC_EHIP = -4,       /* a HIP launch failed */
  SPEC_ETREE = -5,      /* parent array is not a tree in BFS-compatible order */
  SPEC_ESCRATCH = -6    /* shape needs more than SPEC_NOALLOC_SCRATCH_BYTES */
};

/* Human-readable text for a return code (static storage). */
const char* spec_strerror(int code);

/* Workspace bytes needed by any entry point for B requests of n_pos
 * positions (k + 1 for chains, n_nodes for trees) over a vocabulary of V.
 * Returns 0 for invalid sizes. */
size_t spec_workspace_bytes(int B, int n_pos, int V);

/* Uniforms from a seed.  out[i] = (SplitMix64 output number counter0 + i of
 * the stream seeded with `seed`) >> 40, times 2^-24: a float in [0, 1) on
 * the 2^-24 grid.  SplitMix64 as in Steele, Lea & Flood (OOPSLA 2014):
 * output(ctr) = mix(seed + (ctr + 1) * 0x9E3779B97F4A7C15 mod 2^64).
 * The pages tie reproducible sampling to the seed and to the order in which
 * random numbers are used (EAGLE-3 review, sections on interpreting
 * losslessness and on lossless versus numerically identical output); this
 * counter form makes each value independent of the order of use.
 * out: device float[n].  n >= 0. */
int spec_fill_uniforms(uint64_t seed, uint64_t counter0, int64_t n, float* out,
                       void* stream);

/* Greedy chain verification (EAGLE-3 review, greedy bullets of the section
 * on whether a small draft hurts quality; serving chapter, last sentence of
 * the acceptance-rule section).  For each request b:
 *   a_i = argmax_j target[b, i, j] (lowest j on ties), i = 0..k;
 *   n_b = first i < k with draft_tokens[b, i] != a_i, or k;
 *   accepted_len[b] = n_b;
 *   out_tokens[b, 0..n_b-1] = draft_tokens[b, 0..n_b-1];
 *   out_tokens[b, n_b] = a_{n_b};  out_tokens[b, n_b+1..k] = -1.
 * target: [B, k+1, V] of `dtype` (SPEC_F32 or SPEC_BF16).
 * draft_tokens: int32 [B, k] (may be NULL when k == 0).
 * accepted_len: int32 [B].  out_tokens: int32 [B, k+1]. */
int spec_verify_greedy(const void* target, int dtype, int B, int k, int V,
                       const int32_t* draft_tokens, int32_t* accepted_len,
                       int32_t* out_tokens, void* ws, size_t ws_bytes,
                       void* stream);

/* Sampling chain verification with the rule min(1, p(x)/q(x)) (EAGLE-3
 * review, equation A(x) and the residual equation; serving chapter,
 * acceptance-rule section; stop at the first rejection and the bonus token:
 * EAGLE-3 review "Speculative Decoding" step 3, serving chapter "how it
 * works").  For each request b, positions i = 0..k-1 in order:
 *   x = draft_tokens[b, i];  accept iff 0 <= x < V and u_acc < p_i(x)/q_i(x)
 *   (a zero q_i(x) accepts iff p_i(x) > 0);
 *   at the first rejection n: draw t from normalise(max(0, p_n - q_n)) by
 *   inverse CDF with u_res (t = min{ j : C_j > u_res * C_{V-1} }, C the
 *   running sum over ascending token id); if that residual has zero mass,
 *   draw from p_n with the same u_res;
 *   if all k are accepted: n = k and t is drawn from p_k the same way.
 *   accepted_len[b] = n; out_tokens[b] = draft_tokens[b, 0..n-1], t, then -1.
 * Uniforms: u_acc = u[b, i, 0], u_res = u[b, n, 1], where u is `uniforms`
 * (device float [B, k+1, 2]) or, when `uniforms` is NULL, the values
 * spec_fill_uniforms(seed, counter0, ...) would write to such an array.
 * dtype/kind: SPEC_LOGITS with SPEC_F32 or SPEC_BF16 (temperature > 0,
 * finite, 1/temperature finite); SPEC_PROBS with SPEC_F32 (temperature 1).
 * target: [B, k+1, V]; draft: [B, k, V] (may be NULL when k == 0).
 * probe (nullable): float [B, k+1, 4]; for i < k, probe[b,i,0] = p_i(x_i)
 * and probe[b,i,1] = q_i(x_i) (0 for an out-of-range token); probe[b,n,2] =
 * total mass of the distribution drawn from at position n (the residual mass
 * sum max(0, p_n - q_n) after a rejection, sum p_k for the bonus draw); all
 * other entries 0.
 * Arithmetic: row statistics (max, log-sum-exp) in float32 with float64
 * merges; the acceptance ratio in float64; the residual / bonus draw in
 * float64 (normalisers, weights and running sums).
 * flags: one SPEC_SCHED_* value (how the work is scheduled; every schedule
 * gives identical outputs), optionally or-ed with SPEC_FLAG_TEST_GIVE_UP;
 * any other bit is SPEC_EINVAL.  SPEC_PROBS rows always take one draw
 * kernel and ignore the schedule. */
int spec_verify_sample(const void* target, const void* draft, int dtype, int kind,
                       int B, int k, int V, const int32_t* draft_tokens,
                       const float* uniforms, uint64_t seed, uint64_t counter0,
                       float temperature, int flags, int32_t* accepted_len,
                       int32_t* out_tokens, float* probe, void* ws,
                       size_t ws_bytes, void* stream);

/* Schedules of spec_verify_sample for raw logits (the low four bits of
 * `flags`).
 * SPEC_SCHED_ONE_LAUNCH: one kernel that reads every row once.  The rows of
 *   each request's early positions come first; most requests stop at one of
 *   them (stop at the first rejection: EAGLE-3 review "Speculative
 *   Decoding" step 3), so their draws run while the rows of later positions
 *   stream.
 * SPEC_SCHED_TWO_LAUNCH: the row pass, then the draw, as two kernels.
 * SPEC_SCHED_EARLY_EXIT: as SPEC_SCHED_ONE_LAUNCH, except that the row pass
 *   stops reading a row once its request is known to stop before that row's
 *   position (such rows cannot change any output), so fewer bytes are read.
 *   With probe values asked for, every row is read as with
 *   SPEC_SCHED_ONE_LAUNCH.
 * SPEC_SCHED_AUTO: SPEC_SCHED_EARLY_EXIT when the row pass needs more than
 *   one round of resident work-groups (B * (2k+1) * ceil(V / 65536) above
 *   five per compute unit), SPEC_SCHED_TWO_LAUNCH when it needs at most a
 *   third of one, else SPEC_SCHED_ONE_LAUNCH: the fastest for the shape as
 *   measured (every schedule gives the same outputs).
 * Graph capture: on a stream that is being captured (hipStreamIsCapturing),
 * the one-launch schedules take their completion tags from a call epoch in
 * the workspace and add a one-thread kernel that advances it, so every
 * replay of the graph has tags of its own. */
enum {
  SPEC_SCHED_AUTO = 0,
  SPEC_SCHED_ONE_LAUNCH = 1,
  SPEC_SCHED_TWO_LAUNCH = 2,
  SPEC_SCHED_EARLY_EXIT = 3
};
/* Test only: in a one-launch schedule, the row-pass work-group of request 0,
 * position 0, chunk 0 never marks its chunk complete and every bounded wait
 * gives up after 256 polls, so the failure path above runs while every
 * kernel still exits normally. */
#define SPEC_FLAG_TEST_GIVE_UP 0x100

/* Workspace status word: byte offset in the workspace and its bits. */
#define SPEC_WORKSPACE_STATUS_OFFSET 2097152
#define SPEC_STATUS_WAIT_GAVE_UP 1u

/* Waits for `stream` and reads the workspace status word into *status_host
 * (0: no failure since the last reset).  ws: a workspace as above. */
int spec_workspace_status(const void* ws, size_t ws_bytes, uint32_t* status_host,
                          void* stream);

/* Enqueues on `stream` a kernel that zeroes the counter region (per-request
 * words and status word; the call epoch is kept), so a workspace whose
 * status is nonzero can be used again. */
int spec_workspace_reset(void* ws, size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory (code under graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * spec_verify_sample without a workspace argument.  It allocates nothing:
 * its scratch (counters, row statistics, per-request state, draw partials)
 * is a static device array of SPEC_NOALLOC_SCRATCH_BYTES inside the
 * library, one per GPU, held until the process ends.  A shape whose
 * spec_workspace_bytes(B, k+1, V) exceeds that size returns SPEC_ESCRATCH
 * and enqueues nothing.  `stream` must belong to the current device (else
 * SPEC_EINVAL).  Each call first clears, with a kernel on `stream`, the
 * counters its requests use and the status word, so a call whose bounded
 * wait gave up (its outputs are -1) leaves nothing behind for the next.
 * Every call on one GPU shares that GPU's array: calls that overlap in time
 * on one GPU (other streams, other host threads) race and may give wrong
 * outputs.  Arguments, outputs and the other return codes are those of
 * spec_verify_sample. */
#define SPEC_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)
int spec_verify_sample_noalloc(const void* target, const void* draft, int dtype, int kind,
                               int B, int k, int V, const int32_t* draft_tokens,
                               const float* uniforms, uint64_t seed, uint64_t counter0,
                               float temperature, int flags, int32_t* accepted_len,
                               int32_t* out_tokens, float* probe, void* stream);

/* Greedy tree verification (EAGLE-3 review, section on the full inference
 * loop: tree attention gives the target's distribution after every node, and
 * strict acceptance keeps the longest prefix that matches the target's
 * choice).  Node 0 is the root; node j > 0 has parent parent_host[j] < j and
 * carries token node_tokens[b, j] (column 0 is ignored).  target[b, j] is
 * the target's distribution after node j's prefix.  Let a_j = argmax
 * target[b, j] (lowest id on ties).  Node j > 0 is accepted iff its parent
 * is accepted and node_tokens[b, j] == a_{parent(j)}; the root is accepted.
 * d* = the deepest accepted node (lowest index among equal depths).
 *   accepted_len[b] = depth(d*);
 *   out_tokens[b] = tokens of the nodes on the root->d* path (root
 *   excluded), then a_{d*}, then -1 up to D+1 entries (D = tree depth);
 *   out_path[b] (nullable) = node ids of the path from the root (0 first),
 *   then -1 up to D+1 entries.
 * parent_host: HOST int32 [n_nodes], parent[0] = -1, 0 <= parent[j] < j;
 * read during the call only.  target: [B, n_nodes, V] of dtype.
 * node_tokens: int32 [B, n_nodes].  accepted_len: int32 [B].
 * out_tokens, out_path: int32 [B, D+1]. */
int spec_verify_tree_greedy(const void* target, int dtype, int B, int n_nodes,
                            int V, const int32_t* parent_host,
                            const int32_t* node_tokens, int32_t* accepted_len,
                            int32_t* out_tokens, int32_t* out_path, void* ws,
                            size_t ws_bytes, void* stream);

/* Sampling verification over a draft tree (EAGLE-3 review, section on the
 * full inference loop, step 4 "Strict Acceptance": over the tree, the
 * min(1, p/q) test with residual correction, which keeps the target
 * distribution).  The pages give no rule for several siblings; the one used
 * is SpecInfer's multi-step speculative sampling (Miao et al., ASPLOS 2024).
 * Node 0 is the root; node j > 0 has parent parent_host[j] < j and carries
 * token node_tokens[b, j] (column 0 is ignored).  target[b, j] and
 * draft[b, j] are the target's and the draft's rows after node j's prefix
 * (node j's children were drawn from the draft's; draft rows of nodes
 * without children are not read).  For each request b, with p_j, q_j the
 * rows' distributions as in spec_verify_sample:
 *   n := 0 (the root), r := p_0.  For the children c of n in increasing
 *   index, x = node_tokens[b, c]: c is accepted iff 0 <= x < V and
 *   u_acc(c) < r(x) / q_n(x) (a zero q_n(x) accepts iff r(x) > 0).  On
 *   acceptance n := c, r := p_c, and the children of c are tried.  On
 *   rejection r := normalise(max(0, r - q_n)), unless that is all zero
 *   (then r stays).  When no child of n is accepted (or n has none), t is
 *   drawn from r by inverse CDF with u_res(n) (t = min{ j : C_j > u_res *
 *   C_{V-1} }, C the running sum over ascending token id) and the request
 *   stops.
 *   accepted_len[b] = depth(n); out_tokens[b] (int32 [B, D+1], D the tree
 *   depth) = the tokens of the path's nodes below the root, t, then -1;
 *   out_path[b] (nullable, int32 [B, D+1]) = node ids root .. n, then -1.
 * Uniforms: u_acc(c) = u[b, c, 0], u_res(n) = u[b, n, 1], where u is
 * `uniforms` (device float [B, n_nodes, 2]) or, when NULL, the values
 * spec_fill_uniforms(seed, counter0, ...) would write to such an array.
 * dtype, kind and temperature as in spec_verify_sample.  Arithmetic:
 * float32 row statistics (logits); tests, residual masses and the draw in
 * float64.  Workspace: spec_workspace_bytes(B, n_nodes, V).  One call
 * enqueues five kernels (four for SPEC_PROBS) plus one per sibling rank
 * above 0 that occurs in the tree. */
int spec_verify_tree_sample(const void* target, const void* draft, int dtype, int kind, int B,
                            int n_nodes, int V, const int32_t* parent_host,
                            const int32_t* node_tokens, const float* uniforms, uint64_t seed,
                            uint64_t counter0, float temperature, int32_t* accepted_len,
                            int32_t* out_tokens, int32_t* out_path, void* ws, size_t ws_bytes,
                            void* stream);

/* Depth D of the tree described by parent_host (see above), or a negative
 * error code if the array is malformed.  Host only. */
int spec_tree_depth(const int32_t* parent_host, int n_nodes);

/* Rejected drafts of a chain verification, for KV-cache trimming.  The
 * target's forward pass wrote a KV entry for each of the k drafted tokens;
 * only those of the accepted prefix stay, and drafting resumes from the
 * confirmed prefix (EAGLE-3 review, section on the full inference loop,
 * step 5 "KV cache update").  A serving engine marks the others in a
 * rejected-token mask and points their slot-mapping entries at a padding
 * slot ("[vLLM] EAGLE" code walk, sections on rejected-token handling and on
 * slot mapping / KV-cache management).
 *   rejected[b, i] = 1 if i >= accepted_len[b], else 0   (i = 0 .. k-1);
 *   slot_mapping (nullable): slot_mapping[b, i] = pad_slot where
 *   rejected[b, i] = 1, left unchanged elsewhere.
 * accepted_len: int32 [B] (as written by spec_verify_sample or
 * spec_verify_greedy; any value is accepted, a value >= k rejects nothing).
 * rejected: uint8 [B, k].  slot_mapping: int64 [B, k], updated in place.
 * One small kernel on `stream`. */
int spec_rejected_mask(const int32_t* accepted_len, int B, int k, uint8_t* rejected,
                       int64_t* slot_mapping, int64_t pad_slot, void* stream);

/* Rejected nodes of a tree verification, for KV-cache trimming (same
 * sources as spec_rejected_mask).  Node j > 0 is kept iff it lies on the
 * accepted root-to-node path; the root (node 0, the last confirmed token)
 * is never rejected.
 *   rejected[b, j] = 1 if j > 0 and j is not in out_path[b, 0..depth],
 *   else 0;  slot_mapping (nullable) as for spec_rejected_mask.
 * out_path: int32 [B, depth+1] as written by spec_verify_tree_greedy (node
 * ids, -1 after the path's end; entries outside [0, n_nodes) mark nothing).
 * depth: the tree depth D (spec_tree_depth), 0 <= D < n_nodes <= 1024.
 * rejected: uint8 [B, n_nodes].  slot_mapping: int64 [B, n_nodes]. */
int spec_tree_rejected_mask(const int32_t* out_path, int B, int n_nodes, int depth,
                            uint8_t* rejected, int64_t* slot_mapping, int64_t pad_slot,
                            void* stream);

/* Parent array of a draft tree given as a list of choices ("[vLLM] EAGLE"
 * code walk, section on tree-structured drafting: each node is the tuple of
 * child ranks on the path from the root, listed level by level).  Host
 * only.  Choice j is the sequence choices_host[j, 0 .. lengths_host[j]-1]
 * (int32 [n_choices, width], entries >= 0); it becomes node j + 1, whose
 * parent is the node of the same sequence without its last entry, or the
 * root 0 for a one-entry choice.  Writes parent_host[0 .. n_choices]
 * (parent[0] = -1) and returns n_nodes = n_choices + 1.  Errors: SPEC_EINVAL
 * (null pointer, n_choices + 1 > 1024, width < 1, a length outside
 * [1, width]); SPEC_ETREE (a negative entry, a choice listed twice, or a
 * choice whose parent is not listed before it).  parent_host may be
 * partly written on error. */
int spec_tree_from_choices(const int32_t* choices_host, const int32_t* lengths_host,
                           int n_choices, int width, int32_t* parent_host);


/* Optional per-kernel timing for measurement tools (not part of the
 * verification itself).  spec_profile_enable(1) clears the totals and, from
 * then on, times every kernel the library enqueues with a start/stop pair of
 * HIP events on the same stream; spec_profile_enable(0) stops recording.  spec_profile_read
 * waits for the recorded events and returns, for one kernel kind, the number
 * of timed launches and their summed event time in milliseconds.  The events
 * are stamped by each kernel's own dispatch, so an interval covers that
 * kernel alone.  Kinds: */
enum {
  SPEC_KERNEL_ROW_PASS = 0, /* row pass over every logit row + per-request finish
                               (acceptance tests, greedy rule, tree walk) */
  SPEC_KERNEL_DRAW = 1,     /* float64 residual / bonus pass + inverse-CDF draw */
  SPEC_KERNEL_UNIFORMS = 2, /* spec_fill_uniforms */
  SPEC_KERNEL_FUSED = 3,    /* one-launch sampling verification: row pass and draw */
  SPEC_KERNEL_SERVING = 4,  /* rejected-draft masks */
  SPEC_KERNEL_TREE_STATS = 5, /* tree sampling: row statistics */
  SPEC_KERNEL_TREE_MASS = 6,  /* tree sampling: residual-mass rounds */
  SPEC_KERNEL_TREE_WALK = 7,  /* tree sampling: table setup and the walk */
  SPEC_KERNEL_TREE_DRAW = 8,  /* tree sampling: draw weights and the pick */
  SPEC_KERNEL_TREE_LEAF = 9   /* tree sampling: the stop leaves' row statistics */
};
int spec_profile_enable(int on);
int spec_profile_read(int kind, long* launches, double* total_ms);
/* The durations (milliseconds, in launch order) of the timed launches of one
 * kernel kind since spec_profile_enable(1): writes min(cap, count) of them to
 * ms_host (HOST float[cap]) and the count to *n_host.  Waits for the
 * recorded events. */
int spec_profile_durations(int kind, float* ms_host, long cap, long* n_host);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
