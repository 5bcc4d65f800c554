/*
 * specverify -- the verification step of speculative decoding on MI355X (gfx950).
 *
 * What one call computes (per sequence b of a batch):
 *
 *   SV_MODE_SAMPLE -- modified rejection sampling.  Source: the
 *     edgeinferencenotes.hashnode.dev speculative-decoding / EAGLE-3 article,
 *     section "The core idea: draft, then check": with p the target's and q the
 *     draft's probability of a drafted token, accept it outright if p >= q and
 *     otherwise with probability p/q; at the first rejection drop the rest and
 *     draw one replacement from the leftover mass max(0, p - q) renormalised;
 *     if all k drafts are accepted, draw one bonus token from the target's
 *     last row.  Section "Why it changes nothing about the output": temperature,
 *     top-k and nucleus (top-p) apply to both distributions before the test.
 *       p'_j = adjust(target row j), q'_j = adjust(draft row j) with
 *       adjust = z = logits / T, then top-k (exactly top_k entries by value,
 *       lower index first on ties), then softmax, then top-p (the smallest
 *       prefix in (probability desc, index asc) order whose mass reaches
 *       top_p), renormalised.
 *       accept draft j iff  q'_j(x_j) > 0 and u_j < min(1, p'_j(x_j)/q'_j(x_j)),
 *                       or  q'_j(x_j) = 0 and p'_j(x_j) > 0.
 *       n = first rejected j (k if none).  Replacement / bonus drawn with the
 *       per-sequence uniform ur as y = min{v : C_v > ur * C_{V-1}}, C the
 *       running sum of r = max(0, p'_n - q'_n) (n < k; p'_n if that is all
 *       zero) or r = p'_k (n = k), in vocabulary order.
 *       Emitted: x_0 .. x_{n-1}, y.
 *
 *   SV_MODE_GREEDY -- greedy longest agreed prefix.  Source: "Towards Green
 *     Text Generation: Memory-Based Speculative Decoding", section 1 and
 *     section 2.4 "Verifier and Acceptance": the logits of the k+1 positions
 *     are compared greedily with the drafts; a draft is accepted iff it equals
 *     the verifier's argmax (token-ID level).  g_j = argmax row j (lower index
 *     on ties); n = first j with x_j != g_j (k if none); emitted x_0..x_{n-1}, g_n.
 *
 *   SV_MODE_TREE_GREEDY -- greedy token-tree verification.  Source: the same
 *     article, section "One decode round, end to end": the flattened tree is
 *     scored in one target pass, the accept-or-correct rule is applied down
 *     the branches, the longest agreed path is committed plus one correction.
 *     Node 0 is the root; parents[i] < i; row i is the target's distribution
 *     for node i's children.  Node i is accepted iff its parent is accepted
 *     and tokens[i] == argmax(row parents[i]).  d* = accepted node of largest
 *     depth (smallest index on ties).  Emitted: the tokens on the path root ->
 *     d* (root excluded), then argmax(row d*).
 *
 *   SV_MODE_TREE_SAMPLE -- modified rejection sampling down a token tree.
 *     Source: the same article, "One decode round, end to end" (the
 *     accept-or-correct rule of "The core idea" applied down the branches,
 *     one correction resampled at the first rejection) and "Why it changes
 *     nothing about the output".  The pages give no rule for several
 *     children of one node; this library tries them in index order against
 *     a running target: at the accepted node u (root first), r = p'_u;
 *     child c with token x is accepted iff q'_u(x) > 0 and u_c < min(1,
 *     r(x)/q'_u(x)), or q'_u(x) = 0 and r(x) > 0; a rejected child replaces r
 *     by max(0, r - q'_u) renormalised (unless that is all zero).  The
 *     first accepted child becomes the node; when none is, or u has no
 *     child, y is drawn from r with the tree's uniform as in SV_MODE_SAMPLE.
 *     Row i of the target and of the draft is that model's distribution for
 *     node i's children, adjusted as in SV_MODE_SAMPLE (temperature, then
 *     top-k, then top-p, on every row); the children of a node are taken to
 *     be drawn independently from q'_u, which makes the emitted tokens
 *     follow the target.  Emitted: the path's tokens (root excluded), then y.
 *
 * Layout: all arrays are dense, row-major, vocabulary fastest, and live in
 * device memory on the context's device.  Logits are float32 or bf16 (raw
 * 16-bit patterns).  Tokens and outputs are int32; uniforms are float32 in
 * [0, 1).  The library reads inputs and writes outputs only; the caller owns
 * every buffer passed in.  The context owns a device workspace sized at
 * create time from max_batch, k and vocab.
 *
 * Errors: every function returns SV_OK (0) or a negative SV_ERR_* code and
 * never aborts.  Argument errors are found on the host before any HIP call
 * and leave the stream untouched.  Bad data inside device buffers never
 * traps: it sets per-sequence bits in seq_status (SV_STATUS_*):
 *   BAD_TOKEN   a drafted / tree token outside [0, V): treated as rejected
 *   BAD_PARENT  parents[i] not in [0, i) (or parents[0] != -1): node unreachable
 *   BAD_LOGITS  a row the mode reads holds NaN or +inf, or only -inf: the
 *               sequence emits nothing (accepted_len 0, outputs all -1)
 * specverify_run is asynchronous on the given stream and does no host
 * synchronisation; outputs are valid once the stream has reached the call.
 * One context must not be used by two streams at the same time.
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct specverify_ctx specverify_ctx;   /* opaque; owns the workspace only */

enum { SV_MODE_SAMPLE = 0, SV_MODE_GREEDY = 1, SV_MODE_TREE_GREEDY = 2, SV_MODE_TREE_SAMPLE = 3 };
enum { SV_DTYPE_F32 = 0, SV_DTYPE_BF16 = 1 };
enum {
  SV_OK = 0,
  SV_ERR_NULL = -1,      /* a required pointer is NULL */
  SV_ERR_SHAPE = -2,     /* batch / k / vocab out of range */
  SV_ERR_DTYPE = -3,     /* unknown dtype */
  SV_ERR_PARAM = -4,     /* temperature <= 0 or not finite, top_k < 0 or too large, top_p not in (0, 1],
                            an unknown or unsupported option */
  SV_ERR_CAPACITY = -5,  /* batch > max_batch */
  SV_ERR_HIP = -6,       /* a HIP call failed (allocation, launch, no device) */
  SV_ERR_MODE = -7,      /* unknown mode, or a pointer given / missing for this mode */
  SV_ERR_SCRATCH = -8,   /* specverify_run_static: the call needs more than SV_STATIC_SCRATCH_BYTES */
};
enum { SV_STATUS_BAD_TOKEN = 1, SV_STATUS_BAD_PARENT = 2, SV_STATUS_BAD_LOGITS = 4 };

/* Options (sv_config.options).
 *   SV_OPT_LAZY_ROWS  SV_MODE_SAMPLE without top-k / top-p only (else
 *     SV_ERR_PARAM): the rejection fast path.  Source: "Towards Green Text
 *     Generation: Memory-Based Speculative Decoding", section 2.4 "Verifier
 *     and Acceptance" (the first drafted token is checked against the
 *     logits already at hand before the remaining positions are scored) and
 *     section 5.1 (the verifier's cost).  The call first reads only the row
 *     pair of position 0 of every sequence and tests x_0; the rows of
 *     positions 1..k are read only for sequences whose x_0 was accepted.
 *     Outputs equal those without the option, except that a row never read
 *     (every row after position 0 of a sequence that rejected x_0) is not
 *     checked for NaN / +inf. */
enum { SV_OPT_LAZY_ROWS = 1 };

/* Limits checked by create / check_args. */
#define SV_MAX_K 64          /* chain: drafted tokens per sequence */
#define SV_MAX_TREE_NODES 1024
#define SV_MAX_TOP_K 256
#define SV_MAX_VOCAB (1 << 24)

typedef struct {
  int32_t mode;          /* SV_MODE_* */
  int32_t dtype;         /* SV_DTYPE_* of both logit tensors */
  int32_t max_batch;     /* upper bound on the batch passed to run (>= 1) */
  int32_t k;             /* chain: drafted tokens k (1..SV_MAX_K); tree: node count N incl. root */
  int32_t vocab;         /* V (1..SV_MAX_VOCAB) */
  int32_t options;       /* SV_OPT_* bits; 0 = none */
  double temperature;    /* SAMPLE: T > 0 (logits are divided by T in float64); ignored otherwise */
  int32_t top_k;         /* SAMPLE: 0 = off, else 1..SV_MAX_TOP_K (>= V acts as off) */
  double top_p;          /* SAMPLE: 1.0 = off, else in (0, 1) */
} sv_config;

/* Validate cfg and allocate the workspace on `device`; the calling thread's
 * current device is the same afterwards.  On success *out holds a new context.  Errors: SV_ERR_NULL, SV_ERR_SHAPE, SV_ERR_DTYPE,
 * SV_ERR_PARAM, SV_ERR_MODE (no HIP call made), SV_ERR_HIP. */
int specverify_create(const sv_config* cfg, int device, specverify_ctx** out);

/* Host-only argument check that specverify_run performs first; makes no HIP
 * call, so it can run anywhere.  Pointers are only tested for NULL-ness
 * against what `cfg->mode` needs:
 *   SAMPLE: target, draft, draft_tokens, uniforms, resid_uniforms, accepted_len,
 *           out_tokens required; parents and out_nodes must be NULL.
 *   GREEDY: target, draft_tokens, accepted_len, out_tokens required; draft,
 *           parents, uniforms, resid_uniforms, out_nodes must be NULL.
 *   TREE_GREEDY: target, draft_tokens (the node tokens), parents, accepted_len,
 *           out_tokens required; draft, uniforms, resid_uniforms must be NULL;
 *           out_nodes optional.
 *   TREE_SAMPLE: target, draft, draft_tokens (the node tokens), parents,
 *           uniforms, resid_uniforms, accepted_len, out_tokens required;
 *           out_nodes optional.
 * batch = 0 is valid (nothing to do; every pointer may then be NULL);
 * batch > cfg->max_batch is SV_ERR_CAPACITY. */
int specverify_check_args(const sv_config* cfg, int32_t batch,
                          const void* target_logits, const void* draft_logits,
                          const int32_t* draft_tokens, const int32_t* parents,
                          const float* uniforms, const float* resid_uniforms,
                          const int32_t* accepted_len, const int32_t* out_tokens,
                          const int32_t* out_nodes);

/* Verify one batch.  Shapes (B = batch, k and V from the context's config):
 *   target_logits  [B, k+1, V] chain | [B, N, V] tree      dtype per config
 *   draft_logits   [B, k, V]   SAMPLE | [B, N, V] TREE_SAMPLE
 *   draft_tokens   [B, k] chain | [B, N] tree (entry 0, the root, is ignored)
 *   parents        [B, N]      tree modes; parents[b, 0] = -1, parents[b, i] < i
 *   uniforms       [B, k]      SAMPLE: accept-test uniforms u_j | [B, N] TREE_SAMPLE: node i's
 *                             uniform (entry 0 unused)
 *   resid_uniforms [B]         SAMPLE, TREE_SAMPLE: the one uniform for the replacement OR bonus draw
 *   accepted_len   [B]    out: n (tree: depth of the deepest accepted node)
 *   out_tokens     [B, k+1] chain | [B, N] tree   out: n accepted tokens, then the
 *                             replacement / bonus / correction; remaining entries -1
 *   out_nodes      [B, N]  out, tree only, optional: node ids of the path root..d*
 *                             (out_nodes[b, i] is the node whose row gave out_tokens[b, i]); rest -1
 *   resid_probs    [B, V]  out, SAMPLE and TREE_SAMPLE, optional (debug): the normalised
 *                             distribution the last token was drawn from (residual, or p' of the
 *                             last row after full acceptance)
 *   seq_status     [B]     out, optional: SV_STATUS_* bits
 *   stream         hipStream_t the work is queued on (NULL = default stream)
 * Returns SV_OK once the work is queued. */
int specverify_run(specverify_ctx* ctx, int32_t batch,
                   const void* target_logits, const void* draft_logits,
                   const int32_t* draft_tokens, const int32_t* parents,
                   const float* uniforms, const float* resid_uniforms,
                   int32_t* accepted_len, int32_t* out_tokens, int32_t* out_nodes,
                   float* resid_probs, int32_t* seq_status, void* stream);

/* The same verification as specverify_run, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  There is no context: `cfg` describes the call (its
 * max_batch must be >= batch, as for specverify_create), and the workspace is
 * a fixed array of SV_STATIC_SCRATCH_BYTES in device memory that the library
 * holds on every device it runs on until the process ends.  The call runs on
 * the calling thread's current device (the one holding the buffers) and calls
 * no hipMalloc, hipFree or other allocating routine; its first call on a
 * device looks up that device's array address and compute-unit count once.
 * Arguments, outputs and errors as specverify_run, plus SV_ERR_SCRATCH when
 * the call's workspace -- specverify_workspace_bytes of cfg with max_batch set
 * to batch -- exceeds SV_STATIC_SCRATCH_BYTES (no HIP call is made then).
 * Chain sampling with top-p alone is the exception: its workspace holds a
 * 192 KB candidate buffer per row of the nucleus kernel; when those do not
 * fit, one per workgroup of that kernel, with as many workgroups as fit
 * (the same results: fewer rows in flight, and the residual kernel reads the
 * rows instead of the buffers).  Every call on one
 * device shares that device's array and leaves its contents behind; no
 * kernel reads workspace it has not written in the same call, so nothing
 * needs clearing between calls.  Calls that overlap in time on one device
 * (two streams, two threads) race on the array: serialise them. */
#define SV_STATIC_SCRATCH_BYTES (64u << 20)
int specverify_run_static(const sv_config* cfg, int32_t batch,
                          const void* target_logits, const void* draft_logits,
                          const int32_t* draft_tokens, const int32_t* parents,
                          const float* uniforms, const float* resid_uniforms,
                          int32_t* accepted_len, int32_t* out_tokens, int32_t* out_nodes,
                          float* resid_probs, int32_t* seq_status, void* stream);

/* Free the workspace and the context.  NULL is allowed.  The caller must make
 * sure no queued call still uses the context. */
void specverify_destroy(specverify_ctx* ctx);

/* Instrumentation for benchmarks.  On every later specverify_run of this
 * context the dispatch packets of the call's kernels record caller-owned HIP
 * events (hipEvent_t handles created on the context's device):
 *   ev_begin       when the streaming kernel (the call's first kernel, the one
 *                  pass that reads every logit) starts;
 *   ev_stream_end  when the streaming kernel completes (NULL: not recorded);
 *   ev_call_end    when the call's last kernel completes (NULL: not recorded).
 * hipEventElapsedTime(ev_begin, ev_stream_end) is then that kernel's duration
 * and hipEventElapsedTime(ev_begin, ev_call_end) the call's time from its
 * first kernel's start to its last kernel's end.  Pass NULL, NULL, NULL to
 * stop.  Nothing is skipped or reordered.  Errors: SV_ERR_NULL (ctx NULL,
 * ev_begin NULL with another event given, or ev_begin alone). */
int specverify_profile_events(specverify_ctx* ctx, void* ev_begin, void* ev_stream_end,
                              void* ev_call_end);

/* Instrumentation for benchmarks: reads `bytes` of device memory at `src`
 * once (16-byte non-temporal loads, 16 KB per workgroup of 256 threads, the
 * shape of the streaming pass's tiles) and keeps nothing, asynchronously on
 * `stream` (NULL: the current device's null stream).  Timed beside a call
 * on the same logits, it gives the HBM read floor of that call's bytes.
 * `sink` (one device word) is written only if the data XOR to one fixed
 * value, which keeps the loads from being dropped.  src and bytes must be
 * multiples of 16 (SV_ERR_SHAPE otherwise, or for bytes < 0); SV_ERR_NULL
 * for a NULL src or sink with bytes > 0; bytes == 0 launches nothing. */
int specverify_read_floor(const void* src, int64_t bytes, uint32_t* sink, void* stream);

/* Host-only: the streaming pass's tiling that specverify_run would use for
 * `batch` sequences of cfg when the streaming kernel has `grid` resident
 * workgroups on the device and the logit tensors start 16-byte aligned
 * (aligned != 0) or not.  out[6] gets: the tile mode (the library's internal
 * number), tiles per row S, logits per tile L, partials per row P, and the
 * workspace's room per row for tiles (of the mode's candidate lists) and for
 * partials; S * L >= V > (S - 1) * L.  Returns SV_OK, a config or batch
 * error (SV_ERR_NULL / SHAPE / DTYPE / PARAM / MODE / CAPACITY; grid < 1 is
 * SV_ERR_PARAM), or SV_ERR_SHAPE when the tiling would not fit the workspace
 * (specverify_run then refuses the call instead of launching; never
 * expected).  Makes no HIP call, so tests can sweep shapes without a GPU. */
int specverify_tiling(const sv_config* cfg, int32_t batch, int32_t grid, int32_t aligned, int32_t* out);

/* Human-readable name of an SV_OK / SV_ERR_* code (static storage). */
const char* specverify_status_string(int status);

/* Workspace bytes specverify_create would allocate for cfg (0 if cfg is invalid). */
size_t specverify_workspace_bytes(const sv_config* cfg);

/* ---------------------------------------------------------------------------
 * Around the verification step: acceptance statistics, and the token tree's
 * attention mask and commit map.  These need no context; they run on the
 * current HIP device (the one that holds the buffers), asynchronously on
 * `stream`, and allocate nothing.  Argument errors are found on the host
 * before any HIP call (SV_ERR_NULL, SV_ERR_SHAPE, SV_ERR_PARAM); a launch
 * failure is SV_ERR_HIP.  batch = 0 writes the statistics of an empty batch
 * (specverify_accept_stats) or nothing (the tree functions).
 * ------------------------------------------------------------------------- */

/* Layout of specverify_accept_stats' output (doubles; counts are exact). */
enum {
  SV_STATS_SEQUENCES = 0,        /* sequences counted (bad-logits ones left out) */
  SV_STATS_ACCEPTED = 1,         /* sum of accepted_len */
  SV_STATS_DRAFTED = 2,          /* k * sequences */
  SV_STATS_TESTED = 3,           /* sum of min(accepted_len + 1, k) */
  SV_STATS_ACCEPTANCE = 4,       /* accepted / drafted */
  SV_STATS_MAL = 5,              /* accepted / sequences: mean accepted length */
  SV_STATS_TOKENS_PER_STEP = 6,  /* (accepted + sequences) / sequences */
  SV_STATS_ALPHA = 7,            /* accepted / tested: the measured per-token acceptance */
  SV_STATS_EXPECTED_TOKENS = 8,  /* E(alpha, k) = (1 - alpha^(k+1)) / (1 - alpha) */
  SV_STATS_GAMMA_BEST = 9,       /* gamma in 1..12 with the largest speedup (smallest on ties) */
  SV_STATS_SPEEDUP_BEST = 10,    /* that speedup */
  SV_STATS_SPEEDUP_GAMMA1 = 11,  /* speedup(alpha, gamma, c) for gamma = 1..12 at 11..22 */
  SV_STATS_LEN = 23
};

/* Acceptance statistics of one batch of verification results, and the
 * speedup model fed with the measured acceptance.  Sources: "Towards Green
 * Text Generation: Memory-Based Speculative Decoding", Appendix A (acceptance
 * = fraction of drafted tokens accepted; MAL = mean number of draft tokens
 * accepted per verification step); the edgeinferencenotes.hashnode.dev
 * speculative-decoding article, "One decode round, end to end" (a pass
 * commits the accepted tokens plus one); "Speculative Decoding Speedup
 * Calculator", steps 1-3 (alpha = probability that the target accepts a
 * given draft token, measured; E = (1 - alpha^(gamma+1)) / (1 - alpha); cost =
 * gamma c + 1; speedup = E / cost; scan gamma = 1..12).
 *   accepted_len [B] device int32 (specverify_run's output); seq_status [B]
 *   device int32, optional: sequences with SV_STATUS_BAD_LOGITS are left out;
 *   k >= 1: drafted tokens per sequence (a tree caller passes the depth bound
 *   or node count it wants the rate against); draft_cost = c >= 0, finite;
 *   out [SV_STATS_LEN] device doubles, written.  alpha = accepted / tested,
 *   tested counting each sequence's tokens up to and including its first
 *   rejection (min(n + 1, k)); 0 when nothing was tested. */
int specverify_accept_stats(const int32_t* accepted_len, const int32_t* seq_status,
                            int32_t batch, int32_t k, double draft_cost, double* out,
                            void* stream);

/* Tree attention mask.  Source: the edgeinferencenotes.hashnode.dev
 * speculative-decoding article, "One decode round, end to end": the
 * flattened tree is scored under a mask that lets each candidate see only
 * its own ancestors (and the context), never sibling branches.
 *   parents [B, N] device int32 (node 0 is the root; parents[b, i] < i);
 *   mask [B, N, ceil(N/32)] device uint32, written: bit j of row i (word
 *   j / 32, bit j % 32) is set iff j == i or j is an ancestor of i;
 *   depth [B, N] device int32, optional, written.  A node whose parent chain
 *   holds an index outside [0, i) is unreachable: its row holds only itself
 *   and its depth is -1.  1 <= N <= SV_MAX_TREE_NODES. */
int specverify_tree_mask(const int32_t* parents, int32_t batch, int32_t nodes, uint32_t* mask,
                         int32_t* depth, void* stream);

/* Commit map after tree verification.  Sources: the same article (the single
 * longest agreed path is committed, the rest collapse) and "Towards Green
 * Text Generation...", section 2.4 (upon rejection the KV cache is truncated
 * to the accepted prefix).
 *   path_nodes [B, N] device int32 and accepted_len [B]: specverify_run's
 *   out_nodes and accepted_len of a SV_MODE_TREE_GREEDY call;
 *   commit_pos [B, N] device int32, written: node path_nodes[b, d] (d <= n)
 *   goes to position d, every other node to -1.  A sequence whose n is
 *   outside [0, N) or whose path holds a node outside [0, N) (a sequence
 *   that emitted nothing) commits nothing: all -1. */
int specverify_tree_commit(const int32_t* path_nodes, const int32_t* accepted_len, int32_t batch,
                           int32_t nodes, int32_t* commit_pos, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H */
