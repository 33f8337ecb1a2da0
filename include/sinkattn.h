/*
 * sinkattn.h -- C ABI of a gfx950 (MI355X) library for exact sink-aware
 * masked attention, forward and backward.
 *
 * What it computes (sources cited by page title and section):
 *
 *   Mask.  M[q,k] = 1[k <= q] AND 1[q - k <= w OR k < p]: causal, limited to a
 *   local window of w keys behind the query, except that the first p keys of
 *   the sequence stay visible to every later query.  ("Efficient
 *   Reinforcement Learning for Long-Horizon Tool-Use Agentic Tasks", summary
 *   page, paragraph on the sink-aware FlexAttention path.)  The window test
 *   is inclusive (a query sees w + 1 window keys including itself), the
 *   prefix test strict.  Positions are local to each sequence.
 *
 *   Forward.  With S[q,k] = softmax_scale * (q . k) over visible keys,
 *   l[q] = log sum_k exp(S[q,k]) (natural log, content keys only) and
 *   O[q] = sigmoid(l[q] - s_h) * sum_k softmax_k(S[q,:]) v_k,
 *   which equals attention with one extra key of logit s_h and value 0
 *   (arXiv 2608.10357, section 5 "Sink-aware FlexAttention", paragraph
 *   "Zero-value sink equivalence").  One learned sink logit s_h per query
 *   head.  The call returns O and l (same summary-page paragraph: the
 *   attention call returns the output and an auxiliary log-sum-exp).
 *
 *   Backward.  Given dO, returns dQ, dK, dV and dL/ds_h (the per-head sink
 *   gradient of "GPT-OSS Agentic RL training: a practical retrospective",
 *   section on the FlashAttention v3 implementation).  With
 *   L = logaddexp(l, s_h), P' = exp(S - L), D = rowsum(dO * O):
 *     dS = P' * (dO V^T - D),  dQ = scale dS K,  dK = scale dS^T Q,
 *     dV = P'^T dO,            ds_h = -sum_rows exp(s_h - L) D.
 *   dK and dV of a kv-head are summed over the query heads that read it;
 *   ds_h is summed over every row of every sequence.  No O(T^2) buffer is
 *   ever formed.
 *
 * Tensor layouts (all contiguous, last dimension unit-stride, row-major):
 *   fixed length (cu_seqlens == NULL)      varlen (cu_seqlens != NULL)
 *   q, o, dout, dq : [B, T, Hq, d]          [N, Hq, d]
 *   k, v, dk, dv   : [B, T, Hkv, d]         [N, Hkv, d]
 *   lse            : [B, Hq, T]  fp32       [Hq, N]  fp32
 *   sinks, dsinks  : [Hq]        fp32       [Hq]     fp32
 * Element type of q, k, v, o, dout, dq, dk, dv: problem.dtype (bf16 or fp32).
 * Query head h reads kv head h / (Hq / Hkv) (contiguous groups).
 *
 * Conventions:
 *   - Every pointer argument is a DEVICE pointer, except `problem` (host).
 *     The caller owns all memory; the library allocates none.
 *   - Every tensor pointer must be 16-byte aligned (SINKATTN_ERR_MISALIGNED).
 *   - All argument checks run on the host before any HIP call, so an invalid
 *     call returns an error status without touching the device.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *     null stream).  No call synchronises.  A launch failure is reported as
 *     SINKATTN_ERR_HIP.
 *   - Outputs are overwritten, never accumulated into.
 *   - cu_seqlens contents are a caller contract, not checked: cu[0] = 0,
 *     non-decreasing, cu[batch] = total_tokens, every length <= seqlen.
 *   - No global mutable state: concurrent calls on different streams are safe.
 *   - Reproducibility.  bf16: o, lse, dq and dsinks are bitwise the same on
 *     every call (dsinks is added from per-workgroup parts in a fixed order);
 *     dk and dv are too where a kv block's work is one unit, and where it is
 *     cut into several units (long key ranges, prefix keys) those add with
 *     float atomics and agree to rounding only.  fp32: dsinks adds with float
 *     atomics and agrees to rounding only; the other outputs are bitwise
 *     the same.
 */
#ifndef SINKATTN_H
#define SINKATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SINKATTN_OK = 0,
  SINKATTN_ERR_NULL_POINTER = 1, /* a required pointer is NULL */
  SINKATTN_ERR_BAD_SHAPE = 2,    /* negative size, Hq % Hkv != 0, N < 0, Hq * d > 2^24 ... */
  SINKATTN_ERR_BAD_MASK = 3,     /* window < 0 or prefix < 0 */
  SINKATTN_ERR_UNSUPPORTED = 4,  /* dtype / head_dim combination not built */
  SINKATTN_ERR_MISALIGNED = 5,   /* a tensor pointer is not 16-byte aligned */
  SINKATTN_ERR_WORKSPACE = 6,    /* workspace NULL or smaller than required */
  SINKATTN_ERR_HIP = 7,          /* a HIP runtime call or launch failed */
  SINKATTN_ERR_SCRATCH = 8       /* sinkattn_decode_noalloc: problem needs more workspace
                                    than SINKATTN_DECODE_SCRATCH_BYTES */
} sinkattn_status;

typedef enum { SINKATTN_BF16 = 0, SINKATTN_FP32 = 1 } sinkattn_dtype;

/* window value meaning "no window limit": plain causal (plus prefix) */
#define SINKATTN_WINDOW_INF INT32_MAX

typedef struct {
  int32_t dtype;         /* sinkattn_dtype of q, k, v, o, dout, dq, dk, dv */
  int32_t batch;         /* B; or G, the number of packed sequences, if cu_seqlens */
  int32_t seqlen;        /* T; or the maximum sequence length, if cu_seqlens */
  int32_t total_tokens;  /* N, rows of the packed tensors, if cu_seqlens; else ignored */
  int32_t heads_q;       /* Hq >= 1 */
  int32_t heads_kv;      /* Hkv >= 1, Hq % Hkv == 0 */
  int32_t head_dim;      /* d: 64 for bf16; 32 or 64 for fp32 */
  int32_t window;        /* w >= 0, or SINKATTN_WINDOW_INF */
  int32_t prefix;        /* p >= 0 */
  float softmax_scale;   /* scale on q . k (1/sqrt(d) in the usual setting) */
  const int32_t *cu_seqlens; /* device int32[batch + 1], or NULL (fixed length) */
} sinkattn_problem;

/*
 * Forward.  Reads q, k, v, sinks; writes o and (if lse != NULL) lse.
 * lse may be NULL when no backward will follow (inference).  lse is an
 * fp32-accumulated log-sum-exp of the bf16 (or fp32) inputs: for bf16 the
 * probabilities are added in fp32, or (64-key tiles, min(w, seqlen) >= 1024)
 * as fp16 copies on the matrix cores, which keeps lse within
 * ln(1 + 2^-11) = 4.9e-4 of the log of their fp32 sum.
 */
sinkattn_status sinkattn_fwd(const sinkattn_problem *problem, const void *q,
                             const void *k, const void *v, const float *sinks,
                             void *o, float *lse, void *stream);

/* Bytes of device workspace sinkattn_bwd needs for `problem` (0 if invalid). */
size_t sinkattn_bwd_workspace_size(const sinkattn_problem *problem);

/*
 * Backward.  Reads q, k, v, sinks, o and lse (both exactly as written by
 * sinkattn_fwd for the same inputs) and dout; writes dq, dk, dv and dsinks.
 * `workspace` is caller-owned device memory of at least
 * sinkattn_bwd_workspace_size(problem) bytes, 256-byte aligned; its contents
 * on entry do not matter and on return are unspecified.
 */
sinkattn_status sinkattn_bwd(const sinkattn_problem *problem, const void *q,
                             const void *k, const void *v, const float *sinks,
                             const void *o, const float *lse, const void *dout,
                             void *dq, void *dk, void *dv, float *dsinks,
                             void *workspace, size_t workspace_bytes, void *stream);

/*
 * The same backward in stream-ordered phases, for callers that want to place
 * work (or timing events) between them.  `phases` is a non-empty OR of the
 * flags below (other bits: SINKATTN_ERR_BAD_SHAPE); the other arguments are
 * exactly those of sinkattn_bwd and are validated the same way.  Phases must
 * run in flag order (PREPARE, DQ, DKDV, FINISH) across calls on one stream,
 * with the same arguments and workspace; each depends on the one before.
 * The row statistics D = rowsum(dout * o), L = logaddexp(lse, s_h) and the
 * sink gradient dsinks (of "GPT-OSS Agentic RL training: a practical
 * retrospective", FlashAttention v3 implementation section) are computed in
 * PREPARE for fp32 and inside DQ for bf16.
 *   PREPARE: fp32: clears dsinks and runs the row pass; bf16: nothing
 *            (except clearing dsinks for an empty problem);
 *   DQ:      dQ, written to dq (bf16: also the row statistics, each
 *            workgroup's part of dsinks into the workspace, clearing the
 *            fp32 dK/dV workspace accumulators where DKDV adds into them
 *            rather than storing whole rows, and, for short windows with
 *            0 < prefix <= 16, the prefix keys' part of dK, dV from the rows
 *            past the first key block's window, per workgroup into the
 *            workspace);
 *   DKDV:    dK, dV from the recomputed probabilities exp(S - L) (bf16:
 *            into the fp32 workspace accumulators where a key block is
 *            split over several work units, else straight into dk, dv --
 *            with the prefix fold, the prefix keys' rows into the
 *            accumulators; fp32: into dk, dv);
 *   FINISH:  bf16: adds DQ's prefix-key parts into the dK/dV accumulators,
 *            scales and converts what DKDV left there into dk, dv, and
 *            writes dsinks as the sum of DQ's parts; every sum is taken in a
 *            fixed order (so dk, dv and dsinks are the same on every call);
 *            fp32: nothing.
 * sinkattn_bwd(...) == sinkattn_bwd_phases(SINKATTN_BWD_ALL, ...).
 */
enum {
  SINKATTN_BWD_PREPARE = 1,
  SINKATTN_BWD_DQ = 2,
  SINKATTN_BWD_DKDV = 4,
  SINKATTN_BWD_FINISH = 8,
  SINKATTN_BWD_ALL = 15
};
sinkattn_status sinkattn_bwd_phases(uint32_t phases, const sinkattn_problem *problem,
                                    const void *q, const void *k, const void *v,
                                    const float *sinks, const void *o, const float *lse,
                                    const void *dout, void *dq, void *dk, void *dv,
                                    float *dsinks, void *workspace, size_t workspace_bytes,
                                    void *stream);

/* Static, human-readable name of a status code. */
const char *sinkattn_status_string(sinkattn_status status);

/*
 * Host-only helpers exposing the tile schedule the kernels use, so it can be
 * checked against brute-force enumeration of the mask without a GPU.
 *
 * sinkattn_tile_class: for query rows [q0, q1] and key columns [k0, k1]
 * (inclusive, positions local to one sequence) returns 0 if no (q, k) pair
 * in the block is visible, 1 if every pair is visible, 2 otherwise.
 *
 * sinkattn_key_tile_segments: the key tiles of width block_k that query rows
 * [q0, q1] must visit, as at most two half-open tile-index ranges written to
 * out[0..3] (begin0, end0, begin1, end1).  Returns the number of ranges.
 * Every tile holding a visible pair is listed exactly once.
 */
int32_t sinkattn_tile_class(int32_t q0, int32_t q1, int32_t k0, int32_t k1,
                            int32_t window, int32_t prefix);
int32_t sinkattn_key_tile_segments(int32_t q0, int32_t q1, int32_t window,
                                   int32_t prefix, int32_t block_k, int32_t *out);

/*
 * Tile shapes the bf16 kernels use for a problem, chosen from its window
 * (after clamping to seqlen): short windows (w < 1024) get 32-key tiles in
 * the forward and dQ kernels, so that fewer masked pairs are computed at the
 * band's edges, otherwise 64-key tiles; the dK/dV kernel uses 128-row query
 * tiles throughout.  Writes out[0] = forward / dQ key-tile width, out[1] =
 * dK/dV query-tile height.  Host only, no HIP calls.  Returns the problem's
 * validation status (out is written only on SINKATTN_OK).
 */
sinkattn_status sinkattn_tile_config(const sinkattn_problem *problem, int32_t *out);

/*
 * Decode: one new query token per sequence against its key/value cache -- the
 * rollout side of the same attention.  The rollout workers sample from the
 * current policy (arXiv 2608.10357, section 4 "Rollout workers"), and the
 * rollout engine must give the trainer's token probabilities, sink included
 * ("GPT-OSS Agentic RL training: a practical retrospective", section on the
 * training-inference mismatch through attention sinks).  For sequence b with
 * n = cache_seqlens[b] cached tokens (the new token's key and value already
 * written at position n - 1) the query sits at position n - 1 under the same
 * mask M[q,k] = 1[k<=q] AND 1[q-k<=w OR k<p] and sink scaling as sinkattn_fwd:
 * the result equals row n - 1 of sinkattn_fwd on those n tokens (up to bf16
 * rounding of the output).  n = 0 gives o = 0 and lse = -inf; n is clamped to
 * [0, cache_capacity].
 *
 * Layouts (bf16, head_dim 64, contiguous): q and o [batch, heads_q, 64];
 * k_cache and v_cache [batch, cache_capacity, heads_kv, 64];
 * cache_seqlens int32 [batch] (device); sinks fp32 [heads_q];
 * lse fp32 [batch, heads_q] (content-only log-sum-exp, natural log; may be
 * NULL).  heads_q / heads_kv must be at most 16.  The workspace (caller-owned
 * device memory of sinkattn_decode_workspace_size bytes, 256-byte aligned)
 * holds per-block partial results; its contents on entry do not matter.
 * Validation happens on the host before any HIP call, as for sinkattn_fwd.
 */
typedef struct {
  int32_t batch;            /* sequences, one new query token each */
  int32_t cache_capacity;   /* rows per sequence in k_cache / v_cache */
  int32_t heads_q;
  int32_t heads_kv;         /* heads_q / heads_kv <= 16 */
  int32_t head_dim;         /* 64 */
  int32_t window;           /* w >= 0; SINKATTN_WINDOW_INF for plain causal */
  int32_t prefix;           /* p >= 0 */
  float softmax_scale;
} sinkattn_decode_problem;

/* Bytes of device workspace sinkattn_decode needs (0 if the problem is invalid). */
size_t sinkattn_decode_workspace_size(const sinkattn_decode_problem *problem);

sinkattn_status sinkattn_decode(const sinkattn_decode_problem *problem, const void *q,
                                const void *k_cache, const void *v_cache,
                                const int32_t *cache_seqlens, const float *sinks, void *o,
                                float *lse, void *workspace, size_t workspace_bytes,
                                void *stream);

/*
 * Decode without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments (minus the workspace), checks and
 * results as sinkattn_decode.  The per-block partials go to a static device
 * buffer of the library, SINKATTN_DECODE_SCRATCH_BYTES (24 MiB) on each GPU
 * the library runs on, held until the process ends.  That is enough for
 * every problem sinkattn_decode accepts (its workspace is at most
 * 22,282,240 bytes); a problem whose sinkattn_decode_workspace_size exceeded
 * it would return SINKATTN_ERR_SCRATCH (checked on the host, before any HIP
 * call).  The buffer used is that of the
 * current device; the first call on a device looks up its address
 * (hipGetSymbolAddress), and no call allocates memory.  Every call on one GPU
 * shares that buffer and overwrites it: calls that may overlap on one GPU
 * (different streams without ordering between them, or different threads)
 * race and give undefined results.  Nothing in the buffer needs to be zero
 * on entry.
 */
#define SINKATTN_DECODE_SCRATCH_BYTES ((size_t)24 << 20)
sinkattn_status sinkattn_decode_noalloc(const sinkattn_decode_problem *problem, const void *q,
                                        const void *k_cache, const void *v_cache,
                                        const int32_t *cache_seqlens, const float *sinks,
                                        void *o, float *lse, void *stream);

/*
 * GRPO token loss and group-normalised advantage over a packed batch of
 * rollout groups -- the step after the model in the same trainer (arXiv
 * 2608.10357, section 4 "Training pipeline", paragraph "Policy update",
 * eq. 3-7; eq. 3 also on the summary page).  Rollouts g*G .. g*G + G - 1 form
 * group g (G = group_size, M = num_rollouts / G groups); rollout i holds the
 * tokens [cu_seqlens[i], cu_seqlens[i + 1]) of the packed [N] arrays.
 *   A_i  = (R_i - mean_g R) / (std_g R + eps_adv)    std over the group's G
 *          rewards, population form; 0 where R_i equals the mean       (eq. 3)
 *   rho  = exp(logp_new - logp_old)                                     (eq. 4)
 *   J    = min(rho A_i, clip(rho, 1 - eps_clip, 1 + eps_clip) A_i)     (eq. 5, 6)
 *   kl   = logp_new - logp_ref (kl_mode 0), or exp(r) - r - 1 with
 *          r = logp_ref - logp_new (kl_mode 1)
 *   L_g  = (-sum J + beta sum kl) / S_g over the group's optimised tokens
 *          (action_mask != 0), S_g their number; L_g = 0 if S_g = 0     (eq. 7)
 *   loss = (1 / M) sum_g L_g
 * Outputs (device): *loss (fp32); grad [N] fp32 = d loss / d logp_new (0 on
 * tokens that are not optimised); advantages [B] fp32 (may be NULL).  For the
 * gradient the clip counts as active -- and the token's J term contributes 0
 * -- when (A_i > 0 and logp_new - logp_old > log(1 + eps_clip)) or (A_i < 0
 * and logp_new - logp_old < log(1 - eps_clip)), compared in fp32.
 * Inputs (device): logp_new, logp_old fp32 [N]; logp_ref fp32 [N], may be
 * NULL when beta == 0 (then ignored); action_mask uint8 [N], NULL for "every
 * token optimised"; rewards fp32 [B]; cu_seqlens int32 [B + 1], nondecreasing
 * from 0 to N (device memory, not checked; offsets outside [0, N] are
 * clamped, never dereferenced).  Token arrays and grad 16-byte aligned,
 * rewards / advantages / cu_seqlens / loss 4-byte aligned.  The workspace
 * (caller-owned device memory of sinkattn_grpo_workspace_size bytes, 256-byte
 * aligned) holds per-rollout values and per-workgroup partial sums; its
 * contents on entry do not matter.  The result is deterministic: every
 * reduction runs in a fixed order.  Validation happens on the host first.
 */
typedef struct {
  int32_t num_rollouts;     /* B >= 0, a multiple of group_size */
  int32_t group_size;       /* G in [1, 1024] */
  int32_t total_tokens;     /* N >= 0 (0 when B == 0) */
  int32_t kl_mode;          /* 0 or 1 */
  float eps_adv;            /* eps_A >= 0 */
  float eps_clip;           /* eps_c in [0, 1) */
  float beta;               /* KL weight, finite */
} sinkattn_grpo_problem;

/* Bytes of device workspace sinkattn_grpo_loss needs (0 if the problem is invalid). */
size_t sinkattn_grpo_workspace_size(const sinkattn_grpo_problem *problem);

sinkattn_status sinkattn_grpo_loss(const sinkattn_grpo_problem *problem, const float *logp_new,
                                   const float *logp_old, const float *logp_ref,
                                   const uint8_t *action_mask, const float *rewards,
                                   const int32_t *cu_seqlens, float *loss, float *grad,
                                   float *advantages, void *workspace, size_t workspace_bytes,
                                   void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SINKATTN_H */
