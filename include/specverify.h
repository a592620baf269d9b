/*
 * specverify.h -- C ABI of the MI355X (gfx950) speculative-sampling verify
 * library (libspecverify.so).
 *
 * The library implements the verify step of speculative sampling over a large
 * vocabulary, its greedy variant, and the shortlisted drafter head:
 *
 *   - For each sequence b and draft position i < K, the draft token d_i is
 *     accepted with probability min(1, P_t,i(d_i) / P_d,i(d_i)), left to right,
 *     where P = softmax(logits / T) for the target (t) and draft (d) models.
 *     At the first rejection n a replacement is sampled from the normalised
 *     residual (P_t,n - P_d,n)_+; if all K drafts are accepted a bonus token is
 *     sampled from P_t,K.  Speculative Decoding lesson (nextadmin.net),
 *     "Core algorithm" steps 4-6, "Step 1" and "Step 2"; LLMs-from-Scratch
 *     lesson 25 (aiengineeringfromscratch.com), "The exact rule".
 *   - Greedy (temperature 0): accept d_i iff it equals the argmax of target
 *     row i; at the first mismatch emit that argmax and stop.  LLMs-from-Scratch
 *     lesson 25, "Greedy case".
 *   - Shortlisted drafter head: draft logits only on the union of the clusters
 *     each context selects (per context, or per context and draft position),
 *     and verify of a draft stored as those shortlist logits.  DynaSpec
 *     summary (lowest.today, arXiv 2510.13847), "Model architecture", items
 *     1, 3 and 4.
 *   - Drafter head on one static shortlist shared by every context (the
 *     FR-Spec / VocabTrim baselines of the DynaSpec summary).
 *   - KV-cache commit of the accepted drafts after a verify step.
 *     Speculative Decoding lesson, "KV-cache management".
 *
 * Conventions shared by every entry point:
 *   - All array arguments are device pointers (hipMalloc / torch CUDA tensors),
 *     contiguous, row-major, owned by the caller.  The library allocates no
 *     memory and keeps no global state.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Calls
 *     are asynchronous on that stream; nothing is read back to the host.
 *   - Argument errors are returned synchronously before anything is enqueued;
 *     outputs are then left untouched.  SPEC_ERR_HIP reports a failed launch.
 *   - Calls with distinct workspaces may run concurrently.  Two calls that
 *     share a workspace must be ordered (same stream or synchronised).
 */
#ifndef SPECVERIFY_H_
#define SPECVERIFY_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPEC_ABI_VERSION 2
#define SPEC_MAX_K 64

/*
 * The dtype, mode and status arguments are fixed-width integers with named
 * values (not C enum types), so any value a caller passes is well defined on
 * both sides of the ABI; an unknown value is rejected with
 * SPEC_ERR_INVALID_ARG.
 */
typedef int32_t spec_dtype_t;
enum { SPEC_F32 = 0, SPEC_BF16 = 1 };
/*
 * SAMPLE: the Leviathan/Chen rule (accept with probability min(1, P_t/P_d)
 *   left to right, resample (P_t - P_d)_+ at the first rejection, bonus token
 *   from P_t,K when every draft is accepted), reading every row once.
 * GREEDY: argmax verify on the target logits alone.
 * SAMPLE_EARLY_EXIT: the same rule and bit-identical accepted_len and
 *   out_tokens, evaluated position by position so that rows after a
 *   sequence's first rejection are never read (they cannot change its output:
 *   Speculative Decoding lesson, nextadmin.net, "Core algorithm" step 5).
 *   Consequences: p_target/p_draft_at_draft are NaN after the first
 *   rejection, and a non-finite row after it does not mark the sequence
 *   faulty (draft tokens are still checked at every position).
 */
typedef int32_t spec_mode_t;
enum { SPEC_MODE_SAMPLE = 0, SPEC_MODE_GREEDY = 1, SPEC_MODE_SAMPLE_EARLY_EXIT = 2 };
typedef int32_t spec_status_t;
enum {
  SPEC_OK = 0,
  SPEC_ERR_INVALID_ARG = 1, /* NULL pointer, negative size, bad temperature, unknown dtype or mode, overflow */
  SPEC_ERR_UNSUPPORTED = 2, /* K > SPEC_MAX_K, V > 2^30, a grid too large for one launch, V % cluster_size != 0 */
  SPEC_ERR_WORKSPACE = 3,   /* workspace NULL, too small, or not 256-byte aligned */
  SPEC_ERR_HIP = 4          /* a HIP launch failed */
};

/* Library ABI version (SPEC_ABI_VERSION of the build). */
int spec_abi_version(void);

/* Static string naming a status code. */
const char* spec_status_string(spec_status_t status);

/*
 * Workspace bytes spec_verify needs for this shape (0 when B == 0).
 * The workspace holds per-tile partial results between the kernels of one
 * call.  Its contents need no initialisation and carry nothing from one call
 * to the next, so one buffer serves any later call whose size fits.
 */
size_t spec_verify_workspace_bytes(int32_t B, int32_t K, int32_t V, spec_dtype_t dtype,
                                   spec_mode_t mode);

/*
 * Speculative-sampling verify step.
 *
 *   target_logits  [B, K+1, V] of dtype: target logits at the K draft
 *                  positions and the bonus position.
 *   draft_logits   [B, K, V] of dtype: draft-model logits at the K positions.
 *                  Unused (may be NULL) in GREEDY mode or when K == 0.
 *   draft_tokens   [B, K] int32 token ids.  Unused (may be NULL) when K == 0.
 *   uniforms       [B, K+1, 2] float in [0, 1): uniforms[b,i,0] is the accept
 *                  uniform of position i, uniforms[b,i,1] the sampling uniform
 *                  used if the output token at position i is sampled.
 *                  Unused (may be NULL) in GREEDY mode.
 *   temperature    SAMPLE modes: finite and > 0; both softmaxes use logits / T.
 *                  GREEDY: ignored.
 *   accepted_len   [B] int32 out: n in [0, K] accepted drafts, or -1 when the
 *                  sequence is faulty (a draft token outside [0, V), or a row
 *                  the rule reads whose maximum logit is not finite).
 *   out_tokens     [B, K+1] int32 out: d_0..d_{n-1}, then the sampled (or
 *                  argmax) token at position n, then -1.  All -1 when faulty.
 *   p_target_at_draft, p_draft_at_draft
 *                  optional [B, K] float outs (NULL = skip): P_t,i(d_i) and
 *                  P_d,i(d_i) in the SAMPLE modes, NaN in GREEDY mode, where a
 *                  sequence is faulty, and (SAMPLE_EARLY_EXIT) after the
 *                  first rejection.
 *   workspace      device buffer of at least spec_verify_workspace_bytes(),
 *                  256-byte aligned.
 *
 * Logits must be finite or -inf (-inf marks tokens outside a shortlist).
 * The inverse-CDF sample picks the smallest token id v whose cumulative mass,
 * in token-id order, exceeds u * (total mass).
 */
spec_status_t spec_verify(const void* target_logits, const void* draft_logits,
                          const int32_t* draft_tokens, const float* uniforms,
                          int32_t B, int32_t K, int32_t V, spec_dtype_t dtype,
                          float temperature, spec_mode_t mode,
                          int32_t* accepted_len, int32_t* out_tokens,
                          float* p_target_at_draft, float* p_draft_at_draft,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Number of kernel launches spec_verify makes for this shape (0 for an empty
 * or invalid shape).  SAMPLE mode: 4 for large batches (row statistics;
 * accept decisions; the sampled rows' tile sums; token pick), 3 for middle
 * ones (the accept decisions run in the prologue of the tile-sum launch), 2
 * for small ones (whose tile-sum launch also picks the token in its last
 * block per sequence): B=256, K=7, V=262144 takes 4, B=64, K=4, V=151936
 * takes 3, B=8, K=5, V=128256 takes 2; with K = 0, the tile sums and the
 * pick.  SAMPLE_EARLY_EXIT: K + 2 (row
 * statistics of position i for i = 0..K-1, each launch also deciding
 * position i - 1; then the decision of position K - 1 with the sampled rows'
 * tile sums, and the token pick).  GREEDY mode: 2 (per-tile argmax,
 * then per-sequence finalize).
 */
int32_t spec_verify_launch_count(int32_t B, int32_t K, int32_t V, spec_dtype_t dtype, spec_mode_t mode);

/*
 * spec_verify with kernel timing.  Identical work and launches; in addition
 * events[k] (a hipEvent_t passed as void*) is recorded on `stream` before
 * launch k for k < spec_verify_launch_count(), and events[launch count] after
 * the last launch.  Entries at or beyond n_events, and NULL entries, are
 * skipped.
 */
spec_status_t spec_verify_timed(const void* target_logits, const void* draft_logits,
                                const int32_t* draft_tokens, const float* uniforms,
                                int32_t B, int32_t K, int32_t V, spec_dtype_t dtype,
                                float temperature, spec_mode_t mode,
                                int32_t* accepted_len, int32_t* out_tokens,
                                float* p_target_at_draft, float* p_draft_at_draft,
                                void* workspace, size_t workspace_bytes, void* stream,
                                void* const* events, int32_t n_events);

/*
 * spec_verify for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same call without the workspace argument.  Its kernels use the library's
 * own scratch instead, a static device array of SPEC_NOALLOC_SCRATCH_BYTES on
 * every GPU the library runs on (held until the process ends), located once
 * per device on the first call made with that device current.  The call
 * allocates nothing.
 *
 * Arguments, rule, outputs and errors are those of spec_verify, and the
 * outputs are identical to spec_verify's.  In addition:
 *   - SPEC_ERR_WORKSPACE (before anything is enqueued) when the shape needs
 *     more than SPEC_NOALLOC_SCRATCH_BYTES (spec_verify_workspace_bytes()
 *     gives the need; B=256, K=7, V=262144 bf16 SAMPLE needs about 3.4 MB);
 *   - SPEC_ERR_INVALID_ARG when `stream` belongs to another device than the
 *     current one; SPEC_ERR_HIP when the scratch cannot be located.
 * Every call on one GPU shares that GPU's scratch, which keeps the previous
 * call's contents (the kernels need no cleared memory).  Calls ordered on one
 * stream are safe; calls that overlap on one GPU (several streams, or threads
 * without ordering) race on the scratch.
 */
#define SPEC_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
spec_status_t spec_verify_noalloc(const void* target_logits, const void* draft_logits,
                                  const int32_t* draft_tokens, const float* uniforms,
                                  int32_t B, int32_t K, int32_t V, spec_dtype_t dtype,
                                  float temperature, spec_mode_t mode,
                                  int32_t* accepted_len, int32_t* out_tokens,
                                  float* p_target_at_draft, float* p_draft_at_draft, void* stream);

/*
 * Verify with a sparse draft (DynaSpec summary: the drafter's logits exist
 * only on a shortlist, the union of the clusters selected for the context
 * and position; verification keeps the full vocabulary and the exact rule).
 * The rule, outputs, workspace (spec_verify_workspace_bytes with
 * SPEC_MODE_SAMPLE) and errors are those of spec_verify in SAMPLE mode, with
 * P_d at position i = softmax over position i's shortlist and 0 elsewhere.
 * Reads B*K*L draft elements instead of B*K*V.
 *
 *   draft_compact  [B, K, L] of dtype: position i's logits on its shortlist in
 *                  ascending token id (cluster_ids order, then id within the
 *                  cluster); entries past n_sel[i] * cluster_size are ignored.
 *   cluster_ids    [B, K, S] int32 (device): position i's cluster ids,
 *                  strictly ascending in [0, V / cluster_size); the first
 *                  n_sel[i] are used.  Not validated on the host: ids out of
 *                  order give wrong draft values but no access outside the
 *                  compact row.
 *   n_sel          [K] int32 (HOST memory): clusters per position, the same
 *                  for every sequence (for instance DynaSpec's position-aware
 *                  budget), 1 <= n_sel[i] <= S and
 *                  n_sel[i] * cluster_size <= min(L, V).
 *   cluster_size   ids per cluster; V % cluster_size == 0.
 * A draft token off its position's shortlist has P_d = 0 and is accepted.
 */
spec_status_t spec_verify_sparse_draft(const void* target_logits, const void* draft_compact,
                                       const int32_t* cluster_ids, const int32_t* n_sel,
                                       int32_t L, int32_t S, int32_t cluster_size,
                                       const int32_t* draft_tokens, const float* uniforms,
                                       int32_t B, int32_t K, int32_t V, spec_dtype_t dtype,
                                       float temperature, int32_t* accepted_len, int32_t* out_tokens,
                                       float* p_target_at_draft, float* p_draft_at_draft,
                                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Shortlisted drafter head (DynaSpec summary, "Model architecture", items 1,
 * 3 and 4).  The vocabulary is split into V / cluster_size contiguous
 * clusters; cluster c holds ids [c*cluster_size, (c+1)*cluster_size).  Context
 * b (shared by its K positions) selects n_sel clusters.
 *
 *   h             bf16 [B, K, d]   drafter hidden states.
 *   W             bf16 [V, d]      LM-head weight, row-major (one row per token).
 *   cluster_ids   int32 [B, n_sel] strictly ascending ids in [0, V/cluster_size).
 *   logits_compact float [B, K, n_sel*cluster_size] out: the shortlist logits,
 *                 sum_j h[b,k,j] * W[tok,j] accumulated in fp32, ordered by
 *                 ascending token id (cluster_ids order, then id within the
 *                 cluster).  May be NULL if dense_out is given.
 *   dense_out     NULL or [B, K, V] of dense_dtype out: the same logits at
 *                 their token ids and -inf off the shortlist, ready to be the
 *                 draft_logits of spec_verify.
 *   workspace     unused today; pass NULL and 0.
 * Errors: SPEC_ERR_UNSUPPORTED if V % cluster_size != 0; SPEC_ERR_INVALID_ARG
 * for NULL inputs or non-positive sizes.  Cluster ids are not validated on the
 * host (they live on the device): an id out of range or out of order makes the
 * kernel skip that entry and leaves its outputs unwritten.
 */
spec_status_t spec_draft_head_shortlist(const void* h, const void* W, const int32_t* cluster_ids,
                                        int32_t B, int32_t K, int32_t d, int32_t V,
                                        int32_t cluster_size, int32_t n_sel,
                                        float* logits_compact, void* dense_out,
                                        spec_dtype_t dense_dtype,
                                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Clusters selected at draft position t (0-based) under the position-aware
 * budget k_c(t) of the DynaSpec summary ("Model architecture" item 3): k_max
 * at t = 0 and t = 1, floor(k_max / ((t + 1) * 2)) for t >= 2.  The budget
 * reaches 0 at t >= k_max / 2 (t >= 8 for k_max = 16): such a position has no
 * shortlist, so a draft must stop before it (spec_draft_head_positions accepts
 * n_sel = 0 and writes nothing for it; spec_verify_sparse_draft needs
 * n_sel >= 1).  Host function, no GPU work.  Returns -1 if t < 0 or k_max < 1.
 */
int32_t spec_position_budget(int32_t t, int32_t k_max);

/*
 * Shortlisted drafter head with a shortlist per draft position (DynaSpec
 * summary, "Model architecture" item 3: a position-aware budget selects
 * k_c(t) clusters at draft position t).  Position k of context b uses the
 * first n_sel[k] of cluster_ids[b, k, :]; its logits land in the compact
 * layout spec_verify_sparse_draft reads.
 *
 *   h             bf16 [B, K, d]; W bf16 [V, d] row-major.
 *   cluster_ids   int32 [B, K, S] (device): position k's first n_sel[k] ids
 *                 strictly ascending in [0, V / cluster_size).
 *   n_sel         [K] int32 (HOST memory), 0 <= n_sel[k] <= S and
 *                 n_sel[k] * cluster_size <= L.
 *   logits_compact [B, K, L] of compact_dtype out: position k's logits in
 *                 ascending token id, fp32 accumulation (bf16 output rounds
 *                 to nearest even); entries past n_sel[k] * cluster_size are
 *                 not written.
 * Errors: as spec_draft_head_shortlist; SPEC_ERR_UNSUPPORTED if B * K > 1024.
 */
spec_status_t spec_draft_head_positions(const void* h, const void* W, const int32_t* cluster_ids,
                                        const int32_t* n_sel, int32_t B, int32_t K, int32_t d, int32_t V,
                                        int32_t cluster_size, int32_t S, int32_t L, void* logits_compact,
                                        spec_dtype_t compact_dtype, void* stream);

/*
 * Drafter head over a static shortlist shared by every context: the fixed,
 * frequency-ranked subsets (FR-Spec, VocabTrim) that the DynaSpec summary
 * compares against.  A dense bf16 MFMA GEMM with fp32 accumulation:
 *   logits[m, s] = sum_j h[m, j] * W[tok(s), j],  tok(s) = cluster_ids[s / cs] * cs + s % cs,
 * for M = B*K hidden-state rows and N = n_sel * cluster_size shortlist tokens.
 *
 *   h            bf16 [M, d];  W  bf16 [V, d] row-major.
 *   cluster_ids  int32 [n_sel] (device), ids in [0, V / cluster_size) in any
 *                order (the output columns follow it); an id outside that
 *                range contributes zero columns (not checked on the host).
 *   logits       [M, N] of out_dtype out (bf16 rounds to nearest even).
 *   workspace    NULL, or a 256-byte aligned device buffer of at least
 *                spec_draft_head_static_workspace_bytes() bytes.  For narrow
 *                shortlists (fewer than 192 output tiles of 128 x 128: N up
 *                to about 24k at M = 128) it lets the kernel split the d
 *                dimension over several blocks per output tile: the slices'
 *                fp32 partial tiles go to the workspace and a second launch
 *                adds them in a fixed order (results are deterministic, and
 *                differ from the unsplit sum only by fp32 rounding order).
 *                With NULL the head runs in one launch without splitting.
 *                The contents need no initialisation.
 * Any alignment of whole elements works; 16-byte aligned h and W with d % 8 == 0
 * take the vector-load path (the split needs d % 64 == 0 as well).
 * Errors: SPEC_ERR_INVALID_ARG for NULL or misaligned buffers or bad sizes;
 * SPEC_ERR_WORKSPACE for a workspace that is too small or not 256-byte
 * aligned; SPEC_ERR_UNSUPPORTED if V % cluster_size != 0 or the output needs
 * more than 2^31 - 1 output tiles (one block each; tiles are 128 x 128,
 * 128 x 32 or 64 x 32 depending on the shape and alignment).
 */
spec_status_t spec_draft_head_static(const void* h, const void* W, const int32_t* cluster_ids, int32_t M,
                                     int32_t d, int32_t V, int32_t cluster_size, int32_t n_sel, void* logits,
                                     spec_dtype_t out_dtype, void* workspace, size_t workspace_bytes,
                                     void* stream);

/* Workspace bytes that let spec_draft_head_static split d over several blocks
 * per output tile for this shape (0: the shape does not split). */
size_t spec_draft_head_static_workspace_bytes(int32_t M, int32_t d, int32_t V, int32_t cluster_size,
                                             int32_t n_sel);

/*
 * KV-cache commit after a verify step (Speculative Decoding lesson,
 * nextadmin.net, section on KV-cache management and exercise 4).  The
 * target's forward over the K drafts wrote one KV entry per draft position
 * into `staging`; this call moves the entries of the accepted drafts into the
 * cache at each sequence's current length and advances the length, so the
 * cache holds exactly the accepted prefix.  (The token sampled at position n
 * has no entry yet: the next forward computes it.)
 *
 *   cache         [P, B, L_max, E] of dtype, device: P planes (for instance
 *                 layers x {key, value}), E elements per token per plane
 *                 (for instance kv_heads x head_dim).  Updated in place.
 *   staging       [P, B, K, E] of dtype: entries for draft positions 0..K-1.
 *   accepted_len  [B] int32, spec_verify's output: staging entries 0..n-1 are
 *                 committed to cache positions cache_len[b] .. cache_len[b]+n-1.
 *   cache_len     [B] int32 in/out: advanced by n where the commit happens.
 *   status        [B] int32 out, or NULL: 0 committed; 1 no room
 *                 (cache_len + n > L_max); 2 n outside [0, K] (for instance
 *                 -1 from a faulty verify).  Nothing is committed unless 0.
 * Two launches on `stream` (copy; lengths and status).  All buffers are
 * caller-owned device memory; nothing is allocated.  16-byte vector copies
 * when E * size is a multiple of 16 and both buffers are 16-byte aligned,
 * element copies otherwise.
 * Errors: SPEC_ERR_INVALID_ARG for NULL buffers, buffers not aligned to the
 * element size, negative sizes, an unknown dtype or sizes that overflow;
 * SPEC_ERR_UNSUPPORTED for a grid too large for
 * one launch; SPEC_ERR_HIP for a launch failure.
 */
spec_status_t spec_kv_commit(void* cache, const void* staging, const int32_t* accepted_len,
                             int32_t* cache_len, int32_t* status, int32_t P, int32_t B, int32_t K,
                             int32_t L_max, int32_t E, spec_dtype_t dtype, void* stream);

/*
 * Measurement aid, not part of the method: reads `bytes` (a multiple of
 * 32 KiB) of device memory at `src` (16-byte aligned) with the statistics
 * pass's access pattern (each wave 8 KiB contiguous in 16-byte nontemporal
 * loads) and no arithmetic, so its rate is the read-only streaming ceiling
 * the streaming passes compare with.  `sink` is a device int32 that is
 * written only if the data's XOR equals a fixed constant.  One launch.
 */
spec_status_t spec_read_stream_probe(const void* src, size_t bytes, void* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H_ */
