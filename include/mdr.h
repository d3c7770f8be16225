/*
 * mdr.h -- C ABI of the MI355X (gfx950) library for the forward pass of
 * Monodratic routed sparse causal attention.
 *
 * The method (aitechinspire.com write-up of Monodratic, "Snapshot: key facts
 * from the report" and "What's the core idea?"; remio.ai, "Monodratic claims
 * learned routing can make sparse causal attention more selective", section
 * "Monodratic turns sparse attention into a retrieval decision"):
 *   after RoPE, source blocks get learned product addresses and are filed in
 *   bounded causal posting lists; each query probes product addresses, reranks
 *   the returned candidates, keeps a fixed number R of remote blocks, adds
 *   guaranteed local blocks and runs exact causal softmax over the tokens of
 *   those blocks.  The operator is stateless: [batch, sequence, width] in, an
 *   attention delta out; normalisation, residuals, feed-forward layers and
 *   scheduling belong to the host model.
 *
 * Conventions shared by every entry point
 *   - Pointers are device pointers unless stated otherwise.  The caller owns
 *     every buffer; the library allocates nothing and keeps no state between
 *     calls.  Buffers must be 16-byte aligned and contiguous row-major.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  All work is
 *     queued on it asynchronously; nothing synchronises the host.
 *   - Arguments are validated on the host before anything is queued.  A bad
 *     argument returns MDR_ERR_INVALID_ARG, an unsupported size or dtype
 *     MDR_ERR_UNSUPPORTED, a short workspace MDR_ERR_WORKSPACE; in all three
 *     cases nothing is launched.  A failed launch returns MDR_ERR_HIP.  Faults
 *     inside a kernel surface at the caller's next synchronisation.
 *   - Q, K, V, x, out, delta and the projection weights share one dtype
 *     (cfg->dtype: MDR_F32 or MDR_BF16).  Router arithmetic (summaries, logits,
 *     scores) and softmax accumulation are fp32; codebook and bias are fp32.
 *   - Results are bitwise reproducible run to run.  Calls that share a
 *     workspace or output buffers must not overlap in time.
 *
 * Routing semantics (each is a reading of the pages where they leave a step
 * open):
 *   summary of block i      = mean of its post-RoPE key rows
 *   code_g(i)               = argmax_c <codebook[h,g,c,:], summary> + bias[h,g,c]
 *                             (ties to the smaller code)
 *   address(i)              = sum_g code_g * C^(G-1-g)        (A = C^G addresses)
 *   eligibility             = block i is visible to query block j iff i <= j - L
 *   posting view (a, j)     = the newest `capacity` eligible blocks filed under
 *                             address a, newest first; overflow of (b,h) =
 *                             sum_a max(0, n_a - capacity) over blocks i < nb - L
 *   probes of token t       = the P addresses with the largest
 *                             sum_g (<codebook[h,g,c_g,:], q_t> + bias[h,g,c_g]),
 *                             ties to the smaller address
 *   candidates              = views of the probed addresses concatenated in probe
 *                             rank order, cut at M (max_cand; 0 means P*capacity)
 *   selection               = top-R candidates by <q_t, summary_i> (unscaled),
 *                             ties to the smaller block, padded with -1
 *   attention of token t    = softmax(q_t k_s * scale) over s in the selected
 *                             blocks and in the L most recent blocks with s <= t
 */
#ifndef MDR_H
#define MDR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MDR_ABI_VERSION 4

typedef enum {
  MDR_OK = 0,
  MDR_ERR_INVALID_ARG = 1,
  MDR_ERR_UNSUPPORTED = 2,
  MDR_ERR_WORKSPACE = 3,
  MDR_ERR_HIP = 4
} mdr_status;

typedef enum { MDR_F32 = 0, MDR_BF16 = 1 } mdr_dtype;

/* What a full posting list does with its overflow.  The pages name both
 * options, dropping or redirecting blocks, and warn that either may hide
 * relevant blocks (remio.ai, "Monodratic turns sparse attention into a
 * retrieval decision"); they fix no redirect rule.
 *   DROP      query block j reads from address a the newest `capacity`
 *             eligible blocks (i <= j - L) filed under a, newest first.
 *   REDIRECT  the same view, then, while slots remain, the newest blocks
 *             redirected into a.  A block is redirected when it leaves its
 *             own view: when the capacity-th newer block of its address
 *             becomes eligible, i.e. at query block (that block) + L.  It
 *             goes to its alternate address: its own address with, in the
 *             subspace whose two best code logits are closest (fp32 top1 -
 *             top2; ties to the smaller subspace), the runner-up code (ties to
 *             the smaller code) in place of the best one.  Redirected blocks
 *             are read newest arrival first.  Prefill entry points only (the
 *             decode state rejects it with MDR_ERR_UNSUPPORTED). */
typedef enum { MDR_OVERFLOW_DROP = 0, MDR_OVERFLOW_REDIRECT = 1 } mdr_overflow_policy;

/* Sizes of one call.  nb = seq / block blocks per sequence.
 * Supported on gfx950: head_dim in {32, 64, 128}; block in {32, 64, 128};
 * seq % block == 0; 1 <= subspaces <= 4; codes >= 2; subspaces*codes <= 64;
 * codes^subspaces <= 4096; 1 <= probes <= min(16, codes^subspaces);
 * remote <= 16; local >= 1; nb <= 8192; the probe stage's per-token scratch
 * (about 128 * 4 * (G*ceil16(C) + G*min(P,C) + 2P + 2R) bytes) must fit in LDS. */
typedef struct {
  int32_t batch;       /* B */
  int32_t seq;         /* S, tokens per sequence */
  int32_t heads;       /* H */
  int32_t head_dim;    /* D */
  int32_t width;       /* W, mixer only (0 for the core entry points) */
  int32_t block;       /* tokens per block */
  int32_t subspaces;   /* G, code components per product address */
  int32_t codes;       /* C, codes per component */
  int32_t capacity;    /* posting view capacity per address */
  int32_t probes;      /* P, addresses probed per query token */
  int32_t max_cand;    /* M, candidate cut (0 => probes * capacity) */
  int32_t remote;      /* R, remote blocks kept per query token */
  int32_t local;       /* L, local blocks including the current one */
  int32_t dtype;       /* mdr_dtype */
  float rope_base;     /* mixer only: RoPE base (pairs (i, i + D/2), theta_i = base^(-2i/D)) */
  float softmax_scale; /* 0 => 1/sqrt(head_dim) */
  int32_t overflow_policy; /* mdr_overflow_policy (0 = drop) */
} mdr_config;

/* Optional device outputs of the routing stages.  Any NULL member is kept in
 * the workspace instead (n_drop: not computed).  Layouts:
 *   ksum [B,H,nb,D] fp32   addr [B,H,nb]        post_off [B,H,A+1]
 *   post_idx [B,H,nb] (CSR entries: the blocks of address a in ascending order
 *   at post_idx[post_off[a] .. post_off[a+1]); entries past post_off[A] are -1)
 *   overflow [B,H]: blocks no view of the last query block returns
 *   sel [B,H,S,R] (-1 padded)   n_cand [B,H,S]: candidates after the M cut
 *   n_drop [B,H,S]: per token, summed over its probes, the eligible blocks a
 *     probed address holds beyond its capacity (under REDIRECT an address
 *     holds its primaries not redirected away plus the arrivals so far); the
 *     pages ask overflow stress tests to report such dropped candidates
 *     (remio.ai, "What sparse attention researchers should watch next")
 * REDIRECT policy only (written when non-NULL, ignored under DROP):
 *   alt [B,H,nb]: alternate address of each block
 *   redir_off [B,H,A+1], redir_idx [B,H,nb], redir_time [B,H,nb]: per address
 *     the blocks redirected into it in arrival order, at
 *     redir_idx[redir_off[a] .. redir_off[a+1]), with redir_time the query
 *     block at which each arrives; entries past redir_off[A] are -1.
 * Routing diagnostics (each written when non-NULL).  The pages ask for the
 * selected remote blocks per query to be logged and checked against a dense
 * selected-mask oracle (aitechinspire.com, "Practical notes for tinkerers");
 * these outputs let a caller tell which decisions were close to a tie (all
 * fp32, in the kernels' own summation order):
 *   probes [B,H,S,P]: each token's probed addresses, best first
 *   sel_score [B,H,S,R]: <q_t, summary_i> of each selected block (-inf for -1
 *     padding, NaN for a forced block that was not among the candidates)
 *   probe_margin [B,H,S]: the smallest gap between neighbouring address scores
 *     among the min(P + 1, A) best (+inf with fewer than two)
 *   sel_margin [B,H,S]: the smallest gap between neighbouring rerank scores
 *     among the min(R + 1, candidates) best (+inf with fewer than two)
 *   addr_margin [B,H,nb]: per block, the smallest best-minus-second code logit
 *     over its subspaces (+inf when codes == 1)
 *   Asking for any of the first four runs the probe with one more address and
 *   candidate ranked; the routing itself is identical either way. */
typedef struct {
  float* ksum;
  int32_t* addr;
  int32_t* post_off;
  int32_t* post_idx;
  int32_t* overflow;
  int32_t* sel;
  int32_t* n_cand;
  int32_t* n_drop;
  int32_t* alt;
  int32_t* redir_off;
  int32_t* redir_idx;
  int32_t* redir_time;
  int32_t* probes;
  float* sel_score;
  float* probe_margin;
  float* sel_margin;
  float* addr_margin;
} mdr_routing;

/* MDR_ABI_VERSION of the built library. */
int mdr_abi_version(void);

/* Static, human-readable name of a status code (never NULL). */
const char* mdr_status_string(int status);

/* Host-only validation of a configuration.  Returns MDR_OK, MDR_ERR_INVALID_ARG
 * or MDR_ERR_UNSUPPORTED; touches no device. */
mdr_status mdr_check_config(const mdr_config* cfg);

/* Host-only: bytes of device workspace every entry point below needs for `cfg`
 * (mdr_mixer_forward included when cfg->width > 0).  *bytes is set on MDR_OK. */
mdr_status mdr_workspace_size(const mdr_config* cfg, size_t* bytes);

/* Host-only: how the workspace of cfg divides, in bytes.  The pages ask memory
 * to be reported split into weights, routing buffers, posting lists and K/V
 * (remio.ai, "What sparse attention researchers should watch next"); the
 * caller-owned tensors (Q, K, V, out, codebook, bias, projection weights) are
 * not part of the workspace and not counted here.  Regions are 256-byte
 * aligned, so the parts sum to `total` (== mdr_workspace_size). */
typedef struct {
  size_t summaries;     /* block key summaries, addresses (and alternates) */
  size_t posting_lists; /* posting-list CSR, redirect lists, overflow counts */
  size_t selection;     /* sel and n_cand of the workspace copy */
  size_t pair_lists;    /* the selected (token, slot) pairs binned by remote block */
  size_t partials;      /* remote softmax partials (output rows and normalisers) */
  size_t backward;      /* backward-only scratch */
  size_t mixer;         /* mixer-only scratch: projected Q, K, V, O and transposed weights */
  size_t total;
} mdr_workspace_parts;
mdr_status mdr_workspace_breakdown(const mdr_config* cfg, mdr_workspace_parts* parts);

/* Host-only self-check of the kernels' index arithmetic for cfg: the functions
 * the kernels use to map a work-group to its work and to address their buffers
 * are run over every launch index of cfg's kernels (and over extreme
 * distributions of the selected pairs), and each result is checked against the
 * workspace region it addresses (also: regions aligned, disjoint, inside the
 * workspace).  Returns MDR_OK, or MDR_ERR_INVALID_ARG with a description in msg
 * (msg_len bytes, may be 0).  Touches no device. */
mdr_status mdr_selfcheck_indices(const mdr_config* cfg, char* msg, size_t msg_len);

/* The routed attention core on post-RoPE inputs (the whole path: addressing,
 * posting lists, probe + rerank, selected-set attention).
 *   q, k, v    [B,H,S,D] in cfg->dtype
 *   codebook   [H,G,C,D] fp32; code_bias [H,G,C] fp32 or NULL (zero)
 *   force      [B,H,S] int32 or NULL: a block to force into token t's selection
 *              under the same budget R (the pages' forced-target diagnostic,
 *              aitechinspire.com "Snapshot"; remio.ai "Why learned product-hash
 *              routing matters now").  It is used only when 0 <= f <= j - L; it
 *              fills a free slot or replaces the lowest-ranked one.  -1 = none.
 *   out        [B,H,S,D] in cfg->dtype, overwritten
 *   routing    optional outputs (may be NULL)
 *   workspace  >= mdr_workspace_size bytes, 256-byte aligned */
mdr_status mdr_routed_attention(const mdr_config* cfg, const void* q, const void* k, const void* v,
                                const float* codebook, const float* code_bias, const int32_t* force,
                                void* out, const mdr_routing* routing, void* workspace,
                                size_t workspace_bytes, void* stream);

/* mdr_routed_attention without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Its workspace is a static device array
 * of MDR_NOALLOC_SCRATCH_BYTES inside the library, one copy per GPU, held
 * until the process ends; the call allocates nothing.  A configuration whose
 * workspace (mdr_workspace_size) exceeds it returns MDR_ERR_WORKSPACE before
 * anything is launched.  Every call on a GPU shares that GPU's array, so calls
 * that overlap in time on one GPU (other streams, other host threads) race and
 * must be serialised by the caller.  The first call on each device looks up
 * that device's copy (a host-side lookup, no allocation).  Everything else is
 * as in mdr_routed_attention, with identical results. */
#define MDR_NOALLOC_SCRATCH_BYTES (64u << 20)
mdr_status mdr_routed_attention_noalloc(const mdr_config* cfg, const void* q, const void* k, const void* v,
                                        const float* codebook, const float* code_bias, const int32_t* force,
                                        void* out, const mdr_routing* routing, void* stream);

/* Kernels of the core path, in launch order (the profiling form below records
 * an event before each and one after the last). */
#define MDR_CORE_KERNELS 6 /* address, post, probe_rerank, attn_bin, attn_remote, attn_local */

/* Profiling form of mdr_routed_attention, for timing each kernel on `stream`:
 * events[k] (a hipEvent_t created by the caller) is recorded just before the
 * k-th kernel of the core path and events[MDR_CORE_KERNELS] after the last one.
 * attn_bin groups the selected (token, slot) pairs by remote block for
 * attn_remote.  A kernel a configuration does not need (attn_bin and
 * attn_remote when R = 0 or nb <= L; attn_bin up to 8192 tokens with R <= 2,
 * where attn_remote finds each block's pairs itself) gets two adjacent events.  A NULL entry records nothing at that point (so a
 * caller can time one kernel alone); a NULL `events` array is rejected.
 * Everything else is as in mdr_routed_attention. */
mdr_status mdr_routed_attention_profiled(const mdr_config* cfg, const void* q, const void* k, const void* v,
                                         const float* codebook, const float* code_bias, const int32_t* force,
                                         void* out, const mdr_routing* routing, void* workspace,
                                         size_t workspace_bytes, void* const* events, void* stream);

/* The stateless mixer, [B,S,W] -> attention delta [B,S,W] (aitechinspire.com,
 * "Snapshot: key facts from the report"): Q = RoPE(x Wq), K = RoPE(x Wk),
 * V = x Wv (no biases), the routed attention core per head, then
 * delta = concat_h(O) Wo.  The host adds delta to its residual stream.
 *   x [B,S,W]; wq, wk, wv [W, H*D]; wo [H*D, W] (all cfg->dtype, row-major)
 *   codebook, code_bias, routing, workspace as above; delta [B,S,W] overwritten. */
mdr_status mdr_mixer_forward(const mdr_config* cfg, const void* x, const void* wq, const void* wk,
                             const void* wv, const void* wo, const float* codebook,
                             const float* code_bias, void* delta, const mdr_routing* routing,
                             void* workspace, size_t workspace_bytes, void* stream);

/* ---- staged entry points: one stage each, its upstream passed in, so any
 * stage can be fed another implementation's upstream output. ---- */

/* Block summaries and product addresses (remio.ai "Monodratic turns sparse
 * attention into a retrieval decision": a product address combines the
 * decisions of several learned code components).
 *   k [B,H,S,D]; codebook [H,G,C,D]; code_bias [H,G,C] or NULL;
 *   ksum [B,H,nb,D] fp32 out; addr [B,H,nb] out; alt [B,H,nb] out or NULL
 *   (the alternate addresses of the REDIRECT policy; -1 when codes == 1). */
mdr_status mdr_stage_address(const mdr_config* cfg, const void* k, const float* codebook,
                             const float* code_bias, float* ksum, int32_t* addr, int32_t* alt,
                             void* stream);

/* Bounded causal posting lists as CSR plus overflow counts (aitechinspire.com
 * "Snapshot": source blocks assigned to bounded causal posting lists; remio.ai
 * same section: a strict capacity bounds each list, overflow drops blocks).
 *   addr [B,H,nb] in (values must lie in [0, A)); post_off [B,H,A+1],
 *   post_idx [B,H,nb], overflow [B,H] out.  Under REDIRECT also alt
 *   [B,H,nb] in (values in [0, A), or -1 for none) and the redirect lists
 *   redir_off, redir_idx, redir_time out (layouts as in mdr_routing); under
 *   DROP those four may be NULL and are ignored. */
mdr_status mdr_stage_post(const mdr_config* cfg, const int32_t* addr, const int32_t* alt,
                          int32_t* post_off, int32_t* post_idx, int32_t* redir_off,
                          int32_t* redir_idx, int32_t* redir_time, int32_t* overflow, void* stream);

/* Query probe, candidate gathering and rerank to R remote blocks
 * (aitechinspire.com "Snapshot": each query probes product addresses,
 * reranks returned candidates and selects a fixed number of remote blocks).
 *   q [B,H,S,D]; codebook, code_bias as above; ksum [B,H,nb,D] fp32;
 *   post_off [B,H,A+1], post_idx [B,H,nb] (CSR as produced by
 *   mdr_stage_post); redir_off, redir_idx, redir_time as produced by
 *   mdr_stage_post (REDIRECT; ignored under DROP); force [B,H,S] or NULL;
 *   sel [B,H,S,R] out; n_cand [B,H,S] out or NULL; n_drop [B,H,S] out or
 *   NULL (its count assumes every block has an alternate when codes > 1,
 *   as the library's alternates do). */
mdr_status mdr_stage_probe_rerank(const mdr_config* cfg, const void* q, const float* codebook,
                                  const float* code_bias, const float* ksum, const int32_t* post_off,
                                  const int32_t* post_idx, const int32_t* redir_off,
                                  const int32_t* redir_idx, const int32_t* redir_time,
                                  const int32_t* force, int32_t* sel, int32_t* n_cand,
                                  int32_t* n_drop, void* stream);

/* Exact causal softmax over the selected remote blocks plus the L local blocks
 * (aitechinspire.com "Snapshot" and "What's the core idea?": no approximation
 * after selection).
 *   q, k, v [B,H,S,D]; sel [B,H,S,R] in: entry r of token t (block j) is used
 *   when 0 <= sel <= j - L and it does not repeat an earlier entry of the same
 *   token; other entries are ignored.  out [B,H,S,D] overwritten.
 *   workspace >= mdr_workspace_size bytes. */
mdr_status mdr_stage_attend(const mdr_config* cfg, const void* q, const void* k, const void* v,
                            const int32_t* sel, void* out, void* workspace, size_t workspace_bytes,
                            void* stream);

/* mdr_stage_attend that also writes each token's softmax normaliser in base-2
 * log form, the one saved tensor the backward below needs (the selected set is
 * the other):
 *   lse [B,H,S] fp32 out, or NULL (nothing written; the call is then
 *   mdr_stage_attend): lse[t] = log2 sum_s 2^(c q_t.k_s) over the token's
 *   selected keys, c = softmax_scale * log2(e).  Everything else as above. */
mdr_status mdr_stage_attend_lse(const mdr_config* cfg, const void* q, const void* k, const void* v,
                                const int32_t* sel, void* out, float* lse, void* workspace,
                                size_t workspace_bytes, void* stream);

/* Gradient of the selected-set attention with the selection held fixed.  The
 * pages leave training of the router open (remio.ai, "The 99.35% result does
 * not prove language quality"); after selection the attention is an exact
 * softmax (aitechinspire.com "Snapshot"), whose gradient this is:
 *   P = 2^(c q.k - lse) over the selected keys, D_t = dO_t . O_t,
 *   dV = P^T dO, dS = P (dO V^T - D), dQ = scale dS K, dK = scale dS^T Q.
 *   q, k, v, sel  as passed to mdr_stage_attend_lse; out, lse its outputs;
 *   d_out [B,H,S,D] the gradient of out (cfg->dtype);
 *   dq, dk, dv [B,H,S,D] out (cfg->dtype), overwritten -- every row, including
 *   keys no token selected (zero remote share);
 *   workspace >= mdr_workspace_size bytes (its contents are overwritten).
 * Sums are fp32; each remote block's share of dQ is rounded once to the io
 * dtype before the slot-ordered sum.  Deterministic: no atomics. */
mdr_status mdr_stage_attend_backward(const mdr_config* cfg, const void* q, const void* k, const void* v,
                                     const int32_t* sel, const void* out, const float* lse,
                                     const void* d_out, void* dq, void* dk, void* dv, void* workspace,
                                     size_t workspace_bytes, void* stream);

/* Stages of the backward, in launch order: pair binning (count and scatter;
 * empty when R = 0 or nb <= L), row dots D, key blocks (dK, dV, remote dQ
 * shares), query blocks (dQ). */
#define MDR_BACKWARD_KERNELS 4

/* Profiling form of mdr_stage_attend_backward: events[k] (hipEvent_t created
 * by the caller) is recorded on `stream` just before the k-th stage above and
 * events[MDR_BACKWARD_KERNELS] after the last.  A NULL entry records nothing
 * at that point; a NULL `events` array is rejected.  Everything else as in
 * mdr_stage_attend_backward. */
mdr_status mdr_stage_attend_backward_profiled(const mdr_config* cfg, const void* q, const void* k,
                                              const void* v, const int32_t* sel, const void* out,
                                              const float* lse, const void* d_out, void* dq, void* dk,
                                              void* dv, void* workspace, size_t workspace_bytes,
                                              void* const* events, void* stream);

/* ---- streaming decode ----
 * Incremental routing for decoding (remio.ai, "What sparse attention
 * researchers should watch next", names it the open systems question).  Each
 * (b,h)'s posting lists are ring buffers of `capacity` entries per address:
 * block i is filed when it becomes eligible (for query block i + L), evicting
 * the address's oldest entry when full (remio.ai, "Monodratic turns sparse
 * attention into a retrieval decision": strict capacity, overflow drops
 * blocks).  A ring holds exactly the newest `capacity` eligible blocks of its
 * address, the view the prefill path reads, so a decoded token gets the
 * routing and output the prefill path gives the same token.
 *
 * cfg describes the cache: seq = its capacity in tokens; every other field as
 * for mdr_routed_attention (width ignored).  Additionally (remote + local) *
 * block <= 4096 and the candidate cut M <= 1024, else MDR_ERR_UNSUPPORTED.
 *
 * The state is one caller-owned device buffer of mdr_decode_state_size bytes
 * (256-byte aligned); its regions are described by mdr_decode_view.  Calls
 * that share a state must be ordered on one stream. */

/* Bytes of decode state for cfg; 0 when cfg is invalid or unsupported. */
size_t mdr_decode_state_size(const mdr_config* cfg);

/* Device pointers into a decode state (host arithmetic only, nothing launched):
 *   ring [B,H,A,capacity+1]: per address, the number n of blocks filed so far,
 *     then `capacity` slots of block ids, the k-th block filed (k = 0, 1, ...)
 *     sitting in slot k % capacity (-1 while empty);
 *   overflow [B,H] blocks evicted;
 *   summarized [B,H] and filed [B,H] block counts (blocks 0 .. count - 1);
 *   addr [B,H,nb] and ksum [B,H,nb,D] fp32 of the summarised blocks. */
typedef struct {
  int32_t* ring;
  int32_t* overflow;
  int32_t* summarized;
  int32_t* filed;
  int32_t* addr;
  float* ksum;
} mdr_decode_view;
mdr_status mdr_decode_state_view(const mdr_config* cfg, void* state, mdr_decode_view* view);

/* Resets the state for a cache holding n_tokens tokens (0 <= n_tokens < seq):
 * summarises the complete blocks among them and files the blocks a token at
 * position n_tokens may see (i <= n_tokens / block - L).
 *   k_cache [B,H,seq,D] (rows 0 .. n_tokens - 1 read); codebook [H,G,C,D] fp32;
 *   code_bias [H,G,C] or NULL. */
mdr_status mdr_decode_prime(const mdr_config* cfg, const void* k_cache, const float* codebook,
                            const float* code_bias, int32_t n_tokens, void* state, size_t state_bytes,
                            void* stream);

/* Routes and attends the n_new tokens at positions pos .. pos + n_new - 1, which
 * must lie in one block and continue where the prime or the previous step
 * ended.  Their K/V rows must already be in the cache.  Files any block that
 * became eligible first.
 *   q_new [B,H,n_new,D] (post-RoPE); k_cache, v_cache [B,H,seq,D];
 *   force [B,H,n_new] or NULL (as in mdr_routed_attention); out [B,H,n_new,D]
 *   overwritten; sel [B,H,n_new,R] out (-1 padded) or NULL. */
mdr_status mdr_decode_step(const mdr_config* cfg, const void* q_new, const void* k_cache, const void* v_cache,
                           const float* codebook, const float* code_bias, const int32_t* force, int32_t pos,
                           int32_t n_new, void* out, int32_t* sel, void* state, size_t state_bytes,
                           void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MDR_H */
