/*
 * dflash.h — C ABI of the DFlash draft step on AMD Instinct MI355X (gfx950).
 *
 * DFlash drafts for speculative decoding with a small block-diffusion model:
 * from the last verified token plus block-1 mask positions it proposes a whole
 * block of tokens in one non-causal forward pass, conditioned on hidden states
 * taken from five layers of the target model.  The three calls below follow
 * the pages' statement of one drafting round:
 *   - dflash_fuse_inject: fuse the target-layer features and inject them into
 *     every drafter layer's persistent K/V cache
 *     ("DFlash：drafter 的答案，早写在 target model 的隐层里", section 设计:
 *      Feature Fusion and KV Injection);
 *   - dflash_draft_block: one forward pass over [x0, mask x (block-1)] with
 *     non-causal attention inside the block and a shared lm_head
 *     ("DFlash原理深度剖析：块扩散如何用一次前向并行起草整块token", §二.1-§二.3,
 *      §三 step 1);
 *   - dflash_accept_trim: longest matching prefix plus the bonus token, and
 *     the cut of the drafter cache back to the committed length
 *     (same page, §三 step 3 and the paragraph 直观理解).
 *
 * Conventions shared by every call
 *   - Pointers marked "device" are HIP device addresses; everything else is
 *     host memory.  The caller allocates and owns every buffer, including the
 *     workspace; the library never allocates or frees device memory (its one
 *     buffer of its own is the fixed scratch array of dflash_draft_block_noalloc,
 *     a static device variable of the code object).
 *   - Calls are asynchronous and ordered on `stream` (a hipStream_t passed as
 *     void*, NULL = the null stream).  No call synchronises the device.
 *   - Calls on the same dflash_kv must not overlap.
 *   - Return value: 0 on success, or a negative DFLASH_E* code.  A call that
 *     returns an error detected on the host has launched nothing and left all
 *     buffers untouched.  DFLASH_EHIP means a launch failed part-way.
 *   - Errors found on the device (data-dependent) are OR-ed into the sticky
 *     word *kv->err (DFLASH_ERR_* bits); the kernels then clamp instead of
 *     touching memory out of range.  The caller reads err at its own sync
 *     points and clears it.
 *
 * Storage type: cfg->dtype selects fp32 or bf16 for the caller's weights and
 * target features.  With fp32 everything is computed in fp32 (a reference
 * path).  With bf16 the matrix cores run fp16 x fp16 with fp32 accumulation:
 * the weight matrices are converted once to fp16 by dflash_pack_weights, fp32
 * activations are rounded to fp16 where they enter a matrix core, and the K/V
 * cache is fp16; the residual stream, softmax, normalisation statistics and
 * every accumulation stay fp32.  fp16 carries 11 significant bits (bf16: 8)
 * but a smaller range: values must stay below 65504 in magnitude.
 */
#ifndef DFLASH_H
#define DFLASH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* storage types */
#define DFLASH_F32 0
#define DFLASH_BF16 1

/* host-side return codes */
#define DFLASH_OK 0
#define DFLASH_EINVAL (-1) /* null pointer, inconsistent dimensions, batch or rows out of range */
#define DFLASH_ERANGE (-2) /* block outside [2, block_max], unsupported head_dim / dtype / alignment */
#define DFLASH_ENOSPC (-3) /* workspace smaller than dflash_workspace_bytes() */
#define DFLASH_EHIP (-4)   /* a HIP launch failed */

/* device-side sticky error bits in *kv->err */
#define DFLASH_ERR_CTX_OVERFLOW 1 /* a write would pass max_ctx: skipped, len clamped */
#define DFLASH_ERR_TOKEN_RANGE 2  /* a token id outside [0, vocab): replaced by 0 */
#define DFLASH_ERR_NO_BASE 4      /* accept_trim on a sequence with no preceding draft: no trim */
#define DFLASH_ERR_NONFINITE 8    /* a value left the range of its storage type: an injected
                                     K/V value that is not finite in the cache's type, or a
                                     drafted row whose best score is not finite (its draft id
                                     is then 0).  With the bf16 storage type this is how an
                                     fp16 overflow (|x| >= 65520) anywhere in the draft shows:
                                     infinities turn into NaN downstream and reach the pick. */

/* Drafter dimensions.
 * hidden, n_q_heads*head_dim, inter and feat_hidden must be multiples of 256
 * for bf16 (64 for fp32); n_q_heads a multiple of n_kv_heads; head_dim 64 or
 * 128; 2 <= block_max <= 16; for bf16 also vocab a multiple of 16 and
 * (n_q_heads / n_kv_heads) * block_max <= 128; n_layers <= 32,
 * n_feat_layers <= 8.  Violations return DFLASH_ERANGE / DFLASH_EINVAL.
 * mask_token_id: the id whose (shared) embedding marks the block's mask
 * positions (normally vocab-1).  rms_eps: RMSNorm epsilon, x*(mean(x^2)+eps)^-1/2*g.
 * rope_theta: RoPE base; rotate-half pairs (i, i+head_dim/2), frequency
 * rope_theta^(-2i/head_dim), absolute 0-based positions. */
typedef struct dflash_config {
  int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim, inter, vocab;
  int32_t n_feat_layers, feat_hidden, block_max, mask_token_id;
  float rope_theta, rms_eps;
  int32_t dtype; /* DFLASH_F32 or DFLASH_BF16 */
} dflash_config;

/* Drafter weights, all device, caller-owned.  Per-layer
 * fields are HOST arrays of n_layers device pointers.  Shapes are PyTorch
 * Linear [out, in]:
 *   embed, lm_head  [vocab, hidden]   shared with the target
 *   fc              [hidden, n_feat_layers*feat_hidden]  fusion Linear, no bias;
 *                   column block i multiplies target layer i (shallow to deep)
 *   fc_norm, final_norm, in_norm[l], post_norm[l]   [hidden] RMSNorm gains
 *   wq [n_q_heads*head_dim, hidden]; wk, wv [n_kv_heads*head_dim, hidden]
 *   wo [hidden, n_q_heads*head_dim]; w_gate, w_up [inter, hidden];
 *   w_down [hidden, inter]
 * Memory layout (`layout`):
 *   fp32: DFLASH_LAYOUT_ROWMAJOR, every tensor row-major fp32.
 *   bf16: DFLASH_LAYOUT_PACKED: the matrices lm_head, fc, wq, wk, wv, wo,
 *     w_gate, w_up and w_down are fp16 in the fragment-packed layout written by
 *     dflash_pack_weight / dflash_pack_weights (below); embed stays row-major
 *     bf16 (it is gathered by row) and the gains are plain bf16 vectors.
 * Packing is part of the contract of the bf16 storage type: a checkpoint's
 * bf16 matrices are converted once, by the library (dflash_pack_weights), into
 * buffers the caller allocates, and the draft calls take the packed set.
 * Any other combination of dtype and layout returns DFLASH_EINVAL.
 * The calls take the batch size from kv->batch (the cache is sized for it). */
#define DFLASH_LAYOUT_ROWMAJOR 0
#define DFLASH_LAYOUT_PACKED 1
typedef struct dflash_weights {
  const void *embed, *fc, *fc_norm, *final_norm, *lm_head;
  const void *const *in_norm, *const *wq, *const *wk, *const *wv, *const *wo;
  const void *const *post_norm, *const *w_gate, *const *w_up, *const *w_down;
  int32_t layout; /* DFLASH_LAYOUT_* */
} dflash_weights;

/* Converts one bf16 matrix W [n, k] (row-major, device) to fp16 and writes it
 * in the fragment-packed layout the bf16-storage kernels stream (device dst of
 * n*k fp16, caller-owned, must not overlap src):
 *   dst[((c*(k/32) + t)*64 + l)*8 + j] = fp16(W[16c + l%16][32t + 8(l/16) + j])
 * for 16-row groups c, 32-column steps t, lanes l < 64 and j < 8: each 1 KB
 * piece is the B operand of one 16x16x32 fp16 matrix-core instruction over 16
 * output rows, so one wavefront load of it is fully contiguous.  The conversion
 * rounds to nearest even: exact for 2^-14 <= |w| < 65504, values below 2^-14
 * become fp16 subnormals (absolute error < 2^-25); a value that does not fit
 * fp16 (|w| >= 65520, infinities and NaN) is written as infinity or NaN and
 * counted: n_overflow (device int32, nullable) is incremented by the number of
 * such elements, so a caller that loads weights reads it once afterwards (0 =
 * every element converted to a finite fp16).
 * Requires n % 16 == 0 and k % 32 == 0 (DFLASH_ERANGE otherwise); null pointers
 * or n, k <= 0 return DFLASH_EINVAL.  Asynchronous on `stream`; call once when
 * loading weights. */
int dflash_pack_weight(const void *src, int32_t n, int32_t k, void *dst, int32_t *n_overflow,
                       void *stream);

/* The one-time preparation of a bf16 checkpoint: every matrix of `src` (bf16,
 * DFLASH_LAYOUT_ROWMAJOR, PyTorch [out, in] shapes as above) is packed with
 * dflash_pack_weight into the corresponding buffer of `dst` (fp16,
 * DFLASH_LAYOUT_PACKED; n*k elements each, caller-allocated, no overlap with
 * src): lm_head, fc and per layer wq, wk, wv, wo, w_gate, w_up, w_down (fc NULL in
 * both: a target model for dflash_target_verify, skipped).  embed and the gains are
 * not touched (dst may point at src's).  n_overflow as for
 * dflash_pack_weight, summed over all matrices.  cfg->dtype must be DFLASH_BF16
 * (DFLASH_ERANGE otherwise); a wrong layout or a null matrix pointer returns
 * DFLASH_EINVAL before anything is launched.  Asynchronous on `stream`. */
int dflash_pack_weights(const dflash_config *cfg, const dflash_weights *src,
                        const dflash_weights *dst, int32_t *n_overflow, void *stream);

/* Per-sequence drafter K/V cache, caller-owned, one slice of max_ctx*head_dim
 * elements per (sequence b, kv head h) at offset (b*n_kv_heads + h)*max_ctx*head_dim
 * of k[l] and of v[l] (device); RoPE applied to K.
 *   fp32 storage type: fp32, K[pos][dim] and V transposed, V[dim][pos].
 *   bf16 storage type: fp16, fragment-packed so that a 64-position tile of K and
 *   of V is contiguous and in matrix-core operand order (D = head_dim):
 *     K(pos, dim) at ((pos/16)*(D/32) + dim/32)*512 + (pos%16 + 16*((dim%32)/8))*8 + dim%8
 *     V(pos, dim) at ((pos/32)*(D/16) + dim/16)*512 + (dim%16 + 16*g)*8 + j
 *       with r = pos%32, g = (r%16)/4, j = r%4 + (r >= 16 ? 4 : 0).
 *   len   device int32 [batch]  committed (injected) positions
 *   base  device int32 [batch]  len at the last draft; -1 = no draft yet
 *   err   device int32 [1]      sticky DFLASH_ERR_* bits
 * max_ctx must be a multiple of 64.  A draft needs len + block <= max_ctx:
 * the block's own K/V are written to positions [len, len+block) as scratch. */
typedef struct dflash_kv {
  void *const *k;
  void *const *v;
  int32_t *len, *base, *err;
  int32_t batch, max_ctx;
} dflash_kv;

/* Optional parity and timing hooks, passed per call (any field may be NULL / 0;
 * a per-call pointer rather than a process-wide setting, so that calls on
 * different streams or threads never see each other's hooks).  Never needed
 * for drafting.
 * Parity outputs (device, fp32); a non-null `logits` or `top2` switches the
 * lm_head to a variant that also stores every logit / tracks the runner-up:
 *   fused         [total_rows, hidden]       fuse_inject: RMSNorm'd fused feature
 *   final_hidden  [batch, block, hidden]     draft: output of the final RMSNorm
 *   logits        [batch, block-1, vocab]    draft: lm_head outputs of rows 1..block-1
 *   top2          [batch, block-1, 2]        draft: per drafted row the best and the
 *                                            second-best score (logit, or with
 *                                            sampling logit / T + noise) over the
 *                                            vocabulary; equal on a tie
 * Timing: when `timed` names a launch class (DFLASH_TIME_*), the i-th launch
 * of that class (i = n_used, n_used+1, ... while 2i+1 < n_events) records
 * events[2i] when its kernel starts and events[2i+1] when it ends (recorded by
 * the dispatch itself, so the pair brackets the kernel and no launch gap;
 * attention: the split kernel, which reads the cache; fp32: the one kernel), and n_used
 * advances.  events is a host array of hipEvent_t created by the caller. */
#define DFLASH_TIME_NONE 0
#define DFLASH_TIME_GEMM 1   /* projection GEMMs: fusion, injection, QKV, O, gate|up, down */
#define DFLASH_TIME_LMHEAD 2 /* lm_head + fused argmax */
#define DFLASH_TIME_ATTN 3   /* block attention: the split kernel */
typedef struct dflash_debug {
  float *fused, *final_hidden, *logits;
  void *const *events;
  int32_t n_events, n_used, timed;
  float *top2;
} dflash_debug;

/* Bytes of workspace that covers every call below for this config, batch, any
 * fuse_inject row count up to `max_rows`, any block up to cfg->block_max and
 * cache capacity max_ctx.  Non-decreasing in max_rows and max_ctx.  Pure host
 * function; 0 for an invalid configuration. */
size_t dflash_workspace_bytes(const dflash_config *cfg, int32_t batch, int32_t max_rows,
                              int32_t max_ctx);

/* Fuse + inject ("DFlash：drafter 的答案…", section 设计, Feature Fusion and KV
 * Injection; "DFlash原理深度剖析", §二.3).
 * feats: HOST array of n_feat_layers device pointers, each [total_rows, feat_hidden],
 *   target layers in ascending order.  Rows are packed per sequence:
 *   sequence b owns rows row_start[b] .. row_start[b]+row_count[b]-1 (device
 *   int32 [batch] arrays; ranges must not overlap; rows outside every range
 *   are ignored; row_count may be 0).
 * For every row: c = RMSNorm(concat_i feats_i[row] . fc^T; fc_norm), then for
 * every layer l: K = RoPE(c . wk[l]^T) and V = c . wv[l]^T at position
 * len[b] + (row - row_start[b]) are written into k[l], v[l].  Finally
 * len[b] += row_count[b].  Covers the prefill (all context rows) and the
 * per-round re-injection of the accepted rows (row_start = block*b,
 * row_count = accept_len). */
int dflash_fuse_inject(const dflash_config *cfg, const dflash_weights *w,
                       const void *const *feats, const int32_t *row_start,
                       const int32_t *row_count, int32_t total_rows, dflash_kv *kv,
                       void *ws, size_t ws_bytes, dflash_debug *dbg, void *stream);

/* Draft one block per sequence ("DFlash原理深度剖析", §二.1 mask block, §二.2
 * non-causal attention, §三 step 1; "DFlash：drafter 的答案…", section 设计,
 * Parallel Drafting).
 * last_tok: device int32 [kv->batch], the last verified token x0 of each sequence.
 * The block [x0, mask x (block-1)] sits at positions len..len+block-1; every
 * layer attends, without a causal mask, over the injected context keys
 * [0, len) and the block's own keys; the final RMSNorm of rows 1..block-1 goes
 * through the shared lm_head and the greedy pick (lowest id on ties) is
 * written to draft_ids: device int32 [batch, block-1].  Sets base = len;
 * writes the block's K/V to cache positions [len, len+block); len is unchanged. */
int dflash_draft_block(const dflash_config *cfg, const dflash_weights *w, dflash_kv *kv,
                       const int32_t *last_tok, int32_t block, int32_t *draft_ids, void *ws,
                       size_t ws_bytes, dflash_debug *dbg, void *stream);

/* dflash_draft_block for callers that cannot allocate memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same draft, with its workspace in a scratch array of the library's own,
 * DFLASH_NOALLOC_SCRATCH_BYTES per GPU, held from the first call on that GPU
 * until the process ends.  Calls nothing that allocates.  A draft whose
 * workspace (dflash_workspace_bytes(cfg, kv->batch, 0, kv->max_ctx) bounds it)
 * exceeds the scratch returns DFLASH_ENOSPC before anything is launched.
 * Every call on one GPU shares that GPU's scratch: calls that overlap on one
 * GPU (different streams, or threads without ordering) race and must not be
 * made.  The scratch holds no state between calls. */
#define DFLASH_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int dflash_draft_block_noalloc(const dflash_config *cfg, const dflash_weights *w, dflash_kv *kv,
                               const int32_t *last_tok, int32_t block, int32_t *draft_ids,
                               dflash_debug *dbg, void *stream);

/* Sampling parameters of dflash_draft_block_sampled. */
typedef struct dflash_sampling {
  float temperature; /* > 0: sample; <= 0: the greedy pick of dflash_draft_block; must be
                        finite (NaN or infinity: DFLASH_EINVAL); a positive value whose
                        inverse overflows float is the greedy limit */
  uint64_t seed;     /* the Philox key: low half key word 0, high half key word 1 */
  uint64_t offset;   /* Philox counter word 3 (e.g. a round or request counter);
                        below 2^32, else DFLASH_EINVAL */
} dflash_sampling;

/* Draft one block per sequence with temperature sampling instead of the
 * greedy pick.  The pages report drafting under sampling (temperature 1) and
 * verify by comparing the draft position by position with the target's
 * *sampled* tokens, keeping the longest matching prefix
 * ("DFlash：drafter 的答案…", results; "DFlash原理深度剖析", §三 step 3), so
 * dflash_accept_trim is unchanged; the target's sampled tokens go in
 * target_ids.
 * Everything is as in dflash_draft_block except the pick: row r (1..block-1)
 * of sequence b, which drafts position p = len[b] + r, takes
 *   argmax_v ( logit_v / temperature + g_v ),   g_v = -log(-log u_v)
 * (the Gumbel-max form of sampling from softmax(logits / temperature)), with
 *   x   = word (v / 16) mod 4 of the Philox4x32-10 block (Salmon et al.,
 *         SC 2011) at counter (v with bits 4 and 5 cleared, p, b, offset) and
 *         key (seed mod 2^32, seed div 2^32): one block serves ids v, v+16,
 *         v+32, v+48;
 *   u_v = (2 floor(x / 2^9) + 1) / 2^24.
 * Ties go to the lowest id.  The noise is computed in the lm_head's epilogue,
 * so no logits or noise are stored.  smp: host pointer; NULL or temperature <= 0
 * gives the greedy pick.  Repeating a call with the same seed and offset at the
 * same positions repeats the noise; vary `offset` to draw afresh. */
int dflash_draft_block_sampled(const dflash_config *cfg, const dflash_weights *w, dflash_kv *kv,
                               const int32_t *last_tok, int32_t block,
                               const dflash_sampling *smp, int32_t *draft_ids, void *ws,
                               size_t ws_bytes, dflash_debug *dbg, void *stream);

/* Accept + trim ("DFlash原理深度剖析", §三 step 3 and 直观理解).
 * draft_ids: device int32 [batch, block-1]; target_ids: device int32 [batch, block],
 * target_ids[b, i] being the target's token for position base+1+i.
 * n = length of the longest prefix with draft_ids == target_ids;
 * accept_len[b] = n + 1 (device int32 [batch], in [1, block]);
 * bonus[b] = target_ids[b, n] (device int32 [batch]);
 * len[b] = min(len[b], base[b] + accept_len[b]) — so injecting the verified
 * block's rows before or after this call leaves the same cache. */
int dflash_accept_trim(const dflash_config *cfg, const int32_t *draft_ids,
                       const int32_t *target_ids, int32_t block, int32_t *accept_len,
                       int32_t *bonus, dflash_kv *kv, void *stream);

/* ---- beyond the draft step: a synthetic target, and the input-fusion ablation ---- */

/* One causal pass of an autoregressive target model over a block of given tokens
 * per sequence: the verification of a drafted block ("DFlash原理深度剖析", §三
 * step 2: the target scores every position of the block in one pass) and, block by
 * block, a prefill or plain decoding.  The target has the drafter's layer form
 * (pre-norm attention with GQA and RoPE, then SwiGLU; cfg, w and kv describe the
 * target: cfg->n_layers its depth, w its embed / layers / final_norm / lm_head; fc
 * and fc_norm are not read) and is causal: block row r sees the cached positions
 * and rows 0..r.
 * block_ids: device int32 [kv->batch, block], the tokens at positions
 *   len[b] .. len[b] + block - 1 (1 <= block <= cfg->block_max);
 * target_ids: device int32 [batch, block], the greedy next token after each row
 *   (lowest id on ties) -- for a block [x0, d_0, ...] exactly the target_ids of
 *   dflash_accept_trim;
 * capture: NULL, or a host array of cfg->n_feat_layers strictly increasing layer
 *   indices; feats_out[i] (device, [batch * block, hidden] in cfg->dtype) then
 *   receives the residual stream leaving layer capture[i] for every row, the
 *   features dflash_fuse_inject takes (rows b * block ..).
 * Writes the block's K/V at [len, len + block), sets base = len and len += block,
 * so dflash_accept_trim on this cache keeps the accepted prefix.  Workspace:
 * dflash_workspace_bytes(cfg, batch, 0, max_ctx). */
int dflash_target_verify(const dflash_config *cfg, const dflash_weights *w, dflash_kv *kv,
                         const int32_t *block_ids, int32_t block, const int32_t *capture,
                         void *const *feats_out, int32_t *target_ids, void *ws, size_t ws_bytes,
                         void *stream);

/* The injection of the ablation that feeds the target features only into the
 * drafter's first layer input, as EAGLE-3 does, instead of every layer's K/V
 * ("DFlash：drafter 的答案…", 设计 / KV Injection and the first ablation of the
 * results).  Same arguments as dflash_fuse_inject, plus rows_max (host): an upper
 * bound of any sequence's row_count.  Each row's fused feature
 * c = RMSNorm(concat_i feats_i[row] . fc^T; fc_norm) is the first layer's input at
 * its position len[b] + j; the rows run causally through the drafter's layers (row
 * j sees the cache and rows 0..j), each layer appending the K/V it computes; the
 * last layer only contributes its K/V.  Then len[b] += row_count[b].  The draft
 * calls are unchanged.  Rows are processed block_max at a time, ceil(rows_max /
 * block_max) passes.  Workspace: dflash_fuse_inject_input_workspace_bytes. */
size_t dflash_fuse_inject_input_workspace_bytes(const dflash_config *cfg, int32_t batch,
                                                int32_t max_rows, int32_t max_ctx);
int dflash_fuse_inject_input(const dflash_config *cfg, const dflash_weights *w,
                             const void *const *feats, const int32_t *row_start,
                             const int32_t *row_count, int32_t rows_max, int32_t total_rows,
                             dflash_kv *kv, void *ws, size_t ws_bytes, dflash_debug *dbg,
                             void *stream);

/* Static description of a return code. */
const char *dflash_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* DFLASH_H */
