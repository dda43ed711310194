/*
 * tt.h -- C ABI of libtt: the block-denoising step of a two-tower block
 * mask-diffusion language model, hand-written for AMD MI355X (gfx950).
 *
 * Pages cited (title, site):
 *   [keyframe]  "Diffusion Nemotron: Nvidia's "Two Brain" Diffusion Model"
 *               (keyframe.defihacklabs.io)
 *   [news]      "NVIDIA发布Nemotron两塔模型，实现2.42倍文本生成吞吐并保持98.7%质量"
 *               (889990.xyz)
 *   [dothoosh]  "فرآیند انتشار در برابر رمزگشایی متوالی در مدل جدید انویدیا"
 *               (dothoosh.com)
 *   [modelcard] "Nemotron-Labs-TwoTower-30B-A3B-Base-BF16" digest (aitrends.kr)
 *
 * Conventions shared by every entry point:
 *   - Pointers marked "device" are HIP device (or managed) memory; "host"
 *     pointers are ordinary CPU memory.  The caller owns every buffer.  The
 *     library allocates no device memory: scratch space comes from a
 *     caller-provided workspace sized by the matching *_workspace_size().
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL means the null
 *     stream), except tt_denoise_block, which waits on the stream once per
 *     denoising step to read how many slots are still masked.
 *   - Every host-visible argument is validated before anything is launched.
 *     An invalid call returns a status, stores a message readable through
 *     tt_last_error() and launches nothing.  A failing HIP call returns
 *     TT_ERR_HIP.
 *   - Device-side checks (debugging aid): with the environment variable
 *     TT_VALIDATE set to anything but "" or "0", every call that takes the
 *     context arrays (the attention calls, tt_ctx_advance, the denoise and
 *     generation loops, the weighted sublayer) first runs one small kernel
 *     over them and waits for its outcome.  It returns TT_ERR_INVALID_ARG,
 *     naming the first offending sequence, when for an active sequence b
 *     ctx_len[b] < 0, ctx_start[b] < 0, ctx_end[b] < ctx_start[b] +
 *     ctx_len[b], or (with ctx_end, up to 8192 sequences) its reserved
 *     region overlaps another active sequence's; nothing else of the call is
 *     launched then.  Checked calls are synchronous.  The outcome lives in a
 *     small array in each GPU's memory, so two checked calls on one GPU must
 *     not overlap in time.
 *   - No global mutable state besides the thread-local error message (and
 *     the per-GPU arrays of TT_VALIDATE and tt_block_attn_noalloc); calls on
 *     different streams with different workspaces may run concurrently.
 *     Two calls in flight must not share one workspace.
 *   - bf16 is IEEE-754 binary32 truncated to its upper 16 bits (bfloat16).
 *   - Limits: head_dim in {64, 128}; block_size S in [1, 64]; n_q_heads a
 *     multiple of n_kv_heads; temperature finite and > 0; gamma finite.
 */
#ifndef TT_H
#define TT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TT_ABI_VERSION 4
#define TT_TIMESTEP_DIM 256 /* width of the timestep embedding */

typedef enum {
  TT_OK = 0,
  TT_ERR_INVALID_ARG = 1, /* a pointer, size or value outside the contract  */
  TT_ERR_UNSUPPORTED = 2, /* valid but not implemented (e.g. head_dim 96)    */
  TT_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required     */
  TT_ERR_HIP = 4,         /* a HIP runtime call failed                       */
  TT_ERR_CALLBACK = 5     /* a step-provider callback returned non-zero     */
} tt_status;

typedef enum { TT_BF16 = 0, TT_F32 = 1 } tt_dtype;

typedef void* tt_stream; /* hipStream_t */

/* Message of the last failing call on this thread ("" if none).  Valid until
 * the next libtt call on the same thread. */
const char* tt_last_error(void);

/* TT_ABI_VERSION of the loaded library. */
int tt_abi_version(void);

/* Shape of one attention layer of the denoiser.  batch = B sequences, each
 * with one block of block_size = S slots; n_q_heads = Hq, n_kv_heads = Hkv,
 * head_dim = d; dtype (a tt_dtype) is the storage type of q/k/v/residual/out
 * and of the context cache. */
typedef struct {
  int32_t batch;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t block_size;
  int32_t dtype;
} tt_attn_shape;

/* ------------------------------------------------------------------------
 * tt_block_attn -- one denoiser attention layer over [context KV ; block KV].
 *
 * [dothoosh] two-tower mechanism section: inside a block the denoiser
 * attends bidirectionally, and causally to the earlier clean blocks; layer i
 * of the denoiser talks to layer i of the frozen context tower, which keeps
 * the per-layer KV cache of the prompt and committed tokens.  [modelcard]
 * technical features section: bidirectional self-attention inside the block
 * plus layer-aligned cross-attention to the same layer's context KV, with
 * adaLN-single scale/shift/gate per timestep.
 *
 * For sequence b, query head h and its KV head g = h / (Hq/Hkv):
 *   keys   K = [k_ctx[ctx_start[b] .. ctx_start[b]+ctx_len[b]-1, g, :] ;
 *               k_blk[b, 0..S-1, g, :]]          (V likewise)
 *   q'     = q_blk[b, s, h, :] * (1 + ada_scale[b, h*d:(h+1)*d])
 *            + ada_shift[b, h*d:(h+1)*d]
 *   o      = softmax(q' K^T / sqrt(d)) V           (one softmax over all keys)
 *   lse    = ln sum_j exp(q' K_j / sqrt(d))
 *   out    = residual + ada_gate[b, h*d:(h+1)*d] * o
 * (missing shift/scale: 0; missing gate: 1; missing residual: 0).  All S
 * slots are computed alike, masked ones included.
 *
 * Layouts (row-major, contiguous):
 *   q_blk, residual, out  device [B, S, Hq, d]   dtype
 *   k_blk, v_blk          device [B, S, Hkv, d]  dtype
 *   k_ctx, v_ctx          device [T_ctx, Hkv, d] dtype  (this layer's cache;
 *                         sequence b owns tokens ctx_start[b] ..
 *                         ctx_start[b]+ctx_len[b]-1; sequences may share or
 *                         interleave nothing else is assumed)
 *   ctx_start             device [B] int64, ctx_len device [B] int32 (>= 0)
 *   active                device [B] uint8 or NULL (all active); for an
 *                         inactive sequence nothing is read or written
 *   ada_shift/scale/gate  device [B, Hq*d] fp32, each may be NULL
 *   lse                   device [B, S, Hq] fp32 or NULL
 * max_ctx_len (host) sizes the launch; correctness never depends on it, but
 * sequences longer than it run with less parallelism.  residual may alias
 * out.  q_blk/k_blk/v_blk/k_ctx/v_ctx/out/residual and the three ada vectors
 * must be 16-byte aligned.
 * Precision (bf16): q' and the probabilities are rounded to bf16 for the
 * matrix cores, sums are fp32, out is rounded to nearest-even.  (fp32: all
 * fp32.)  Deterministic: identical inputs give identical bits.
 * Errors: TT_ERR_INVALID_ARG (null required pointer, bad shape, Hq % Hkv,
 * max_ctx_len < 0), TT_ERR_UNSUPPORTED (head_dim not 64/128),
 * TT_ERR_WORKSPACE (workspace NULL or smaller than
 * tt_block_attn_workspace_size(shape, max_ctx_len)), TT_ERR_HIP.
 * The workspace needs no initialisation; its contents are dead after the
 * call's kernels finish.
 * ---------------------------------------------------------------------- */
size_t tt_block_attn_workspace_size(const tt_attn_shape* shape, int32_t max_ctx_len);

tt_status tt_block_attn(const tt_attn_shape* shape,
                        const void* q_blk, const void* k_blk, const void* v_blk,
                        const void* k_ctx, const void* v_ctx,
                        const int64_t* ctx_start, const int32_t* ctx_len,
                        int32_t max_ctx_len, const uint8_t* active,
                        const float* ada_shift, const float* ada_scale,
                        const float* ada_gate, const void* residual,
                        void* out, float* lse,
                        void* workspace, size_t workspace_bytes, tt_stream stream);

/* ------------------------------------------------------------------------
 * tt_block_attn_noalloc -- tt_block_attn for callers that cannot allocate:
 * code under HIP graph capture, tight serving loops and harnesses that forbid
 * hipMalloc.  It computes exactly what tt_block_attn computes (same kernels,
 * same launch, identical bits) but takes no workspace: its partial results go
 * to a scratch array of TT_BLOCK_ATTN_SCRATCH_BYTES that the library keeps in
 * each GPU's memory until the process ends.  The call allocates nothing
 * (no hipMalloc, hipFree or allocating library routine); its first call on a
 * device looks up that device's copy of the array.
 * Arguments, layouts, precision and errors are tt_block_attn's, plus
 * TT_ERR_WORKSPACE when tt_block_attn_workspace_size(shape, max_ctx_len)
 * exceeds TT_BLOCK_ATTN_SCRATCH_BYTES (64 MiB: every shape whose
 * B * Hkv * ceil(S * Hq / Hkv / 256) stays within the compute-unit count,
 * e.g. B = 64, S = 16, Hq = 32, Hkv = 2, d = 128 at any context length,
 * needs at most 17 MiB).  The scratch needs no initialisation.
 * All calls on one GPU share its scratch: two calls that overlap in time on
 * one GPU (different streams or threads without ordering between them) race
 * and may return wrong results; calls in one stream's order are safe.
 * ---------------------------------------------------------------------- */
#define TT_BLOCK_ATTN_SCRATCH_BYTES (64ull << 20)

tt_status tt_block_attn_noalloc(const tt_attn_shape* shape,
                                const void* q_blk, const void* k_blk, const void* v_blk,
                                const void* k_ctx, const void* v_ctx,
                                const int64_t* ctx_start, const int32_t* ctx_len,
                                int32_t max_ctx_len, const uint8_t* active,
                                const float* ada_shift, const float* ada_scale,
                                const float* ada_gate, const void* residual,
                                void* out, float* lse, tt_stream stream);

/* ------------------------------------------------------------------------
 * tt_ctx_block_attn -- one attention layer of the frozen context tower over
 * a block that has just been committed, with the append of that block's K/V
 * to the layer's cache.
 *
 * [dothoosh] two-tower mechanism section: the context tower runs causally
 * over the prompt and the committed tokens and produces every layer's KV
 * cache, which the denoiser reads layer by layer.  [news] architecture
 * details section: the autoregressive context tower is the part that
 * generates the KV cache.  (Reading: once a block is final, the context tower
 * consumes its S tokens like an autoregressive prefill chunk.)
 *
 * For sequence b, query head h, KV head g = h / (Hq/Hkv) and block token s:
 *   keys   K_s = [k_ctx[ctx_start[b] .. ctx_start[b]+ctx_len[b]-1, g, :] ;
 *                 k_blk[b, 0..s, g, :]]          (V likewise: causal in the block)
 *   o      = softmax(q_blk[b, s, h, :] K_s^T / sqrt(d)) V_s
 *   lse    = ln sum_j exp(q_blk[b, s, h, :] K_s,j / sqrt(d))
 *   out    = residual + o                     (no adaLN: denoiser only)
 * Append: when ctx_end is non-NULL, every active sequence b with
 * ctx_len[b] + S <= ctx_end[b] - ctx_start[b] also gets
 *   k_ctx[ctx_start[b] + ctx_len[b] + s, g, :] = k_blk[b, s, g, :]  (s < S, all g)
 * (v likewise).  ctx_len is NOT changed (call tt_ctx_advance once after the
 * last layer); a sequence without room is not written, and its attention is
 * still computed.  Sequences' reserved regions [ctx_start[b], ctx_end[b])
 * must not overlap.  NULL ctx_end: attention only, the cache is read-only.
 *
 * Layouts, alignment, precision, determinism and errors are those of
 * tt_block_attn (ada vectors absent); ctx_end is device [B] int64.  The
 * workspace is sized by tt_block_attn_workspace_size(shape, max_ctx_len).
 * ---------------------------------------------------------------------- */
tt_status tt_ctx_block_attn(const tt_attn_shape* shape,
                            const void* q_blk, const void* k_blk, const void* v_blk,
                            void* k_ctx, void* v_ctx,
                            const int64_t* ctx_start, const int32_t* ctx_len,
                            const int64_t* ctx_end, int32_t max_ctx_len,
                            const uint8_t* active, const void* residual,
                            void* out, float* lse,
                            void* workspace, size_t workspace_bytes, tt_stream stream);

/* ------------------------------------------------------------------------
 * tt_ctx_advance -- grow every context that took the block: for each active
 * sequence b (active NULL = all) with ctx_len[b] + block_size <=
 * ctx_end[b] - ctx_start[b]: ctx_len[b] += block_size and appended[b] = 1;
 * otherwise ctx_len[b] is unchanged and appended[b] = 0.  The room test is
 * the one tt_ctx_block_attn's append uses, so after the layers' append calls
 * and this call the caches and lengths agree ([dothoosh] two-tower mechanism
 * section: the context tower's cache covers the prompt and every committed
 * token).
 *   ctx_start, ctx_end device [B] int64; ctx_len device [B] int32 in/out;
 *   active device [B] uint8 or NULL; appended device [B] uint8 out or NULL.
 * Errors: TT_ERR_INVALID_ARG (batch < 0, block_size outside [1, 64], NULL
 * or misaligned ctx_start/ctx_end/ctx_len), TT_ERR_HIP.
 * ---------------------------------------------------------------------- */
tt_status tt_ctx_advance(int32_t batch, int32_t block_size, const int64_t* ctx_start,
                         const int64_t* ctx_end, int32_t* ctx_len, const uint8_t* active,
                         uint8_t* appended, tt_stream stream);

/* Zero-fill `bytes` of device memory at `workspace` on `stream` with a
 * kernel (no memset node, so the call can sit inside captured graphs). */
tt_status tt_workspace_clear(void* workspace, size_t bytes, tt_stream stream);

/* ------------------------------------------------------------------------
 * tt_timestep_embed -- the 256-wide sinusoidal embedding of the diffusion
 * timestep that feeds adaLN-single ([dothoosh] two-tower mechanism section:
 * every layer is modulated by the diffusion timestep through adaLN-single;
 * the embedding is not on the pages: DiT's sinusoid is used):
 *   emb[b, i]       = cos(1000 * t[b] * 10000^(-i/128)),  i < 128
 *   emb[b, 128 + i] = sin(1000 * t[b] * 10000^(-i/128))
 * t device [B] fp32, emb device [B, 256] fp32.  Computed in fp64.
 * ---------------------------------------------------------------------- */
tt_status tt_timestep_embed(int32_t batch, const float* t, float* emb, tt_stream stream);

/* ------------------------------------------------------------------------
 * tt_adaln_single -- per-layer (shift, scale, gate) vectors from the timestep
 * embedding ([dothoosh] two-tower mechanism section: adaLN-single adds about
 * 1.5 M parameters; [modelcard] technical features section: scale, shift and
 * gate per timestep for every denoiser layer):
 *   u[b, :]          = SiLU(t_emb[b, :]) @ w + bias           (fp32 sums)
 *   ada[l, j, b, c]  = u[b, j*width + c] + table[l, j, c]
 * with j = 0 shift, 1 scale, 2 gate.
 *   t_emb device [B, 256] fp32;  w device [256, 3*width] bf16;
 *   bias device [3*width] fp32 or NULL;  table device [n_layers, 3, width]
 *   fp32 or NULL;  ada device [n_layers, 3, B, width] fp32.
 * width must be a multiple of 4; w must be 8-byte aligned; ada, bias and
 * table must be 16-byte aligned.
 * ---------------------------------------------------------------------- */
tt_status tt_adaln_single(int32_t batch, int32_t width, int32_t n_layers,
                          const float* t_emb, const void* w, const float* bias,
                          const float* table, float* ada, tt_stream stream);

/* ------------------------------------------------------------------------
 * tt_confidence_unmask -- one unmasking pass over B blocks.
 *
 * [keyframe] key point 3: all masked slots of the block are predicted at
 * once, confident tokens are committed step by step and the undetermined
 * rest is masked again.  [dothoosh] benchmark paragraph: the confidence
 * threshold gamma sets how many tokens a step commits.  [news] code example:
 * confidence_threshold=0.8, mask_token_id=3, temperature=0.1.
 *
 * For every slot (b, s) with masked[b, s] != 0 on entry:
 *   pred = lowest v with logits[b, s, v] = max_v logits[b, s, v]
 *   p    = 1 / sum_v exp((logits[b, s, v] - max) / temperature)
 * Commit set of sequence b: C = {s : p >= gamma}; if C is empty and some
 * slot is masked, C = {the slot of largest p, lowest s on ties}.  For s in
 * C: tokens = pred, masked = 0, committed_now = 1, commit_step = step.
 * Other masked slots: tokens = mask_token_id, committed_now = 0.  Slots not
 * masked on entry are left alone (committed_now 0, conf NaN, pred -1).
 * n_masked[b] = masked slots left.
 * Decisions are exact with respect to fp64 arithmetic: p is computed in fp32
 * and every p within 2^-14 of gamma (or of the best p, when the one-commit
 * rule applies) is recomputed in fp64 before it decides anything.
 *   logits   device, element (b, s, v) at ((b*S + s) * row_stride + v),
 *            dtype TT_BF16 or TT_F32, finite (or -inf with one finite
 *            value per row)
 *   tokens   device [B, S] int32 in/out;  masked device [B, S] uint8 in/out
 *   committed_now, conf (fp32), pred (int32), commit_step (int8): device
 *            [B, S], each may be NULL; commit_step is only written at
 *            committed slots
 *   n_masked device [B] int32 out, may be NULL
 * Errors: TT_ERR_INVALID_ARG (null logits/tokens/masked, block_size outside
 * [1, 64], vocab < 1, row_stride < vocab, temperature not > 0, gamma NaN),
 * TT_ERR_WORKSPACE, TT_ERR_HIP.
 * ---------------------------------------------------------------------- */
size_t tt_unmask_workspace_size(int32_t batch, int32_t block_size, int32_t vocab);

tt_status tt_confidence_unmask(int32_t batch, int32_t block_size, int32_t vocab,
                               const void* logits, int32_t dtype, int64_t row_stride,
                               float gamma, float temperature, int32_t mask_token_id,
                               int32_t step, int32_t* tokens, uint8_t* masked,
                               uint8_t* committed_now, float* conf, int32_t* pred,
                               int8_t* commit_step, int32_t* n_masked,
                               void* workspace, size_t workspace_bytes, tt_stream stream);

/* ------------------------------------------------------------------------
 * tt_sample_unmask -- tt_confidence_unmask with temperature sampling.
 *
 * [news] training and inference section, code example: the generation call
 * takes a temperature (0.1) next to the confidence threshold (0.8).
 * [keyframe] key point 3: all masked slots are predicted at once and the
 * confident ones are committed.  (Reading: the prediction of a masked slot
 * is drawn from softmax(l / temperature); its confidence is the probability
 * of the drawn token under that distribution.)
 *
 * For every slot (b, s) with masked[b, s] != 0 on entry:
 *   G_v  = -ln(-ln u_v),  u_v = (2 * (w_v >> 9) + 1) / 2^24,  where w_v is
 *          word v % 4 of Philox4x32-10 (Salmon et al., SC 2011) with
 *          key = (seed & 0xffffffff, seed >> 32) and
 *          counter = (v / 4, b * S + s, step, block_index)
 *   pred = lowest v maximising logits[b, s, v] + temperature * G_v
 *          (the Gumbel-max draw from softmax(logits / temperature))
 *   p    = exp((logits[b, s, pred] - max) / temperature)
 *          / sum_v exp((logits[b, s, v] - max) / temperature)
 * and then the commit rule of tt_confidence_unmask, unchanged (gamma <= 0
 * commits every masked slot).  Decisions are exact with respect to fp64:
 * rows whose two best perturbed scores lie within 2^-17 (1 + |max| +
 * 20 temperature) are rescored in fp64, and p is rechecked in fp64 near
 * gamma as in tt_confidence_unmask.
 * Arguments, layouts and errors are those of tt_confidence_unmask, plus
 * TT_ERR_INVALID_ARG for step < 0 or block_index < 0.  The workspace is
 * sized by tt_unmask_workspace_size (the same size serves both calls).
 * Cost: one read of every masked row; only the tokens within
 * 20 * temperature of their slice's maximum draw noise, so large
 * temperatures over flat logits cost more arithmetic.
 * ---------------------------------------------------------------------- */
tt_status tt_sample_unmask(int32_t batch, int32_t block_size, int32_t vocab,
                           const void* logits, int32_t dtype, int64_t row_stride,
                           float gamma, float temperature, uint64_t seed,
                           int32_t block_index, int32_t mask_token_id, int32_t step,
                           int32_t* tokens, uint8_t* masked, uint8_t* committed_now,
                           float* conf, int32_t* pred, int8_t* commit_step,
                           int32_t* n_masked, void* workspace, size_t workspace_bytes,
                           tt_stream stream);

/* ------------------------------------------------------------------------
 * tt_denoise_block -- the block denoising loop ([dothoosh] two-tower
 * mechanism section: a block starts as [MASK] tokens and is refined over T
 * steps until final; [news] code example: steps_per_block = block_size =
 * 16).  For step k = 0 .. max_steps-1 while any slot is masked:
 *   1. t[b] = n_masked[b] / S; emb = tt_timestep_embed(t);
 *      ada = tt_adaln_single(emb, ada_w, ada_bias, ada_table)  (skipped,
 *      identity modulation, when ada_w is NULL);
 *   2. for layer l: provider->layer_inputs(user, k, l, prev_out, q_blk,
 *      k_blk, v_blk, stream) fills the block's q/k/v, then tt_block_attn
 *      over layer l's context cache with layer l's (shift, scale, gate), no
 *      residual, and active[b] = (n_masked[b] > 0), writing `out`;
 *   3. provider->logits(user, k, out, logits, stream) fills [B, S, vocab]
 *      logits of the shape's dtype; tt_confidence_unmask(step = k).
 * Sequences with nothing masked are inactive.  Slots still masked after
 * max_steps stay masked.  The provider stands for the rest of the denoiser
 * (the pages' weights are not part of this library); its buffers live in the
 * workspace and it must enqueue its work on `stream`.
 *   k_ctx_layers, v_ctx_layers  host arrays of n_layers device pointers
 *   ctx_start, ctx_len          device [B]
 *   ada_w [256, 3*Hq*d] bf16, ada_bias [3*Hq*d] fp32, ada_table
 *   [n_layers, 3, Hq*d] fp32 (device; bias/table may be NULL; w 8-byte,
 *   bias and table 16-byte aligned)
 *   tokens [B,S] int32, masked [B,S] uint8 device in/out; commit_step
 *   [B,S] int8 device in/out or NULL; steps_taken host int32 out or NULL.
 * Errors: as tt_block_attn and tt_confidence_unmask, plus TT_ERR_CALLBACK
 * when a callback returns non-zero (state is that of the last completed
 * step), TT_ERR_INVALID_ARG for max_steps outside [0, S] or n_layers < 1.
 * ---------------------------------------------------------------------- */
typedef struct {
  void* user;
  int (*layer_inputs)(void* user, int32_t step, int32_t layer, const void* prev_out,
                      void* q_blk, void* k_blk, void* v_blk, tt_stream stream);
  int (*logits)(void* user, int32_t step, const void* last_out, void* logits,
                tt_stream stream);
} tt_step_provider;

size_t tt_denoise_workspace_size(const tt_attn_shape* shape, int32_t n_layers,
                                 int32_t max_ctx_len, int32_t vocab);

tt_status tt_denoise_block(const tt_attn_shape* shape, int32_t n_layers, int32_t max_steps,
                           float gamma, float temperature, int32_t mask_token_id,
                           int32_t vocab, const void* const* k_ctx_layers,
                           const void* const* v_ctx_layers, const int64_t* ctx_start,
                           const int32_t* ctx_len, int32_t max_ctx_len,
                           const void* ada_w, const float* ada_bias, const float* ada_table,
                           const tt_step_provider* provider, int32_t* tokens,
                           uint8_t* masked, int8_t* commit_step, int32_t* steps_taken,
                           void* workspace, size_t workspace_bytes, tt_stream stream);

/* ------------------------------------------------------------------------
 * tt_denoise_block_resume -- the same loop started at step first_step: the
 * block refined step by step until final ([dothoosh] two-tower mechanism
 * section) can be stopped after any step and continued later from its state
 * (tokens, masked, commit_step), which is all the loop carries between steps
 * (the timestep of a step is the masked fraction at its start).  It runs
 * steps k = first_step .. first_step + max_steps - 1 while any slot is
 * masked: the provider is called with the absolute step k, commit_step
 * records k, and with sample != 0 the unmasking pass is tt_sample_unmask
 * (seed, block_index, step = k), else the argmax of tt_confidence_unmask.
 * A run of n steps therefore gives bit for bit the state that a run of j
 * steps followed by a resumed run from first_step = j with n - j steps gives,
 * whatever j.  tt_denoise_block is this call with first_step = 0, sample = 0.
 *   first_step  in [0, S]; max_steps in [0, S - first_step]
 *   *steps_taken (host, may be NULL): steps run by this call.
 * Arguments, layouts, workspace (tt_denoise_workspace_size) and errors are
 * those of tt_denoise_block, plus TT_ERR_INVALID_ARG for first_step or
 * max_steps outside their ranges, or block_index < 0 with sample != 0.
 * ---------------------------------------------------------------------- */
tt_status tt_denoise_block_resume(const tt_attn_shape* shape, int32_t n_layers,
                                  int32_t first_step, int32_t max_steps, float gamma,
                                  float temperature, int32_t sample, uint64_t seed,
                                  int32_t block_index, int32_t mask_token_id, int32_t vocab,
                                  const void* const* k_ctx_layers,
                                  const void* const* v_ctx_layers, const int64_t* ctx_start,
                                  const int32_t* ctx_len, int32_t max_ctx_len,
                                  const void* ada_w, const float* ada_bias,
                                  const float* ada_table, const tt_step_provider* provider,
                                  int32_t* tokens, uint8_t* masked, int8_t* commit_step,
                                  int32_t* steps_taken, void* workspace, size_t workspace_bytes,
                                  tt_stream stream);

/* ------------------------------------------------------------------------
 * tt_generate -- multi-block generation: denoise a block, let the context
 * tower take it, go on to the next block, stop at EOS.
 *
 * [news] training and inference section, code example: the generation call
 * takes max_new_tokens=128, block_size=16, steps_per_block=16,
 * mask_token_id=3, temperature=0.1, confidence_threshold=0.8 and
 * eos_token_id.  [dothoosh] two-tower mechanism section: generation goes
 * block by block, each block starting as [MASK] tokens refined over T steps
 * until final; the context tower runs causally over the prompt and the
 * committed tokens and keeps every layer's KV cache.
 *
 * For block k = 0 .. n_blocks-1 while some sequence is unfinished:
 *   1. every unfinished sequence gets a fully masked block; the loop of
 *      tt_denoise_block runs up to steps_per_block steps (callbacks
 *      layer_inputs(k, step, layer, ...) and logits(k, step, ...)), with
 *      tt_sample_unmask (block_index k) when `sample` is non-zero, else the
 *      argmax of tt_confidence_unmask; the last allowed step commits every
 *      slot still masked, so every generated block is final;
 *   2. the context tower takes the block: for each layer,
 *      ctx_inputs(k, layer, tokens, prev_out, q, k_blk, v_blk) fills its
 *      q/k/v and tt_ctx_block_attn runs with the append; then
 *      tt_ctx_advance grows the contexts;
 *   3. out_tokens[b, k*S .. k*S+S-1] = the block's tokens and
 *      n_generated[b] += S; a sequence stops after a block that holds
 *      eos_token_id (stop_reason 1) or whose append found no room
 *      (stop_reason 2); otherwise stop_reason stays 0.
 * The denoiser's attention reads the caches as they grow, with no adaLN when
 * ada_w is NULL.  Positions of out_tokens past n_generated[b] are not
 * written.  The callbacks enqueue on `stream`; their buffers live in the
 * workspace; `tokens` is device [B, S] int32.
 *   k_ctx_layers, v_ctx_layers  host arrays of n_layers device caches
 *   ctx_start, ctx_end          device [B] int64 (reserved regions, disjoint)
 *   ctx_len                     device [B] int32 in/out
 *   max_ctx_len                 host: the longest initial context
 *   out_tokens  device [B, n_blocks*S] int32; n_generated device [B] int32;
 *   stop_reason device [B] int8 or NULL; blocks_taken host int32 or NULL.
 * eos_token_id < 0: no EOS stop.  Waits on the stream once per step and once
 * per block.
 * Errors: as tt_denoise_block and tt_ctx_block_attn, plus
 * TT_ERR_INVALID_ARG for steps_per_block outside [1, S], n_blocks < 0, a
 * NULL callback, NULL out_tokens/n_generated/ctx_end; TT_ERR_CALLBACK when a
 * callback returns non-zero (the state is that of the last completed call).
 * ---------------------------------------------------------------------- */
typedef struct {
  void* user;
  int (*layer_inputs)(void* user, int32_t block, int32_t step, int32_t layer,
                      const void* prev_out, void* q_blk, void* k_blk, void* v_blk,
                      tt_stream stream);
  int (*logits)(void* user, int32_t block, int32_t step, const void* last_out, void* logits,
                tt_stream stream);
  int (*ctx_inputs)(void* user, int32_t block, int32_t layer, const int32_t* tokens,
                    const void* prev_out, void* q_blk, void* k_blk, void* v_blk,
                    tt_stream stream);
} tt_gen_provider;

size_t tt_generate_workspace_size(const tt_attn_shape* shape, int32_t n_layers, int32_t n_blocks,
                                  int32_t max_ctx_len, int32_t vocab);

tt_status tt_generate(const tt_attn_shape* shape, int32_t n_layers, int32_t n_blocks,
                      int32_t steps_per_block, float gamma, float temperature, int32_t sample,
                      uint64_t seed, int32_t mask_token_id, int32_t eos_token_id, int32_t vocab,
                      void* const* k_ctx_layers, void* const* v_ctx_layers,
                      const int64_t* ctx_start, const int64_t* ctx_end, int32_t* ctx_len,
                      int32_t max_ctx_len, const void* ada_w, const float* ada_bias,
                      const float* ada_table, const tt_gen_provider* provider,
                      int32_t* out_tokens, int32_t* n_generated, int8_t* stop_reason,
                      int32_t* blocks_taken, void* workspace, size_t workspace_bytes,
                      tt_stream stream);

/* ------------------------------------------------------------------------
 * tt_mamba_block_scan -- one Mamba-2 layer's sequence mixer over a block of
 * S slots, seeded with the context tower's conv and SSM boundary states.
 *
 * [dothoosh] two-tower mechanism section: the context tower produces every
 * layer's KV cache and final Mamba-2 states; the denoiser's Mamba-2 layers
 * take their initial state directly from the context tower's Mamba state.
 * [modelcard] notes: the seeding injects the context tower's conv/SSM
 * boundary states as the initial states of the denoiser's Mamba layers,
 * causally (no future leakage).  The mixer is the published Mamba-2 one
 * (T. Dao, A. Gu, "Transformers are SSMs", ICML 2024); the pages give no
 * layer sizes.
 *
 * For sequence b, with u = [conv_state[b] ; xbc[b]] along the slots:
 *   v[s, c]  = SiLU(sum_{j<W} conv_w[c, j] u[s + j, c] + conv_b[c])
 *   x, B, C  = channels [0, H*P), [H*P, H*P+G*N), [H*P+G*N, C) of v
 *   dt[s, h] = softplus(dt_raw[b, s, h] + dt_bias[h]),  A[h] = -exp(A_log[h])
 *   Hs       = exp(dt A[h]) H{s-1} + dt x[s, h] B[s, g]^T   (H0 = ssm_state[b, h])
 *   y[b, s, h*P + p] = sum_n Hs[p, n] C[s, g, n] + D[h] x[s, h, p]
 * with g = h / (H/G).  The denoiser reads the seed (NULL outputs); the
 * context tower taking a committed block passes ssm_state_out (may alias
 * ssm_state: the final H) and conv_state_out (must not overlap conv_state:
 * the last W-1 rows of u).
 *   shape: batch B, n_heads H, head_dim P in {32, 64}, d_state N in
 *          {64, 128}, n_groups G (divides H), conv_width W in [2, 4]
 *          (Mamba-2's is 4; [5, 8] returns TT_ERR_UNSUPPORTED),
 *          block_size S in [1, 64], dtype of xbc / conv states / y.
 *   xbc [B, S, C] and y [B, S, H*P] (dtype; y aligned to 4 elements),
 *   C = H*P + 2*G*N;
 *   dt_raw [B, S, H] fp32; conv_state [B, C, W-1] (dtype);
 *   ssm_state [B, H, P, N] fp32 (16-byte aligned);
 *   conv_w [C, W], conv_b [C] or NULL, A_log [H], dt_bias [H] or NULL,
 *   D [H] or NULL: fp32;  active [B] uint8 or NULL (inactive: untouched).
 * All device pointers.  fp32 arithmetic throughout; y rounded to nearest
 * even for bf16.  The workspace (tt_mamba_workspace_size bytes, 16-byte
 * aligned, no initialisation) holds the B/C conv outputs and C.B products
 * the heads of a group share; it is left untouched where one kernel does
 * the whole layer (S <= 16 and N = 2P), but must still be passed.  Errors: TT_ERR_INVALID_ARG (NULL required
 * pointer, bad sizes, G not dividing H, misaligned state or y),
 * TT_ERR_UNSUPPORTED (P, N or W outside the sets above), TT_ERR_WORKSPACE,
 * TT_ERR_HIP.
 * ---------------------------------------------------------------------- */
typedef struct {
  int32_t batch;
  int32_t n_heads;
  int32_t head_dim;
  int32_t d_state;
  int32_t n_groups;
  int32_t conv_width;
  int32_t block_size;
  int32_t dtype;
} tt_mamba_shape;

size_t tt_mamba_workspace_size(const tt_mamba_shape* shape);

tt_status tt_mamba_block_scan(const tt_mamba_shape* shape, const void* xbc, const float* dt_raw,
                              const void* conv_state, const float* ssm_state,
                              const float* conv_w, const float* conv_b, const float* A_log,
                              const float* dt_bias, const float* D, const uint8_t* active,
                              void* y, void* conv_state_out, float* ssm_state_out,
                              void* workspace, size_t workspace_bytes, tt_stream stream);

/* ------------------------------------------------------------------------
 * The weighted adaLN-single attention sublayer of a denoiser layer.
 *
 * [dothoosh] "two-tower mechanism" section and [modelcard] "technical
 * features": every denoiser layer is conditioned on the diffusion timestep
 * through adaLN-single, which injects a scale, a shift and a gate per
 * timestep.  The pages do not show the layer around the three vectors; the
 * published adaLN-single placement (PixArt-alpha / DiT) is taken:
 *   h       = LayerNorm(x) * (1 + scale[b]) + shift[b]   (no affine, eps 1e-6)
 *   q|k|v   = h W_qkv^T                                   (no bias)
 *   o       = block attention of q over [context KV ; k, v] (tt_block_attn
 *             with identity modulation and no residual)
 *   out     = x + gate[b] * (o W_o^T)                     (no bias)
 * The pages give no hidden size: `width` (D) is a parameter.
 *
 * Shapes (M = batch * block_size token rows, row m = (b, s), b = m / S):
 *   x, h, out  [B, S, D] bf16;  shift, scale, gate [B, D] fp32 (for layer l
 *              of tt_adaln_single's output: ada + (3l + j) * B * D, j = 0,
 *              1, 2);
 *   w_qkv      [(Hq + 2 Hkv) d, D] bf16, rows in the order q heads, k heads,
 *              v heads (PyTorch Linear (out, in) storage);
 *   w_o        [D, Hq d] bf16;
 *   q_blk [B, S, Hq, d], k_blk / v_blk [B, S, Hkv, d], o [B, S, Hq, d] bf16;
 *   the context arguments are those of tt_block_attn.
 * Requirements: shape->dtype == TT_BF16 (else TT_ERR_UNSUPPORTED); D a
 * multiple of 64 in [64, 8192]; every buffer 16-byte aligned.  Arithmetic:
 * fp32 (LayerNorm statistics by exact two-pass sums; projections on the bf16
 * matrix cores with fp32 accumulation); every bf16 output rounded to nearest
 * even.  Sequences with active[b] == 0 are not written.  All calls are
 * asynchronous on `stream`; deterministic.  Errors: TT_ERR_INVALID_ARG (NULL
 * required pointer, misalignment, overlapping buffers as stated),
 * TT_ERR_UNSUPPORTED, TT_ERR_WORKSPACE, TT_ERR_HIP.
 * ---------------------------------------------------------------------- */

/* h = LayerNorm(x) (1 + scale) + shift.  h may be x itself (in place) but
 * must not overlap it otherwise. */
tt_status tt_ln_modulate(const tt_attn_shape* shape, int32_t width, const void* x,
                         const float* shift, const float* scale, const uint8_t* active, void* h,
                         tt_stream stream);

/* q|k|v = h W_qkv^T, written as the attention's q_blk, k_blk, v_blk (none
 * may overlap h). */
tt_status tt_qkv_proj(const tt_attn_shape* shape, int32_t width, const void* h, const void* w_qkv,
                      const uint8_t* active, void* q_blk, void* k_blk, void* v_blk,
                      tt_stream stream);

/* out = x + gate (o W_o^T).  out may be x itself (in place); it must not
 * overlap o, nor x otherwise. */
tt_status tt_out_proj(const tt_attn_shape* shape, int32_t width, const void* o, const void* w_o,
                      const float* gate, const void* x, const uint8_t* active, void* out,
                      tt_stream stream);

/* Workspace of tt_adaln_attn_sublayer (256-byte aligned, no
 * initialisation): h, q, k, v, o and the attention's partials.  0 on
 * invalid arguments (tt_last_error says why). */
size_t tt_adaln_sublayer_workspace_size(const tt_attn_shape* shape, int32_t width,
                                        int32_t max_ctx_len);

/* The whole sublayer: tt_ln_modulate, tt_qkv_proj, the block attention and
 * tt_out_proj in stream order, intermediates in the workspace.  out may be x
 * itself. */
tt_status tt_adaln_attn_sublayer(const tt_attn_shape* shape, int32_t width, const void* x,
                                 const float* shift, const float* scale, const float* gate,
                                 const void* w_qkv, const void* w_o, const void* k_ctx,
                                 const void* v_ctx, const int64_t* ctx_start,
                                 const int32_t* ctx_len, int32_t max_ctx_len,
                                 const uint8_t* active, void* out, void* workspace,
                                 size_t workspace_bytes, tt_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* TT_H */
