/*
 * wq_decode.h -- C ABI of libwq's decode-step kernels: the work of a Llama-style decode step
 * around its weight-only-quantized linears (which are wq_linear / wq_linear_grouped, wq.h).
 *
 * The pages name this loop without defining it: the gpt-fast write-up (m.greenbasetech.com,
 * part on torch.compile) captures a whole decode step as one region so that the CPU no longer
 * feeds the GPU piece by piece, and its part on GPU quantization notes that every weight is
 * loaded once per generated token; the speed-up strategies page (sharktoolz.top, section 6 "KV
 * cache and multi-query attention") keeps the keys and values of processed tokens in a cache
 * and lets several query heads share one key/value head. The calls below implement the Llama
 * decoder layer those pages discuss; each one states the definition it follows. A decode step
 * of M sequences (all at the same position) is, per layer:
 *
 *   wq_add_rmsnorm      x += delta (the previous block's output); h = rmsnorm(x) * g
 *   wq_linear_grouped   q, k, v = h . Wq^T, h . Wk^T, h . Wv^T
 *   wq_rope_attention   rotate q, k at pos; cache[pos] = (k, v); a = attention(q, cache[0..pos])
 *   wq_linear           o = a . Wo^T
 *   wq_add_rmsnorm      x += o; h = rmsnorm(x) * g
 *   wq_linear_grouped   gate, up
 *   wq_silu_mul         m = silu(gate) * up
 *   wq_linear           down = m . Wdown^T        (added to x by the next wq_add_rmsnorm)
 *
 * then wq_add_rmsnorm (final norm), wq_linear (output layer) and wq_argmax_next (next tokens,
 * pos += 1). wq_embed starts a step from token ids. Every device call reads the position and
 * the token ids from device memory, so the whole step can be captured once as a HIP graph and
 * replayed step after step.
 *
 * Types: fp16 values as uint16_t bits; the residual stream x is float32; token ids and the
 * position are int32 in device memory. Row-major [M, width] buffers. Conventions as in wq.h:
 * errors are returned before any launch, device calls are asynchronous on `stream` and never
 * synchronize, memory is owned by the caller, device pointers must be 16-byte aligned.
 */
#ifndef WQ_DECODE_H_
#define WQ_DECODE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Host: the rotary-embedding table, cos_out[p * (head_dim/2) + i] = cos(p * theta^(-2i/head_dim))
 * and sin_out likewise, for positions p = 0 .. positions-1, computed in float64 and rounded to
 * float32. head_dim even and >= 2, positions >= 1, theta > 0; else WQ_ERR_SHAPE / WQ_ERR_ARG. */
int wq_rope_table(double theta, int64_t head_dim, int64_t positions, float* cos_out, float* sin_out);

/* Device: x[m, :] = float(table[tokens[m], :]) for m < M. table [vocab, d] fp16; x [M, d]
 * float32. A token id outside [0, vocab) is clamped into it. d a multiple of 8. */
int wq_embed(const uint16_t* table, const int32_t* tokens, float* x, int64_t M, int64_t d, int64_t vocab, void* stream);

/* Device: RMSNorm with the residual add in front. If delta is not NULL, x += float(delta) first
 * (x is updated in place). Then out[m, i] = fp16(x[m, i] * g[i] / sqrt(mean_i(x[m, i]^2) + eps)),
 * in float32 (the sum of squares in a fixed order). x [M, d] float32; delta, out [M, d] fp16;
 * g [d] fp16. d a multiple of 8, eps >= 0. */
int wq_add_rmsnorm(float* x, const uint16_t* delta, const uint16_t* g, float eps, uint16_t* out, int64_t M, int64_t d,
                   void* stream);

/* Host: bytes of the workspace wq_rope_attention needs for these sizes (the partial results of the
 * position chunks); 0 when max_seq <= 4096 (one workgroup per head, nothing leaves it). */
size_t wq_attention_workspace_bytes(int64_t M, int64_t n_heads, int64_t head_dim, int64_t max_seq);

/* Device: rotary embedding, key/value cache append and attention of one new token per sequence.
 * p = *pos (device int32, clamped into [0, max_seq)). For each sequence m and query head h, with
 * key/value head kh = h / (n_heads / n_kv_heads):
 *   q' = rope(q[m, h]) at p; k' = fp16(rope(k[m, kh])) at p; the pair (2i, 2i+1) of a head is
 *        rotated by the angle whose cosine and sine are rope_cos / rope_sin[p * head_dim/2 + i];
 *   cache_k[m, p, kh] = k', cache_v[m, p, kh] = v[m, kh];
 *   out[m, h] = fp16( sum_{t<=p} softmax_t(q'.cache_k[m, t, kh] / sqrt(head_dim)) cache_v[m, t, kh] )
 * in float32. q, out [M, n_heads*head_dim] fp16; k, v [M, n_kv_heads*head_dim] fp16; cache_k,
 * cache_v [M, max_seq, n_kv_heads*head_dim] fp16 (this layer's); rope_cos, rope_sin float32
 * [max_seq, head_dim/2] (wq_rope_table). head_dim 64 or 128; n_heads a multiple of n_kv_heads.
 * Caches of up to 4096 positions (max_seq <= 4096): one launch, one workgroup per (query head,
 * sequence), and `workspace` is not used (it may be NULL). Longer caches: the positions are split
 * over workgroups of 64, whose partial results meet in `workspace` (wq_attention_workspace_bytes;
 * WQ_ERR_ARG if smaller; no initial contents needed), and a second launch combines them; calls
 * that share a workspace must not overlap in time. The two paths sum in different orders, so their
 * results may differ in the last bits; each is deterministic. */
int wq_rope_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* cache_k, uint16_t* cache_v,
                      const float* rope_cos, const float* rope_sin, const int32_t* pos, uint16_t* out, int64_t M,
                      int64_t n_heads, int64_t n_kv_heads, int64_t head_dim, int64_t max_seq, void* workspace,
                      size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture that may not
 * call hipMalloc, tight serving loops, harnesses that forbid allocation): wq_rope_attention with
 * its workspace taken from a buffer the library holds in device memory, WQ_NOALLOC_SCRATCH_BYTES
 * per GPU, kept until the process ends. It allocates nothing and computes exactly what
 * wq_rope_attention computes. Sizes whose workspace (wq_attention_workspace_bytes) exceeds the
 * buffer return WQ_ERR_SCRATCH before any launch; other errors as wq_rope_attention, and
 * WQ_ERR_DEVICE if the buffer's address cannot be found on the current device. Every call on a
 * GPU shares that GPU's buffer (no contents need clearing: each call writes the partial results it
 * reads), so calls that overlap in time on one GPU race. */
#define WQ_NOALLOC_SCRATCH_BYTES (8u << 20)
int wq_rope_attention_noalloc(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* cache_k,
                              uint16_t* cache_v, const float* rope_cos, const float* rope_sin, const int32_t* pos,
                              uint16_t* out, int64_t M, int64_t n_heads, int64_t n_kv_heads, int64_t head_dim,
                              int64_t max_seq, void* stream);

/* Device: out[i] = fp16(gate[i] / (1 + exp(-gate[i])) * up[i]) in float32, i < n. n a multiple of 8. */
int wq_silu_mul(const uint16_t* gate, const uint16_t* up, uint16_t* out, int64_t n, void* stream);

/* Device: tokens[m] = the lowest index of the largest of logits[m, 0 .. vocab-1] (fp16, NaN never
 * chosen), for m < M; then *pos += 1 (the step is done). vocab a multiple of 8. */
int wq_argmax_next(const uint16_t* logits, int64_t M, int64_t vocab, int32_t* tokens, int32_t* pos, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* WQ_DECODE_H_ */
