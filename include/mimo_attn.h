/*
 * mimo_attn.h — C ABI of the MiMo-V2.6-Flash attention hot path on MI355X (gfx950).
 *
 * The layer (miles MiMo-V2.6-Flash page, section 1 Model Introduction, and the
 * Model techniques map page, rows Grouped-query attention, Sliding-window
 * attention, Learnable attention sink, Partial RoPE):
 *   - 64 query heads; sliding-window layers have 8 KV heads, a 128-key window
 *     and one sink logit per query head; global layers have 4 KV heads, full
 *     causal attention and no sink;
 *   - q/k head dim 192, v head dim 128; the output is scaled by 0.707;
 *   - partial RoPE rotates the first 64 of the 192 q/k dims (rotate-half
 *     pairing: dim i with dim i+32), base 1e4 (sliding) or 1e7 (global);
 *   - GQA: query head h reads KV head h / (num_q_heads / num_kv_heads).
 *
 * For query position p and head h the library computes
 *     s_j = softmax_scale * <rope(q, p), rope(k_j, pos_j)>   for visible keys j
 *     visible: pos_j <= p and (window == 0 or p - pos_j < window)
 *     o   = v_scale * sum_j exp(s_j) v_j / (sum_j exp(s_j) + exp(sink_h))
 * where the sink term is present only when a sink array is given (it joins the
 * normaliser and contributes no value: techniques map page, Learnable attention
 * sink).  A row with no visible key and no sink gets o = 0.
 *
 * Conventions for every entry point
 *   - bf16 tensors are passed as uint16_t bit patterns; all layouts are dense,
 *     row-major, token-major: [batch or sequence, token or slot, head, dim].
 *   - Every pointer is a DEVICE pointer owned by the caller, except cfg, which is
 *     a host pointer read during the call only.  The library allocates nothing
 *     and keeps no state between calls.
 *   - Every bf16 or fp8 tensor and every workspace must be 16-byte aligned (the
 *     kernels move rows in 16-byte pieces; a tensor PyTorch allocates, and any
 *     view of it that starts on a token or slot row, is); otherwise the call
 *     returns MIMO_ERR_INVALID_ARGUMENT.  fp32 and integer arrays need only
 *     their natural alignment.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Success means the
 *     work is enqueued on that stream; no call synchronises the host, so every
 *     call can be captured into a HIP graph.
 *   - All arguments are validated on the host before anything is enqueued.  On
 *     error nothing is launched, outputs are untouched, and mimo_last_error()
 *     returns a message (thread-local, valid until the thread's next call).
 *   - Sizes of 0 (no tokens, no sequences) are valid and enqueue nothing.
 *   - Supported head geometry: head_dim_qk 192, head_dim_v 128, rope_dim 64,
 *     num_q_heads a multiple of num_kv_heads; prefill needs a GQA group size
 *     (num_q_heads / num_kv_heads) that is a multiple of 4; decode needs a
 *     group size of at most 16, at most 8 KV heads, at most 65535 sequences
 *     and caches of at most 2^30 slots.  Anything else returns
 *     MIMO_ERR_UNSUPPORTED.
 */
#ifndef MIMO_ATTN_H
#define MIMO_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mimo_status {
    MIMO_OK = 0,
    MIMO_ERR_INVALID_ARGUMENT = 1, /* null or misaligned pointer, negative size, inconsistent sizes */
    MIMO_ERR_UNSUPPORTED = 2,      /* head geometry the kernels are not built for */
    MIMO_ERR_WORKSPACE = 3,        /* workspace missing or too small */
    MIMO_ERR_HIP = 4               /* the HIP runtime refused a launch */
} mimo_status;

/* Layer configuration (mirrors the model config keys). */
typedef struct mimo_attn_cfg {
    int32_t num_q_heads;   /* 64 */
    int32_t num_kv_heads;  /* 8 on sliding-window layers, 4 on global layers */
    int32_t head_dim_qk;   /* 192 */
    int32_t head_dim_v;    /* 128 */
    int32_t rope_dim;      /* 64: int(192 * 0.334), the first 64 dims rotate */
    double rope_base;      /* 1e4 sliding, 1e7 global */
    float softmax_scale;   /* 1/sqrt(192) */
    float v_scale;         /* 0.707 */
    int32_t window;        /* keys visible counting the query itself: 128; 0 = unbounded */
} mimo_attn_cfg;

/*
 * Partial RoPE of a batch of head vectors (techniques map page, Partial RoPE;
 * the angle of pair i is pos * rope_base^(-2i/rope_dim), computed by exact
 * fixed-point turn reduction so it stays accurate at any position, which the
 * Gaudi recipe page's section on required fixes shows an fp32 angle does not).
 *   x_in, x_out : [n_tokens, n_heads, head_dim_qk] bf16; x_out may equal x_in
 *                 (in place: then only the 64 rotated dims are rewritten).
 *   pos         : [n_tokens] int64 positions, >= 0.
 */
mimo_status mimo_rope_partial(const mimo_attn_cfg *cfg, const uint16_t *x_in, uint16_t *x_out,
                              int64_t n_tokens, int32_t n_heads, const int64_t *pos,
                              void *stream);

/*
 * Sliding-window prefill with the per-head sink (techniques map page, rows
 * Sliding-window attention and Learnable attention sink; window convention of
 * the miles page, section 5.4 Notable quirks: window keys in total, the query
 * included).  q/k are unrotated; RoPE is applied on load.
 *   q     : [B, T, num_q_heads, 192]   token t has position pos0 + t
 *   k     : [B, T, num_kv_heads, 192]  the same tokens as q
 *   v     : [B, T, num_kv_heads, 128]
 *   sinks : [num_q_heads] fp32 sink logits, or NULL for none
 *   out   : [B, T, num_q_heads, 128] bf16
 *   lse   : [B, num_q_heads, T] fp32 natural-log normaliser (sink included), or NULL
 * Needs cfg->window >= 1.
 */
mimo_status mimo_attn_prefill_swa(const mimo_attn_cfg *cfg, const uint16_t *q, const uint16_t *k,
                                  const uint16_t *v, const float *sinks, int32_t B, int32_t T,
                                  int64_t pos0, uint16_t *out, float *lse, void *stream);

/*
 * Workspace of the global-layer prefill calls (mimo_attn_prefill_global, and
 * mimo_attn_prefill_varlen with cfg->window == 0): room for one image per 64-key
 * tile and KV head, holding the tile's rotated K and transposed V exactly as the
 * attention kernel keeps them in LDS (so that each tile is rotated and transposed
 * once per call rather than once per workgroup that reads it), and the tile's
 * largest key norm.  total_k is the
 * number of key tokens over the batch (B * Tk for a dense call, the row count of k
 * for a packed one).  Returns 0 where the images are not used (sliding windows,
 * GQA groups that are not a multiple of 8) or the arguments are invalid.
 */
size_t mimo_attn_prefill_workspace_size(const mimo_attn_cfg *cfg, int32_t B, int64_t total_k);

/*
 * Global causal prefill of one query chunk against its whole prefix (the tiled
 * global-attention prefill of the Gaudi recipe page, Launch section: query tiles
 * instead of a dense bias).
 *   q     : [B, Tq, num_q_heads, 192]   query t has position q_pos0 + t
 *   k, v  : [B, Tk, num_kv_heads, 192|128], key j has position j
 *   Tk must equal q_pos0 + Tq (each chunk sees its full prefix).
 *   out   : [B, Tq, num_q_heads, 128] bf16;  lse : [B, num_q_heads, Tq] fp32 or NULL.
 *   ws    : device workspace of at least mimo_attn_prefill_workspace_size(cfg, B,
 *           B * Tk) bytes, not overlapping any other argument, owned by the caller and
 *           overwritten by the call; or NULL, which stages every tile inside the
 *           attention kernel instead (same results up to the rounding of the
 *           rotated keys, slower).  A smaller non-NULL ws is MIMO_ERR_WORKSPACE.
 * Needs cfg->window == 0.
 */
mimo_status mimo_attn_prefill_global(const mimo_attn_cfg *cfg, const uint16_t *q, const uint16_t *k,
                                     const uint16_t *v, int32_t B, int32_t Tq, int32_t Tk,
                                     int64_t q_pos0, uint16_t *out, float *lse, void *ws,
                                     size_t ws_bytes, void *stream);

/*
 * Prefill of packed variable-length sequences (THD layout), which also covers
 * continuing a sequence chunk by chunk (Gaudi recipe page, Launch and Buckets
 * sections: prompts are prefilled in chunks of up to 8,192 tokens against the
 * context before them; a sliding layer's chunk needs only the window - 1 keys
 * before it, a global layer's chunk its whole prefix).
 *   Sequence b owns query tokens cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 and key
 *   tokens cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1 (Tq_b and Tk_b of them).  Its
 *   first key sits at position P_b = k_pos0[b] (0 if k_pos0 is NULL) and its
 *   queries are its last Tq_b keys: query t is at position P_b + Tk_b - Tq_b + t.
 *   Visibility, RoPE and the sink are as in the dense calls, with cfg->window
 *   (0 = causal only) and sinks optional on either layer type.
 *   q   : [total_q, num_q_heads, 192] unrotated;  k : [total_k, num_kv_heads, 192]
 *   unrotated;  v : [total_k, num_kv_heads, 128];  out : [total_q, num_q_heads, 128];
 *   lse : [num_q_heads, total_q] fp32 or NULL (natural-log LSE of each row,
 *   sink included).
 *   cu_seqlens_q / cu_seqlens_k : [B+1] int32 device arrays, non-decreasing,
 *   starting at 0;  k_pos0 : [B] int64 device array or NULL.
 *   total_k : rows of k and v.
 *   ws      : with cfg->window == 0, as for mimo_attn_prefill_global with
 *             mimo_attn_prefill_workspace_size(cfg, B, total_k) bytes (or NULL);
 *             ignored on sliding layers.
 * The caller guarantees, for every b: 0 <= Tq_b <= Tk_b, Tq_b <= max_seqlen_q,
 * cu_seqlens_q[B] <= total_q, cu_seqlens_k[B] <= total_k, and positions >= 0.
 * These device values are not read on the host; rows of a sequence past
 * max_seqlen_q are left unwritten.
 * The attention runs over the keys given: a sliding chunk must carry the
 * min(window - 1, P) keys before its first query, a global chunk its whole
 * prefix (P_b = 0).
 */
mimo_status mimo_attn_prefill_varlen(const mimo_attn_cfg *cfg, const uint16_t *q, const uint16_t *k,
                                     const uint16_t *v, const float *sinks, int32_t B,
                                     const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k,
                                     const int64_t *k_pos0, int32_t max_seqlen_q, int32_t total_q,
                                     int64_t total_k, uint16_t *out, float *lse, void *ws,
                                     size_t ws_bytes, void *stream);

/*
 * One decode query per sequence over a KV cache (window-sized ring on sliding
 * layers, Gaudi recipe page, Launch section; a long cache on global layers).
 * Split-K flash decoding balanced over the batch: the visible slots of all
 * sequences are cut into 32-slot steps and split evenly over a fixed set of
 * workgroups; a sequence shared by several workgroups gets one partial result
 * per workgroup in `ws`, and a combine pass merges them by their log-sum-exp.
 * Three kernels are enqueued (plan, partial, combine); `ws` also holds the plan.
 *   q       : [S, num_q_heads, 192] unrotated; q_pos : [S] int64 positions
 *   k_cache : [S, cap, num_kv_heads, 192] rotated keys (as mimo_kv_ring_append writes)
 *   v_cache : [S, cap, num_kv_heads, 128]
 *   Cache rule: the token at position t lives in slot t mod cap.  window > 0:
 *   the query sees positions max(0, p-window+1)..p, which needs cap >= window.
 *   window == 0: it sees 0..p, which needs p < cap (later positions are cut off
 *   at cap).  A negative position sees nothing.
 *   sinks   : [num_q_heads] fp32 or NULL.   out : [S, num_q_heads, 128] bf16.
 *   ws      : device workspace of at least mimo_attn_decode_workspace_size() bytes.
 */
mimo_status mimo_attn_decode(const mimo_attn_cfg *cfg, int32_t S, const uint16_t *q,
                             const int64_t *q_pos, const uint16_t *k_cache, const uint16_t *v_cache,
                             int32_t cap, const float *sinks, uint16_t *out, void *ws,
                             size_t ws_bytes, void *stream);

/* Workspace bytes mimo_attn_decode needs for S sequences over caches of cap
 * slots (the size does not depend on cap; 0 for an unsupported cfg). */
size_t mimo_attn_decode_workspace_size(const mimo_attn_cfg *cfg, int32_t S, int32_t cap);

/*
 * Allocation-free variant of mimo_attn_decode, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  The same kernels and results as mimo_attn_decode;
 * the split-K partials and the plan go to a scratch array that the library
 * holds on every GPU it runs on (MIMO_DECODE_NOALLOC_MAX_BYTES, kept until the
 * process ends) instead of a caller workspace.  Arguments as in
 * mimo_attn_decode without ws / ws_bytes.
 *   - A call whose workspace (mimo_attn_decode_workspace_size) exceeds the
 *     scratch returns MIMO_ERR_WORKSPACE; at 64 query heads that is more than
 *     751 sequences with 4 KV heads or 879 with 8.
 *   - `stream` must belong to the current device (else MIMO_ERR_INVALID_ARGUMENT).
 *   - Every call on one GPU uses that GPU's one scratch array: calls that may
 *     overlap in time on the same GPU (other streams, other threads) race and
 *     give wrong results.  Calls in order on one stream are safe.  Nothing in
 *     the scratch has to start at zero: each call writes all it reads.
 */
#define MIMO_DECODE_NOALLOC_MAX_BYTES ((size_t)32 << 20)
mimo_status mimo_attn_decode_noalloc(const mimo_attn_cfg *cfg, int32_t S, const uint16_t *q,
                                     const int64_t *q_pos, const uint16_t *k_cache, const uint16_t *v_cache,
                                     int32_t cap, const float *sinks, uint16_t *out, void *stream);

/*
 * Multi-query decode for speculative verification: n_q query tokens per
 * sequence, the newest at q_pos[s] and token i at q_pos[s] - (n_q - 1 - i),
 * each attending causally to the cache (a draft token sees the tokens before
 * it, the earlier drafts included, and itself).  The pages' engines verify 4
 * draft tokens (EAGLE through the MTP layers: miles MiMo-V2.6-Flash page,
 * section 4.2) or 7 to 8 (DFlash: vLLM recipe page, DFlash launch; SGLang
 * cookbook page, DFlash and caching section).
 *   q   : [S, n_q, num_q_heads, 192] unrotated;  out : [S, n_q, num_q_heads, 128].
 *   The cache holds every token up to q_pos[s] (the drafts appended first), with
 *   the cache rule of mimo_attn_decode; a ring needs cap >= window + n_q - 1 so
 *   that the oldest draft's window is still in it.  A token at a negative
 *   position sees nothing and gets a zero row.
 *   Needs (num_q_heads / num_kv_heads) * n_q <= 128.  n_q = 1 is mimo_attn_decode.
 *   ws  : device workspace of at least mimo_attn_decode_multi_workspace_size() bytes.
 */
mimo_status mimo_attn_decode_multi(const mimo_attn_cfg *cfg, int32_t S, int32_t n_q, const uint16_t *q,
                                   const int64_t *q_pos, const uint16_t *k_cache, const uint16_t *v_cache,
                                   int32_t cap, const float *sinks, uint16_t *out, void *ws,
                                   size_t ws_bytes, void *stream);

/* Workspace bytes mimo_attn_decode_multi needs (independent of cap; 0 for an
 * unsupported cfg or n_q). */
size_t mimo_attn_decode_multi_workspace_size(const mimo_attn_cfg *cfg, int32_t S, int32_t n_q, int32_t cap);

/*
 * Backward of dense prefill attention (both layer types; cfg->window > 0 is a
 * sliding window, 0 causal): the trainer's path of the sliding-window layers
 * with their learned sink (miles MiMo-V2.6-Flash page, section 5.4: the sink is
 * trained through the fused attention).  Inputs are the forward's q, k, v (as
 * given to mimo_attn_prefill_swa / _global with Tq = Tk = T, token t at
 * pos0 + t), sinks or NULL, its output `out` and its `lse` ([B, num_q_heads, T],
 * the forward's lse output), and the upstream gradient dout [B, T, num_q_heads,
 * 128].  Outputs (overwritten): dq [B, T, num_q_heads, 192], dk [B, T,
 * num_kv_heads, 192], dv [B, T, num_kv_heads, 128] (gradients of the unrotated
 * inputs, bf16) and, when sinks are given, dsinks [num_q_heads] fp32 (summed
 * over the batch).  ws: at least mimo_attn_backward_workspace_size() bytes.
 * Deterministic: nothing is accumulated across workgroups.  B * T * num_q_heads
 * above 2^30 returns MIMO_ERR_UNSUPPORTED.
 */
mimo_status mimo_attn_prefill_backward(const mimo_attn_cfg *cfg, const uint16_t *q, const uint16_t *k,
                                       const uint16_t *v, const float *sinks, int32_t B, int32_t T, int64_t pos0,
                                       const uint16_t *out, const float *lse, const uint16_t *dout, uint16_t *dq,
                                       uint16_t *dk, uint16_t *dv, float *dsinks, void *ws, size_t ws_bytes,
                                       void *stream);

/* Workspace bytes of mimo_attn_prefill_backward: per (token, query head) the 64 rotated dims
 * of q (bf16) and one fp32 value, per (token, KV head) the 64 rotated dims of k (bf16), and
 * one fp32 value per (batch row, block of 32 tokens, query head); 0 for an invalid cfg or
 * B, T <= 0. */
size_t mimo_attn_backward_workspace_size(const mimo_attn_cfg *cfg, int32_t B, int32_t T);

/* Element type of a paged KV cache. */
typedef enum mimo_kv_dtype {
    MIMO_KV_BF16 = 0,      /* bf16 bit patterns */
    MIMO_KV_FP8_E4M3 = 1   /* OCP fp8 e4m3 (e4m3fn) codes; value = code * scale */
} mimo_kv_dtype;

/*
 * Decode over a paged KV cache: the cache of every sequence is a list of
 * blocks of block_size token slots taken from shared pools, and a block table
 * maps a sequence's logical block to its pool block (vLLM recipe page,
 * Launch command for AMD MI355X: --block-size 128 and --kv-cache-dtype fp8;
 * Gaudi recipe page, Launch: --block-size 128).  Position t of sequence s
 * lives in pool block block_table[s * max_blocks + t / block_size], slot
 * t % block_size.  Queries as in mimo_attn_decode_multi (n_q >= 1 tokens, the
 * newest at q_pos[s]); a sequence holds positions 0..q_pos[s], and with a
 * window only the blocks that hold some query's window are read (blocks
 * before them may have been released).
 *   k_pool  : [n_blocks, block_size, num_kv_heads, 192] rotated keys;
 *   v_pool  : [n_blocks, block_size, num_kv_heads, 128];  elements of kv_dtype.
 *   k_scale, v_scale : dequantisation scales of fp8 pools (ignored for bf16).
 *   block_table : [S, max_blocks] int32 device array; entries outside
 *   [0, n_blocks) are clamped into it (never read outside the pools).
 *   block_size : a multiple of 32;  q_pos[s] < max_blocks * block_size.
 *   out : [S, n_q, num_q_heads, 128] bf16;  ws as for mimo_attn_decode_multi
 *   (mimo_attn_decode_multi_workspace_size with the same S and n_q).
 */
mimo_status mimo_attn_decode_paged(const mimo_attn_cfg *cfg, int32_t S, int32_t n_q, const uint16_t *q,
                                   const int64_t *q_pos, const void *k_pool, const void *v_pool,
                                   int32_t n_blocks, int32_t block_size, mimo_kv_dtype kv_dtype,
                                   float k_scale, float v_scale, const int32_t *block_table,
                                   int32_t max_blocks, const float *sinks, uint16_t *out, void *ws,
                                   size_t ws_bytes, void *stream);

/*
 * Append one new token per sequence to a paged cache: k_new is rotated at
 * pos[s] (partial RoPE) and written with v_new into the slot of position
 * pos[s] (layout as in mimo_attn_decode_paged).  fp8 pools store
 * code = round-to-nearest-even(x / scale), saturated to +-448, where x is the
 * fp32 rotated key (or the bf16 value); bf16 pools store the bf16-rounded
 * rotation, as mimo_kv_ring_append does.  A negative position writes nothing.
 */
mimo_status mimo_kv_paged_append(const mimo_attn_cfg *cfg, int32_t S, const uint16_t *k_new,
                                 const uint16_t *v_new, const int64_t *pos, void *k_pool, void *v_pool,
                                 int32_t n_blocks, int32_t block_size, mimo_kv_dtype kv_dtype,
                                 float k_scale, float v_scale, const int32_t *block_table,
                                 int32_t max_blocks, void *stream);

/*
 * Append one new token per sequence: rotate k_new at pos (partial RoPE) and
 * write it and v_new into slot pos mod cap (the window-sized KV of the Gaudi
 * recipe page keeps only the window; a global cache with cap above every
 * position never wraps).
 *   k_new : [S, num_kv_heads, 192] unrotated;  v_new : [S, num_kv_heads, 128]
 *   pos   : [S] int64, >= 0;  k_cache / v_cache as in mimo_attn_decode.
 */
mimo_status mimo_kv_ring_append(const mimo_attn_cfg *cfg, int32_t S, const uint16_t *k_new,
                                const uint16_t *v_new, const int64_t *pos, uint16_t *k_cache,
                                uint16_t *v_cache, int32_t cap, void *stream);

/* Message for the calling thread's last error ("" if none). */
const char *mimo_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MIMO_ATTN_H */
