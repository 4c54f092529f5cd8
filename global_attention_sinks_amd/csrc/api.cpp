// C ABI of the attention hot path: argument validation on the host, then one
// or two kernel launches on the caller's stream.  No allocation, no host
// synchronisation, no state beyond a thread-local error message.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "../../include/mimo_attn.h"
#include "kernels.hpp"

#include <initializer_list>

using namespace mimo;

namespace {

thread_local char g_err[512] = "";

mimo_status fail(mimo_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

mimo_status ok() {
    g_err[0] = '\0';
    return MIMO_OK;
}

mimo_status from_hip(hipError_t e, const char *what) {
    if (e == hipSuccess) return ok();
    return fail(MIMO_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// The kernels move bf16 and fp8 rows and workspaces in 16-byte pieces (vector loads,
// and buffer loads that write LDS): every such pointer must be 16-byte aligned.
// NULL pointers pass (their own checks report them).
mimo_status check_aligned(const char *names, std::initializer_list<const void *> ptrs) {
    for (const void *p : ptrs)
        if (p && (reinterpret_cast<uintptr_t>(p) & 15u) != 0)
            return fail(MIMO_ERR_INVALID_ARGUMENT, "%s must be 16-byte aligned", names);
    return MIMO_OK;
}

// Shared checks of the layer configuration.
mimo_status check_cfg(const mimo_attn_cfg *cfg) {
    if (!cfg) return fail(MIMO_ERR_INVALID_ARGUMENT, "cfg is NULL");
    if (cfg->num_q_heads <= 0 || cfg->num_kv_heads <= 0)
        return fail(MIMO_ERR_INVALID_ARGUMENT, "head counts must be positive (got %d q, %d kv)",
                    cfg->num_q_heads, cfg->num_kv_heads);
    if (cfg->num_q_heads % cfg->num_kv_heads != 0)
        return fail(MIMO_ERR_INVALID_ARGUMENT, "num_q_heads %d is not a multiple of num_kv_heads %d",
                    cfg->num_q_heads, cfg->num_kv_heads);
    if (cfg->head_dim_qk != kDqk || cfg->head_dim_v != kDv || cfg->rope_dim != kRope)
        return fail(MIMO_ERR_UNSUPPORTED, "head geometry qk=%d v=%d rope=%d is not 192/128/64",
                    cfg->head_dim_qk, cfg->head_dim_v, cfg->rope_dim);
    if (!(cfg->rope_base > 1.0) || !isfinite(cfg->rope_base))
        return fail(MIMO_ERR_INVALID_ARGUMENT, "rope_base must be finite and > 1");
    if (!(cfg->softmax_scale > 0.0f) || !isfinite(cfg->softmax_scale))
        return fail(MIMO_ERR_INVALID_ARGUMENT, "softmax_scale must be finite and > 0");
    if (!isfinite(cfg->v_scale)) return fail(MIMO_ERR_INVALID_ARGUMENT, "v_scale must be finite");
    if (cfg->window < 0) return fail(MIMO_ERR_INVALID_ARGUMENT, "window must be >= 0");
    return ok();
}

// Fixed-point rotary turns for a base, recomputed only when the base changes.
const RopeTurns &rope_turns(double base) {
    thread_local double cached_base = 0.0;
    thread_local RopeTurns rt;
    if (base != cached_base) {
        const long double two_pi = 6.283185307179586476925286766559005768L;
        for (int i = 0; i < kPairs; ++i) {
            long double theta = powl((long double)base, -(long double)(2 * i) / (long double)kRope);
            long double frac = theta / two_pi;           // in (0, 1/(2 pi)]
            rt.turn[i] = (uint64_t)llroundl(ldexpl(frac, 64));
        }
        cached_base = base;
    }
    return rt;
}

float scale_log2(const mimo_attn_cfg *cfg) { return cfg->softmax_scale * 1.4426950408889634f; }

bool overlap(const void *a, size_t na, const void *b, size_t nb) {
    const char *pa = (const char *)a, *pb = (const char *)b;
    return pa < pb + nb && pb < pa + na;
}

}  // namespace

extern "C" {

const char *mimo_last_error(void) { return g_err; }

mimo_status mimo_rope_partial(const mimo_attn_cfg *cfg, const uint16_t *x_in, uint16_t *x_out,
                              int64_t n_tokens, int32_t n_heads, const int64_t *pos, void *stream) {
    mimo_status st = check_cfg(cfg);
    if (st != MIMO_OK) return st;
    if (n_tokens < 0 || n_heads <= 0)
        return fail(MIMO_ERR_INVALID_ARGUMENT, "n_tokens must be >= 0 and n_heads > 0");
    if (n_tokens == 0) return ok();
    if (!x_in || !x_out || !pos) return fail(MIMO_ERR_INVALID_ARGUMENT, "x_in, x_out and pos must be non-NULL");
    if (check_aligned("x_in and x_out", {x_in, x_out}) != MIMO_OK) return MIMO_ERR_INVALID_ARGUMENT;
    const size_t bytes = (size_t)n_tokens * n_heads * kDqk * 2;
    if (x_in != x_out && overlap(x_in, bytes, x_out, bytes))
        return fail(MIMO_ERR_INVALID_ARGUMENT, "x_out must equal x_in or not overlap it");
    return from_hip(launch_rope_partial(rope_turns(cfg->rope_base), x_in, x_out,
                                        n_tokens * (int64_t)n_heads, n_heads, pos,
                                        (hipStream_t)stream),
                    "rope_partial launch");
}

static mimo_status prefill_common(const mimo_attn_cfg *cfg, const uint16_t *q, const uint16_t *k,
                                  const uint16_t *v, uint16_t *out, int32_t B, int32_t Tq,
                                  int32_t Tk) {
    mimo_status st = check_cfg(cfg);
    if (st != MIMO_OK) return st;
    if (B < 0 || Tq < 0 || Tk < 0) return fail(MIMO_ERR_INVALID_ARGUMENT, "sizes must be >= 0");
    if ((cfg->num_q_heads / cfg->num_kv_heads) % 4 != 0)
        return fail(MIMO_ERR_UNSUPPORTED, "prefill needs a GQA group size that is a multiple of 4 (got %d)",
                    cfg->num_q_heads / cfg->num_kv_heads);
    if (B == 0 || Tq == 0) return ok();
    if (!q || !k || !v || !out) return fail(MIMO_ERR_INVALID_ARGUMENT, "q, k, v and out must be non-NULL");
    if (check_aligned("q, k, v and out", {q, k, v, out}) != MIMO_OK) return MIMO_ERR_INVALID_ARGUMENT;
    return ok();
}

mimo_status mimo_attn_prefill_swa(const mimo_attn_cfg *cfg, const uint16_t *q, const uint16_t *k,
                                  const uint16_t *v, const float *sinks, int32_t B, int32_t T,
                                  int64_t pos0, uint16_t *out, float *lse, void *stream) {
    mimo_status st = prefill_common(cfg, q, k, v, out, B, T, T);
    if (st != MIMO_OK) return st;
    if (cfg->window < 1) return fail(MIMO_ERR_INVALID_ARGUMENT, "sliding-window prefill needs window >= 1");
    if (pos0 < 0) return fail(MIMO_ERR_INVALID_ARGUMENT, "pos0 must be >= 0");
    if (B == 0 || T == 0) return ok();
    PrefillArgs a{};
    a.q = q; a.k = k; a.v = v; a.out = out; a.lse = lse; a.sinks = sinks;
    a.B = B; a.Tq = T; a.Tk = T; a.Hq = cfg->num_q_heads; a.Hkv = cfg->num_kv_heads;
    a.q_pos0 = pos0; a.k_pos0 = pos0; a.window = cfg->window; a.lse_hstride = T;
    a.scale_log2 = scale_log2(cfg); a.v_scale = cfg->v_scale;
    a.rt = rope_turns(cfg->rope_base);
    return from_hip(launch_prefill(a, (hipStream_t)stream), "prefill_swa launch");
}

// Bytes of the K/V tile images a global-layer prefill uses (0 where the layer does
// not use them: sliding windows, GQA groups that are not a multiple of 8).
static size_t image_bytes(const mimo_attn_cfg *cfg, int32_t B, int64_t total_k) {
    if (cfg->window != 0 || (cfg->num_q_heads / cfg->num_kv_heads) % 8 != 0 || B <= 0 || total_k <= 0) return 0;
    return prefill_image_bytes(B, total_k, cfg->num_kv_heads);
}

size_t mimo_attn_prefill_workspace_size(const mimo_attn_cfg *cfg, int32_t B, int64_t total_k) {
    if (check_cfg(cfg) != MIMO_OK) return 0;
    return image_bytes(cfg, B, total_k);
}

// ws == NULL: no images (the attention kernel stages each tile itself).
static mimo_status attach_images(PrefillArgs &a, const mimo_attn_cfg *cfg, int32_t B, int64_t total_k,
                                 void *ws, size_t ws_bytes) {
    const size_t need = image_bytes(cfg, B, total_k);
    if (!ws || need == 0) return ok();
    if (check_aligned("ws", {ws}) != MIMO_OK) return MIMO_ERR_INVALID_ARGUMENT;
    if (ws_bytes < need)
        return fail(MIMO_ERR_WORKSPACE, "prefill workspace needs %zu bytes (got %zu)", need, ws_bytes);
    a.kv_img = static_cast<uint16_t *>(ws);
    a.kv_norm = reinterpret_cast<float *>(static_cast<char *>(ws) +
                                          prefill_image_norm_offset(B, total_k, cfg->num_kv_heads));
    return ok();
}

mimo_status mimo_attn_prefill_global(const mimo_attn_cfg *cfg, const uint16_t *q, const uint16_t *k,
                                     const uint16_t *v, int32_t B, int32_t Tq, int32_t Tk,
                                     int64_t q_pos0, uint16_t *out, float *lse, void *ws,
                                     size_t ws_bytes, void *stream) {
    mimo_status st = prefill_common(cfg, q, k, v, out, B, Tq, Tk);
    if (st != MIMO_OK) return st;
    if (cfg->window != 0) return fail(MIMO_ERR_INVALID_ARGUMENT, "global prefill needs window == 0");
    if (q_pos0 < 0) return fail(MIMO_ERR_INVALID_ARGUMENT, "q_pos0 must be >= 0");
    if ((int64_t)Tk != q_pos0 + Tq)
        return fail(MIMO_ERR_INVALID_ARGUMENT, "Tk (%d) must equal q_pos0 + Tq (%lld)", Tk,
                    (long long)(q_pos0 + Tq));
    if (B == 0 || Tq == 0) return ok();
    PrefillArgs a{};
    a.q = q; a.k = k; a.v = v; a.out = out; a.lse = lse; a.sinks = nullptr;
    a.B = B; a.Tq = Tq; a.Tk = Tk; a.Hq = cfg->num_q_heads; a.Hkv = cfg->num_kv_heads;
    a.q_pos0 = q_pos0; a.k_pos0 = 0; a.window = 0; a.lse_hstride = Tq;
    a.scale_log2 = scale_log2(cfg); a.v_scale = cfg->v_scale;
    a.rt = rope_turns(cfg->rope_base);
    st = attach_images(a, cfg, B, (int64_t)B * Tk, ws, ws_bytes);
    if (st != MIMO_OK) return st;
    return from_hip(launch_prefill(a, (hipStream_t)stream), "prefill_global launch");
}

mimo_status mimo_attn_prefill_varlen(const mimo_attn_cfg *cfg, const uint16_t *q, const uint16_t *k,
                                     const uint16_t *v, const float *sinks, int32_t B,
                                     const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k,
                                     const int64_t *k_pos0, int32_t max_seqlen_q, int32_t total_q,
                                     int64_t total_k, uint16_t *out, float *lse, void *ws,
                                     size_t ws_bytes, void *stream) {
    mimo_status st = check_cfg(cfg);
    if (st != MIMO_OK) return st;
    if (B < 0 || max_seqlen_q < 0 || total_q < 0 || total_k < 0)
        return fail(MIMO_ERR_INVALID_ARGUMENT, "B, max_seqlen_q, total_q and total_k must be >= 0");
    if ((cfg->num_q_heads / cfg->num_kv_heads) % 4 != 0)
        return fail(MIMO_ERR_UNSUPPORTED, "prefill needs a GQA group size that is a multiple of 4 (got %d)",
                    cfg->num_q_heads / cfg->num_kv_heads);
    if (max_seqlen_q > total_q)
        return fail(MIMO_ERR_INVALID_ARGUMENT, "max_seqlen_q (%d) exceeds total_q (%d)", max_seqlen_q, total_q);
    if (B == 0 || max_seqlen_q == 0) return ok();
    if (!q || !k || !v || !out || !cu_seqlens_q || !cu_seqlens_k)
        return fail(MIMO_ERR_INVALID_ARGUMENT, "q, k, v, out, cu_seqlens_q and cu_seqlens_k must be non-NULL");
    if (check_aligned("q, k, v and out", {q, k, v, out}) != MIMO_OK) return MIMO_ERR_INVALID_ARGUMENT;
    PrefillArgs a{};
    a.q = q; a.k = k; a.v = v; a.out = out; a.lse = lse; a.sinks = sinks;
    a.B = B; a.Tq = max_seqlen_q; a.Hq = cfg->num_q_heads; a.Hkv = cfg->num_kv_heads;
    a.Tk = total_k > INT32_MAX ? INT32_MAX : (int32_t)total_k;   // packed: bounds every sequence's keys
    a.window = cfg->window; a.lse_hstride = total_q;
    a.cu_q = cu_seqlens_q; a.cu_k = cu_seqlens_k; a.kpos = k_pos0;
    a.scale_log2 = scale_log2(cfg); a.v_scale = cfg->v_scale;
    a.rt = rope_turns(cfg->rope_base);
    st = attach_images(a, cfg, B, total_k, ws, ws_bytes);
    if (st != MIMO_OK) return st;
    return from_hip(launch_prefill(a, (hipStream_t)stream), "prefill_varlen launch");
}

// Paged layout of a decode call (table == NULL: per-sequence caches).
struct PagedLayout {
    const int32_t *table = nullptr;
    int32_t max_blocks = 0, block_shift = 0, n_blocks = 0, fp8 = 0;
    float k_scale = 1.0f, v_scale = 1.0f;
};

size_t mimo_attn_backward_workspace_size(const mimo_attn_cfg *cfg, int32_t B, int32_t T) {
    if (check_cfg(cfg) != MIMO_OK || B <= 0 || T <= 0) return 0;
    return backward_workspace_bytes(B, T, cfg->num_q_heads, cfg->num_kv_heads);
}

mimo_status mimo_attn_prefill_backward(const mimo_attn_cfg *cfg, const uint16_t *q, const uint16_t *k,
                                       const uint16_t *v, const float *sinks, int32_t B, int32_t T, int64_t pos0,
                                       const uint16_t *out, const float *lse, const uint16_t *dout, uint16_t *dq,
                                       uint16_t *dk, uint16_t *dv, float *dsinks, void *ws, size_t ws_bytes,
                                       void *stream) {
    mimo_status st = prefill_common(cfg, q, k, v, dq, B, T, T);
    if (st != MIMO_OK) return st;
    if (pos0 < 0) return fail(MIMO_ERR_INVALID_ARGUMENT, "pos0 must be >= 0");
    if ((int64_t)B * T * cfg->num_q_heads > ((int64_t)1 << 31) / 2)
        return fail(MIMO_ERR_UNSUPPORTED, "B * T * num_q_heads is too large");
    if (B == 0 || T == 0) return ok();
    if (!out || !lse || !dout || !dk || !dv)
        return fail(MIMO_ERR_INVALID_ARGUMENT, "out, lse, dout, dq, dk and dv must be non-NULL");
    if (sinks && !dsinks) return fail(MIMO_ERR_INVALID_ARGUMENT, "dsinks must be non-NULL when sinks are given");
    if (check_aligned("out, dout, dq, dk, dv and ws", {out, dout, dq, dk, dv, ws}) != MIMO_OK)
        return MIMO_ERR_INVALID_ARGUMENT;
    const size_t need = backward_workspace_bytes(B, T, cfg->num_q_heads, cfg->num_kv_heads);
    if (!ws || ws_bytes < need)
        return fail(MIMO_ERR_WORKSPACE, "backward workspace needs %zu bytes (got %zu)", need,
                    ws ? ws_bytes : (size_t)0);
    BwdArgs a{};
    a.q = q; a.k = k; a.v = v; a.out = out; a.dout = dout; a.lse = lse; a.sinks = sinks;
    const size_t rows = (size_t)B * T * cfg->num_q_heads, krows = (size_t)B * T * cfg->num_kv_heads;
    a.qrot = (uint16_t *)ws;
    a.krot = a.qrot + rows * 64;
    a.D = (float *)(a.krot + krows * 64);
    a.csink = a.D + rows;
    a.dq = dq; a.dk = dk; a.dv = dv; a.dsinks = sinks ? dsinks : nullptr;
    a.B = B; a.T = T; a.Hq = cfg->num_q_heads; a.Hkv = cfg->num_kv_heads; a.window = cfg->window; a.pos0 = pos0;
    a.scale = cfg->softmax_scale; a.scale_log2 = scale_log2(cfg); a.v_scale = cfg->v_scale;
    a.rt = rope_turns(cfg->rope_base);
    return from_hip(launch_backward(a, (hipStream_t)stream), "prefill_backward launch");
}

// Validation shared by the decode calls; fills everything of `a` but the
// workspace.  All checks run before any HIP call.
static mimo_status decode_prepare(const mimo_attn_cfg *cfg, int32_t S, int32_t n_q, const uint16_t *q,
                                  const int64_t *q_pos, const void *k_cache, const void *v_cache,
                                  int32_t cap, const float *sinks, uint16_t *out, const PagedLayout &pl,
                                  DecodeArgs &a) {
    mimo_status st = check_cfg(cfg);
    if (st != MIMO_OK) return st;
    if (S < 0 || cap < 1) return fail(MIMO_ERR_INVALID_ARGUMENT, "S must be >= 0 and cap >= 1");
    if (n_q < 1) return fail(MIMO_ERR_INVALID_ARGUMENT, "n_q must be >= 1");
    const int G = cfg->num_q_heads / cfg->num_kv_heads;
    if (G > 16) return fail(MIMO_ERR_UNSUPPORTED, "decode needs a GQA group size <= 16 (got %d)", G);
    if (G * n_q > 128)
        return fail(MIMO_ERR_UNSUPPORTED, "decode needs group size x n_q <= 128 (got %d x %d)", G, n_q);
    if (!pl.table && cfg->window > 0 && (int64_t)cap < (int64_t)cfg->window + n_q - 1)
        return fail(MIMO_ERR_INVALID_ARGUMENT, "a ring cache needs cap (%d) >= window + n_q - 1 (%d)", cap,
                    cfg->window + n_q - 1);
    if (cfg->num_kv_heads > 8)
        return fail(MIMO_ERR_UNSUPPORTED, "decode needs num_kv_heads <= 8 (got %d)", cfg->num_kv_heads);
    if (S > 65535) return fail(MIMO_ERR_UNSUPPORTED, "decode needs S <= 65535");
    if (cap > kDecodeMaxCap) return fail(MIMO_ERR_UNSUPPORTED, "decode needs cap <= %d", kDecodeMaxCap);
    if (S == 0) return ok();
    if (!q || !q_pos || !k_cache || !v_cache || !out)
        return fail(MIMO_ERR_INVALID_ARGUMENT, "q, q_pos, the caches and out must be non-NULL");
    if (check_aligned("q, the caches and out", {q, k_cache, v_cache, out}) != MIMO_OK)
        return MIMO_ERR_INVALID_ARGUMENT;
    a = DecodeArgs{};
    a.q = q; a.k_cache = k_cache; a.v_cache = v_cache; a.pos = q_pos; a.sinks = sinks; a.out = out;
    a.S = S; a.Hq = cfg->num_q_heads; a.Hkv = cfg->num_kv_heads; a.cap = cap; a.window = cfg->window;
    a.n_q = n_q;
    a.scale_log2 = scale_log2(cfg); a.v_scale = cfg->v_scale;
    a.table = pl.table; a.max_blocks = pl.max_blocks; a.block_shift = pl.block_shift; a.n_blocks = pl.n_blocks;
    a.fp8 = pl.fp8;
    if (pl.fp8) {   // scores and outputs of the codes, scaled back
        a.scale_log2 *= pl.k_scale;
        a.v_scale *= pl.v_scale;
    }
    a.rt = rope_turns(cfg->rope_base);
    return ok();
}

static mimo_status decode_common(const mimo_attn_cfg *cfg, int32_t S, int32_t n_q, const uint16_t *q,
                                 const int64_t *q_pos, const void *k_cache, const void *v_cache,
                                 int32_t cap, const float *sinks, uint16_t *out, void *ws, size_t ws_bytes,
                                 void *stream, const PagedLayout &pl = PagedLayout()) {
    DecodeArgs a;
    mimo_status st = decode_prepare(cfg, S, n_q, q, q_pos, k_cache, v_cache, cap, sinks, out, pl, a);
    if (st != MIMO_OK || S == 0) return st;
    const size_t need = decode_workspace_bytes(S, cfg->num_q_heads, cfg->num_kv_heads, n_q);
    if (!ws || ws_bytes < need)
        return fail(MIMO_ERR_WORKSPACE, "decode workspace needs %zu bytes (got %zu)", need,
                    ws ? ws_bytes : (size_t)0);
    if (check_aligned("ws", {ws}) != MIMO_OK) return MIMO_ERR_INVALID_ARGUMENT;
    a.ws_o = (float *)ws;
    return from_hip(launch_decode(a, (hipStream_t)stream), "decode launch");
}

static size_t decode_ws_size(const mimo_attn_cfg *cfg, int32_t S, int32_t n_q) {
    if (!cfg || S <= 0 || n_q < 1 || cfg->num_q_heads <= 0 || cfg->num_kv_heads <= 0 ||
        cfg->num_kv_heads > 8 || cfg->num_q_heads % cfg->num_kv_heads != 0)
        return 0;
    const int G = cfg->num_q_heads / cfg->num_kv_heads;
    if (G > 16 || G * n_q > 128) return 0;
    return decode_workspace_bytes(S, cfg->num_q_heads, cfg->num_kv_heads, n_q);
}

size_t mimo_attn_decode_workspace_size(const mimo_attn_cfg *cfg, int32_t S, int32_t cap) {
    (void)cap;
    return decode_ws_size(cfg, S, 1);
}

mimo_status mimo_attn_decode(const mimo_attn_cfg *cfg, int32_t S, const uint16_t *q,
                             const int64_t *q_pos, const uint16_t *k_cache, const uint16_t *v_cache,
                             int32_t cap, const float *sinks, uint16_t *out, void *ws,
                             size_t ws_bytes, void *stream) {
    return decode_common(cfg, S, 1, q, q_pos, k_cache, v_cache, cap, sinks, out, ws, ws_bytes, stream);
}

mimo_status mimo_attn_decode_noalloc(const mimo_attn_cfg *cfg, int32_t S, const uint16_t *q,
                                     const int64_t *q_pos, const uint16_t *k_cache, const uint16_t *v_cache,
                                     int32_t cap, const float *sinks, uint16_t *out, void *stream) {
    static_assert(kDecodeScratchBytes == MIMO_DECODE_NOALLOC_MAX_BYTES, "scratch size in the header");
    DecodeArgs a;
    mimo_status st = decode_prepare(cfg, S, 1, q, q_pos, k_cache, v_cache, cap, sinks, out, PagedLayout(), a);
    if (st != MIMO_OK || S == 0) return st;
    const size_t need = decode_workspace_bytes(S, cfg->num_q_heads, cfg->num_kv_heads, 1);
    if (need > kDecodeScratchBytes)
        return fail(MIMO_ERR_WORKSPACE,
                    "allocation-free decode: %d sequences need %zu bytes of scratch, more than the %zu the "
                    "library holds per GPU; use mimo_attn_decode with a workspace", S, need,
                    kDecodeScratchBytes);
    void *ptr = nullptr;
    const hipError_t e = decode_scratch((hipStream_t)stream, &ptr);
    if (e == hipErrorInvalidDevice)
        return fail(MIMO_ERR_INVALID_ARGUMENT, "allocation-free decode: the stream must belong to the current device");
    if (e != hipSuccess) return from_hip(e, "decode scratch lookup");
    a.ws_o = (float *)ptr;
    return from_hip(launch_decode(a, (hipStream_t)stream), "decode launch");
}

size_t mimo_attn_decode_multi_workspace_size(const mimo_attn_cfg *cfg, int32_t S, int32_t n_q, int32_t cap) {
    (void)cap;
    return decode_ws_size(cfg, S, n_q);
}

mimo_status mimo_attn_decode_multi(const mimo_attn_cfg *cfg, int32_t S, int32_t n_q, const uint16_t *q,
                                   const int64_t *q_pos, const uint16_t *k_cache, const uint16_t *v_cache,
                                   int32_t cap, const float *sinks, uint16_t *out, void *ws,
                                   size_t ws_bytes, void *stream) {
    return decode_common(cfg, S, n_q, q, q_pos, k_cache, v_cache, cap, sinks, out, ws, ws_bytes, stream);
}

// Checks of a paged layout shared by decode and append.
static mimo_status check_paged(int32_t n_blocks, int32_t block_size, mimo_kv_dtype kv_dtype, float k_scale,
                               float v_scale, int32_t max_blocks, PagedLayout &pl) {
    if (kv_dtype != MIMO_KV_BF16 && kv_dtype != MIMO_KV_FP8_E4M3)
        return fail(MIMO_ERR_INVALID_ARGUMENT, "kv_dtype must be MIMO_KV_BF16 or MIMO_KV_FP8_E4M3");
    if (block_size < 32 || (block_size & (block_size - 1)) != 0 || block_size > (1 << 16))
        return fail(MIMO_ERR_UNSUPPORTED, "block_size must be a power of two in [32, 65536] (got %d)", block_size);
    if (n_blocks < 1 || max_blocks < 1)
        return fail(MIMO_ERR_INVALID_ARGUMENT, "n_blocks and max_blocks must be >= 1");
    if ((int64_t)max_blocks * block_size > (1 << 30))
        return fail(MIMO_ERR_UNSUPPORTED, "max_blocks * block_size must be <= 2^30");
    if (kv_dtype == MIMO_KV_FP8_E4M3 &&
        (!(k_scale > 0.0f) || !(v_scale > 0.0f) || !isfinite(k_scale) || !isfinite(v_scale)))
        return fail(MIMO_ERR_INVALID_ARGUMENT, "fp8 scales must be finite and > 0");
    int shift = 0;
    while ((1 << shift) < block_size) ++shift;
    pl.max_blocks = max_blocks;
    pl.block_shift = shift;
    pl.n_blocks = n_blocks;
    pl.fp8 = kv_dtype == MIMO_KV_FP8_E4M3;
    pl.k_scale = pl.fp8 ? k_scale : 1.0f;
    pl.v_scale = pl.fp8 ? v_scale : 1.0f;
    return ok();
}

mimo_status mimo_attn_decode_paged(const mimo_attn_cfg *cfg, int32_t S, int32_t n_q, const uint16_t *q,
                                   const int64_t *q_pos, const void *k_pool, const void *v_pool,
                                   int32_t n_blocks, int32_t block_size, mimo_kv_dtype kv_dtype,
                                   float k_scale, float v_scale, const int32_t *block_table,
                                   int32_t max_blocks, const float *sinks, uint16_t *out, void *ws,
                                   size_t ws_bytes, void *stream) {
    mimo_status st = check_cfg(cfg);
    if (st != MIMO_OK) return st;
    PagedLayout pl;
    st = check_paged(n_blocks, block_size, kv_dtype, k_scale, v_scale, max_blocks, pl);
    if (st != MIMO_OK) return st;
    if (S > 0 && !block_table) return fail(MIMO_ERR_INVALID_ARGUMENT, "block_table must be non-NULL");
    pl.table = block_table;
    return decode_common(cfg, S, n_q, q, q_pos, k_pool, v_pool, max_blocks * block_size, sinks, out, ws,
                         ws_bytes, stream, pl);
}

mimo_status mimo_kv_paged_append(const mimo_attn_cfg *cfg, int32_t S, const uint16_t *k_new,
                                 const uint16_t *v_new, const int64_t *pos, void *k_pool, void *v_pool,
                                 int32_t n_blocks, int32_t block_size, mimo_kv_dtype kv_dtype,
                                 float k_scale, float v_scale, const int32_t *block_table,
                                 int32_t max_blocks, void *stream) {
    mimo_status st = check_cfg(cfg);
    if (st != MIMO_OK) return st;
    PagedLayout pl;
    st = check_paged(n_blocks, block_size, kv_dtype, k_scale, v_scale, max_blocks, pl);
    if (st != MIMO_OK) return st;
    if (S < 0) return fail(MIMO_ERR_INVALID_ARGUMENT, "S must be >= 0");
    if ((int64_t)S * cfg->num_kv_heads > 0x7fffffff)
        return fail(MIMO_ERR_UNSUPPORTED, "S * num_kv_heads is too large");
    if (S == 0) return ok();
    if (!k_new || !v_new || !pos || !k_pool || !v_pool || !block_table)
        return fail(MIMO_ERR_INVALID_ARGUMENT, "k_new, v_new, pos, the pools and block_table must be non-NULL");
    if (check_aligned("k_new, v_new and the pools", {k_new, v_new, k_pool, v_pool}) != MIMO_OK)
        return MIMO_ERR_INVALID_ARGUMENT;
    PagedAppendArgs a{};
    a.k_new = k_new; a.v_new = v_new; a.pos = pos; a.k_pool = k_pool; a.v_pool = v_pool; a.table = block_table;
    a.S = S; a.Hkv = cfg->num_kv_heads; a.n_blocks = n_blocks; a.block_shift = pl.block_shift;
    a.max_blocks = max_blocks; a.fp8 = pl.fp8; a.k_scale = pl.k_scale; a.v_scale = pl.v_scale;
    return from_hip(launch_kv_paged_append(rope_turns(cfg->rope_base), a, (hipStream_t)stream),
                    "kv_paged_append launch");
}

mimo_status mimo_kv_ring_append(const mimo_attn_cfg *cfg, int32_t S, const uint16_t *k_new,
                                const uint16_t *v_new, const int64_t *pos, uint16_t *k_cache,
                                uint16_t *v_cache, int32_t cap, void *stream) {
    mimo_status st = check_cfg(cfg);
    if (st != MIMO_OK) return st;
    if (S < 0 || cap < 1) return fail(MIMO_ERR_INVALID_ARGUMENT, "S must be >= 0 and cap >= 1");
    if ((int64_t)S * cfg->num_kv_heads > 0x7fffffff)
        return fail(MIMO_ERR_UNSUPPORTED, "S * num_kv_heads is too large");
    if (S == 0) return ok();
    if (!k_new || !v_new || !pos || !k_cache || !v_cache)
        return fail(MIMO_ERR_INVALID_ARGUMENT, "k_new, v_new, pos, k_cache and v_cache must be non-NULL");
    if (check_aligned("k_new, v_new and the caches", {k_new, v_new, k_cache, v_cache}) != MIMO_OK)
        return MIMO_ERR_INVALID_ARGUMENT;
    return from_hip(launch_kv_ring_append(rope_turns(cfg->rope_base), S, cfg->num_kv_heads, k_new,
                                          v_new, pos, k_cache, v_cache, cap, (hipStream_t)stream),
                    "kv_ring_append launch");
}

}  // extern "C"
