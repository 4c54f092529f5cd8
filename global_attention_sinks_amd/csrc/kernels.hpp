// Launch interface between the C ABI layer and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace mimo {

// ---- partial RoPE and ring append (rope.hip)
hipError_t launch_rope_partial(const RopeTurns &rt, const uint16_t *x_in, uint16_t *x_out,
                               int64_t n_rows, int32_t n_heads, const int64_t *pos,
                               hipStream_t stream);
hipError_t launch_kv_ring_append(const RopeTurns &rt, int32_t S, int32_t Hkv, const uint16_t *k_new,
                                 const uint16_t *v_new, const int64_t *pos, uint16_t *k_cache,
                                 uint16_t *v_cache, int32_t cap, hipStream_t stream);
// Paged pools [n_blocks, 1 << block_shift, Hkv, D] of bf16 (fp8 == 0) or fp8 e4m3 codes.
struct PagedAppendArgs {
    const uint16_t *k_new, *v_new;
    const int64_t *pos;
    void *k_pool, *v_pool;
    const int32_t *table;
    int32_t S, Hkv, n_blocks, block_shift, max_blocks, fp8;
    float k_scale, v_scale;
};
hipError_t launch_kv_paged_append(const RopeTurns &rt, const PagedAppendArgs &a, hipStream_t stream);

// ---- prefill (prefill.hip)
struct PrefillArgs {
    const uint16_t *q, *k, *v;
    uint16_t *out;
    float *lse;           // nullable
    const float *sinks;   // nullable
    int32_t B, Tq, Tk, Hq, Hkv;
    int64_t q_pos0;       // position of query 0
    int64_t k_pos0;       // position of key 0
    int32_t window;       // 0 = causal only
    float scale_log2;     // softmax_scale * log2(e)
    float v_scale;
    RopeTurns rt;
    // packed sequences (all NULL for dense batches): sequence b owns query tokens
    // cu_q[b]..cu_q[b+1]-1 and key tokens cu_k[b]..cu_k[b+1]-1, its first key sits
    // at position kpos[b] (0 if kpos is NULL) and its queries are its last keys;
    // Tq is then the longest query count and Tk the total key count
    const int32_t *cu_q, *cu_k;
    const int64_t *kpos;
    int64_t lse_hstride;  // lse element stride between heads
    // filled by the launcher
    int32_t n_qblk, n_hgrp, xcd_remap;
    int32_t band_runs;    // sliding band kernel: runs of query blocks per (sequence, KV head)
    // global layers (window 0, GQA group a multiple of 8): device buffer of at least
    // prefill_image_bytes() for the rotated-K / transposed-V tile images, or NULL to
    // stage each tile inside the attention kernel
    uint16_t *kv_img;
    float *kv_norm;       // largest key norm of each tile image (same index), with kv_img
};
// Tile images a global prefill over B sequences of total_k keys may use, and the
// workspace they take: the images, then one fp32 norm per image.
size_t prefill_image_count(int32_t B, int64_t total_k, int32_t Hkv);
size_t prefill_image_norm_offset(int32_t B, int64_t total_k, int32_t Hkv);   // bytes before the norms
size_t prefill_image_bytes(int32_t B, int64_t total_k, int32_t Hkv);
hipError_t launch_prefill(PrefillArgs a, hipStream_t stream);

// ---- prefill backward (backward.hip)
struct BwdArgs {
    const uint16_t *q, *k, *v, *out, *dout;   // [B, T, H, D] bf16, q/k unrotated
    const float *lse;                         // [B, Hq, T] natural-log LSE of the forward
    const float *sinks;                       // nullable
    uint16_t *qrot;                           // workspace [B, Hq, T, 64]: the rotated dims of Q~ (bf16)
    uint16_t *krot;                           // workspace [B, Hkv, T, 64]: the rotated dims of K~ (bf16)
    float *D;                                 // workspace [B, Hq, T]: rowsum(dO o O)
    float *csink;                             // workspace [B * 32-query blocks, Hq]: sink-term partials
    uint16_t *dq, *dk, *dv;
    float *dsinks;                            // [Hq], written when sinks != NULL
    int32_t B, T, Hq, Hkv, window;
    int64_t pos0;
    float scale, scale_log2, v_scale;
    RopeTurns rt;
    int32_t n_qblk, n_hgrp, n_kblk;           // filled by the launcher
};
size_t backward_workspace_bytes(int32_t B, int32_t T, int32_t Hq, int32_t Hkv);
hipError_t launch_backward(BwdArgs a, hipStream_t stream);

// ---- decode (decode.hip)
// The batch's 32-slot steps are split evenly over step ranges, each taking at
// least kDecodeMinSteps steps; the partial pass runs kDecodeWaves waves in all
// (one per SIMD of the 256 CUs).
constexpr int kDecodeWaves = 1024;
constexpr int kDecodeMinSteps = 1;
constexpr int kDecodeMaxCap = 1 << 30;
struct DecodeArgs {
    const uint16_t *q;
    const void *k_cache, *v_cache;   // per-sequence caches [S, cap, Hkv, D], or paged pools
    const int64_t *pos;   // newest query's position per sequence
    const float *sinks;   // nullable
    uint16_t *out;
    float *ws_o;          // [n_groups + S, n_q, Hq, 128] partial outputs
    float *ws_ml;         // [n_groups + S, n_q, Hq, 2] partial (max, sum)
    int64_t *plan_start;  // [S + 1] first step of each sequence; [S] = total steps
    int32_t *plan_first;  // [S] first workgroup on the sequence
    int32_t *plan_cover;  // [S] workgroups on the sequence (0: nothing visible)
    int32_t *plan_part;   // [S] first partial slot of the sequence
    int32_t *plan_wg_seq; // [n_groups] sequence holding each workgroup's first step
    int32_t S, Hq, Hkv, cap, window, n_q;
    // paged caches (table == NULL: per-sequence caches of cap slots): position t of
    // sequence s is in pool block table[s * max_blocks + (t >> block_shift)]
    const int32_t *table;
    int32_t max_blocks, block_shift, n_blocks;
    int32_t fp8;                   // pools hold fp8 e4m3 codes (scales folded into scale_log2, v_scale)
    int32_t n_groups, wph, kvpw;   // filled by the launcher
    int32_t direct;                // 1: workgroup x = sequence x, all its steps, no plan / combine
    float scale_log2, v_scale;
    RopeTurns rt;
};
// Launch shape of the decode partial pass for a head geometry and query count.
struct DecodeGeom {
    int nc;        // 16-column (query token, head) tiles per wave
    int wph;       // waves per KV head
    int kvpw;      // KV heads per workgroup
    int n_hsub;    // workgroups side by side on one step range (KV head subsets)
    int threads;   // workgroup size
    int n_groups;  // step ranges
};
DecodeGeom decode_geometry(int32_t Hq, int32_t Hkv, int32_t n_q);
size_t decode_workspace_bytes(int32_t S, int32_t Hq, int32_t Hkv, int32_t n_q);
hipError_t launch_decode(DecodeArgs a, hipStream_t stream);
// Scratch of the allocation-free decode call: a device array of this many bytes
// that the library holds on every GPU it runs on.  decode_scratch() returns its
// address on the current device (looked up once per device); hipErrorInvalidDevice
// if `stream` belongs to another device.
constexpr size_t kDecodeScratchBytes = (size_t)32 << 20;
hipError_t decode_scratch(hipStream_t stream, void **ptr);

}  // namespace mimo
