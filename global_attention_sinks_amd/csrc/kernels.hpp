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
    // filled by the launcher
    int32_t n_qblk, n_hgrp, xcd_remap;
};
hipError_t launch_prefill(PrefillArgs a, hipStream_t stream);

// ---- decode (decode.hip)
#ifndef MIMO_DECODE_CHUNK
#define MIMO_DECODE_CHUNK 1024
#endif
constexpr int kDecodeChunk = MIMO_DECODE_CHUNK;   // cache slots per split
constexpr int kDecodeMaxSplits = 1024;   // so caches of up to 1M slots
struct DecodeArgs {
    const uint16_t *q, *k_cache, *v_cache;
    const int64_t *pos;
    const float *sinks;   // nullable
    uint16_t *out;
    float *ws_o;          // [S, Hq, n_split_max, 128]
    float *ws_ml;         // [S, Hq, n_split_max, 2]
    int32_t S, Hq, Hkv, cap, window, n_split_max;
    float scale_log2, v_scale;
    RopeTurns rt;
};
size_t decode_workspace_bytes(int32_t S, int32_t Hq, int32_t cap);
hipError_t launch_decode(DecodeArgs a, hipStream_t stream);

}  // namespace mimo
