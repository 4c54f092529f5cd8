// Partial RoPE (techniques map page, Partial RoPE: the first 64 of 192 dims
// rotate) and the window-sized ring append (Gaudi recipe page, Launch section:
// sliding layers keep only their window of KV).  Both are HBM-bound copies with
// a rotation on 64 dims; the angles use exact fixed-point turn reduction.
#include "kernels.hpp"

namespace mimo {

// One thread per unit of a 192-dim row: units 0..3 rotate the 16-byte chunk
// pair (c, c+4) = dims [8c, 8c+8) with [8c+32, 8c+40); units 4..19 copy the
// pass-through chunks 8..23.  In place, only the 4 rotating units run.
__global__ __launch_bounds__(256) void rope_partial_kernel(RopeTurns rt, const uint16_t *x_in,
                                                           uint16_t *x_out, int64_t n_rows,
                                                           int32_t n_heads, const int64_t *pos,
                                                           int32_t units) {
    int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
    int64_t row = u / units;
    int unit = (int)(u - row * units);
    if (row >= n_rows) return;
    const uint16_t *src = x_in + row * kDqk;
    uint16_t *dst = x_out + row * kDqk;
    if (unit < 4) {
        int64_t p = pos[row / n_heads];
        u32x4 x = ldg128(src + 8 * unit);
        u32x4 y = ldg128(src + 8 * unit + 32);
        rope_rotate8(x, y, rt, 8 * unit, p);
        stg128(dst + 8 * unit, x);
        stg128(dst + 8 * unit + 32, y);
    } else {
        int c = 8 + (unit - 4);
        stg128(dst + 8 * c, ldg128(src + 8 * c));
    }
}

hipError_t launch_rope_partial(const RopeTurns &rt, const uint16_t *x_in, uint16_t *x_out,
                               int64_t n_rows, int32_t n_heads, const int64_t *pos,
                               hipStream_t stream) {
    int units = (x_in == x_out) ? 4 : 20;
    int64_t threads = n_rows * units;
    int64_t blocks = (threads + 255) / 256;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(rope_partial_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, rt, x_in,
                       x_out, n_rows, n_heads, pos, units);
    return hipGetLastError();
}

// One block of 64 threads per (sequence, KV head): threads 0..3 rotate the k
// chunk pairs, 4..19 copy the k pass-through chunks, 20..35 copy v.
__global__ __launch_bounds__(64) void kv_ring_append_kernel(RopeTurns rt, int32_t Hkv,
                                                            const uint16_t *k_new,
                                                            const uint16_t *v_new,
                                                            const int64_t *pos, uint16_t *k_cache,
                                                            uint16_t *v_cache, int32_t cap) {
    int row = blockIdx.x;
    int s = row / Hkv, g = row - s * Hkv;
    int t = threadIdx.x;
    int64_t p = pos[s];
    if (p < 0) return;   // outside the contract: write nothing
    int64_t slot = p % cap;
    size_t dst_row = ((size_t)s * cap + slot) * Hkv + g;
    const uint16_t *ks = k_new + (size_t)row * kDqk;
    uint16_t *kd = k_cache + dst_row * kDqk;
    if (t < 4) {
        u32x4 x = ldg128(ks + 8 * t);
        u32x4 y = ldg128(ks + 8 * t + 32);
        rope_rotate8(x, y, rt, 8 * t, p);
        stg128(kd + 8 * t, x);
        stg128(kd + 8 * t + 32, y);
    } else if (t < 20) {
        int c = 8 + (t - 4);
        stg128(kd + 8 * c, ldg128(ks + 8 * c));
    } else if (t < 36) {
        int c = t - 20;
        stg128(v_cache + dst_row * kDv + 8 * c, ldg128(v_new + (size_t)row * kDv + 8 * c));
    }
}

hipError_t launch_kv_ring_append(const RopeTurns &rt, int32_t S, int32_t Hkv, const uint16_t *k_new,
                                 const uint16_t *v_new, const int64_t *pos, uint16_t *k_cache,
                                 uint16_t *v_cache, int32_t cap, hipStream_t stream) {
    hipLaunchKernelGGL(kv_ring_append_kernel, dim3((unsigned)(S * Hkv)), dim3(64), 0, stream, rt,
                       Hkv, k_new, v_new, pos, k_cache, v_cache, cap);
    return hipGetLastError();
}

// Four fp32 values -> four fp8 e4m3 codes (round to nearest even; values
// beyond +-448 saturate), packed in one dword, value e in byte e.
__device__ __forceinline__ uint32_t fp8x4(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

__device__ __forceinline__ float clamp448(float x) { return fminf(fmaxf(x, -448.0f), 448.0f); }

// 8 bf16 values, each divided by scale, as 8 fp8 codes
__device__ __forceinline__ u32x2 quant8(u32x4 x, float scale) {
    u32x2 r;
    r[0] = fp8x4(clamp448(bf_lo(x[0]) / scale), clamp448(bf_hi(x[0]) / scale), clamp448(bf_lo(x[1]) / scale),
                 clamp448(bf_hi(x[1]) / scale));
    r[1] = fp8x4(clamp448(bf_lo(x[2]) / scale), clamp448(bf_hi(x[2]) / scale), clamp448(bf_lo(x[3]) / scale),
                 clamp448(bf_hi(x[3]) / scale));
    return r;
}

// One workgroup of 64 threads per (sequence, KV head), as for the ring append.
__global__ __launch_bounds__(64) void kv_paged_append_kernel(RopeTurns rt, PagedAppendArgs a) {
    const int row = blockIdx.x;
    const int s = row / a.Hkv, g = row - s * a.Hkv;
    const int t = threadIdx.x;
    const int64_t p = a.pos[s];
    if (p < 0) return;                              // outside the contract: write nothing
    const int64_t lb = p >> a.block_shift;
    if (lb >= a.max_blocks) return;
    int blk = a.table[(size_t)s * a.max_blocks + lb];
    blk = blk < 0 ? 0 : (blk >= a.n_blocks ? a.n_blocks - 1 : blk);
    const size_t dst_row = ((((size_t)blk << a.block_shift) + (size_t)(p & ((1 << a.block_shift) - 1))) * a.Hkv) + g;
    const uint16_t *ks = a.k_new + (size_t)row * kDqk;
    const uint16_t *vs = a.v_new + (size_t)row * kDv;
    if (!a.fp8) {
        uint16_t *kd = static_cast<uint16_t *>(a.k_pool) + dst_row * kDqk;
        uint16_t *vd = static_cast<uint16_t *>(a.v_pool) + dst_row * kDv;
        if (t < 4) {
            u32x4 x = ldg128(ks + 8 * t);
            u32x4 y = ldg128(ks + 8 * t + 32);
            rope_rotate8(x, y, rt, 8 * t, p);
            stg128(kd + 8 * t, x);
            stg128(kd + 8 * t + 32, y);
        } else if (t < 20) {
            const int c = 8 + (t - 4);
            stg128(kd + 8 * c, ldg128(ks + 8 * c));
        } else if (t < 36) {
            const int c = t - 20;
            stg128(vd + 8 * c, ldg128(vs + 8 * c));
        }
        return;
    }
    uint8_t *kd = static_cast<uint8_t *>(a.k_pool) + dst_row * kDqk;
    uint8_t *vd = static_cast<uint8_t *>(a.v_pool) + dst_row * kDv;
    if (t < 4) {
        // rotate pairs (8t + e, 8t + e + 32) in fp32 and quantise the fp32 result
        const u32x4 x = ldg128(ks + 8 * t), y = ldg128(ks + 8 * t + 32);
        float xr[8], yr[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float sn, cs;
            rope_sincos(rt.turn[8 * t + e], p, sn, cs);
            const float x0 = (e & 1) ? bf_hi(x[e >> 1]) : bf_lo(x[e >> 1]);
            const float y0 = (e & 1) ? bf_hi(y[e >> 1]) : bf_lo(y[e >> 1]);
            xr[e] = clamp448((x0 * cs - y0 * sn) / a.k_scale);
            yr[e] = clamp448((y0 * cs + x0 * sn) / a.k_scale);
        }
        const u32x2 qx = {fp8x4(xr[0], xr[1], xr[2], xr[3]), fp8x4(xr[4], xr[5], xr[6], xr[7])};
        const u32x2 qy = {fp8x4(yr[0], yr[1], yr[2], yr[3]), fp8x4(yr[4], yr[5], yr[6], yr[7])};
        *reinterpret_cast<u32x2 *>(kd + 8 * t) = qx;
        *reinterpret_cast<u32x2 *>(kd + 8 * t + 32) = qy;
    } else if (t < 20) {
        const int c = 8 + (t - 4);
        *reinterpret_cast<u32x2 *>(kd + 8 * c) = quant8(ldg128(ks + 8 * c), a.k_scale);
    } else if (t < 36) {
        const int c = t - 20;
        *reinterpret_cast<u32x2 *>(vd + 8 * c) = quant8(ldg128(vs + 8 * c), a.v_scale);
    }
}

hipError_t launch_kv_paged_append(const RopeTurns &rt, const PagedAppendArgs &a, hipStream_t stream) {
    hipLaunchKernelGGL(kv_paged_append_kernel, dim3((unsigned)(a.S * a.Hkv)), dim3(64), 0, stream, rt, a);
    return hipGetLastError();
}

}  // namespace mimo
