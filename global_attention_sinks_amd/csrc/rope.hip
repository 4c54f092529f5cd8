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

}  // namespace mimo
