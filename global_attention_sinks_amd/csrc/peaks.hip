// On-box peaks for the roofline: a bf16 MFMA throughput loop and HBM stream
// kernels (copy, read).  Measurement only: nothing on the attention path calls
// these; the benchmark reports its kernels against both the vendor peaks and
// what these reach on the same card.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mimo_peaks.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kOps = 8;     // operand registers per side, rotated so consecutive MFMAs see new data
constexpr int kChains = 8;  // independent accumulators per wave (covers the MFMA's latency)

// Each wave loads kOps A and kOps B operands (16 bytes per lane each) from
// `operands`, then issues iters * 64 MFMA 32x32x16 bf16 in kChains chains whose
// operands change from one MFMA to the next.  One float per wave is written so
// the work cannot be dropped.
__global__ __launch_bounds__(256) void mfma_loop_kernel(const uint16_t *operands, int64_t n_elems, int iters,
                                                        float *sink) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    u32x4 A[kOps], B[kOps];
#pragma unroll
    for (int i = 0; i < kOps; ++i) {
        const int64_t ea = (((wave * 2 * kOps + i) * 64 + lane) * 8) % (n_elems - 7);
        const int64_t eb = (((wave * 2 * kOps + kOps + i) * 64 + lane) * 8) % (n_elems - 7);
        A[i] = *reinterpret_cast<const u32x4 *>(operands + (ea & ~(int64_t)7));
        B[i] = *reinterpret_cast<const u32x4 *>(operands + (eb & ~(int64_t)7));
    }
    f32x16 acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[c][e] = 0.0f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int c = 0; c < kChains; ++c)
                acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8, A[(c + u) % kOps]), __builtin_bit_cast(bf16x8, B[(3 * c + u) % kOps]),
                    acc[c], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += acc[c][e];
    if (lane == 0) sink[wave] = s;
}

// Grid-stride streams of 16-byte elements, four loads in flight per thread
// before their stores (or their use), marked non-temporal: streamed once.
constexpr int kUnroll = 4;

__global__ __launch_bounds__(256) void copy_kernel(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + (kUnroll - 1) * stride < n; i += kUnroll * stride) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) __builtin_nontemporal_store(v[u], dst + i + u * stride);
    }
    for (; i < n; i += stride) dst[i] = src[i];
}

__global__ __launch_bounds__(256) void read_kernel(const u32x4 *__restrict__ src, int64_t n, uint32_t *out) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t x = 0;
    for (; i + (kUnroll - 1) * stride < n; i += kUnroll * stride) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    for (; i < n; i += stride) {
        const u32x4 v = src[i];
        x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    if (x == 0x9e3779b9u) out[0] = x;   // keeps the loads; practically never stores
}

__global__ __launch_bounds__(256) void write_kernel(u32x4 *__restrict__ dst, int64_t n, uint32_t value) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const u32x4 v = {value, value, value, value};
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + (kUnroll - 1) * stride < n; i += kUnroll * stride) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) __builtin_nontemporal_store(v, dst + i + u * stride);
    }
    for (; i < n; i += stride) dst[i] = v;
}

}  // namespace

extern "C" {

int mimo_peak_mfma_waves(void) { return 256 * 4 * 2; }

int mimo_peak_mfma_bf16(const uint16_t *operands, int64_t n_elems, int32_t iters, float *sink, void *stream) {
    if (!operands || !sink || n_elems < 64 || iters < 1) return (int)hipErrorInvalidValue;
    const int waves = mimo_peak_mfma_waves();   // two waves per SIMD on every CU
    hipLaunchKernelGGL(mfma_loop_kernel, dim3(waves / 4), dim3(256), 0, (hipStream_t)stream, operands, n_elems,
                       iters, sink);
    return (int)hipGetLastError();
}

int mimo_peak_copy(const void *src, void *dst, int64_t bytes, void *stream) {
    if (!src || !dst || bytes < 16 || bytes % 16) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(copy_kernel, dim3(256 * 16), dim3(256), 0, (hipStream_t)stream,
                       static_cast<const u32x4 *>(src), static_cast<u32x4 *>(dst), bytes / 16);
    return (int)hipGetLastError();
}

int mimo_peak_read(const void *src, int64_t bytes, uint32_t *out, void *stream) {
    if (!src || !out || bytes < 16 || bytes % 16) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(read_kernel, dim3(256 * 16), dim3(256), 0, (hipStream_t)stream,
                       static_cast<const u32x4 *>(src), bytes / 16, out);
    return (int)hipGetLastError();
}

int mimo_peak_write(void *dst, int64_t bytes, uint32_t value, void *stream) {
    if (!dst || bytes < 16 || bytes % 16) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(write_kernel, dim3(256 * 16), dim3(256), 0, (hipStream_t)stream, static_cast<u32x4 *>(dst),
                       bytes / 16, value);
    return (int)hipGetLastError();
}

}  // extern "C"
