// Decode attention: one query token per sequence over a KV cache, for both
// layer types (sliding layers over their window-sized ring, Gaudi recipe page,
// Launch section; global layers over a long cache).  Split-K flash decoding:
//
//   pass 1 (decode_partial_kernel): one workgroup per (sequence, chunk of
//     kDecodeChunk cache slots) with one wave per KV head, so a workgroup
//     streams whole token rows [slot][all KV heads] of the cache.  Per 32-key
//     step a wave computes S^T = K Q^T for its GQA group's query heads (<= 16,
//     the N side of a 16x16x32 bf16 MFMA) and O^T += V^T P^T.  K is read
//     straight from HBM in operand layout: the contraction order over the 192
//     dims is chosen so that the 4 lanes of a key row read 64 contiguous bytes
//     per load and consecutive loads finish each 128-byte line; V is read
//     row-major and transposed in registers with byte permutes.  The next step's K/V loads are in flight while the current step
//     is computed.  A sequence whose live slots fit one chunk writes its output
//     directly; otherwise the wave writes its (max, sum, O) partial.
//   pass 2 (decode_combine_kernel): merges the chunk partials by their
//     log-sum-exp.
//
// The sink logit (techniques map page, Learnable attention sink) is folded into
// chunk 0 as the initial (max, sum) = (sink * log2 e, 1).
#include "kernels.hpp"

namespace mimo {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// Number of cache slots a query at position p can see (slots >= this hold nothing).
__device__ __forceinline__ int live_slots(int64_t p, int32_t cap) {
    if (p < 0) return 0;
    return p + 1 < cap ? (int)(p + 1) : cap;
}

#ifndef MIMO_DECODE_NT
#define MIMO_DECODE_NT 0
#endif
// K/V cache rows are read exactly once: stream them past the caches
__device__ __forceinline__ u32x4 ldg_stream(const uint16_t *p) {
#if MIMO_DECODE_NT
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
#else
    return *reinterpret_cast<const u32x4 *>(p);
#endif
}

struct StepBuf {
    u32x4 k[2][6];   // [16-key sub-block][chunk]: dims 32*ch + 8*lg .. +8 of one key row
    u32x4 v[8];      // 8 key rows x 8 dv
};

}  // namespace

__global__ __launch_bounds__(512) void decode_partial_kernel(DecodeArgs a) {
    const int sp = blockIdx.x;
    const int s = blockIdx.y;
    const int lane = threadIdx.x & 63, g = threadIdx.x >> 6;   // one wave per KV head
    const int lg = lane >> 4, r16 = lane & 15;
    const int G = a.Hq / a.Hkv;

    const int64_t p = a.pos[s];
    const int n = live_slots(p, a.cap);
    const int nsplit = (n + kDecodeChunk - 1) / kDecodeChunk;
    if (sp >= (nsplit > 0 ? nsplit : 1)) return;

    const int head = g * G + r16;
    const bool head_ok = r16 < G;

    // ---- q (B operand): head r16; contraction slot (ch, lg, e) is dim 32*ch + 8*lg + e,
    // so the 4 lanes of a K row read 64 contiguous bytes per load instruction.
    // Chunks 0 and 1 of a lane are rotate-half partners (dims i and i+32).
    u32x4 qf[6];
    if (head_ok && p >= 0) {
        const uint16_t *qrow = a.q + ((size_t)s * a.Hq + head) * kDqk + 8 * lg;
#pragma unroll
        for (int ch = 0; ch < 6; ++ch) qf[ch] = ldg128(qrow + 32 * ch);
        rope_rotate8(qf[0], qf[1], a.rt, 8 * lg, p);
    } else {
#pragma unroll
        for (int ch = 0; ch < 6; ++ch) qf[ch] = u32x4{0, 0, 0, 0};
    }

    float m_run, l_run;
    if (sp == 0 && a.sinks && head_ok) {
        m_run = a.sinks[head] * kLog2e;
        l_run = (lg == 0) ? 1.0f : 0.0f;
    } else {
        m_run = kNegInf;
        l_run = 0.0f;
    }
    f32x4 O[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) O[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    const size_t krs = (size_t)a.Hkv * kDqk, vrs = (size_t)a.Hkv * kDv;
    const uint16_t *kbase = a.k_cache + (size_t)s * a.cap * krs + (size_t)g * kDqk + 8 * lg;
    const uint16_t *vbase = a.v_cache + (size_t)s * a.cap * vrs + (size_t)g * kDv + 8 * r16;
    const int kbeg = sp * kDecodeChunk;
    const int kend = (kbeg + kDecodeChunk < n) ? kbeg + kDecodeChunk : n;
    const float cl2 = a.scale_log2;
    // ring rule: slot j holds position p - ((p - j) mod cap); with pm = p mod cap
    // that distance is pm - j, or pm - j + cap when j > pm
    const int pm = p >= 0 ? (int)(p % a.cap) : 0;
    const int win = a.window > 0 ? a.window : 0x7fffffff;
    const int64_t pcap = p;

    auto load = [&](StepBuf &bf, int j0) {
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            const int j = j0 + 16 * sb + r16;
#pragma unroll
            for (int ch = 0; ch < 6; ++ch)
                bf.k[sb][ch] = (j < a.cap) ? ldg_stream(kbase + (size_t)j * krs + 32 * ch) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            const int j = j0 + 16 * (jj >> 2) + 4 * lg + (jj & 3);
            bf.v[jj] = (j < a.cap) ? ldg_stream(vbase + (size_t)j * vrs) : u32x4{0, 0, 0, 0};
        }
    };

    auto visible = [&](int j) -> bool {
        if (j >= n) return false;
        if (a.window > 0) {
            int d = pm - j;
            if (d < 0) d += a.cap;
            return d < win && (int64_t)d <= pcap;
        }
        return true;
    };

    auto compute = [&](StepBuf &bf, int j0) {
        f32x4 S[2];
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            S[sb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ch = 0; ch < 6; ++ch) S[sb] = mfma16(bf.k[sb][ch], qf[ch], S[sb]);
        }
        // lane's keys: j0 + 16*sb + 4*lg + i  (rows of its S^T registers and of its V loads)
        if (j0 + 32 > kend || a.window > 0) {
#pragma unroll
            for (int sb = 0; sb < 2; ++sb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (!visible(j0 + 16 * sb + 4 * lg + i)) {
                        S[sb][i] = kNegInf;
                        bf.v[4 * sb + i] = u32x4{0, 0, 0, 0};
                    }
                }
        }
        float mx = fmaxf(fmaxf(fmaxf(S[0][0], S[0][1]), fmaxf(S[0][2], S[0][3])),
                         fmaxf(fmaxf(S[1][0], S[1][1]), fmaxf(S[1][2], S[1][3])));
        mx = max_xor16(mx);
        mx = max_xor32(mx);
        const float mc = mx * cl2;
        const bool need = mc > m_run + 8.0f;
        if (__any(need)) {
            const float alpha = need ? __builtin_amdgcn_exp2f(m_run - mc) : 1.0f;
            if (need) m_run = mc;
            l_run *= alpha;
#pragma unroll
            for (int t = 0; t < 8; ++t) O[t] *= alpha;
        }
        const float mu = (m_run == kNegInf) ? 0.0f : m_run;
        float ls = 0.0f;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(S[sb][i], cl2, -mu));
                S[sb][i] = pv;
                ls += pv;
            }
        l_run += ls;
        u32x4 pf;
        pf[0] = pack_bf16(S[0][0], S[0][1]);
        pf[1] = pack_bf16(S[0][2], S[0][3]);
        pf[2] = pack_bf16(S[1][0], S[1][1]);
        pf[3] = pack_bf16(S[1][2], S[1][3]);
        // O^T tile t covers dv = 8*r + t (r = 0..15): lane's V chunk is dv 8*r16..8*r16+7
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const uint32_t sel = (t & 1) ? 0x07060302u : 0x05040100u;
            u32x4 vt;
#pragma unroll
            for (int u = 0; u < 4; ++u)
                vt[u] = __builtin_amdgcn_perm(bf.v[2 * u + 1][t >> 1], bf.v[2 * u][t >> 1], sel);
            O[t] = mfma16(vt, pf, O[t]);
        }
    };

    {
        StepBuf A, B;
        int j0 = kbeg;
        if (j0 < kend) load(A, j0);
        while (j0 < kend) {
            int j1 = j0 + 32;
            if (j1 < kend) load(B, j1);
            compute(A, j0);
            j0 = j1;
            if (j0 >= kend) break;
            j1 = j0 + 32;
            if (j1 < kend) load(A, j1);
            compute(B, j0);
            j0 = j1;
        }
    }

    // ---- this wave's partial for its heads: lane (lg, r16) holds, for each i,
    // dv [32*lg + 8*i, +8) of head r16 in O[0..7][i]
    l_run = sum_xor16(l_run);
    l_run = sum_xor32(l_run);
    if (!head_ok) return;
    if (nsplit <= 1) {
        const float inv = l_run > 0.0f ? a.v_scale / l_run : 0.0f;
        uint16_t *dst = a.out + ((size_t)s * a.Hq + head) * kDv + 32 * lg;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            u32x4 r;
#pragma unroll
            for (int e = 0; e < 4; ++e) r[e] = pack_bf16(O[2 * e][i] * inv, O[2 * e + 1][i] * inv);
            stg128(dst + 8 * i, r);
        }
    } else {
        const size_t part = ((size_t)s * a.Hq + head) * a.n_split_max + sp;
        float *dst = a.ws_o + part * kDv + 32 * lg;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f32x4 lo = {O[0][i], O[1][i], O[2][i], O[3][i]};
            f32x4 hi = {O[4][i], O[5][i], O[6][i], O[7][i]};
            *reinterpret_cast<f32x4 *>(dst + 8 * i) = lo;
            *reinterpret_cast<f32x4 *>(dst + 8 * i + 4) = hi;
        }
        if (lg == 0) {
            a.ws_ml[2 * part] = m_run;
            a.ws_ml[2 * part + 1] = l_run;
        }
    }
}

// One workgroup of 128 threads (one per dv) per (sequence, query head).
__global__ __launch_bounds__(128) void decode_combine_kernel(DecodeArgs a) {
    __shared__ float wsc[kDecodeMaxSplits];
    __shared__ float red[2][4];
    const int s = blockIdx.x / a.Hq;
    const int qh = blockIdx.x - s * a.Hq;
    const int n = live_slots(a.pos[s], a.cap);
    const int nsplit = (n + kDecodeChunk - 1) / kDecodeChunk;
    if (nsplit <= 1) return;
    const size_t part0 = ((size_t)s * a.Hq + qh) * a.n_split_max;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    // 1) max over the chunk maxima
    float M = kNegInf;
    for (int i = tid; i < nsplit; i += 128) M = fmaxf(M, a.ws_ml[2 * (part0 + i)]);
    for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    if (lane == 0) red[0][w] = M;
    __syncthreads();
    M = fmaxf(red[0][0], red[0][1]);
    // 2) chunk weights and the total sum
    float L = 0.0f;
    for (int i = tid; i < nsplit; i += 128) {
        const float mi = a.ws_ml[2 * (part0 + i)];
        const float sc = (mi == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f(mi - M);
        wsc[i] = sc;
        L += a.ws_ml[2 * (part0 + i) + 1] * sc;
    }
    for (int o = 32; o > 0; o >>= 1) L += __shfl_xor(L, o);
    if (lane == 0) red[1][w] = L;
    __syncthreads();
    L = red[1][0] + red[1][1];
    // 3) weighted sum of the partial outputs
    float o = 0.0f;
    const float *src = a.ws_o + part0 * kDv + tid;
    for (int i = 0; i < nsplit; ++i) o += src[(size_t)i * kDv] * wsc[i];
    const float r = L > 0.0f ? o * (a.v_scale / L) : 0.0f;
    const uint32_t pk = pack_bf16(r, 0.0f);
    a.out[((size_t)s * a.Hq + qh) * kDv + tid] = (uint16_t)(pk & 0xffffu);
}

size_t decode_workspace_bytes(int32_t S, int32_t Hq, int32_t cap) {
    const int64_t nsm = ((int64_t)cap + kDecodeChunk - 1) / kDecodeChunk;
    if (nsm <= 1) return 0;
    return (size_t)S * Hq * nsm * (kDv + 2) * sizeof(float);
}

hipError_t launch_decode(DecodeArgs a, hipStream_t stream) {
    a.n_split_max = (int)(((int64_t)a.cap + kDecodeChunk - 1) / kDecodeChunk);
    if (a.n_split_max > kDecodeMaxSplits) return hipErrorInvalidValue;
    if (a.n_split_max > 1) a.ws_ml = a.ws_o + (size_t)a.S * a.Hq * a.n_split_max * kDv;
    hipLaunchKernelGGL(decode_partial_kernel, dim3(a.n_split_max, a.S), dim3(64 * a.Hkv), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.n_split_max <= 1) return e;
    hipLaunchKernelGGL(decode_combine_kernel, dim3(a.S * a.Hq), dim3(kDv), 0, stream, a);
    return hipGetLastError();
}

}  // namespace mimo
