// Decode attention: one query token per sequence over a KV cache, for both
// layer types (sliding layers over their window-sized ring, Gaudi recipe page,
// Launch section; global layers over a long cache).  Split-K flash decoding
// with the whole batch's work split evenly over the GPU:
//
//   plan (decode_plan_kernel, one workgroup): each sequence's live slots are
//     cut into 32-slot steps; prefix sums over the sequences put every step of
//     the batch on one line, which is cut into equal contiguous ranges, one per
//     workgroup of the next pass.  Per sequence it records the first workgroup
//     on it, how many workgroups share it and where their partials go.
//   pass 1 (decode_partial_kernel): each workgroup walks its range, which may
//     end one sequence and start the next, with one wave per KV head.  Per
//     step a wave computes S^T = K Q^T for its GQA group's query heads (<= 16,
//     the N side of a 16x16x32 bf16 MFMA) and O^T += V^T P^T.  K is read
//     straight from HBM in operand layout: the contraction order over the 192
//     dims is chosen so that the 4 lanes of a key row read 64 contiguous bytes
//     per load and consecutive loads finish each 128-byte line; V is read
//     row-major and transposed in registers with byte permutes.  The next
//     step's loads are in flight during the current step's math.  A sequence
//     held by one workgroup gets its output written here; otherwise each piece
//     writes its (max, sum, O) partial.
//   pass 2 (decode_combine_kernel): merges a sequence's partials by their
//     log-sum-exp, and writes zeros for a sequence that sees no slot.
//
// The sink logit (techniques map page, Learnable attention sink) is folded into
// the piece holding a sequence's first step as the initial (max, sum) =
// (sink * log2 e, 1).
#include <atomic>
#include <mutex>

#include "kernels.hpp"

namespace mimo {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();
constexpr int kStep = 32;              // cache slots per step
constexpr int kPlanThreads = 1024;
constexpr int kMaxGroups = kDecodeWaves;   // workgroups of one wave when Hkv = 1
// Steps whose loads are in flight per wave: the computed one and the next; fp8
// steps are half the bytes, so one-token fp8 decode keeps three in flight to
// cover the same HBM latency.
constexpr int kDepth = 2;
constexpr int kFp8Depth = 3;

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// The logical key slots [lo, hi) a sequence whose newest query sits at p reads.
// Per-sequence caches: slot = position mod cap, slots 0 .. min(p+1, cap) - 1.
// Paged caches: slot = position; with a window only the 32-aligned range from
// the oldest query's window start on (earlier blocks may be released).
__device__ __forceinline__ void key_range(const DecodeArgs &a, int64_t p, int &lo, int &hi) {
    lo = 0;
    hi = 0;
    if (p < 0) return;
    if (a.table) {
        const int64_t end = (int64_t)a.max_blocks << a.block_shift;
        hi = (int)(p + 1 < end ? p + 1 : end);
        if (a.window > 0) {
            const int64_t first = p - (a.n_q - 1) - a.window + 1;
            lo = first > 0 ? (int)(first & ~(int64_t)(kStep - 1)) : 0;
        }
    } else {
        hi = p + 1 < a.cap ? (int)(p + 1) : a.cap;
    }
}

__device__ __forceinline__ int64_t steps_of(const DecodeArgs &a, int64_t p) {
    int lo, hi;
    key_range(a, p, lo, hi);
    return (hi - lo + kStep - 1) / kStep;
}

// 8 fp8 e4m3 codes (two dwords, code e in byte e) -> 8 bf16, two codes per
// v_cvt_scalef32_pk_bf16_fp8 at scale 1 (exact: every e4m3 value is a bf16 value;
// checked on all 256 codes against the format's definition)
__device__ __forceinline__ u32x4 fp8x8_to_bf16(uint32_t w0, uint32_t w1) {
    u32x4 r;
    r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false));
    r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true));
    r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false));
    r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true));
    return r;
}

// Workgroups used for Ts steps: at most n_groups, each with >= kDecodeMinSteps
// steps, so every workgroup below the result has a non-empty range.
__device__ __forceinline__ int64_t groups_used(int64_t Ts, int32_t n_groups) {
    const int64_t by_steps = (Ts + kDecodeMinSteps - 1) / kDecodeMinSteps;
    return by_steps < n_groups ? by_steps : n_groups;
}

// Workgroup w takes steps [floor(w*Ts/ng), floor((w+1)*Ts/ng)); this is the
// w whose range holds step x.
__device__ __forceinline__ int64_t step_owner(int64_t x, int64_t Ts, int64_t ng) {
    return ((x + 1) * ng - 1) / Ts;
}

// Inclusive prefix sum over one value per thread of a kPlanThreads block
// (wave scans, then the wave totals); also returns the block total.
template <typename T>
__device__ T block_scan(T v, T *wsum, T &total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const T u = __shfl_up(v, off);
        if (lane >= off) v += u;
    }
    if (lane == 63) wsum[w] = v;
    __syncthreads();
    T before = 0, all = 0;
#pragma unroll
    for (int i = 0; i < kPlanThreads / 64; ++i) {
        const T x = wsum[i];
        before += i < w ? x : T(0);
        all += x;
    }
    total = all;
    return v + before;
}

// One step's K/V registers of a lane.  bf16: k[sb][ch] holds dims 32*ch + 8*lg
// .. +8 of key row 16*sb + r16; v[jj] 8 dv of a key row.  fp8: k[sb][c] holds
// 16 codes, dims 16*(lg + 4*c) .. +16 (two MFMA chunks); v[jj] 8 codes.
template <bool FP8> struct StepBuf;
template <> struct StepBuf<false> {
    u32x4 k[2][6];
    u32x4 v[8];
};
template <> struct StepBuf<true> {
    u32x4 k[2][3];
    u32x2 v[8];
};

}  // namespace

// One workgroup; thread t plans a contiguous run of sequences, then the
// starting sequence of workgroups t and t + kPlanThreads, ...
__global__ __launch_bounds__(kPlanThreads) void decode_plan_kernel(DecodeArgs a) {
    __shared__ int64_t run_end[kPlanThreads];
    __shared__ int64_t wsum64[kPlanThreads / 64];
    __shared__ int32_t wsum32[kPlanThreads / 64];
    const int t = threadIdx.x;
    const int per = (a.S + kPlanThreads - 1) / kPlanThreads;
    const int s0 = min(a.S, t * per), s1 = min(a.S, s0 + per);
    int64_t mine = 0;
    for (int s = s0; s < s1; ++s) mine += steps_of(a, a.pos[s]);
    int64_t Ts;
    const int64_t incl = block_scan<int64_t>(mine, wsum64, Ts);
    run_end[t] = incl;
    const int64_t ng = groups_used(Ts, a.n_groups);
    int64_t start = incl - mine;
    int32_t parts = 0;
    for (int s = s0; s < s1; ++s) {
        const int64_t steps = steps_of(a, a.pos[s]);
        int32_t first = 0, cover = 0;
        if (steps > 0) {
            first = (int32_t)step_owner(start, Ts, ng);
            cover = (int32_t)step_owner(start + steps - 1, Ts, ng) - first + 1;
        }
        a.plan_start[s] = start;
        a.plan_first[s] = first;
        a.plan_cover[s] = cover;
        parts += cover > 1 ? cover : 0;
        start += steps;
    }
    if (t == kPlanThreads - 1) a.plan_start[a.S] = Ts;
    int32_t ptot;
    const int32_t pincl = block_scan<int32_t>(parts, wsum32, ptot);
    int32_t base = pincl - parts;
    for (int s = s0; s < s1; ++s) {
        a.plan_part[s] = base;
        const int32_t cover = a.plan_cover[s];
        base += cover > 1 ? cover : 0;
    }
    // the sequence holding each workgroup's first step: the thread run whose
    // steps reach it (LDS), then the last sequence of that run starting at or
    // before it (this block's plan_start writes, visible after the barrier)
    __syncthreads();
    for (int64_t w = t; w < ng; w += kPlanThreads) {
        const int64_t x = w * Ts / ng;
        int lo = 0, hi = kPlanThreads - 1;   // first run with run_end > x
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (run_end[mid] > x) hi = mid;
            else lo = mid + 1;
        }
        int sl = min(a.S - 1, lo * per), sh = min(a.S, lo * per + per) - 1;
        while (sl < sh) {
            const int mid = (sl + sh + 1) >> 1;
            if (a.plan_start[mid] <= x) sl = mid;
            else sh = mid - 1;
        }
        a.plan_wg_seq[w] = sl;
    }
}

// NC column tiles of 16 (query token, query head) pairs per wave, which all
// use the K/V rows the wave loads once per step; more tiles go to more waves
// of the same KV head.  MAXT: workgroup size bound (512: eight KV-head waves,
// two per SIMD; 256: up to four waves, one per SIMD with the whole register
// file, for the tiles of multi-query decode).
template <int NC, int MAXT, bool FP8, bool PAGED, int DEPTH, int SW = 0>
__global__ __attribute__((amdgpu_flat_work_group_size(64, MAXT), amdgpu_waves_per_eu(MAXT / 256, MAXT / 256)))
void decode_partial_kernel(DecodeArgs a) {
    // SW > 0: the workgroup is the SW waves of one KV head; each step's K/V rows
    // are read from HBM once, by all of them, staged in LDS and read from there
    constexpr int kKRowB = FP8 ? kDqk : 2 * kDqk;        // bytes of one K / V row
    constexpr int kVRowB = FP8 ? kDv : 2 * kDv;
    constexpr int kStepB = kStep * (kKRowB + kVRowB);
    __shared__ __attribute__((aligned(16))) uint8_t sring[SW > 0 ? 2 * kStepB : 16];
    const int64_t wg = blockIdx.x;
    // step range of the workgroup: its share of the planned line, or (direct) the
    // whole of sequence blockIdx.x
    int lo, s_end;
    int64_t r_lo, r_hi;
    if (a.direct) {
        lo = (int)wg;
        s_end = lo + 1;
        r_lo = 0;
        r_hi = INT64_MAX;
    } else {
        const int64_t Ts = a.plan_start[a.S];
        lo = a.plan_wg_seq[wg];   // meaningful only below the groups used
        const int64_t ng = groups_used(Ts, a.n_groups);
        if (wg >= ng) return;
        r_lo = wg * Ts / ng;
        r_hi = (wg + 1) * Ts / ng;
        s_end = a.S;
    }

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int gl = w / a.wph, sub = w - gl * a.wph;
    const int g = blockIdx.y * a.kvpw + gl;            // this wave's KV head
    const int lg = lane >> 4, r16 = lane & 15;
    const int G = a.Hq / a.Hkv;
    const int nq = a.n_q;
    // column r16 of tile t is (query token tok, query head hd): col = G * tok + head in group
    int tok[NC], hd[NC];
    bool ok[NC];
#pragma unroll
    for (int t = 0; t < NC; ++t) {
        const int col = 16 * (NC * sub + t) + r16;
        tok[t] = col / G;
        hd[t] = g * G + (col - tok[t] * G);
        ok[t] = tok[t] < nq;
    }
    const float cl2 = a.scale_log2;
    // row strides of the caches in elements (bf16) or bytes (fp8): one element each
    const size_t krs = (size_t)a.Hkv * kDqk, vrs = (size_t)a.Hkv * kDv;
    const int win = a.window > 0 ? a.window : 0x7fffffff;
    constexpr bool paged = PAGED;
    const int bmask = (1 << a.block_shift) - 1;
    using Buf = StepBuf<FP8>;
    // per-lane bases: K dims of the contraction slots, V dv chunk of the lane
    const uint16_t *k16 = static_cast<const uint16_t *>(a.k_cache) + (size_t)g * kDqk + 8 * lg;
    const uint16_t *v16 = static_cast<const uint16_t *>(a.v_cache) + (size_t)g * kDv + 8 * r16;
    const uint8_t *k8 = static_cast<const uint8_t *>(a.k_cache) + (size_t)g * kDqk + 16 * lg;
    const uint8_t *v8 = static_cast<const uint8_t *>(a.v_cache) + (size_t)g * kDv + 8 * r16;

    for (int s = lo; s < s_end; ++s) {
        int64_t st0 = 0, st1;
        if (a.direct) {
            // a sequence without slots still gets its (zero) output written below
            st1 = a.pos[s] >= 0 ? steps_of(a, a.pos[s]) : 0;
        } else {
            st0 = a.plan_start[s];
            if (st0 >= r_hi) break;
            st1 = a.plan_start[s + 1];
        }
        const int64_t seg_lo = st0 > r_lo ? st0 : r_lo;
        const int64_t seg_hi = st1 < r_hi ? st1 : r_hi;
        if (seg_lo >= seg_hi && !a.direct) continue;

        const int64_t p = a.pos[s];   // newest query's position (>= 0: the sequence has steps)
        int jlo, n;
        key_range(a, p, jlo, n);      // logical slots [jlo, n)

        u32x4 qf[NC][6];
        float m_run[NC], l_run[NC];
        f32x4 O[NC][8];

        const int kbeg = jlo + (int)(seg_lo - st0) * kStep;
        const int kseg = jlo + (int)(seg_hi - st0) * kStep;
        const int kend = kseg < n ? kseg : n;
        // ring rule: slot j holds position p - ((p - j) mod cap); with pm = p mod cap
        // that distance is pm - j, or pm - j + cap when j > pm.  Paged: slot j is position j.
        const int pm = paged ? 0 : (int)(p % a.cap);
        const size_t seq_rows = paged ? 0 : (size_t)s * a.cap;
        const int32_t *btab = paged ? a.table + (size_t)s * a.max_blocks : nullptr;

        // physical cache row of slot j: per-sequence caches re-read their last row
        // for slots past the end (last step of a full cache); a paged step lies in
        // one block.  Every slot at or past n is masked out of the step anyway.
        auto load = [&](Buf &bf, int j0) {
            size_t blk_row = 0;
            if constexpr (PAGED) {
                int blk = btab[j0 >> a.block_shift];
                blk = blk < 0 ? 0 : (blk >= a.n_blocks ? a.n_blocks - 1 : blk);
                blk_row = (size_t)blk << a.block_shift;
            }
            auto row = [&](int j) -> size_t {
                return paged ? blk_row + (size_t)(j & bmask) : seq_rows + (size_t)min(j, a.cap - 1);
            };
#pragma unroll
            for (int sb = 0; sb < 2; ++sb) {
                const size_t r = row(j0 + 16 * sb + r16);
                if constexpr (FP8) {
#pragma unroll
                    for (int c = 0; c < 3; ++c) bf.k[sb][c] = *reinterpret_cast<const u32x4 *>(k8 + r * krs + 64 * c);
                } else {
#pragma unroll
                    for (int ch = 0; ch < 6; ++ch) bf.k[sb][ch] = ldg128(k16 + r * krs + 32 * ch);
                }
            }
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                const size_t r = row(j0 + 16 * (jj >> 2) + 4 * lg + (jj & 3));
                if constexpr (FP8) bf.v[jj] = *reinterpret_cast<const u32x2 *>(v8 + r * vrs);
                else bf.v[jj] = ldg128(v16 + r * vrs);
            }
        };

        auto compute = [&](Buf &bf, int j0) {
            // the lane's 8 keys are j0 + 16*sb + 4*lg + i (rows of its S^T registers and
            // of its V loads); d = how many positions each lies before the newest query
            // unmasked: a global layer's step wholly inside this piece, before the
            // newest n_q - 1 positions, in a cache whose slot j holds position j
            const bool masked = a.window > 0 || j0 + kStep > kend ||
                                (nq > 1 && (!(paged || p < a.cap) || (int64_t)j0 + kStep > p - nq + 2));
            // K operands in bf16 (fp8 codes widened once per step)
            u32x4 kop8[2][FP8 ? 6 : 1];
            if constexpr (FP8) {
#pragma unroll
                for (int sb = 0; sb < 2; ++sb)
#pragma unroll
                    for (int ch = 0; ch < 6; ++ch) {
                        const u32x4 wv = bf.k[sb][ch >> 1];
                        kop8[sb][ch] = (ch & 1) ? fp8x8_to_bf16(wv[2], wv[3]) : fp8x8_to_bf16(wv[0], wv[1]);
                    }
            }
            auto kop = [&](int sb, int ch) -> u32x4 {
                if constexpr (FP8) return kop8[sb][ch];
                else return bf.k[sb][ch];
            };
            u32x4 pf[NC];
#pragma unroll
            for (int t = 0; t < NC; ++t) {
                f32x4 S[2];
#pragma unroll
                for (int sb = 0; sb < 2; ++sb) {
                    S[sb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ch = 0; ch < 6; ++ch) S[sb] = mfma16(kop(sb, ch), qf[t][ch], S[sb]);
                }
                if (masked) {
                    const int delta = nq - 1 - tok[t];   // the column's query lies delta before the newest
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int j = j0 + 16 * (e >> 2) + 4 * lg + (e & 3);
                        int d;
                        if constexpr (PAGED) {
                            d = (int)(p - j);
                        } else {
                            d = pm - j;
                            if (d < 0) d += a.cap;
                        }
                        const bool live = j < n && (int64_t)d <= p;
                        const int dd = d - delta;
                        if (!(live && dd >= 0 && dd < win)) S[e >> 2][e & 3] = kNegInf;
                        // no query of the sequence sees it: drop its value row (it may hold NaN)
                        if (t == 0 && !(live && d - (nq - 1) < win)) {
                            if constexpr (FP8) bf.v[e] = u32x2{0, 0};
                            else bf.v[e] = u32x4{0, 0, 0, 0};
                        }
                    }
                }
                float mx = fmaxf(fmaxf(fmaxf(S[0][0], S[0][1]), fmaxf(S[0][2], S[0][3])),
                                 fmaxf(fmaxf(S[1][0], S[1][1]), fmaxf(S[1][2], S[1][3])));
                mx = max_xor16(mx);
                mx = max_xor32(mx);
                const float mc = mx * cl2;
                const bool need = mc > m_run[t] + 8.0f;
                if (__any(need)) {
                    const float alpha = need ? __builtin_amdgcn_exp2f(m_run[t] - mc) : 1.0f;
                    if (need) m_run[t] = mc;
                    l_run[t] *= alpha;
#pragma unroll
                    for (int tt = 0; tt < 8; ++tt) O[t][tt] *= alpha;
                }
                const float mu = (m_run[t] == kNegInf) ? 0.0f : m_run[t];
                float ls = 0.0f;
#pragma unroll
                for (int sb = 0; sb < 2; ++sb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(S[sb][i], cl2, -mu));
                        S[sb][i] = pv;
                        ls += pv;
                    }
                l_run[t] += ls;
                pf[t][0] = pack_bf16(S[0][0], S[0][1]);
                pf[t][1] = pack_bf16(S[0][2], S[0][3]);
                pf[t][2] = pack_bf16(S[1][0], S[1][1]);
                pf[t][3] = pack_bf16(S[1][2], S[1][3]);
            }
            u32x4 vr8[FP8 ? 8 : 1];
            if constexpr (FP8) {
#pragma unroll
                for (int e = 0; e < 8; ++e) vr8[e] = fp8x8_to_bf16(bf.v[e][0], bf.v[e][1]);
            }
            auto vr = [&](int e) -> u32x4 {
                if constexpr (FP8) return vr8[e];
                else return bf.v[e];
            };
            // O^T tile tt covers dv = 8*r + tt (r = 0..15): lane's V chunk is dv 8*r16..8*r16+7
#pragma unroll
            for (int tt = 0; tt < 8; ++tt) {
                const uint32_t sel = (tt & 1) ? 0x07060302u : 0x05040100u;
                u32x4 vt;
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    vt[u] = __builtin_amdgcn_perm(vr(2 * u + 1)[tt >> 1], vr(2 * u)[tt >> 1], sel);
#pragma unroll
                for (int t = 0; t < NC; ++t) O[t][tt] = mfma16(vt, pf[t], O[t][tt]);
            }
        };

        auto init_q = [&]() {
            // ---- q (B operand) of each tile, in the contraction order of the K operand:
            // bf16: slot (ch, lg, e) is dim 32*ch + 8*lg + e, so chunks 0 and 1 of a lane
            // are rotate-half partners (dims i and i+32); fp8: slot (ch = 2c+h, lg, e) is
            // dim 16*(lg + 4*c) + 8*h + e, and the partner of chunk h of c = 0 sits two
            // lanes over, so it is read from memory as well
#pragma unroll
            for (int t = 0; t < NC; ++t) {
                if (ok[t]) {
                    const int64_t qp = p - (nq - 1 - tok[t]);
                    const uint16_t *qrow = a.q + (((size_t)s * nq + tok[t]) * a.Hq + hd[t]) * kDqk;
                    if constexpr (FP8) {
#pragma unroll
                        for (int c = 0; c < 3; ++c)
#pragma unroll
                            for (int h = 0; h < 2; ++h) qf[t][2 * c + h] = ldg128(qrow + 16 * (lg + 4 * c) + 8 * h);
                        const int pl = lg < 2 ? lg + 2 : lg - 2;
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            const u32x4 own = qf[t][h], partner = ldg128(qrow + 16 * pl + 8 * h);
                            u32x4 x = lg < 2 ? own : partner, y = lg < 2 ? partner : own;
                            rope_rotate8(x, y, a.rt, 16 * (lg & 1) + 8 * h, qp);
                            qf[t][h] = lg < 2 ? x : y;
                        }
                    } else {
#pragma unroll
                        for (int ch = 0; ch < 6; ++ch) qf[t][ch] = ldg128(qrow + 8 * lg + 32 * ch);
                        rope_rotate8(qf[t][0], qf[t][1], a.rt, 8 * lg, qp);
                    }
                } else {
#pragma unroll
                    for (int ch = 0; ch < 6; ++ch) qf[t][ch] = u32x4{0, 0, 0, 0};
                }
                if (seg_lo == st0 && a.sinks && ok[t]) {
                    m_run[t] = a.sinks[hd[t]] * kLog2e;
                    l_run[t] = (lg == 0) ? 1.0f : 0.0f;
                } else {
                    m_run[t] = kNegInf;
                    l_run[t] = 0.0f;
                }
#pragma unroll
                for (int tt = 0; tt < 8; ++tt) O[t][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        };

        if constexpr (SW > 0) {
            // Staging: per step, 32 K rows and 32 V rows cut into 16-byte (bf16) or
            // 8-byte (fp8) chunks, 768 of K and 512 of V, spread evenly over the
            // workgroup; each thread holds its chunks of the next RS steps in
            // registers, so RS steps per KV head are in flight from HBM.
            constexpr int NT = 64 * SW;
            constexpr int KCH = 768, TOT = 1280, PER = TOT / NT, KPER = KCH / NT;
            static_assert(TOT % NT == 0 && KCH % NT == 0, "chunk split");
            constexpr int CB = FP8 ? 8 : 16;
            constexpr int RS = SW == 2 ? 2 : 3;
            using Chunk = typename std::conditional<FP8, u32x2, u32x4>::type;
            const int tid = threadIdx.x;
            const uint8_t *kb8 = static_cast<const uint8_t *>(a.k_cache) + (size_t)g * kKRowB;
            const uint8_t *vb8 = static_cast<const uint8_t *>(a.v_cache) + (size_t)g * kVRowB;
            const size_t krb = (size_t)a.Hkv * kKRowB, vrb = (size_t)a.Hkv * kVRowB;
            Chunk rs[RS][PER];
            auto gload = [&](Chunk (&r)[PER], int j0) {
                size_t blk_row = 0;
                if constexpr (PAGED) {
                    int blk = btab[j0 >> a.block_shift];
                    blk = blk < 0 ? 0 : (blk >= a.n_blocks ? a.n_blocks - 1 : blk);
                    blk_row = (size_t)blk << a.block_shift;
                }
                auto row = [&](int j) -> size_t {
                    return paged ? blk_row + (size_t)(j & bmask) : seq_rows + (size_t)min(j, a.cap - 1);
                };
#pragma unroll
                for (int i = 0; i < PER; ++i) {
                    const int u = tid + i * NT;
                    if (i < KPER) r[i] = *reinterpret_cast<const Chunk *>(kb8 + row(j0 + u / 24) * krb + CB * (u % 24));
                    else r[i] = *reinterpret_cast<const Chunk *>(vb8 + row(j0 + (u - KCH) / 16) * vrb + CB * ((u - KCH) % 16));
                }
            };
            // LDS step image: K rows of kKRowB bytes, their 16-byte chunks XOR-swizzled
            // by row (conflict-free operand reads), then V rows of kVRowB bytes
            auto kslot = [](int row, int c16) {
                return FP8 ? row * kKRowB + 16 * (c16 ^ ((row >> 2) & 3)) : row * kKRowB + 16 * (c16 ^ ((row >> 1) & 7));
            };
            auto lstore = [&](const Chunk (&r)[PER], int buf) {
                uint8_t *base = sring + buf * kStepB;
#pragma unroll
                for (int i = 0; i < PER; ++i) {
                    const int u = tid + i * NT;
                    if (i < KPER) {
                        const int row = u / 24, c = u % 24;
                        const int off = FP8 ? kslot(row, c >> 1) + 8 * (c & 1) : kslot(row, c);
                        *reinterpret_cast<Chunk *>(base + off) = r[i];
                    } else {
                        const int row = (u - KCH) / 16, c = (u - KCH) % 16;
                        *reinterpret_cast<Chunk *>(base + kStep * kKRowB + row * kVRowB + CB * c) = r[i];
                    }
                }
            };
            // the operand registers of a step, as the per-wave loads would give them
            auto lfetch = [&](Buf &bf, int buf) {
                const uint8_t *base = sring + buf * kStepB;
#pragma unroll
                for (int sb = 0; sb < 2; ++sb) {
                    const int row = 16 * sb + r16;
#pragma unroll
                    for (int ch = 0; ch < (FP8 ? 3 : 6); ++ch)
                        bf.k[sb][ch] = *reinterpret_cast<const u32x4 *>(base + kslot(row, 4 * ch + lg));
                }
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) {
                    const int row = 16 * (jj >> 2) + 4 * lg + (jj & 3);
                    bf.v[jj] = *reinterpret_cast<const std::remove_reference_t<decltype(bf.v[0])> *>(base + kStep * kKRowB + row * kVRowB + CB * r16);
                }
            };
            // (loads past the last step re-read the last step, and their stores land in
            // a buffer nobody reads: no load sits under a data-dependent branch, which
            // keeps the compiler's memory waits per register set)
            const int nsteps = (kend - kbeg + kStep - 1) / kStep;   // >= 1
            auto step_j0 = [&](int i) { return kbeg + min(i, nsteps - 1) * kStep; };
            gload(rs[0], step_j0(0));   // first step's loads go out before q's
            init_q();
#pragma unroll
            for (int i = 1; i < RS; ++i) gload(rs[i], step_j0(i));
            lstore(rs[0], 0);
            gload(rs[0], step_j0(RS));
            __syncthreads();
            // step i: computed from LDS buffer i & 1; its successor is stored to the
            // other buffer from register set (i + 1) % RS, which then loads step i + 1 + RS
            auto phase = [&](int i, int ph) {
                Buf bf;
                lfetch(bf, i & 1);
                compute(bf, kbeg + i * kStep);
                lstore(rs[(ph + 1) % RS], (i + 1) & 1);
                gload(rs[(ph + 1) % RS], step_j0(i + 1 + RS));
                __syncthreads();
            };
            // whole rounds of RS steps without branches around the loads, then the rest
            int i0 = 0;
            for (; i0 + RS <= nsteps; i0 += RS) {
#pragma unroll
                for (int ph = 0; ph < RS; ++ph) phase(i0 + ph, ph);
            }
#pragma unroll
            for (int ph = 0; ph < RS - 1; ++ph)
                if (i0 + ph < nsteps) phase(i0 + ph, ph);
        } else {
            // Loads are unconditional: a step past the last re-reads the last one (in
            // bounds, never computed). A load under a data-dependent branch made the
            // compiler wait for every load in flight, the next step's included.
            const int klast = kend > kbeg ? kbeg + (kend - kbeg - 1) / kStep * kStep : kbeg;
            auto lstep = [&](int j) { return j < klast ? j : klast; };
            Buf A, B;
            int j0 = kbeg;
            load(A, j0);   // first step's loads go out before q's
            init_q();
            if constexpr (DEPTH == 3) {
                // three steps' loads in flight: the one computed and the next two
                Buf C;
                load(B, lstep(j0 + kStep));
                while (j0 < kend) {
                    load(C, lstep(j0 + 2 * kStep));
                    compute(A, j0);
                    j0 += kStep;
                    if (j0 >= kend) break;
                    load(A, lstep(j0 + 2 * kStep));
                    compute(B, j0);
                    j0 += kStep;
                    if (j0 >= kend) break;
                    load(B, lstep(j0 + 2 * kStep));
                    compute(C, j0);
                    j0 += kStep;
                }
            } else {
                while (j0 < kend) {
                    load(B, lstep(j0 + kStep));
                    compute(A, j0);
                    j0 += kStep;
                    if (j0 >= kend) break;
                    load(A, lstep(j0 + kStep));
                    compute(B, j0);
                    j0 += kStep;
                }
            }
        }

        // ---- this piece: lane (lg, r16) holds, for each i, dv [32*lg + 8*i, +8) of
        // its column in O[t][0..7][i]
        const int cover = a.direct ? 1 : a.plan_cover[s];
#pragma unroll
        for (int t = 0; t < NC; ++t) {
            float lt = sum_xor16(l_run[t]);
            lt = sum_xor32(lt);
            if (!ok[t]) continue;
            const size_t row = ((size_t)s * nq + tok[t]) * a.Hq + hd[t];
            if (cover == 1) {
                const float inv = lt > 0.0f ? a.v_scale / lt : 0.0f;
                uint16_t *dst = a.out + row * kDv + 32 * lg;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    u32x4 r;
#pragma unroll
                    for (int e = 0; e < 4; ++e) r[e] = pack_bf16(O[t][2 * e][i] * inv, O[t][2 * e + 1][i] * inv);
                    stg128(dst + 8 * i, r);
                }
            } else {
                const size_t part = (size_t)(a.plan_part[s] + (int32_t)(wg - a.plan_first[s]));
                const size_t idx = (part * nq + tok[t]) * a.Hq + hd[t];
                float *dst = a.ws_o + idx * kDv + 32 * lg;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const f32x4 lo4 = {O[t][0][i], O[t][1][i], O[t][2][i], O[t][3][i]};
                    const f32x4 hi4 = {O[t][4][i], O[t][5][i], O[t][6][i], O[t][7][i]};
                    *reinterpret_cast<f32x4 *>(dst + 8 * i) = lo4;
                    *reinterpret_cast<f32x4 *>(dst + 8 * i + 4) = hi4;
                }
                if (lg == 0) {
                    a.ws_ml[2 * idx] = m_run[t];
                    a.ws_ml[2 * idx + 1] = lt;
                }
            }
        }
    }
}

// One workgroup of 128 threads (one per dv) per (sequence, query token, query head).
__global__ __launch_bounds__(128) void decode_combine_kernel(DecodeArgs a) {
    __shared__ float wsc[kMaxGroups];
    __shared__ float red[2][2];
    const int rows = a.n_q * a.Hq;                  // output rows of one sequence
    const int s = blockIdx.x / rows;
    const int rr = blockIdx.x - s * rows;           // token * Hq + head
    const int cover = a.plan_cover[s];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    uint16_t *dst = a.out + (size_t)blockIdx.x * kDv + tid;
    if (cover == 0) {   // no visible slot: zero output (the sink carries no value)
        *dst = 0;
        return;
    }
    if (cover == 1) return;
    const size_t part0 = (size_t)a.plan_part[s];
    // 1) max over the pieces' maxima
    float M = kNegInf;
    for (int i = tid; i < cover; i += 128) M = fmaxf(M, a.ws_ml[2 * ((part0 + i) * rows + rr)]);
    for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    if (lane == 0) red[0][w] = M;
    __syncthreads();
    M = fmaxf(red[0][0], red[0][1]);
    // 2) piece weights and the total sum
    float L = 0.0f;
    for (int i = tid; i < cover; i += 128) {
        const size_t pi = (part0 + i) * rows + rr;
        const float mi = a.ws_ml[2 * pi];
        const float sc = (mi == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f(mi - M);
        wsc[i] = sc;
        L += a.ws_ml[2 * pi + 1] * sc;
    }
    for (int o = 32; o > 0; o >>= 1) L += __shfl_xor(L, o);
    if (lane == 0) red[1][w] = L;
    __syncthreads();
    L = red[1][0] + red[1][1];
    // 3) weighted sum of the partial outputs
    const float *src = a.ws_o + (part0 * rows + rr) * kDv + tid;
    const size_t stride = (size_t)rows * kDv;
    float o = 0.0f;
#pragma unroll 8
    for (int i = 0; i < cover; ++i) o += src[i * stride] * wsc[i];
    const float r = L > 0.0f ? o * (a.v_scale / L) : 0.0f;
    *dst = (uint16_t)(pack_bf16(r, 0.0f) & 0xffffu);
}

DecodeGeom decode_geometry(int32_t Hq, int32_t Hkv, int32_t n_q) {
    DecodeGeom m{};
    const int G = Hq / Hkv;
    const int tiles = (G * n_q + 15) / 16;
    if (n_q == 1) {   // one tile per wave, one wave per KV head
        // at most 4 KV heads (waves) per workgroup, so every workgroup runs one wave
        // per SIMD and the step ranges cover all CUs (8 KV heads in one workgroup
        // left half the CUs idle on sliding layers)
        m.nc = 1; m.wph = 1; m.kvpw = Hkv < 4 ? Hkv : 4;
        while (Hkv % m.kvpw) --m.kvpw;
    } else if (tiles <= 2) {   // up to 2 tiles per wave, at most four waves per workgroup
        m.wph = (tiles + 1) / 2;
        m.nc = (tiles + m.wph - 1) / m.wph;
        m.kvpw = m.wph >= 4 ? 1 : 4 / m.wph;
        while (Hkv % m.kvpw) --m.kvpw;
    } else {          // 2 tiles per wave; the 2 or 4 waves of a KV head share its steps through LDS
        m.nc = 2;
        m.wph = tiles <= 4 ? 2 : 4;
        m.kvpw = 1;
    }
    m.n_hsub = Hkv / m.kvpw;
    m.threads = 64 * m.kvpw * m.wph;
    m.n_groups = kDecodeWaves / (Hkv * m.wph);
    if (m.n_groups < 1) m.n_groups = 1;
    return m;
}

namespace {

// partials: every sequence shared by several workgroups has one piece per
// workgroup on it, and the pieces of all sequences number < groups + S
size_t decode_partial_slots(int32_t S, const DecodeGeom &m) { return (size_t)m.n_groups + (size_t)S; }

template <int SW>
void launch_shared(const DecodeArgs &a, const DecodeGeom &m, hipStream_t stream) {
    const dim3 grid(m.n_groups, m.n_hsub), block(64 * SW);
    if (!a.table)
        hipLaunchKernelGGL((decode_partial_kernel<2, 256, false, false, 2, SW>), grid, block, 0, stream, a);
    else if (a.fp8)
        hipLaunchKernelGGL((decode_partial_kernel<2, 256, true, true, 2, SW>), grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((decode_partial_kernel<2, 256, false, true, 2, SW>), grid, block, 0, stream, a);
}

template <int NC, int MAXT, int DEPTH = kDepth>
void launch_partial(const DecodeArgs &a, const DecodeGeom &m, hipStream_t stream) {
    const dim3 grid(m.n_groups, m.n_hsub), block(m.threads);
    if (!a.table)
        hipLaunchKernelGGL((decode_partial_kernel<NC, MAXT, false, false, DEPTH>), grid, block, 0, stream, a);
    else if (a.fp8)
        hipLaunchKernelGGL((decode_partial_kernel<NC, MAXT, true, true, (NC == 1 ? kFp8Depth : DEPTH)>), grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((decode_partial_kernel<NC, MAXT, false, true, DEPTH>), grid, block, 0, stream, a);
}

}  // namespace

size_t decode_workspace_bytes(int32_t S, int32_t Hq, int32_t Hkv, int32_t n_q) {
    const DecodeGeom m = decode_geometry(Hq, Hkv, n_q);
    const size_t parts = decode_partial_slots(S, m) * (size_t)n_q * Hq * (kDv + 2) * sizeof(float);
    const size_t plan = (size_t)(S + 1) * sizeof(int64_t) + ((size_t)3 * S + m.n_groups) * sizeof(int32_t);
    return parts + plan;
}

// Direct mode: a cache whose sequences read at most kDirectMaxSteps steps (a
// sliding layer's ring, or a windowed paged cache) is walked one workgroup per
// (sequence, KV head), each writing its output itself: no plan, no partials, no
// combine.  Splitting such short sequences only added two launches and a merge.
constexpr int kDirectMaxSteps = 8;

static bool decode_direct(const DecodeArgs &a, const DecodeGeom &m) {
    if (m.wph != 1) return false;
    int64_t steps;
    if (a.table) {
        if (a.window <= 0) return false;
        steps = (a.window + a.n_q - 2 + kStep - 1) / kStep + 1;   // 32-aligned start of the oldest window
    } else {
        steps = (a.cap + kStep - 1) / kStep;
    }
    return steps <= kDirectMaxSteps;
}

hipError_t launch_decode(DecodeArgs a, hipStream_t stream) {
    if (a.Hkv < 1 || a.Hkv > 8 || a.n_q < 1 || a.Hq / a.Hkv * a.n_q > 128) return hipErrorInvalidValue;
    DecodeGeom m = decode_geometry(a.Hq, a.Hkv, a.n_q);
    if (decode_direct(a, m)) {
        if (a.S == 0) return hipSuccess;
        // one wave (one KV head) per workgroup: S * Hkv workgroups
        a.direct = 1;
        a.wph = 1;
        a.kvpw = 1;
        a.n_groups = a.S;
        m.kvpw = 1;
        m.n_hsub = a.Hkv;
        m.threads = 64;
        m.n_groups = a.S;
        if (m.nc == 1) launch_partial<1, 256>(a, m, stream);
        else launch_partial<2, 256>(a, m, stream);
        return hipGetLastError();
    }
    a.direct = 0;
    a.n_groups = m.n_groups;
    a.wph = m.wph;
    a.kvpw = m.kvpw;
    const size_t parts = decode_partial_slots(a.S, m);
    const size_t rows = (size_t)a.n_q * a.Hq;
    a.ws_ml = a.ws_o + parts * rows * kDv;
    a.plan_start = reinterpret_cast<int64_t *>(a.ws_ml + parts * rows * 2);
    a.plan_first = reinterpret_cast<int32_t *>(a.plan_start + a.S + 1);
    a.plan_cover = a.plan_first + a.S;
    a.plan_part = a.plan_cover + a.S;
    a.plan_wg_seq = a.plan_part + a.S;
    hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.n_q == 1) {
        launch_partial<1, 256>(a, m, stream);   // at most 4 KV heads: 256 threads
    }
    else if (m.wph == 2 && m.kvpw == 1) launch_shared<2>(a, m, stream);
    else if (m.wph == 4 && m.kvpw == 1) launch_shared<4>(a, m, stream);
    else if (m.nc == 1) launch_partial<1, 256>(a, m, stream);
    else launch_partial<2, 256>(a, m, stream);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(decode_combine_kernel, dim3((unsigned)(a.S * rows)), dim3(kDv), 0, stream, a);
    return hipGetLastError();
}

// ---- scratch of the allocation-free decode call
// One file-scope device array; every GPU the library runs on holds its own copy
// at its own address until the process ends (zero-initialised storage: it takes
// no space in the library file).  In host code the array's name is not a device
// address, so it is only ever used to look that address up.
static __device__ __align__(256) uint8_t scratch[kDecodeScratchBytes];

hipError_t decode_scratch(hipStream_t stream, void **ptr) {
    constexpr int kMaxDevices = 64;
    static std::atomic<void *> addr[kMaxDevices];
    static std::mutex mu;
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (stream) {
        hipDevice_t sdev = cur;
        e = hipStreamGetDevice(stream, &sdev);
        if (e != hipSuccess) return e;
        if (sdev != cur) return hipErrorInvalidDevice;
    }
    if (cur < 0 || cur >= kMaxDevices) return hipErrorInvalidDevice;
    void *p = addr[cur].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(mu);
        p = addr[cur].load(std::memory_order_relaxed);
        if (!p) {   // first call on this device, which is current
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (!p) return hipErrorInvalidSymbol;
            addr[cur].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return hipSuccess;
}

}  // namespace mimo
