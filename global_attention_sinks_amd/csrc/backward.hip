// Backward of prefill attention with a learned sink, for the trainer's path
// (miles MiMo-V2.6-Flash page, section 5.4: the sink is trained through the
// fused attention).  Given the forward's output O, its row log-sum-exp L
// (natural log, sink included) and the upstream gradient dO, with
// P = exp(c S - L), dP = v_scale dO V^T and D = rowsum(dO o O):
//   dS = P o (dP - D);  dQ~ = c dS K~;  dK~ = c dS^T Q~;  dV = v_scale P^T dO;
//   d sink_h = -sum over rows of exp(sink_h - L) D;
// and dq, dk are dQ~, dK~ turned back by the transpose of the partial RoPE
// rotation (the same angle, negated).
//
//   bwd_dq_kernel      query-major: a workgroup owns 32 queries x 4 heads of a
//                      GQA group; it forms D per (row, head) from O and dO and
//                      per head the sum of its rows' sink terms, then per 32-key
//                      tile (K rotated, K^T and V staged in LDS, shared by the 4
//                      heads) rebuilds S^T and dP^T and accumulates
//                      dQ~^T = K~^T dS^T in registers
//   bwd_sink_kernel    one workgroup per head sums the sink partials (fixed order)
//   bwd_dkdv_kernel    key-major: a workgroup owns 128 keys of one KV head (one
//                      wave per 32 keys, the keys' K~ and V held in registers);
//                      it walks every query head of the group and every 32-query
//                      block that sees its keys (Q~, Q~^T, dO, dO^T staged in
//                      LDS, double-buffered) and accumulates dK~^T = Q~^T dS
//                      and dV^T = dO^T P
// Both contractions reuse the forward's layout trick: the A-operand rows of the
// first product are read with bits 2 and 3 of the row index swapped, so each
// lane's accumulators are directly the B operand of the second product.  The
// dk/dv stages are written transposed straight from registers: a staging
// thread holds both rows of a row pair and stores each column pair as a dword.
// Nothing is accumulated across workgroups, so the results are deterministic.
#include "kernels.hpp"

namespace mimo {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kPosInf = __builtin_inff();
constexpr int RSTR = kDqk + 8;   // LDS row stride of a 192-dim tile (bf16)
constexpr int VSTR = kDv + 8;    // LDS row stride of a 128-dim tile
constexpr int TSTR = 32 + 8;     // LDS row stride of a transposed 32-column tile

__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

__device__ __forceinline__ u32x4 lds128(const uint16_t *p) { return *reinterpret_cast<const u32x4 *>(p); }

// Transpose a staged 32-row tile (row stride sstr, nch chunks of 8 columns) into
// dst[col][row] (row stride TSTR): each unit takes two rows x 8 columns and
// writes 8 dwords of two rows each.
__device__ __forceinline__ void transpose32(uint16_t *dst, const uint16_t *src, int sstr, int nch, int tid,
                                            int nthreads) {
    for (int u = tid; u < 16 * nch; u += nthreads) {
        const int rp = u % 16, c = u / 16;
        const u32x4 a = lds128(src + (2 * rp) * sstr + 8 * c);
        const u32x4 b = lds128(src + (2 * rp + 1) * sstr + 8 * c);
#pragma unroll
        for (int d = 0; d < 8; ++d) {
            const uint32_t sel = (d & 1) ? 0x07060302u : 0x05040100u;
            *reinterpret_cast<uint32_t *>(dst + (8 * c + d) * TSTR + 2 * rp) = __builtin_amdgcn_perm(b[d >> 1], a[d >> 1], sel);
        }
    }
}

// One 32-row stage held in registers between its global loads and its LDS
// stores (256 threads): a 192-dim row piece that rotates (threads < 128), two
// pass-through 192-dim chunks and two 128-dim chunks per thread.
struct StageRegs {
    u32x4 rx, ry;
    u32x4 pl[2];
    u32x4 r128[2];
};

__device__ __forceinline__ void stage_load(StageRegs &st, const uint16_t *src192, size_t s192,
                                           const uint16_t *src128, size_t s128, int nvalid, int tid) {
    // rows past the end re-read the last valid row: they are masked out of every
    // product (zero probability), and finite values keep 0 * value = 0; the loads
    // stay unconditional so that they are all in flight together
    const int last = nvalid - 1;
    if (tid < 128) {
        const int row = min(tid >> 2, last), cc = tid & 3;
        st.rx = ldg128(src192 + row * s192 + 8 * cc);
        st.ry = ldg128(src192 + row * s192 + 8 * cc + 32);
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int u = tid + 256 * r;
        const int row = min(u >> 4, last), c = 8 + (u & 15), c2 = u & 15;
        st.pl[r] = ldg128(src192 + row * s192 + 8 * c);
        st.r128[r] = ldg128(src128 + row * s128 + 8 * c2);
    }
}

// Rotate (rows at positions pos0 + row) and store a loaded stage into LDS.
__device__ __forceinline__ void stage_store(const StageRegs &st, uint16_t *d192, uint16_t *d128, int64_t pos0,
                                            const RopeTurns &rt, int tid) {
    if (tid < 128) {
        const int row = tid >> 2, cc = tid & 3;
        u32x4 x = st.rx, y = st.ry;
        rope_rotate8(x, y, rt, 8 * cc, pos0 + row);
        *reinterpret_cast<u32x4 *>(d192 + row * RSTR + 8 * cc) = x;
        *reinterpret_cast<u32x4 *>(d192 + row * RSTR + 8 * cc + 32) = y;
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int u = tid + 256 * r;
        const int row = u >> 4, c = 8 + (u & 15), c2 = u & 15;
        *reinterpret_cast<u32x4 *>(d192 + row * RSTR + 8 * c) = st.pl[r];
        *reinterpret_cast<u32x4 *>(d128 + row * VSTR + 8 * c2) = st.r128[r];
    }
}

// Turn a rotated-space gradient held as (dims d, d + 32) pairs back: the
// transpose of the rotation by pos * theta_d.
__device__ __forceinline__ void rope_back(float &x, float &y, uint64_t turn, int64_t pos) {
    float sn, cs;
    rope_sincos(turn, pos, sn, cs);
    const float nx = x * cs + y * sn;
    const float ny = y * cs - x * sn;
    x = nx;
    y = ny;
}

}  // namespace

// ---- d sink_h: one workgroup per head, fixed-order tree sum over the workgroup partials
__global__ __launch_bounds__(256) void bwd_sink_kernel(BwdArgs a) {
    __shared__ float red[256];
    const int h = blockIdx.x;
    const int64_t nblk = (int64_t)a.B * a.n_qblk;   // (batch, query block) partials
    float s_ = 0.0f;
    for (int64_t i = threadIdx.x; i < nblk; i += 256) s_ += a.csink[i * a.Hq + h];
    red[threadIdx.x] = s_;
    __syncthreads();
    for (int off = 128; off > 0; off >>= 1) {
        if (threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
        __syncthreads();
    }
    if (threadIdx.x == 0) a.dsinks[h] = red[0];
}

// ---- dq: 4 heads x 32 queries per workgroup, 32-key tiles
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2, 2))) void bwd_dq_kernel(BwdArgs a) {
    constexpr int NW = 4;
    __shared__ __attribute__((aligned(16))) uint16_t Ks[32 * RSTR];
    __shared__ __attribute__((aligned(16))) uint16_t KTs[kDqk * TSTR];
    __shared__ __attribute__((aligned(16))) uint16_t Vs[32 * VSTR];
    // each wave's dO rows: the B operand of dP^T, parked in LDS (each lane reads
    // back only what it wrote) to keep the kernel at two waves per SIMD
    __shared__ __attribute__((aligned(16))) uint16_t DOs[NW][32 * VSTR];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int h2 = lane >> 5, l32 = lane & 31;
    const int combos = a.B * a.Hkv * a.n_hgrp;
    const int qb = a.n_qblk - 1 - (int)(blockIdx.x / combos);   // longest key range first
    const int c = blockIdx.x % combos;
    const int b = c % a.B, pair = c / a.B;
    const int hg = pair % a.n_hgrp, g = pair / a.n_hgrp;
    const int G = a.Hq / a.Hkv;
    const int head = g * G + hg * NW + w;
    const int q0 = qb * 32;
    const int t = q0 + l32;
    const bool tval = t < a.T;

    // key range of the block (indices; positions are pos0 + index for q and k alike)
    const int jlo = a.window > 0 ? max(0, q0 - a.window + 1) : 0;
    const int jhi = min(q0 + 31, a.T - 1);

    // per lane: Q~ (B operand of S^T = K~ Q~^T, dims 96*h2 + 8*s), dO (B operand of dP^T = V dO^T)
    const size_t qrow = ((size_t)b * a.T + t) * a.Hq + head;
    u32x4 qf[12], dof[8];
    uint16_t *dos = DOs[w] + l32 * VSTR + 64 * h2;
    float L2 = kPosInf, Dq = 0.0f;
    if (tval) {
        const uint16_t *src = a.q + qrow * kDqk + 96 * h2;
#pragma unroll
        for (int s = 0; s < 12; ++s) qf[s] = ldg128(src + 8 * s);
        if (h2 == 0) {
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) rope_rotate8(qf[cc], qf[cc + 4], a.rt, 8 * cc, a.pos0 + t);
        }
        const uint16_t *gs = a.dout + qrow * kDv + 64 * h2;
#pragma unroll
        for (int s = 0; s < 8; ++s) dof[s] = ldg128(gs + 8 * s);
        L2 = a.lse[((size_t)b * a.Hq + head) * a.T + t] * kLog2e;
        // D = <dO, O> of the row: this lane's 64 dims, then its h2 partner's
        const uint16_t *os = a.out + qrow * kDv + 64 * h2;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const u32x4 o = ldg128(os + 8 * s);
#pragma unroll
            for (int x = 0; x < 4; ++x) Dq += bf_lo(o[x]) * bf_lo(dof[s][x]) + bf_hi(o[x]) * bf_hi(dof[s][x]);
        }
    } else {
#pragma unroll
        for (int s = 0; s < 12; ++s) qf[s] = u32x4{0, 0, 0, 0};
#pragma unroll
        for (int s = 0; s < 8; ++s) dof[s] = u32x4{0, 0, 0, 0};
    }
    Dq = sum_xor32(Dq);
#pragma unroll
    for (int s = 0; s < 8; ++s) *reinterpret_cast<u32x4 *>(dos + 8 * s) = dof[s];
    if (tval && h2 == 0) a.D[qrow] = Dq;   // for the dk/dv pass
    if (a.sinks) {
        // this head's sink terms -exp(sink - L) D summed over the block's 32 rows
        // (fixed order), one partial per (batch, query block, head)
        float term = (tval && h2 == 0) ? -__builtin_amdgcn_exp2f(a.sinks[head] * kLog2e - L2) * Dq : 0.0f;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) term += __shfl_xor(term, o);
        if (lane == 0) a.csink[((size_t)b * a.n_qblk + qb) * a.Hq + head] = term;
    }

    f32x16 acc[6];
#pragma unroll
    for (int mb = 0; mb < 6; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[mb][e] = 0.0f;

    const int prow = (l32 & 0x13) | ((l32 & 4) << 1) | ((l32 & 8) >> 1);
    const float cl2 = a.scale_log2;
    const int win = a.window > 0 ? a.window : 0x7fffffff;
    const size_t krs = (size_t)a.Hkv * kDqk, vrs = (size_t)a.Hkv * kDv;

    // the next tile's K / V rows are loaded into registers while this one is computed
    auto load_tile = [&](StageRegs &st, int j0) {
        stage_load(st, a.k + ((size_t)b * a.T + j0) * krs + (size_t)g * kDqk, krs,
                   a.v + ((size_t)b * a.T + j0) * vrs + (size_t)g * kDv, vrs, min(32, a.T - j0), tid);
    };
    const int j_first = (jlo / 32) * 32;
    StageRegs st;
    load_tile(st, j_first);
    for (int j0 = j_first; j0 <= jhi; j0 += 32) {
        __syncthreads();   // the previous tile's reads are done
        stage_store(st, Ks, Vs, a.pos0 + j0, a.rt, tid);
        if (j0 + 32 <= jhi) load_tile(st, j0 + 32);
        __syncthreads();
        transpose32(KTs, Ks, RSTR, kDqk / 8, tid, 64 * NW);
        __syncthreads();

        f32x16 S, DP;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            S[e] = 0.0f;
            DP[e] = 0.0f;
        }
#pragma unroll
        for (int s = 0; s < 12; ++s) S = mfma32(lds128(Ks + prow * RSTR + 96 * h2 + 8 * s), qf[s], S);
#pragma unroll
        for (int s = 0; s < 8; ++s) DP = mfma32(lds128(Vs + prow * VSTR + 64 * h2 + 8 * s), lds128(dos + 8 * s), DP);

        // element e: key j0 + 16*(e>>3) + 8*h2 + (e&7), query t
        u32x4 dsb[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            float v8[8];
#pragma unroll
            for (int x = 0; x < 8; ++x) {
                const int e = 8 * s + x;
                const int j = j0 + 16 * s + 8 * h2 + x;
                const bool vis = tval && j < a.T && j <= t && t - j < win;
                const float p = vis ? __builtin_amdgcn_exp2f(__builtin_fmaf(S[e], cl2, -L2)) : 0.0f;
                v8[x] = p * (DP[e] * a.v_scale - Dq);
            }
#pragma unroll
            for (int x = 0; x < 4; ++x) dsb[s][x] = pack_bf16(v8[2 * x], v8[2 * x + 1]);
        }
        // dQ~^T (192 x 32 queries) += K~^T (192 x 32 keys) dS^T
#pragma unroll
        for (int mb = 0; mb < 6; ++mb)
#pragma unroll
            for (int s = 0; s < 2; ++s)
                acc[mb] = mfma32(lds128(KTs + (32 * mb + l32) * TSTR + 16 * s + 8 * h2), dsb[s], acc[mb]);
    }

    // ---- epilogue: acc[mb][e] holds dim 32*mb + 8*(e/4) + 4*h2 + (e%4) of query t
    if (!tval) return;
    const float cs = a.scale;
#pragma unroll
    for (int mb = 0; mb < 6; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[mb][e] *= cs;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int d = 8 * (e / 4) + 4 * h2 + (e % 4);   // < 32: rotary pair (d, d + 32)
        float x = acc[0][e], y = acc[1][e];
        rope_back(x, y, a.rt.turn[d], a.pos0 + t);
        acc[0][e] = x;
        acc[1][e] = y;
    }
    uint16_t *dst = a.dq + qrow * kDqk;
#pragma unroll
    for (int mb = 0; mb < 6; ++mb)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
            u32x2 o;
            o[0] = pack_bf16(acc[mb][4 * e4], acc[mb][4 * e4 + 1]);
            o[1] = pack_bf16(acc[mb][4 * e4 + 2], acc[mb][4 * e4 + 3]);
            *reinterpret_cast<u32x2 *>(dst + 32 * mb + 8 * e4 + 4 * h2) = o;
        }
}

// ---- dk, dv: 128 keys of one KV head per workgroup (one wave per 32 keys)
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void bwd_dkdv_kernel(BwdArgs a) {
    // two stage buffers: one is computed on while the next is written
    __shared__ __attribute__((aligned(16))) uint16_t Qsb[2][32 * RSTR];
    __shared__ __attribute__((aligned(16))) uint16_t QTsb[2][kDqk * TSTR];
    __shared__ __attribute__((aligned(16))) uint16_t Osb[2][32 * VSTR];
    __shared__ __attribute__((aligned(16))) uint16_t OTsb[2][kDv * TSTR];
    __shared__ __attribute__((aligned(16))) float Lsb[2][32], Dsb[2][32];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int h2 = lane >> 5, l32 = lane & 31;
    const int per_b = a.Hkv * a.n_kblk;
    const int b = blockIdx.x / per_b;
    const int r = blockIdx.x - b * per_b;
    const int g = r % a.Hkv;
    const int kb = a.n_kblk - 1 - r / a.Hkv;          // later keys see fewer queries under a causal mask
    const int jb0 = kb * 128;
    const int jw0 = jb0 + 32 * w;                      // this wave's keys
    const int j = jw0 + l32;
    const bool jval = j < a.T;
    const int G = a.Hq / a.Hkv;
    const size_t qrs = (size_t)a.Hq * kDqk, ors = (size_t)a.Hq * kDv;

    // per lane: K~ (B operand of S = Q~ K~^T), V (B operand of dP = dO V^T) of key j
    const size_t krow = ((size_t)b * a.T + j) * a.Hkv + g;
    u32x4 kf[12], vf[8];
    if (jval) {
        const uint16_t *src = a.k + krow * kDqk + 96 * h2;
#pragma unroll
        for (int s = 0; s < 12; ++s) kf[s] = ldg128(src + 8 * s);
        if (h2 == 0) {
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) rope_rotate8(kf[cc], kf[cc + 4], a.rt, 8 * cc, a.pos0 + j);
        }
        const uint16_t *vs = a.v + krow * kDv + 64 * h2;
#pragma unroll
        for (int s = 0; s < 8; ++s) vf[s] = ldg128(vs + 8 * s);
    } else {
#pragma unroll
        for (int s = 0; s < 12; ++s) kf[s] = u32x4{0, 0, 0, 0};
#pragma unroll
        for (int s = 0; s < 8; ++s) vf[s] = u32x4{0, 0, 0, 0};
    }

    f32x16 dK[6], dV[4];
#pragma unroll
    for (int mb = 0; mb < 6; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) dK[mb][e] = 0.0f;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) dV[mb][e] = 0.0f;

    const int prow = (l32 & 0x13) | ((l32 & 4) << 1) | ((l32 & 8) >> 1);
    const float cl2 = a.scale_log2;
    const int win = a.window > 0 ? a.window : 0x7fffffff;
    // queries that see some key of the workgroup, and of this wave
    const int qlo = jb0;
    const int qhi = a.window > 0 ? min(a.T - 1, jb0 + 127 + a.window - 1) : a.T - 1;
    const int wq_hi = a.window > 0 ? jw0 + 31 + a.window - 1 : 0x7fffffff;

    // stages (query head, 32-query block), head-major; the next stage's rows are
    // loaded into registers while this one is computed
    const int q_first = (qlo / 32) * 32;
    const int n_qb = (qhi - q_first) / 32 + 1;
    const int n_stage = G * n_qb;
    // Staging of a stage (32 query rows of one head): thread u < 64 takes rows
    // (2*(u%16), +1) x rotating chunks (u/16, u/16 + 4) of Q; every thread takes
    // rows (2*(t%16), +1) x one pass-through Q chunk 8 + t/16 and x dO chunk t/16.
    // Holding both rows of a pair, a thread writes its chunks row-major and, two
    // rows per dword, transposed: no LDS-to-LDS transpose pass.
    struct DkStage {
        u32x4 rq[2][2];   // [row of pair][chunk c, c + 4], threads < 64
        u32x4 pq[2];      // [row of pair] pass-through Q chunk
        u32x4 po[2];      // [row of pair] dO chunk
        float lv, dv;     // L and D of query row tid (threads < 32)
    };
    const int rp = tid & 15, rc = tid >> 4;
    auto load_stage = [&](DkStage &st, int s_) {
        s_ = min(s_, n_stage - 1);   // past the last stage: re-read it (unused)
        const int head = g * G + s_ / n_qb, q0 = q_first + 32 * (s_ % n_qb);
        const int last = min(32, a.T - q0) - 1;
        const uint16_t *qb_ = a.q + ((size_t)b * a.T + q0) * qrs + (size_t)head * kDqk;
        const uint16_t *ob_ = a.dout + ((size_t)b * a.T + q0) * ors + (size_t)head * kDv;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            // rows past the end re-read the last valid row: masked out of every product
            const int row = min(2 * rp + i, last);
            if (tid < 64) {
                st.rq[i][0] = ldg128(qb_ + row * qrs + 8 * rc);
                st.rq[i][1] = ldg128(qb_ + row * qrs + 8 * rc + 32);
            }
            st.pq[i] = ldg128(qb_ + row * qrs + 8 * (8 + rc));
            st.po[i] = ldg128(ob_ + row * ors + 8 * rc);
        }
        if (tid < 32) {
            const bool ok = tid <= last;
            st.lv = ok ? a.lse[((size_t)b * a.Hq + head) * a.T + q0 + tid] * kLog2e : kPosInf;
            st.dv = ok ? a.D[((size_t)b * a.T + q0 + tid) * a.Hq + head] : 0.0f;
        }
    };
    // chunk x0 (row 2*rp) and x1 (row 2*rp + 1) of 8 columns starting at col:
    // row-major into d (row stride sstr), transposed into dT (column-major pairs)
    auto put2 = [&](uint16_t *d, uint16_t *dT, int sstr, int col, const u32x4 &x0, const u32x4 &x1) {
        *reinterpret_cast<u32x4 *>(d + (2 * rp) * sstr + col) = x0;
        *reinterpret_cast<u32x4 *>(d + (2 * rp + 1) * sstr + col) = x1;
#pragma unroll
        for (int dd = 0; dd < 8; ++dd) {
            const uint32_t sel = (dd & 1) ? 0x07060302u : 0x05040100u;
            *reinterpret_cast<uint32_t *>(dT + (col + dd) * TSTR + 2 * rp) = __builtin_amdgcn_perm(x1[dd >> 1], x0[dd >> 1], sel);
        }
    };
    auto store_stage = [&](DkStage &st, int s_, int buf) {
        const int q0 = q_first + 32 * (s_ % n_qb);
        if (tid < 64) {
#pragma unroll
            for (int i = 0; i < 2; ++i) rope_rotate8(st.rq[i][0], st.rq[i][1], a.rt, 8 * rc, a.pos0 + q0 + 2 * rp + i);
            put2(Qsb[buf], QTsb[buf], RSTR, 8 * rc, st.rq[0][0], st.rq[1][0]);
            put2(Qsb[buf], QTsb[buf], RSTR, 8 * rc + 32, st.rq[0][1], st.rq[1][1]);
        }
        put2(Qsb[buf], QTsb[buf], RSTR, 8 * (8 + rc), st.pq[0], st.pq[1]);
        put2(Osb[buf], OTsb[buf], VSTR, 8 * rc, st.po[0], st.po[1]);
        if (tid < 32) {
            Lsb[buf][tid] = st.lv;
            Dsb[buf][tid] = st.dv;
        }
    };
    DkStage st;
    load_stage(st, 0);
    store_stage(st, 0, 0);
    load_stage(st, 1);
    __syncthreads();
    for (int s_ = 0; s_ < n_stage; ++s_) {
        const int q0 = q_first + 32 * (s_ % n_qb);
        const int buf = s_ & 1;
        const uint16_t *Qs = Qsb[buf], *QTs = QTsb[buf], *Os = Osb[buf], *OTs = OTsb[buf];
        const float *Ls = Lsb[buf], *Ds = Dsb[buf];
        // does this wave's key range meet the block's queries? (wave-uniform)
        if (!(jw0 > q0 + 31 || q0 > wq_hi)) {

            f32x16 S, DP;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                S[e] = 0.0f;
                DP[e] = 0.0f;
            }
#pragma unroll
            for (int s = 0; s < 12; ++s) S = mfma32(lds128(Qs + prow * RSTR + 96 * h2 + 8 * s), kf[s], S);
#pragma unroll
            for (int s = 0; s < 8; ++s) DP = mfma32(lds128(Os + prow * VSTR + 64 * h2 + 8 * s), vf[s], DP);

            // element e: query q0 + 16*(e>>3) + 8*h2 + (e&7), key j
            u32x4 pb[2], dsb[2];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                float p8[8], d8[8];
                // the lane's 8 query rows are consecutive: their L and D in two 16-byte reads each
                const float4 l0 = *reinterpret_cast<const float4 *>(Ls + 16 * s + 8 * h2);
                const float4 l1 = *reinterpret_cast<const float4 *>(Ls + 16 * s + 8 * h2 + 4);
                const float4 d0 = *reinterpret_cast<const float4 *>(Ds + 16 * s + 8 * h2);
                const float4 d1 = *reinterpret_cast<const float4 *>(Ds + 16 * s + 8 * h2 + 4);
                const float lrow[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
                const float drow[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
#pragma unroll
                for (int x = 0; x < 8; ++x) {
                    const int e = 8 * s + x;
                    const int q = q0 + 16 * s + 8 * h2 + x;
                    const bool vis = jval && q < a.T && j <= q && q - j < win;
                    const float p = vis ? __builtin_amdgcn_exp2f(__builtin_fmaf(S[e], cl2, -lrow[x])) : 0.0f;
                    p8[x] = p;
                    d8[x] = p * (DP[e] * a.v_scale - drow[x]);
                }
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    pb[s][x] = pack_bf16(p8[2 * x], p8[2 * x + 1]);
                    dsb[s][x] = pack_bf16(d8[2 * x], d8[2 * x + 1]);
                }
            }
            // dV^T (128 x 32 keys) += dO^T P;  dK~^T (192 x 32 keys) += Q~^T dS
#pragma unroll
            for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                for (int s = 0; s < 2; ++s)
                    dV[mb] = mfma32(lds128(OTs + (32 * mb + l32) * TSTR + 16 * s + 8 * h2), pb[s], dV[mb]);
#pragma unroll
            for (int mb = 0; mb < 6; ++mb)
#pragma unroll
                for (int s = 0; s < 2; ++s)
                    dK[mb] = mfma32(lds128(QTs + (32 * mb + l32) * TSTR + 16 * s + 8 * h2), dsb[s], dK[mb]);
        }
        // the next stage goes to the other buffer, read last in the previous stage
        store_stage(st, s_ + 1 < n_stage ? s_ + 1 : s_, buf ^ 1);
        load_stage(st, s_ + 2);
        __syncthreads();
    }

    // ---- epilogue: dK[mb][e] / dV[mb][e] hold dim 32*mb + 8*(e/4) + 4*h2 + (e%4) of key j
    if (!jval) return;
#pragma unroll
    for (int mb = 0; mb < 6; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) dK[mb][e] *= a.scale;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int d = 8 * (e / 4) + 4 * h2 + (e % 4);
        float x = dK[0][e], y = dK[1][e];
        rope_back(x, y, a.rt.turn[d], a.pos0 + j);
        dK[0][e] = x;
        dK[1][e] = y;
    }
    uint16_t *dk = a.dk + krow * kDqk;
    uint16_t *dv = a.dv + krow * kDv;
#pragma unroll
    for (int mb = 0; mb < 6; ++mb)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
            u32x2 o;
            o[0] = pack_bf16(dK[mb][4 * e4], dK[mb][4 * e4 + 1]);
            o[1] = pack_bf16(dK[mb][4 * e4 + 2], dK[mb][4 * e4 + 3]);
            *reinterpret_cast<u32x2 *>(dk + 32 * mb + 8 * e4 + 4 * h2) = o;
        }
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
            u32x2 o;
            o[0] = pack_bf16(dV[mb][4 * e4] * a.v_scale, dV[mb][4 * e4 + 1] * a.v_scale);
            o[1] = pack_bf16(dV[mb][4 * e4 + 2] * a.v_scale, dV[mb][4 * e4 + 3] * a.v_scale);
            *reinterpret_cast<u32x2 *>(dv + 32 * mb + 8 * e4 + 4 * h2) = o;
        }
}

size_t backward_workspace_bytes(int32_t B, int32_t T, int32_t Hq) {
    const size_t rows = (size_t)B * T * Hq;
    return (rows + (size_t)B * ((T + 31) / 32) * Hq) * sizeof(float);
}

hipError_t launch_backward(BwdArgs a, hipStream_t stream) {
    const int G = a.Hq / a.Hkv;
    if (G % 4 != 0) return hipErrorInvalidValue;
    a.n_qblk = (a.T + 31) / 32;
    a.n_hgrp = G / 4;
    a.n_kblk = (a.T + 127) / 128;
    // dq also forms D and the sink partials; d sink and dk/dv read them
    const int64_t qblocks = (int64_t)a.B * a.Hkv * a.n_hgrp * a.n_qblk;
    hipLaunchKernelGGL(bwd_dq_kernel, dim3((unsigned)qblocks), dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.sinks) {
        hipLaunchKernelGGL(bwd_sink_kernel, dim3(a.Hq), dim3(256), 0, stream, a);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int64_t kblocks = (int64_t)a.B * a.Hkv * a.n_kblk;
    hipLaunchKernelGGL(bwd_dkdv_kernel, dim3((unsigned)kblocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace mimo
