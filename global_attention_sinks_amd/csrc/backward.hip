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
//   bwd_krot_kernel    writes the rotated dims 0..63 of K~ into the workspace
//   bwd_dq_kernel      query-major: a workgroup owns 32 queries x 4 heads of a
//                      GQA group; it forms D per (row, head) from O and dO and
//                      per head the sum of its rows' sink terms, writes D and
//                      the rotated dims 0..63 of Q~ for dk/dv, then per 32-key
//                      tile (K~ and V rows copied into LDS by buffer loads that
//                      write LDS, double-buffered, shared by the 4 heads)
//                      rebuilds S^T and dP^T and accumulates dQ~^T = K~^T dS^T
//                      in registers, reading K~^T with LDS transpose loads
//   bwd_sink_kernel    one workgroup per head sums the sink partials (fixed order)
//   bwd_dkdv_kernel    key-major: a workgroup owns 64 keys of one KV head (one
//                      wave per 16 keys, 16x16x32 MFMAs, the keys' K~ and V held
//                      in registers; two workgroups per CU); it walks every query
//                      head of the group and every 32-query block that sees its
//                      keys (Q~ and dO rows copied into LDS by buffer loads that
//                      write LDS, double-buffered; the rotated dims of Q~ come
//                      from the dq pass) and accumulates dK~^T = Q~^T dS and
//                      dV^T = dO^T P, reading Q~^T and dO^T with LDS transpose loads
// Both kernels reuse the forward's layout trick: the A-operand rows of the first
// product are read in a permuted order, so each lane's accumulators are directly
// the B operand of the second product.
// Nothing is accumulated across workgroups, so the results are deterministic.
#include "kernels.hpp"

namespace mimo {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kPosInf = __builtin_inff();

__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

__device__ __forceinline__ u32x4 lds128(const uint16_t *p) { return *reinterpret_cast<const u32x4 *>(p); }

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

namespace {
// Both kernels copy their LDS tiles with buffer loads that write LDS (a buffer
// resource per source, 16 or 4 bytes per lane landing at lds + bytes * lane).
// A tile's rows are split by source: the rotated dims 0..63 (rows of 64 + 8 pad
// elements, 144 bytes, 9 copies of 16 bytes per row) and 128-dim rows (pass-
// through dims of q / k, dO, V: 128 + 8 pad, 272 bytes, 17 copies per row), each
// region whole 1 KiB copies (lanes past the region's rows re-read the last row
// into slack).  Rows past the sequence re-read its last row: the masks zero them.
constexpr int kRotStr = 72, kRowStr = 136;   // row strides (elements)
constexpr int kRotBytes = 5120, kRowBytes = 9216;   // 32-row regions, whole 1 KiB copies
constexpr int kRotCopies = 5, kRowCopies = 9;
constexpr uint32_t kRsrcFlags = 0x00020000u;

// dk/dv stage: Q~ dims 0..63, Q dims 64..191, dO, then L and D (32 floats each)
constexpr int kQaOff = 0, kQbOff = kRotBytes, kObOff = kRotBytes + kRowBytes, kLOff = kRotBytes + 2 * kRowBytes;
constexpr int kDOff = kLOff + 256, kStageBytes = kDOff + 256;
constexpr int kStageCopies = kRotCopies + 2 * kRowCopies + 2;   // + L, D (4 bytes per lane)
// dq tile: K~ dims 0..63, K dims 64..191, V
constexpr int kKaOff = 0, kKbOff = kRotBytes, kVOff = kRotBytes + kRowBytes, kTileBytes = kRotBytes + 2 * kRowBytes;
constexpr int kTileCopies = kRotCopies + 2 * kRowCopies;

// Lane offsets of copy k of a region (c = 64 k + lane): rotated rows and 128-dim rows.
__device__ __forceinline__ int rot_voff(int k, int lane, int last) {
    const int c = 64 * k + lane, row = c / 9, piece = c - 9 * row;
    return min(row, last) * 128 + 16 * min(piece, 7);
}
__device__ __forceinline__ int row_voff(int k, int lane, int last, int row_bytes) {
    const int c = 64 * k + lane, row = c / 17, piece = c - 17 * row;
    return min(row, last) * row_bytes + 16 * min(piece, 15);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ void lds_copy(__amdgpu_buffer_rsrc_t rsrc, const unsigned char *lds_dst, int bytes,
                                         int voffset) {
    auto *d = (__attribute__((address_space(3))) void *)(const_cast<unsigned char *>(lds_dst));
    if (bytes == 16) __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, d, 16, voffset, 0, 0, 0);
    else __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, d, 4, voffset, 0, 0, 0);
}

// 8 consecutive rows (queries) x this lane's column of a row-major bf16 stage, as
// one MFMA operand: two transpose loads, rows row0 .. row0 + 3 and row0 + 4 .. + 7
// of the lane group.  p0 is this lane's address for the first four rows.
__device__ __forceinline__ u32x4 lds_tr8(const uint16_t *p0, int str) {
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(const_cast<uint16_t *>(p0)));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(const_cast<uint16_t *>(p0 + 4 * str)));
    const u32x2 a = __builtin_bit_cast(u32x2, lo), c = __builtin_bit_cast(u32x2, hi);
    return u32x4{a[0], a[1], c[0], c[1]};
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

// ---- rotated dims 0..63 of K for dq: krot [B, Hkv, T, 64], one thread per (key
// row, KV head, 8 rotary pairs)
__global__ __launch_bounds__(256) void bwd_krot_kernel(BwdArgs a) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)a.B * a.T * a.Hkv * 4) return;
    const int cc = (int)(i & 3);
    const int64_t rg = i >> 2;   // (b * T + t) * Hkv + g
    const int g = (int)(rg % a.Hkv);
    const int64_t bt = rg / a.Hkv;
    const int t = (int)(bt % a.T), b = (int)(bt / a.T);
    const uint16_t *src = a.k + rg * kDqk;
    u32x4 x = ldg128(src + 8 * cc), y = ldg128(src + 32 + 8 * cc);
    rope_rotate8(x, y, a.rt, 8 * cc, a.pos0 + t);
    uint16_t *dst = a.krot + (((size_t)b * a.Hkv + g) * a.T + t) * kRope;
    stg128(dst + 8 * cc, x);
    stg128(dst + 32 + 8 * cc, y);
}

// ---- dq: 4 heads x 32 queries per workgroup, 32-key tiles copied into LDS (double-
// buffered) by buffer loads: K~ dims 0..63 from krot, K dims 64..191, V.  S^T = K~ Q~^T
// and dP^T = V dO^T read the key rows in the bit-2/3-swapped order prow, so dS^T packs
// straight into the B operand of dQ~^T = K~^T dS^T, whose A operand (a dim x 8
// consecutive keys per lane) comes from the row-major tile by LDS transpose loads.
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2, 2))) void bwd_dq_kernel(BwdArgs a) {
    constexpr int NW = 4;
    __shared__ __attribute__((aligned(1024))) unsigned char tiles[2][kTileBytes];
    // each wave's dO rows: the B operand of dP^T, parked in LDS (each lane reads back
    // only what it wrote) to keep the kernel at two waves per SIMD; the 16-byte chunks
    // of row r are XOR-swizzled by r % 16 so that 16 rows read at once hit distinct banks
    __shared__ __attribute__((aligned(16))) uint16_t DOs[NW][32 * kDv];

    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h2 = lane >> 5, l32 = lane & 31;
    const int combos = a.B * a.Hkv * a.n_hgrp;
    const int qb = a.n_qblk - 1 - (int)(blockIdx.x / combos);   // longest key range first
    const int c = blockIdx.x % combos;
    // consecutive workgroups land on different XCDs (each with its own L2): the
    // head groups of one (sequence, KV head) sit combos / n_hgrp apart, a multiple
    // of 8 when B * Hkv is, so they share an XCD and its copy of the K/V tiles
    const int bg = c % (a.B * a.Hkv), hg = c / (a.B * a.Hkv);
    const int b = bg % a.B, g = bg / a.B;
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
    uint16_t *dos = DOs[w] + l32 * kDv;
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
    for (int s = 0; s < 8; ++s) *reinterpret_cast<u32x4 *>(dos + 8 * ((8 * h2 + s) ^ (l32 & 15))) = dof[s];
    if (tval && h2 == 0) {
        // for the dk/dv pass, head-major so that a 32-query stage is contiguous: D and
        // the rotated dims 0..63 of Q~ (this lane's qf[0..7])
        const size_t hrow = ((size_t)b * a.Hq + head) * a.T + t;
        a.D[hrow] = Dq;
        uint16_t *qr = a.qrot + hrow * kRope;
#pragma unroll
        for (int s = 0; s < 8; ++s) stg128(qr + 8 * s, qf[s]);
    }
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
    const int Hkv = a.Hkv;
    // transpose loads: this lane addresses key row 8 (lane / 32) + (lane % 16) / 4 and
    // the 4 dims from 16 ((lane / 16) % 2) + 4 (lane % 4) of a 32-dim block
    const int trow = 8 * h2 + ((lane & 15) >> 2), tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

    auto copy_tile = [&](int j0, int buf) {
        const int last = min(32, a.T - j0) - 1;
        const unsigned char *dst = tiles[buf];
        const size_t trow0 = ((size_t)b * a.T + j0) * Hkv + g;
#pragma unroll
        for (int m = 0; m < (kTileCopies + NW - 1) / NW; ++m) {
            const int id = w + NW * m;   // wave-uniform
            if (id < kRotCopies) {
                const auto rs = __builtin_amdgcn_make_buffer_rsrc(
                    a.krot + (((size_t)b * Hkv + g) * a.T + j0) * kRope, 0, (last + 1) * 128, kRsrcFlags);
                lds_copy(rs, dst + kKaOff + 1024 * id, 16, rot_voff(id, lane, last));
            } else if (id < kRotCopies + kRowCopies) {
                const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(a.k + trow0 * kDqk), 0,
                                                                  last * Hkv * 384 + 384, kRsrcFlags);
                const int k = id - kRotCopies;
                lds_copy(rs, dst + kKbOff + 1024 * k, 16, row_voff(k, lane, last, Hkv * 384) + 128);
            } else if (id < kTileCopies) {
                const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(a.v + trow0 * kDv), 0,
                                                                  last * Hkv * 256 + 256, kRsrcFlags);
                const int k = id - kRotCopies - kRowCopies;
                lds_copy(rs, dst + kVOff + 1024 * k, 16, row_voff(k, lane, last, Hkv * 256));
            }
        }
    };

    const int j_first = (jlo / 32) * 32;
    copy_tile(j_first, 0);
    // Q~ is complete here (its loads are older than the copies): no wait of the
    // compiler's for it inside the loop, where copies would be in flight
    asm volatile("" ::"v"(qf[0]), "v"(qf[1]), "v"(qf[2]), "v"(qf[3]), "v"(qf[4]), "v"(qf[5]), "v"(qf[6]),
                 "v"(qf[7]), "v"(qf[8]), "v"(qf[9]), "v"(qf[10]), "v"(qf[11]));
    __syncthreads();   // also waits for this wave's copies
    int buf = 0;
    for (int j0 = j_first; j0 <= jhi; j0 += 32) {
        // the next tile goes to the other buffer, last read before the previous barrier
        if (j0 + 32 <= jhi) copy_tile(j0 + 32, buf ^ 1);
        const uint16_t *Ka = reinterpret_cast<const uint16_t *>(tiles[buf] + kKaOff);
        const uint16_t *Kb = reinterpret_cast<const uint16_t *>(tiles[buf] + kKbOff);
        const uint16_t *Vs = reinterpret_cast<const uint16_t *>(tiles[buf] + kVOff);

        f32x16 S, DP;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            S[e] = 0.0f;
            DP[e] = 0.0f;
        }
        // S^T: chunk s of this lane is dims 96 h2 + 8 s .. + 7 of key row prow
        const uint16_t *klo = h2 ? Kb + prow * kRowStr + 32 : Ka + prow * kRotStr;        // s < 8
        const uint16_t *khi = h2 ? Kb + prow * kRowStr + 32 : Kb + prow * kRowStr - 64;   // s >= 8
#pragma unroll
        for (int s = 0; s < 12; ++s) S = mfma32(lds128((s < 8 ? klo : khi) + 8 * s), qf[s], S);
#pragma unroll
        for (int s = 0; s < 8; ++s)
            DP = mfma32(lds128(Vs + prow * kRowStr + 64 * h2 + 8 * s), lds128(dos + 8 * ((8 * h2 + s) ^ (l32 & 15))), DP);

        // element e: key j0 + 16*(e>>3) + 8*h2 + (e&7), query t.  A tile whose every
        // key every query of the block sees needs no mask; otherwise, less j0 + 8 h2,
        // the keys query t sees form a range [lo, hi] and key c is in it when
        // c - lo <= hi - lo as unsigned (c a constant: no per-key registers).
        // (Rows past T have L = +inf, so their p is 0 either way.)
        const bool full = (j0 + 32 <= a.T) && (j0 + 31 <= q0) && (q0 + 31 - j0 < win);
        int lo = 0;
        uint32_t span = 0xffffffffu;
        if (!full) {
            const int hi = min(t, a.T - 1) - j0 - 8 * h2;
            lo = (int)max((int64_t)t - j0 - 8 * h2 - win + 1, (int64_t)-64);   // keys before the tile: c >= 0 > lo
            span = (uint32_t)(hi - lo);
            if (hi < lo) {   // nothing visible
                lo = 0x40000000;
                span = 0;
            }
        }
        u32x4 dsb[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            float v8[8];
#pragma unroll
            for (int x = 0; x < 8; ++x) {
                const int e = 8 * s + x;
                float p = __builtin_amdgcn_exp2f(__builtin_fmaf(S[e], cl2, -L2));
                if (!full && (uint32_t)(16 * s + x - lo) > span) p = 0.0f;
                v8[x] = p * (DP[e] * a.v_scale - Dq);
            }
#pragma unroll
            for (int x = 0; x < 4; ++x) dsb[s][x] = pack_bf16(v8[2 * x], v8[2 * x + 1]);
        }
        // dQ~^T (192 x 32 queries) += K~^T (192 x 32 keys) dS^T; A operand of block
        // (mb, s): dims 32 mb + l32, keys 16 s + 8 h2 .. + 7 (transpose loads)
#pragma unroll
        for (int mb = 0; mb < 6; ++mb)
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const u32x4 kt = mb < 2 ? lds_tr8(Ka + (16 * s + trow) * kRotStr + 32 * mb + tcol, kRotStr)
                                        : lds_tr8(Kb + (16 * s + trow) * kRowStr + 32 * (mb - 2) + tcol, kRowStr);
                acc[mb] = mfma32(kt, dsb[s], acc[mb]);
            }
        __syncthreads();   // this tile's reads are done; also waits for this wave's copies of the next
        buf ^= 1;
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

// ---- dk, dv: 16 NWV keys of one KV head per workgroup, one wave per 16 keys (two
// waves per SIMD), 16x16x32 MFMAs.  Lane (g4 = lane / 16, l16 = lane % 16) holds,
// for key kw0 + l16 of its wave, dims 32 c + 8 g4 .. + 7 of K~ and V (B operands of
// S = Q~ K~^T and dP = dO V^T).  The A operands of S and dP are Q~ / dO rows read
// in the order pi: in query block qb of the stage's 32 queries, MFMA row 4 u + i
// is query 8 u + 4 qb + i, so that a lane's accumulators of the two blocks hold
// queries 8 g4 .. 8 g4 + 7 of its key: exactly the B operand (8 consecutive
// queries) of dV^T = dO^T P and dK~^T = Q~^T dS.  The A operands of those two
// (dO^T, Q~^T: 16 dims x 8 consecutive queries per lane) are read from the same
// row-major stage with LDS transpose loads (ds_read_b64_tr_b16: within each 16
// lanes, output lane 16 G + r, element e comes from element r % 4 of the 8 bytes
// that lane 16 G + 4 e + r / 4 addresses).
//
// A stage (32 queries of one head) is copied into LDS by buffer loads that write
// LDS directly, gathering its rows from q, dout, lse and the dq pass's workspace
// (rotated dims of Q~ and D): no staging registers, no RoPE, no transpose.  Stage
// layout in bytes, per buffer: Q~ dims 0..63 rows of 144 (64 + 8 pad), Q dims
// 64..191 rows of 272, dO rows of 272, L and D 32 floats each; each region is
// whole 1 KiB copies (16 bytes per lane; lanes past the region's rows re-read
// the last row into slack).

template <int NWV>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * NWV, 64 * NWV), amdgpu_waves_per_eu(2, 2)))
void bwd_dkdv_kernel(BwdArgs a) {
    constexpr int KPW = 16;   // keys per wave
    constexpr int KPB = KPW * NWV;
    // two stage buffers: one is computed on while the next is copied in
    __shared__ __attribute__((aligned(1024))) unsigned char stg[2][kStageBytes];

    // w through readfirstlane: the compiler then knows it (and the copies' choice of
    // source and LDS region) to be wave-uniform
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g4 = lane >> 4, l16 = lane & 15;
    const int per_b = a.Hkv * a.n_kblk;
    const int b = blockIdx.x / per_b;
    const int r = blockIdx.x - b * per_b;
    const int g = r % a.Hkv;
    const int kb = a.n_kblk - 1 - r / a.Hkv;          // later keys see fewer queries under a causal mask
    const int jb0 = kb * KPB;
    const int kw0 = jb0 + KPW * w;                     // this wave's keys
    const int j = kw0 + l16;
    const bool jval = j < a.T;
    const int G = a.Hq / a.Hkv;

    const size_t krow = ((size_t)b * a.T + (jval ? j : a.T - 1)) * a.Hkv + g;
    u32x4 kf[6], vf[4];
    {
        const uint16_t *src = a.k + krow * kDqk + 8 * g4;
#pragma unroll
        for (int c = 0; c < 6; ++c) kf[c] = ldg128(src + 32 * c);
        rope_rotate8(kf[0], kf[1], a.rt, 8 * g4, a.pos0 + (jval ? j : a.T - 1));
        const uint16_t *vs = a.v + krow * kDv + 8 * g4;
#pragma unroll
        for (int c = 0; c < 4; ++c) vf[c] = ldg128(vs + 32 * c);
    }

    f32x4 dK[12], dV[8];
#pragma unroll
    for (int mb = 0; mb < 12; ++mb) dK[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) dV[mb] = f32x4{0.f, 0.f, 0.f, 0.f};

    const float cl2 = a.scale_log2;
    const int win = a.window > 0 ? a.window : 0x7fffffff;
    // queries that see some key of the workgroup, and of this wave
    const int qlo = jb0;
    const int qhi = a.window > 0 ? min(a.T - 1, jb0 + KPB - 1 + a.window - 1) : a.T - 1;
    const int wq_hi = a.window > 0 ? kw0 + KPW - 1 + a.window - 1 : 0x7fffffff;
    // query row of MFMA row l16 in query block qb (the order pi above)
    const int prow0 = 8 * (l16 >> 2) + (l16 & 3);
    // transpose loads: this lane addresses row 8 (lane / 16) + (lane % 16) / 4 and
    // the 4 columns from 4 (lane % 4) of a 16-column block
    const int trow = 8 * g4 + (l16 >> 2), tcol = 4 * (lane & 3);

    // stages (query head, 32-query block), head-major
    const int q_first = (qlo / 32) * 32;
    const int n_qb = (qhi - q_first) / 32 + 1;
    const int n_stage = G * n_qb;
    const int Hq = a.Hq;
    // block order within a head: step t takes the block congruent to (last block of the
    // sequence - t) mod n_qb, so workgroups of neighbouring keys copy the same stage at
    // the same step (one L2 fetch serves them all); under a causal mask, all later blocks
    const int boff = ((a.T - 1) / 32 - q_first / 32) % n_qb;
    auto stage_q0 = [&](int s_) {
        int i = boff - s_ % n_qb;
        if (i < 0) i += n_qb;
        return q_first + 32 * i;
    };
    auto copy_stage = [&](int s_, int buf) {
        const int head = g * G + s_ / n_qb, q0 = stage_q0(s_);
        const int last = min(32, a.T - q0) - 1;   // rows past it re-read it: masked out of every product
        const size_t hrow = ((size_t)b * Hq + head) * a.T + q0;
        const size_t trow0 = ((size_t)b * a.T + q0) * Hq + head;
        const unsigned char *dst = stg[buf];
#pragma unroll
        for (int m = 0; m < (kStageCopies + NWV - 1) / NWV; ++m) {
            const int id = w + NWV * m;   // wave-uniform
            if (id < kRotCopies) {
                const auto rs = __builtin_amdgcn_make_buffer_rsrc(a.qrot + hrow * kRope, 0, (last + 1) * 128, kRsrcFlags);
                lds_copy(rs, dst + kQaOff + 1024 * id, 16, rot_voff(id, lane, last));
            } else if (id < kRotCopies + kRowCopies) {
                const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(a.q + trow0 * kDqk), 0,
                                                                  last * Hq * 384 + 384, kRsrcFlags);
                const int k = id - kRotCopies;
                lds_copy(rs, dst + kQbOff + 1024 * k, 16, row_voff(k, lane, last, Hq * 384) + 128);
            } else if (id < kRotCopies + 2 * kRowCopies) {
                const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(a.dout + trow0 * kDv), 0,
                                                                  last * Hq * 256 + 256, kRsrcFlags);
                const int k = id - kRotCopies - kRowCopies;
                lds_copy(rs, dst + kObOff + 1024 * k, 16, row_voff(k, lane, last, Hq * 256));
            } else if (id < kStageCopies) {
                const bool isL = id == kStageCopies - 2;
                const float *src = isL ? a.lse + hrow : a.D + hrow;
                const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(src), 0, (last + 1) * 4, kRsrcFlags);
                lds_copy(rs, dst + (isL ? kLOff : kDOff), 4, min(lane, last) * 4);
            }
        }
    };

    copy_stage(0, 0);
    __syncthreads();   // also waits for this wave's copies
    for (int s_ = 0; s_ < n_stage; ++s_) {
        const int q0 = stage_q0(s_);
        const int buf = s_ & 1;
        // the next stage goes to the other buffer, last read in the previous stage
        if (s_ + 1 < n_stage) copy_stage(s_ + 1, buf ^ 1);
        const uint16_t *Qa = reinterpret_cast<const uint16_t *>(stg[buf] + kQaOff);
        const uint16_t *Qb = reinterpret_cast<const uint16_t *>(stg[buf] + kQbOff);
        const uint16_t *Ob = reinterpret_cast<const uint16_t *>(stg[buf] + kObOff);
        const float *Ls = reinterpret_cast<const float *>(stg[buf] + kLOff);
        const float *Ds = reinterpret_cast<const float *>(stg[buf] + kDOff);
        // does this wave's key range meet the block's queries? (wave-uniform)
        if (!(kw0 > q0 + 31 || q0 > wq_hi)) {
            f32x4 S[2], DP[2];
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                S[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
                DP[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
            {
                // S (2 query blocks x 6 chunks) and dP (2 x 4) interleaved, RS fragment
                // reads in flight
                constexpr int RS = 8;
                auto faddr = [&](int i) {   // i < 12: S (qb, c); else dP
                    const int u = i < 12 ? i : i - 12;
                    const int qb = i < 12 ? u / 6 : u / 4, c = i < 12 ? u % 6 : u % 4;
                    const int row = prow0 + 4 * qb;
                    return i < 12 ? (c < 2 ? Qa + row * kRotStr + 32 * c : Qb + row * kRowStr + 32 * (c - 2)) + 8 * g4
                                  : Ob + row * kRowStr + 32 * c + 8 * g4;
                };
                auto order = [](int i) { return i < 16 ? ((i & 1) ? 12 + (i >> 1) : (i >> 1)) : i - 8; };
                u32x4 fr[RS];
#pragma unroll
                for (int i = 0; i < RS; ++i) fr[i] = lds128(faddr(order(i)));
#pragma unroll
                for (int i = 0; i < 20; ++i) {
                    const int u = order(i);
                    if (u < 12) S[u / 6] = mfma16(fr[i % RS], kf[u % 6], S[u / 6]);
                    else DP[(u - 12) / 4] = mfma16(fr[i % RS], vf[(u - 12) % 4], DP[(u - 12) / 4]);
                    if (i + RS < 20) fr[i % RS] = lds128(faddr(order(i + RS)));
                }
                __builtin_amdgcn_sched_group_barrier(0x100, RS, 0);
#pragma unroll
                for (int i = 0; i < 20 - RS; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, RS, 0);
            }

            // element i of block qb: query q0 + 8 g4 + 4 qb + i, key j.  A stage whose
            // every query sees every key of the wave needs no mask; otherwise, less
            // q0 + 8 g4, the queries key j is seen by form a range [lo, hi] and query c
            // is in it when c - lo <= hi - lo as unsigned.
            const bool full = (kw0 + KPW <= a.T) && (q0 + 32 <= a.T) && (kw0 + KPW - 1 <= q0) && (q0 + 31 - kw0 < win);
            int lo = 0;
            uint32_t span = 0xffffffffu;
            if (!full) {
                lo = j - q0 - 8 * g4;
                const int hi = (int)min((int64_t)j + win - 1, (int64_t)a.T - 1) - q0 - 8 * g4;
                span = (uint32_t)(hi - lo);
                if (!jval || hi < lo) {   // nothing visible
                    lo = 0x40000000;
                    span = 0;
                }
            }
            u32x4 pb, dsb;
            {
                // the lane's 8 query rows are consecutive: their L and D in two 16-byte reads
                // each, read as integer vectors (as float vectors the compiler could not tell
                // them from the next stage's copies in flight and waited for those first)
                const u32x4 l0 = *reinterpret_cast<const u32x4 *>(Ls + 8 * g4);
                const u32x4 l1 = *reinterpret_cast<const u32x4 *>(Ls + 8 * g4 + 4);
                const u32x4 d0 = *reinterpret_cast<const u32x4 *>(Ds + 8 * g4);
                const u32x4 d1 = *reinterpret_cast<const u32x4 *>(Ds + 8 * g4 + 4);
                float lrow[8], drow[8];
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    lrow[x] = __uint_as_float(l0[x]);
                    lrow[4 + x] = __uint_as_float(l1[x]);
                    drow[x] = __uint_as_float(d0[x]);
                    drow[4 + x] = __uint_as_float(d1[x]);
                }
                float p8[8], d8[8];
#pragma unroll
                for (int x = 0; x < 8; ++x) {
                    const float sx = S[x >> 2][x & 3], dpx = DP[x >> 2][x & 3];
                    float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sx, cl2, -lrow[x] * kLog2e));
                    if (!full && (uint32_t)(x - lo) > span) p = 0.0f;
                    p8[x] = p;
                    d8[x] = p * (dpx * a.v_scale - drow[x]);
                }
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    pb[x] = pack_bf16(p8[2 * x], p8[2 * x + 1]);
                    dsb[x] = pack_bf16(d8[2 * x], d8[2 * x + 1]);
                }
            }
            // dV^T (128 x 16 keys) += dO^T P;  dK~^T (192 x 16 keys) += Q~^T dS: 20
            // MFMAs, RD fragments (two transpose loads each) in flight
            __builtin_amdgcn_sched_barrier(0);
            {
                constexpr int RD = 8;
                auto fload = [&](int i) {   // i < 8: dV block i; else dK block i - 8
                    if (i < 8) return lds_tr8(Ob + trow * kRowStr + 16 * i + tcol, kRowStr);
                    const int mb = i - 8;
                    return mb < 4 ? lds_tr8(Qa + trow * kRotStr + 16 * mb + tcol, kRotStr)
                                  : lds_tr8(Qb + trow * kRowStr + 16 * (mb - 4) + tcol, kRowStr);
                };
                u32x4 fr[RD];
#pragma unroll
                for (int i = 0; i < RD; ++i) fr[i] = fload(i);
#pragma unroll
                for (int i = 0; i < 20; ++i) {
                    if (i < 8) dV[i] = mfma16(fr[i % RD], pb, dV[i]);
                    else dK[i - 8] = mfma16(fr[i % RD], dsb, dK[i - 8]);
                    if (i + RD < 20) fr[i % RD] = fload(i + RD);
                }
                __builtin_amdgcn_sched_group_barrier(0x100, 2 * RD, 1);
#pragma unroll
                for (int i = 0; i < 20 - RD; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
                    __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, RD, 1);
            }
        }
        __syncthreads();   // this stage's reads are done; also waits for this wave's copies of the next
    }

    // ---- epilogue: dK[mb][i] / dV[mb][i] hold dim 16 mb + 4 g4 + i of key j
    if (!jval) return;
#pragma unroll
    for (int mb = 0; mb < 12; ++mb) dK[mb] *= a.scale;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int d = 16 * mb + 4 * g4 + i;   // < 32: rotary pair (d, d + 32) = blocks mb, mb + 2
            float x = dK[mb][i], y = dK[mb + 2][i];
            rope_back(x, y, a.rt.turn[d], a.pos0 + j);
            dK[mb][i] = x;
            dK[mb + 2][i] = y;
        }
    const size_t orow = ((size_t)b * a.T + j) * a.Hkv + g;
    uint16_t *dk = a.dk + orow * kDqk + 4 * g4;
    uint16_t *dv = a.dv + orow * kDv + 4 * g4;
#pragma unroll
    for (int mb = 0; mb < 12; ++mb) {
        u32x2 o;
        o[0] = pack_bf16(dK[mb][0], dK[mb][1]);
        o[1] = pack_bf16(dK[mb][2], dK[mb][3]);
        *reinterpret_cast<u32x2 *>(dk + 16 * mb) = o;
    }
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
        u32x2 o;
        o[0] = pack_bf16(dV[mb][0] * a.v_scale, dV[mb][1] * a.v_scale);
        o[1] = pack_bf16(dV[mb][2] * a.v_scale, dV[mb][3] * a.v_scale);
        *reinterpret_cast<u32x2 *>(dv + 16 * mb) = o;
    }
}

size_t backward_workspace_bytes(int32_t B, int32_t T, int32_t Hq, int32_t Hkv) {
    const size_t rows = (size_t)B * T * Hq, krows = (size_t)B * T * Hkv;
    return (rows + krows) * kRope * sizeof(uint16_t) + (rows + (size_t)B * ((T + 31) / 32) * Hq) * sizeof(float);
}

hipError_t launch_backward(BwdArgs a, hipStream_t stream) {
    const int G = a.Hq / a.Hkv;
    if (G % 4 != 0) return hipErrorInvalidValue;
    a.n_qblk = (a.T + 31) / 32;
    a.n_hgrp = G / 4;
    constexpr int kDkdvWaves = 4;
    a.n_kblk = (a.T + 16 * kDkdvWaves - 1) / (16 * kDkdvWaves);
    const int64_t krot_threads = (int64_t)a.B * a.T * a.Hkv * 4;
    hipLaunchKernelGGL(bwd_krot_kernel, dim3((unsigned)((krot_threads + 255) / 256)), dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // dq also forms D and the sink partials; d sink and dk/dv read them
    const int64_t qblocks = (int64_t)a.B * a.Hkv * a.n_hgrp * a.n_qblk;
    hipLaunchKernelGGL(bwd_dq_kernel, dim3((unsigned)qblocks), dim3(256), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.sinks) {
        hipLaunchKernelGGL(bwd_sink_kernel, dim3(a.Hq), dim3(256), 0, stream, a);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int64_t kblocks = (int64_t)a.B * a.Hkv * a.n_kblk;
    hipLaunchKernelGGL(bwd_dkdv_kernel<kDkdvWaves>, dim3((unsigned)kblocks), dim3(64 * kDkdvWaves), 0, stream, a);
    return hipGetLastError();
}

}  // namespace mimo
