// Prefill attention for both layer types of MiMo-V2.6-Flash on gfx950.
//
// Sliding-window layers: 64 query heads over 8 KV heads, a 128-key window and a
// per-head sink (techniques map page, rows Sliding-window attention, Learnable
// attention sink, Grouped-query attention).  Global layers: 64 over 4 KV heads,
// full causal attention, run one query chunk at a time against its whole
// prefix (Gaudi recipe page, Launch section: tiled global prefill).
//
// Design (one workgroup = NW query heads of one GQA group x 32 query tokens;
// one wave per head, two waves per SIMD):
//   * S^T = K Q^T and O^T = V^T P^T on 32x32x16 bf16 MFMA.  With keys on the
//     MFMA's M side, every lane owns one query column, so the row max / row sum
//     of the softmax are in-lane plus one permlane32 swap.
//   * Q lives in registers for the whole kernel (B operand), rotated once on
//     load.  Each K/V tile of NK keys is staged once per workgroup in LDS
//     (double-buffered) and read by all NW heads: K rotated on its way in
//     (fused RoPE; angle = exact fixed-point tile base + per-row offset), V
//     transposed on its way in (the PV contraction runs over keys).
//   * K rows are read from LDS in a bit-permuted order (bits 2 and 3 of the row
//     swapped) so that the S^T accumulator registers of a lane hold 8
//     consecutive keys, which are exactly its P^T operand for the PV MFMA, with
//     no data movement between the two products.
//   * Online softmax in the exp2 domain with the sink folded in as the initial
//     (max, sum) = (sink * log2 e, 1); the running max is only raised when it
//     grows by more than 2^8, which keeps every exponent <= 2^8.
//   * Tiles wholly outside the causal band are never visited; only edge tiles
//     evaluate the mask.  Workgroups are mapped XCD-aware (each XCD streams the
//     K/V of one set of KV heads, sequence after sequence of the batch) and
//     longest-first for causal balance.
//   * Two shapes: 8 heads x 64-key tiles (88 KB of LDS, one workgroup per CU;
//     long global prefixes) and 4 heads x 32-key tiles (46 KB, two workgroups
//     per CU so one's prologue and stores overlap the other's math; the short
//     sliding-window band, where 32-key tiles also waste fewer masked keys).
#include "kernels.hpp"

namespace mimo {

namespace {

constexpr int KSTR = kDqk + 8;          // LDS row stride of a K tile (bf16)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();
constexpr int RING = 4;                 // LDS fragment reads issued ahead of their MFMA

__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

__device__ __forceinline__ u32x4 lds128(const uint16_t *p) {
    return *reinterpret_cast<const u32x4 *>(p);
}

// ---- one query row's output, o = inv * O, as bf16 with 16-byte stores.  In the
// O^T accumulators lane half h2 holds dims 32 mb + 8 a4 + 4 h2 + (0..3); one lane
// swap per pair of 4-dim pieces gives the lower half all 8 dims of the even pieces
// and the upper half those of the odd ones.
__device__ __forceinline__ void store_out_row(const f32x16 (&O)[4], float inv, uint16_t *dst, int h2) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int a2 = 0; a2 < 2; ++a2) {
            u32x2 pe, po;   // pieces a4 = 2 a2 and 2 a2 + 1
            pe[0] = pack_bf16(O[mb][8 * a2] * inv, O[mb][8 * a2 + 1] * inv);
            pe[1] = pack_bf16(O[mb][8 * a2 + 2] * inv, O[mb][8 * a2 + 3] * inv);
            po[0] = pack_bf16(O[mb][8 * a2 + 4] * inv, O[mb][8 * a2 + 5] * inv);
            po[1] = pack_bf16(O[mb][8 * a2 + 6] * inv, O[mb][8 * a2 + 7] * inv);
            // upper lanes' pe <-> lower lanes' po
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                const auto r = __builtin_amdgcn_permlane32_swap(pe[x], po[x], false, false);
                pe[x] = r[0];
                po[x] = r[1];
            }
            const u32x4 o = {pe[0], pe[1], po[0], po[1]};
            *reinterpret_cast<u32x4 *>(dst + 32 * mb + 8 * (2 * a2 + h2)) = o;
        }
}

// ---- which (query block, batch, KV head, head group) workgroup blockIdx.x owns.
// With the (KV head, head group) pairs split evenly over the 8 XCDs, an XCD walks
// its pairs sequence by sequence, query blocks longest-first: its resident
// workgroups then sweep the same K/V rows together (L2 reuse), and every XCD gets
// the same share of every sequence.
__device__ __forceinline__ void map_block(const PrefillArgs &a, int &qb, int &b, int &pair) {
    const int P = a.Hkv * a.n_hgrp;
    const int i = blockIdx.x;
    if (a.xcd_remap == 2) {
        const int x = i & 7, j = i >> 3, ppx = P >> 3;
        const int per_b = ppx * a.n_qblk;
        b = j / per_b;
        const int r = j - b * per_b;
        pair = x * ppx + r % ppx;
        qb = a.n_qblk - 1 - r / ppx;
    } else if (a.xcd_remap == 1) {
        const int combos = a.B * P;
        const int x = i & 7, j = i >> 3, cpx = combos >> 3;
        const int c = x * cpx + j % cpx;
        qb = a.n_qblk - 1 - j / cpx;
        b = c % a.B;
        pair = c / a.B;
    } else {
        const int combos = a.B * P;
        const int c = i % combos;
        qb = a.n_qblk - 1 - i / combos;
        b = c % a.B;
        pair = c / a.B;
    }
}

}  // namespace

template <int NW, int NK>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * NW, 64 * NW), amdgpu_waves_per_eu(2, 2)))
void prefill_kernel(PrefillArgs a) {
    constexpr int QW = 32;                          // queries per wave (one MFMA column block)
    constexpr int NT = 64 * NW;
    constexpr int KB = NK / 32;                     // 32-key MFMA row blocks per tile
    constexpr int VSTR = NK + 8;                    // LDS row stride of a V^T tile (bf16)
    constexpr int K_TILE = NK * KSTR;
    constexpr int V_TILE = kDv * VSTR;
    constexpr int STAGE = K_TILE + V_TILE;
    // staging work per tile, spread evenly over the NT threads
    constexpr int ROT_UNITS = NK * 8;               // (row, 4 rotating pairs): 8-byte pieces
    constexpr int PLAIN_UNITS = NK * 16;            // (row, 16-byte pass-through chunk)
    constexpr int V_UNITS = (NK / 2) * 16;          // (key pair, 8-dv chunk)
    constexpr int ROT_PER = ROT_UNITS / NT, PLAIN_PER = PLAIN_UNITS / NT, V_PER = V_UNITS / NT;
    static_assert(ROT_UNITS % NT == 0 && PLAIN_UNITS % NT == 0 && V_UNITS % NT == 0, "staging split");
    static_assert(NK % 32 == 0, "tile of whole MFMA blocks");

    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * STAGE];
    __shared__ float2 rope_base[2][kPairs];

    const int tid = threadIdx.x;
    // w through readfirstlane: the head, and so its sink, are then known to be
    // wave-uniform, and the sink comes by a scalar load whose wait is not a wait
    // for Q's vector loads
    const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h2 = lane >> 5, l32 = lane & 31;

    int qb, b, pair;
    map_block(a, qb, b, pair);
    const int hg = pair % a.n_hgrp;
    const int g = pair / a.n_hgrp;
    const int G = a.Hq / a.Hkv;
    const int head = g * G + hg * NW + w;
    const int q0 = qb * QW;

    // ---- this sequence's tokens: dense [B, T, H, D] batches, or packed
    // sequences (offsets cu_q / cu_k) whose queries are the last Tq of their keys
    int Tq, Tk;
    size_t q_tok0, k_tok0, lse_off;
    int64_t q_pos0, k_pos0;
    if (a.cu_q) {
        const int qs = a.cu_q[b], ks = a.cu_k[b];
        Tq = a.cu_q[b + 1] - qs;
        Tk = a.cu_k[b + 1] - ks;
        q_tok0 = (size_t)qs;
        k_tok0 = (size_t)ks;
        k_pos0 = a.kpos ? a.kpos[b] : 0;
        q_pos0 = k_pos0 + Tk - Tq;
        lse_off = (size_t)qs;
    } else {
        Tq = a.Tq;
        Tk = a.Tk;
        q_tok0 = (size_t)b * a.Tq;
        k_tok0 = (size_t)b * a.Tk;
        q_pos0 = a.q_pos0;
        k_pos0 = a.k_pos0;
        lse_off = (size_t)b * a.Hq * a.Tq;
    }
    if (q0 >= Tq) return;   // whole workgroup: a packed sequence shorter than the longest

    const size_t krow_stride = (size_t)a.Hkv * kDqk;
    const size_t vrow_stride = (size_t)a.Hkv * kDv;
    const uint16_t *kbase = a.k + k_tok0 * krow_stride + (size_t)g * kDqk;
    const uint16_t *vbase = a.v + k_tok0 * vrow_stride + (size_t)g * kDv;

    // ---- key range of the block
    const int t_last = min(q0 + QW, Tq) - 1;
    const int64_t qp_lo = q_pos0 + q0;
    const int64_t qp_hi = q_pos0 + t_last;
    int64_t jlo = 0;
    if (a.window > 0) jlo = qp_lo - a.window + 1 - k_pos0;
    if (jlo < 0) jlo = 0;
    int64_t jhi = qp_hi - k_pos0;
    if (jhi > Tk - 1) jhi = Tk - 1;
    const int tile_lo = (int)(jlo / NK);
    const int tile_hi = jhi >= jlo ? (int)(jhi / NK) : tile_lo - 1;

    // ---- Q in registers (B operand): lane holds dims [96*h2, 96*h2+96) of query q0 + l32;
    // rotated below, once the first tile's loads are in flight beside these
    u32x4 qr[12];
    const bool q_valid = q0 + l32 < Tq;
    if (q_valid) {
        const uint16_t *src = a.q + ((q_tok0 + q0 + l32) * a.Hq + head) * kDqk + 96 * h2;
#pragma unroll
        for (int ks = 0; ks < 12; ++ks) qr[ks] = ldg128(src + 8 * ks);
    } else {
#pragma unroll
        for (int ks = 0; ks < 12; ++ks) qr[ks] = u32x4{0, 0, 0, 0};
    }

    // ---- softmax state of this lane's query column
    float m_run = a.sinks ? a.sinks[head] * kLog2e : kNegInf;
    float l_run = (a.sinks && h2 == 0) ? 1.0f : 0.0f;
    f32x16 O[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) O[mb][e] = 0.0f;

    // ---- staging: fixed per-thread pieces of every tile
    // rotating K piece r: row u>>3, pairs 4*(u&7)..+3; pass-through chunk r: row u>>4,
    // chunk 8+(u&15); V block r: key pair u%(NK/2) (consecutive lanes), 8-dv chunk u/(NK/2)
    int k_rot_off[ROT_PER], k_rot_row[ROT_PER], k_pl_off[PLAIN_PER], v_off[V_PER];
    float rope_oc[ROT_PER][4], rope_os[ROT_PER][4];   // cos/sin(row * theta) of the piece's pairs
#pragma unroll
    for (int r = 0; r < ROT_PER; ++r) {
        const int u = tid + r * NT, row = u >> 3, hq = u & 7;
        k_rot_row[r] = row;
        k_rot_off[r] = row * (int)krow_stride + 4 * hq;
#pragma unroll
        for (int e = 0; e < 4; ++e) turn_sincos((uint64_t)row * a.rt.turn[4 * hq + e], rope_os[r][e], rope_oc[r][e]);
    }
#pragma unroll
    for (int r = 0; r < PLAIN_PER; ++r) {
        const int u = tid + r * NT;
        k_pl_off[r] = (u >> 4) * (int)krow_stride + 8 * (8 + (u & 15));
    }
#pragma unroll
    for (int r = 0; r < V_PER; ++r) {
        const int u = tid + r * NT;
        v_off[r] = 2 * (u % (NK / 2)) * (int)vrow_stride + 8 * (u / (NK / 2));
    }
    // exact cos/sin(tile position * theta_i) for the 32 pairs, one tile ahead, two
    // slots; lane i < 32 of wave 0 loads pair i's frequency once
    const uint64_t my_turn = a.rt.turn[tid & (kPairs - 1)];
    auto tile_bases = [&](int jt) {
        if (tid < kPairs) {
            float sn, cs;
            turn_sincos((uint64_t)(k_pos0 + (int64_t)jt * NK) * my_turn, sn, cs);
            rope_base[jt & 1][tid] = float2{cs, sn};
        }
    };

    u32x2 k_rx[ROT_PER], k_ry[ROT_PER];
    u32x4 k_pl[PLAIN_PER], v_st[V_PER][2];

    auto load_tile = [&](int jt) {
        const int j0 = jt * NK;
        const uint16_t *kt = kbase + (size_t)j0 * krow_stride;
        const uint16_t *vt = vbase + (size_t)j0 * vrow_stride;
        if (j0 + NK <= Tk) {
#pragma unroll
            for (int r = 0; r < ROT_PER; ++r) {
                k_rx[r] = *reinterpret_cast<const u32x2 *>(kt + k_rot_off[r]);
                k_ry[r] = *reinterpret_cast<const u32x2 *>(kt + k_rot_off[r] + 32);
            }
#pragma unroll
            for (int r = 0; r < PLAIN_PER; ++r) k_pl[r] = ldg128(kt + k_pl_off[r]);
#pragma unroll
            for (int r = 0; r < V_PER; ++r) {
                v_st[r][0] = ldg128(vt + v_off[r]);
                v_st[r][1] = ldg128(vt + v_off[r] + vrow_stride);
            }
        } else {   // ragged last tile: rows past Tk are zero
            const int nrow = Tk - j0;
#pragma unroll
            for (int r = 0; r < ROT_PER; ++r) {
                const bool ok = k_rot_row[r] < nrow;
                k_rx[r] = ok ? *reinterpret_cast<const u32x2 *>(kt + k_rot_off[r]) : u32x2{0, 0};
                k_ry[r] = ok ? *reinterpret_cast<const u32x2 *>(kt + k_rot_off[r] + 32) : u32x2{0, 0};
            }
#pragma unroll
            for (int r = 0; r < PLAIN_PER; ++r) {
                const int u = tid + r * NT;
                k_pl[r] = ((u >> 4) < nrow) ? ldg128(kt + k_pl_off[r]) : u32x4{0, 0, 0, 0};
            }
#pragma unroll
            for (int r = 0; r < V_PER; ++r) {
                const int u = tid + r * NT, k2 = 2 * (u % (NK / 2));
                v_st[r][0] = (k2 < nrow) ? ldg128(vt + v_off[r]) : u32x4{0, 0, 0, 0};
                v_st[r][1] = (k2 + 1 < nrow) ? ldg128(vt + v_off[r] + vrow_stride) : u32x4{0, 0, 0, 0};
            }
        }
    };

    auto store_tile = [&](int jt, int buf) {
        uint16_t *Ks = smem + buf * STAGE;
        uint16_t *Vs = Ks + K_TILE;
#pragma unroll
        for (int r = 0; r < ROT_PER; ++r) {
            const int u = tid + r * NT;
            const int row = u >> 3, hq = u & 7;
            u32x2 x = k_rx[r], y = k_ry[r];
            const float4 b01 = *reinterpret_cast<const float4 *>(&rope_base[jt & 1][4 * hq]);
            const float4 b23 = *reinterpret_cast<const float4 *>(&rope_base[jt & 1][4 * hq + 2]);
            const float bc[4] = {b01.x, b01.z, b23.x, b23.z}, bs[4] = {b01.y, b01.w, b23.y, b23.w};
#pragma unroll
            for (int wd = 0; wd < 2; ++wd) {
                // angle(tile position + row) = base(tile) + offset(row)
                const int e0 = 2 * wd, e1 = 2 * wd + 1;
                const float c0 = bc[e0] * rope_oc[r][e0] - bs[e0] * rope_os[r][e0];
                const float s0 = bs[e0] * rope_oc[r][e0] + bc[e0] * rope_os[r][e0];
                const float c1 = bc[e1] * rope_oc[r][e1] - bs[e1] * rope_os[r][e1];
                const float s1 = bs[e1] * rope_oc[r][e1] + bc[e1] * rope_os[r][e1];
                const float x0 = bf_lo(x[wd]), x1 = bf_hi(x[wd]);
                const float y0 = bf_lo(y[wd]), y1 = bf_hi(y[wd]);
                x[wd] = pack_bf16(x0 * c0 - y0 * s0, x1 * c1 - y1 * s1);
                y[wd] = pack_bf16(y0 * c0 + x0 * s0, y1 * c1 + x1 * s1);
            }
            *reinterpret_cast<u32x2 *>(Ks + row * KSTR + 4 * hq) = x;
            *reinterpret_cast<u32x2 *>(Ks + row * KSTR + 4 * hq + 32) = y;
        }
#pragma unroll
        for (int r = 0; r < PLAIN_PER; ++r) {
            const int u = tid + r * NT;
            const int row = u >> 4, cc = 8 + (u & 15);
            *reinterpret_cast<u32x4 *>(Ks + row * KSTR + 8 * cc) = k_pl[r];
        }
#pragma unroll
        for (int r = 0; r < V_PER; ++r) {
            const int u = tid + r * NT;
            const int kp = u % (NK / 2), cc = u / (NK / 2);
            // 2 keys x 8 dv -> 8 dv rows of V^T, one dword (2 keys) each
#pragma unroll
            for (int d = 0; d < 8; ++d) {
                const uint32_t sel = (d & 1) ? 0x07060302u : 0x05040100u;
                const uint32_t wv = __builtin_amdgcn_perm(v_st[r][1][d >> 1], v_st[r][0][d >> 1], sel);
                *reinterpret_cast<uint32_t *>(Vs + (8 * cc + d) * VSTR + 2 * kp) = wv;
            }
        }
    };

    const float cl2 = a.scale_log2;
    // K row read order: bits 2 and 3 of the row index swapped
    const int prow = (l32 & 0x13) | ((l32 & 4) << 1) | ((l32 & 8) >> 1);
    const int64_t qp = q_pos0 + q0 + l32;

    // the first tile's loads go out beside Q's, so the two round trips overlap
    if (tile_hi >= tile_lo) load_tile(tile_lo);
    if (q_valid && h2 == 0) {
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) rope_rotate8(qr[cc], qr[cc + 4], a.rt, 8 * cc, qp);
    }
    if (tile_hi >= tile_lo) {
        tile_bases(tile_lo);
        if (tile_lo + 1 <= tile_hi) tile_bases(tile_lo + 1);
        __syncthreads();
        store_tile(tile_lo, 0);
    }
    __syncthreads();

    for (int jt = tile_lo; jt <= tile_hi; ++jt) {
        const int buf = (jt - tile_lo) & 1;
        const bool has_next = jt < tile_hi;
        if (has_next) load_tile(jt + 1);
        if (jt + 2 <= tile_hi) tile_bases(jt + 2);   // slot jt&1: last read by store_tile(jt)

        const uint16_t *Ks = smem + buf * STAGE;
        const uint16_t *Vs = Ks + K_TILE;
        const int j0 = jt * NK;

        // ---- S^T = K Q^T: KB key blocks of 32 x 32 queries, RING fragment reads in flight
        f32x16 S[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int e = 0; e < 16; ++e) S[kb][e] = 0.0f;
        {
            const uint16_t *kr0 = Ks + prow * KSTR + 96 * h2;
            auto kaddr = [&](int i) { return kr0 + (i % KB) * 32 * KSTR + 8 * (i / KB); };
            u32x4 kf[RING];
#pragma unroll
            for (int i = 0; i < RING; ++i) kf[i] = lds128(kaddr(i));
#pragma unroll
            for (int i = 0; i < 12 * KB; ++i) {
                S[i % KB] = mfma32(kf[i % RING], qr[i / KB], S[i % KB]);
                if (i + RING < 12 * KB) kf[i % RING] = lds128(kaddr(i + RING));
            }
            // keep RING reads in flight (the 64-key shape has no registers to spare for
            // it: pinned there, it spills)
            if constexpr (NK == 32) {
                __builtin_amdgcn_sched_group_barrier(0x100, RING, 0);   // LDS reads
    #pragma unroll
                for (int i = 0; i < 12 * KB - RING; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, RING, 0);
            }
        }

        // ---- mask on edge tiles only (offsets are small there, so 32-bit)
        const int64_t kp0 = k_pos0 + j0;
        const bool full = (j0 + NK <= Tk) && (kp0 + NK - 1 <= qp_lo) &&
                          (a.window == 0 || qp_hi - kp0 < a.window);
        if (!full) {
            int64_t d64 = qp - kp0;
            d64 = d64 < -(1 << 30) ? -(1 << 30) : (d64 > (1 << 30) ? (1 << 30) : d64);
            const int d = (int)d64;                 // query position - first key position
            const int kmax = Tk - j0;             // keys past the end of k/v
            const int win = a.window > 0 ? a.window : 0x7fffffff;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int jrel = 32 * kb + 16 * (e >> 3) + 8 * h2 + (e & 7);
                    const bool vis = (jrel < kmax) && (jrel <= d) && (d - jrel < win);
                    if (!vis) S[kb][e] = kNegInf;
                }
        }

        // ---- online softmax (exp2 domain), lazy rescale
        float mx = kNegInf;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int e = 0; e < 16; ++e) mx = fmaxf(mx, S[kb][e]);
        mx = max_xor32(mx);
        const float mc = mx * cl2;
        const bool need = mc > m_run + 8.0f;
        if (__any(need)) {
            const float alpha = need ? __builtin_amdgcn_exp2f(m_run - mc) : 1.0f;
            if (need) m_run = mc;
            l_run *= alpha;
#pragma unroll
            for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                for (int e = 0; e < 16; ++e) O[mb][e] *= alpha;
        }
        const float mu = (m_run == kNegInf) ? 0.0f : m_run;
        u32x4 P[KB][2];   // [kb][s]
        float ls[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kb][e], cl2, -mu));
                S[kb][e] = p;
                ls[e & 3] += p;
            }
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int x = 0; x < 4; ++x)
                    P[kb][s][x] = pack_bf16(S[kb][8 * s + 2 * x], S[kb][8 * s + 2 * x + 1]);
        }
        l_run += (ls[0] + ls[1]) + (ls[2] + ls[3]);

        // ---- O^T += V^T P^T, RING fragment reads in flight
        {
            const uint16_t *vr0 = Vs + l32 * VSTR + 8 * h2;
            // i = (mb, kb, s): dv block mb, key block kb, 16-key step s
            auto vaddr = [&](int i) {
                const int mb = i / (2 * KB), kb = (i / 2) % KB, s = i & 1;
                return vr0 + mb * 32 * VSTR + 32 * kb + 16 * s;
            };
            u32x4 vf[RING];
#pragma unroll
            for (int i = 0; i < RING; ++i) vf[i] = lds128(vaddr(i));
#pragma unroll
            for (int i = 0; i < 8 * KB; ++i) {
                O[i / (2 * KB)] = mfma32(vf[i % RING], P[(i / 2) % KB][i & 1], O[i / (2 * KB)]);
                if (i + RING < 8 * KB) vf[i % RING] = lds128(vaddr(i + RING));
            }
            if constexpr (NK == 32) {
                __builtin_amdgcn_sched_group_barrier(0x100, RING, 1);
    #pragma unroll
                for (int i = 0; i < 8 * KB - RING; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, RING, 1);
            }
        }

        if (has_next) store_tile(jt + 1, buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: o = v_scale * O / l, bf16
    const float lt = sum_xor32(l_run);
    const int t = q0 + l32;
    if (t < Tq) {
        const float inv = lt > 0.0f ? a.v_scale / lt : 0.0f;
        uint16_t *dst = a.out + ((q_tok0 + t) * a.Hq + head) * kDv;
        store_out_row(O, inv, dst, h2);
        if (a.lse && h2 == 0)
            a.lse[lse_off + (size_t)head * a.lse_hstride + t] = lt > 0.0f ? (m_run + log2f(lt)) * kLn2 : kNegInf;
    }
}


// ---- K/V tile images for the global kernel below.  Every workgroup whose queries
// follow a key stages that key again (thousands of times over a long chunk), so
// rotating K and transposing V once per call, instead of once per workgroup and
// tile, takes that work out of the attention loop.  One workgroup
// per 64-key tile of one (sequence, KV head) writes the tile's exact LDS image:
// K rotated (rows padded to KSTR), then V^T (rows padded to kImgVS); rows past the
// sequence's end are zero.  Tiles of sequence b start at tile index
// floor(cu_k[b] / 64) + b (packed) or b * ceil(Tk / 64) (dense), and tile t of KV
// head g is image (start + t) * Hkv + g.
constexpr int kImgNK = 64;
constexpr int kPrepVS = kDv + 8;                             // V row stride while transposing
constexpr int kImgVS = kImgNK + 8;                           // V^T row stride in the image
constexpr int kImgK = kImgNK * KSTR;                         // bf16 elements
constexpr int kImgTile = kImgK + kDv * kImgVS;               // 22016 bf16 = 43 KiB
constexpr float kSkipMax = 32.0f;   // exp2-domain headroom before the row max is needed

// Sum of squares of 8 bf16 values.
__device__ __forceinline__ float sumsq8(u32x4 x) {
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float lo = bf_lo(x[i]), hi = bf_hi(x[i]);
        s = __builtin_fmaf(lo, lo, s);
        s = __builtin_fmaf(hi, hi, s);
    }
    return s;
}

__global__ __launch_bounds__(256) void kv_image_kernel(PrefillArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t vs[kImgNK * kPrepVS];
    // squared norms of each rotated key row's pieces: 4 rotating (row, 8 pairs)
    // pieces, then the 16 pass-through chunks; summed in this order by one lane
    __shared__ float rn[kImgNK][4 + 16];
    const int b = blockIdx.y, g = blockIdx.z, tid = threadIdx.x;
    int Tk, tile_base;
    size_t k_tok0;
    int64_t k_pos0;
    if (a.cu_k) {
        const int ks = a.cu_k[b];
        Tk = a.cu_k[b + 1] - ks;
        k_tok0 = (size_t)ks;
        k_pos0 = a.kpos ? a.kpos[b] : 0;
        tile_base = ks / kImgNK + b;
    } else {
        Tk = a.Tk;
        k_tok0 = (size_t)b * a.Tk;
        k_pos0 = a.k_pos0;
        tile_base = b * ((a.Tk + kImgNK - 1) / kImgNK);
    }
    const int ntile = (Tk + kImgNK - 1) / kImgNK;
    const size_t krow = (size_t)a.Hkv * kDqk, vrow = (size_t)a.Hkv * kDv;
    for (int t = blockIdx.x; t < ntile; t += gridDim.x) {
        const size_t tile_id = (size_t)(tile_base + t) * a.Hkv + g;
        uint16_t *wk = a.kv_img + tile_id * kImgTile;
        uint16_t *wv = wk + kImgK;
        const int j0 = t * kImgNK;
        {   // rotating chunks: row tid/4, pairs 8*(tid%4)..+7
            const int row = tid >> 2, cc = tid & 3, j = j0 + row;
            u32x4 x = {0, 0, 0, 0}, y = {0, 0, 0, 0};
            if (j < Tk) {
                const uint16_t *src = a.k + (k_tok0 + j) * krow + (size_t)g * kDqk;
                x = ldg128(src + 8 * cc);
                y = ldg128(src + 32 + 8 * cc);
                rope_rotate8(x, y, a.rt, 8 * cc, k_pos0 + j);
            }
            *reinterpret_cast<u32x4 *>(wk + row * KSTR + 8 * cc) = x;
            *reinterpret_cast<u32x4 *>(wk + row * KSTR + 32 + 8 * cc) = y;
            rn[row][cc] = sumsq8(x) + sumsq8(y);
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) {   // pass-through chunks 8..23
            const int u = tid + 256 * m, row = u >> 4, c = 8 + (u & 15), j = j0 + row;
            u32x4 x = {0, 0, 0, 0};
            if (j < Tk) x = ldg128(a.k + (k_tok0 + j) * krow + (size_t)g * kDqk + 8 * c);
            *reinterpret_cast<u32x4 *>(wk + row * KSTR + 8 * c) = x;
            rn[row][4 + (u & 15)] = sumsq8(x);
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) {   // V rows into LDS
            const int u = tid + 256 * m, row = u >> 4, c = u & 15, j = j0 + row;
            u32x4 x = {0, 0, 0, 0};
            if (j < Tk) x = ldg128(a.v + (k_tok0 + j) * vrow + (size_t)g * kDv + 8 * c);
            *reinterpret_cast<u32x4 *>(vs + row * kPrepVS + 8 * c) = x;
        }
        __syncthreads();
        if (tid < kImgNK) {   // wave 0: the tile's largest key norm, summed in a fixed order
            float ss = 0.0f;
#pragma unroll
            for (int i = 0; i < 4 + 16; ++i) ss += rn[tid][i];
            float n = sqrtf(ss);
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) n = fmaxf(n, __shfl_xor(n, off));
            if (tid == 0) a.kv_norm[tile_id] = n;
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) {   // V^T rows: dv, keys 8c..8c+7
            const int u = tid + 256 * m, dv = u >> 3, c = u & 7;
            u32x4 o;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                o[i] = (uint32_t)vs[(8 * c + 2 * i) * kPrepVS + dv] |
                       ((uint32_t)vs[(8 * c + 2 * i + 1) * kPrepVS + dv] << 16);
            *reinterpret_cast<u32x4 *>(wv + dv * kImgVS + 8 * c) = o;
        }
        __syncthreads();
    }
}

// ---- Global prefill over the tile images: the math of prefill_kernel<8, 64>
// (same workgroup shape, block mapping, MFMA layout and online softmax), with each
// tile moved HBM -> LDS by buffer loads that write LDS: 43 copies of 1 KiB, 16
// bytes per lane, straight into LDS.  No staging registers, no RoPE or transpose VALU
// work and no LDS stores remain in the loop.
template <int NW>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * NW, 64 * NW), amdgpu_waves_per_eu(2, 2)))
void prefill_image_kernel(PrefillArgs a) {
    constexpr int NK = 64;
    constexpr int QW = 32;
    constexpr int KB = NK / 32;
    constexpr int VSTR = NK + 8;
    constexpr int K_TILE = NK * KSTR;               // 25600 bytes
    constexpr int V_TILE = kDv * VSTR;              // 18432 bytes
    constexpr int STAGE = K_TILE + V_TILE;
    constexpr int K_OPS = K_TILE * 2 / 1024, V_OPS = V_TILE * 2 / 1024;   // 25 + 18 copies of 1 KiB
    constexpr int OPS = K_OPS + V_OPS;
    constexpr int OPW = (OPS + NW - 1) / NW;        // per wave
    constexpr int RQ = 6, RV = 8;                   // K / V^T fragment reads in flight
    static_assert(K_TILE * 2 % 1024 == 0 && V_TILE * 2 % 1024 == 0, "whole 1 KiB copies");
    static_assert(STAGE == kImgTile && VSTR == kImgVS, "prepared image = LDS stage");

    __shared__ __attribute__((aligned(1024))) uint16_t smem[2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h2 = lane >> 5, l32 = lane & 31;

    int qb, b, pair;
    map_block(a, qb, b, pair);
    const int hg = pair % a.n_hgrp;
    const int g = pair / a.n_hgrp;
    const int G = a.Hq / a.Hkv;
    const int head = g * G + hg * NW + w;
    const int q0 = qb * QW;

    int Tq, Tk, tile_base;
    size_t q_tok0, lse_off;
    int64_t q_pos0, k_pos0;
    if (a.cu_q) {
        const int qs = a.cu_q[b], ks = a.cu_k[b];
        Tq = a.cu_q[b + 1] - qs;
        Tk = a.cu_k[b + 1] - ks;
        q_tok0 = (size_t)qs;
        k_pos0 = a.kpos ? a.kpos[b] : 0;
        q_pos0 = k_pos0 + Tk - Tq;
        lse_off = (size_t)qs;
        tile_base = ks / NK + b;
    } else {
        Tq = a.Tq;
        Tk = a.Tk;
        q_tok0 = (size_t)b * a.Tq;
        q_pos0 = a.q_pos0;
        k_pos0 = a.k_pos0;
        lse_off = (size_t)b * a.Hq * a.Tq;
        tile_base = b * ((a.Tk + NK - 1) / NK);
    }
    if (q0 >= Tq) return;

    const int t_last = min(q0 + QW, Tq) - 1;
    const int64_t qp_lo = q_pos0 + q0;
    const int64_t qp_hi = q_pos0 + t_last;
    int64_t jlo = 0;
    if (a.window > 0) jlo = qp_lo - a.window + 1 - k_pos0;
    if (jlo < 0) jlo = 0;
    int64_t jhi = qp_hi - k_pos0;
    if (jhi > Tk - 1) jhi = Tk - 1;
    const int tile_lo = (int)(jlo / NK);
    const int tile_hi = jhi >= jlo ? (int)(jhi / NK) : tile_lo - 1;

    u32x4 qr[12];
    {
        const int t = q0 + l32;
        if (t < Tq) {
            const uint16_t *src = a.q + ((q_tok0 + t) * a.Hq + head) * kDqk + 96 * h2;
#pragma unroll
            for (int ks = 0; ks < 12; ++ks) qr[ks] = ldg128(src + 8 * ks);
            if (h2 == 0) {
                const int64_t qp = q_pos0 + t;
#pragma unroll
                for (int cc = 0; cc < 4; ++cc) rope_rotate8(qr[cc], qr[cc + 4], a.rt, 8 * cc, qp);
            }
        } else {
#pragma unroll
            for (int ks = 0; ks < 12; ++ks) qr[ks] = u32x4{0, 0, 0, 0};
        }
    }

    // |q| * scale * log2(e): with a tile's largest |k| it bounds every score of the
    // tile in the exp2 domain (Cauchy-Schwarz)
    float qbound;
    {
        float qss = 0.0f;
#pragma unroll
        for (int ks = 0; ks < 12; ++ks) qss += sumsq8(qr[ks]);
        qbound = sqrtf(sum_xor32(qss)) * a.scale_log2;
    }
    float m_run = a.sinks ? a.sinks[head] * kLog2e : kNegInf;
    float l_run = (a.sinks && h2 == 0) ? 1.0f : 0.0f;
    f32x16 O[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) O[mb][e] = 0.0f;

    // ---- a tile's image is STAGE contiguous elements: OPS copies of 1 KiB, op i
    // landing at LDS byte 1024 * i of the stage; wave w issues ops w, w + NW, ...
    // The copies are buffer loads (a resource spanning the one tile) rather than
    // global ones: a global load into LDS counts as both a vector-memory and an LDS
    // access, and while one is in flight every LDS wait is compiled as a full
    // drain, which would leave the fragment reads below one batch deep.
    auto copy_tile = [&](int jt, int buf) {
        const size_t tile_id = (size_t)(tile_base + jt) * a.Hkv + g;
        const __amdgpu_buffer_rsrc_t rsrc =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(a.kv_img + tile_id * STAGE), 0, STAGE * 2,
                                              0x00020000);
        uint16_t *dst = smem + buf * STAGE;
#pragma unroll
        for (int m = 0; m < OPW; ++m) {
            const int op = w + NW * m;
            if (op < OPS)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void *)(dst + op * 512),
                                                         16, lane * 16, op * 1024, 0, 0);
        }
    };

    const float cl2 = a.scale_log2;
    const int prow = (l32 & 0x13) | ((l32 & 4) << 1) | ((l32 & 8) >> 1);
    const int64_t qp = q_pos0 + q0 + l32;

    auto qk = [&](int buf, f32x16 (&S)[KB]) {
        const uint16_t *Ks = smem + buf * STAGE;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int e = 0; e < 16; ++e) S[kb][e] = 0.0f;
        const uint16_t *kr0 = Ks + prow * KSTR + 96 * h2;
        auto kaddr = [&](int i) { return kr0 + (i % KB) * 32 * KSTR + 8 * (i / KB); };
        u32x4 kf[RQ];
#pragma unroll
        for (int i = 0; i < RQ; ++i) kf[i] = lds128(kaddr(i));
#pragma unroll
        for (int i = 0; i < 12 * KB; ++i) {
            S[i % KB] = mfma32(kf[i % RQ], qr[i / KB], S[i % KB]);
            if (i + RQ < 12 * KB) kf[i % RQ] = lds128(kaddr(i + RQ));
        }
        // keep RQ reads in flight (left alone, the scheduler let them drain to one
        // or two and waited before most MFMAs)
        __builtin_amdgcn_sched_group_barrier(0x100, RQ, 0);   // LDS reads
#pragma unroll
        for (int i = 0; i < 12 * KB - RQ; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, RQ, 0);
    };

    auto softmax_pv = [&](f32x16 (&S)[KB], int jt, int buf, float kn) {
        const uint16_t *Vs = smem + buf * STAGE + K_TILE;
        const int j0 = jt * NK;
        const int64_t kp0 = k_pos0 + j0;
        const bool full = (j0 + NK <= Tk) && (kp0 + NK - 1 <= qp_lo) &&
                          (a.window == 0 || qp_hi - kp0 < a.window);
        if (!full) {
            int64_t d64 = qp - kp0;
            d64 = d64 < -(1 << 30) ? -(1 << 30) : (d64 > (1 << 30) ? (1 << 30) : d64);
            const int d = (int)d64;
            const int kmax = Tk - j0;
            const int win = a.window > 0 ? a.window : 0x7fffffff;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int jrel = 32 * kb + 16 * (e >> 3) + 8 * h2 + (e & 7);
                    const bool vis = (jrel < kmax) && (jrel <= d) && (d - jrel < win);
                    if (!vis) S[kb][e] = kNegInf;
                }
        }
        // The row max is only needed when a score could exceed the running max by
        // more than 2^kSkipMax in the exp2 domain (fp32 holds such terms easily):
        // interior tiles whose norm bound rules that out skip it.
        if (!full || __any(qbound * kn > m_run + kSkipMax)) {
            float mx = kNegInf;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int e = 0; e < 16; ++e) mx = fmaxf(mx, S[kb][e]);
            mx = max_xor32(mx);
            const float mc = mx * cl2;
            const bool need = mc > m_run + 8.0f;
            if (__any(need)) {
                const float alpha = need ? __builtin_amdgcn_exp2f(m_run - mc) : 1.0f;
                if (need) m_run = mc;
                l_run *= alpha;
#pragma unroll
                for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                    for (int e = 0; e < 16; ++e) O[mb][e] *= alpha;
            }
        }
        const float mu = (m_run == kNegInf) ? 0.0f : m_run;
        u32x4 Pm[KB][2];
        float ls[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kb][e], cl2, -mu));
                S[kb][e] = p;
                ls[e & 3] += p;
            }
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int x = 0; x < 4; ++x)
                    Pm[kb][s][x] = pack_bf16(S[kb][8 * s + 2 * x], S[kb][8 * s + 2 * x + 1]);
        }
        l_run += (ls[0] + ls[1]) + (ls[2] + ls[3]);
        const uint16_t *vr0 = Vs + l32 * VSTR + 8 * h2;
        auto vaddr = [&](int i) {
            const int mb = i / (2 * KB), kb = (i / 2) % KB, s = i & 1;
            return vr0 + mb * 32 * VSTR + 32 * kb + 16 * s;
        };
        u32x4 vf[RV];
#pragma unroll
        for (int i = 0; i < RV; ++i) vf[i] = lds128(vaddr(i));
#pragma unroll
        for (int i = 0; i < 8 * KB; ++i) {
            O[i / (2 * KB)] = mfma32(vf[i % RV], Pm[(i / 2) % KB][i & 1], O[i / (2 * KB)]);
            if (i + RV < 8 * KB) vf[i % RV] = lds128(vaddr(i + RV));
        }
        __builtin_amdgcn_sched_group_barrier(0x100, RV, 1);
#pragma unroll
        for (int i = 0; i < 8 * KB - RV; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, RV, 1);
    };

    // a tile's key norm (uniform: a scalar load) is fetched one tile ahead, with the
    // tile's copies, so no wait in the loop has to cover copies still in flight
    auto tile_norm = [&](int jt) {
        return a.kv_norm[__builtin_amdgcn_readfirstlane((tile_base + jt) * a.Hkv + g)];
    };
    f32x16 S[KB];
    float kn = 0.0f;
    if (tile_hi >= tile_lo) {
        copy_tile(tile_lo, 0);
        kn = tile_norm(tile_lo);
    }
    __syncthreads();
    for (int jt = tile_lo; jt <= tile_hi; ++jt) {
        const int buf = (jt - tile_lo) & 1;
        if (jt < tile_hi) copy_tile(jt + 1, buf ^ 1);   // buffer buf ^ 1 was last read before the barrier
        const float kn_next = tile_norm(min(jt + 1, tile_hi));
        qk(buf, S);
        softmax_pv(S, jt, buf, kn);
        __syncthreads();   // also waits for this wave's copies of tile jt + 1
        kn = kn_next;
    }

    const float lt = sum_xor32(l_run);
    const int t = q0 + l32;
    if (t < Tq) {
        const float inv = lt > 0.0f ? a.v_scale / lt : 0.0f;
        uint16_t *dst = a.out + ((q_tok0 + t) * a.Hq + head) * kDv;
        store_out_row(O, inv, dst, h2);
        if (a.lse && h2 == 0)
            a.lse[lse_off + (size_t)head * a.lse_hstride + t] = lt > 0.0f ? (m_run + log2f(lt)) * kLn2 : kNegInf;
    }
}

// ---- RoPE of a block's 32 query rows with both wave halves at work.  Lane (l, 0)
// holds dims 0..95 of row l and lane (l, 1) dims 96..191, so all 32 rotating pairs
// (dims i and i + 32, i < 32) sit in the lower half.  Pairs 16..31 move to the upper
// half (lane swaps, undone at the end) and every lane rotates 16 pairs.  The angle
// of pair i for row l is the block's base angle (position pos0, exact fixed-point
// turns, the same for every lane) plus l * theta_i (under 32 positions: fp32 keeps
// it to ~3e-7 turns), which saves the per-row 64-bit turn products.
__device__ __forceinline__ void swap_halves(u32x4 &lo_keep, u32x4 &hi_keep) {
    // upper lanes' lo_keep <-> lower lanes' hi_keep
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const auto r = __builtin_amdgcn_permlane32_swap(lo_keep[i], hi_keep[i], false, false);
        lo_keep[i] = r[0];
        hi_keep[i] = r[1];
    }
}

__device__ __forceinline__ void rope_rotate_block(u32x4 (&qr)[12], int64_t pos0, int l32, int h2,
                                                  const RopeTurns &rt) {
    swap_halves(qr[0], qr[2]);
    swap_halves(qr[1], qr[3]);
    swap_halves(qr[4], qr[6]);
    swap_halves(qr[5], qr[7]);
    const float lf = (float)l32;
    const bool up = h2 != 0;
    constexpr float k2m32 = 2.3283064365386963e-10f;   // 2^-32
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            float cs[2], sn[2];
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int i = 8 * c + 2 * w + k;   // pair in the lower half; i + 16 in the upper
                // the block's base angles (uniform, scalar unit) and theta's high words,
                // picked per half; recomputed per block rather than held in registers
                uint32_t th_lo = (uint32_t)(rt.turn[i] >> 32), th_hi = (uint32_t)(rt.turn[i + 16] >> 32);
                uint32_t b_lo = (uint32_t)(((uint64_t)pos0 * rt.turn[i]) >> 32);
                uint32_t b_hi = (uint32_t)(((uint64_t)pos0 * rt.turn[i + 16]) >> 32);
                asm volatile("" : "+s"(th_lo), "+s"(th_hi), "+s"(b_lo), "+s"(b_hi));
                const float th = (float)(up ? th_hi : th_lo) * k2m32;
                const float b = (float)(int32_t)(up ? b_hi : b_lo) * k2m32;
                const float r = __builtin_fmaf(lf, th, b);
                sn[k] = __builtin_amdgcn_sinf(r);
                cs[k] = __builtin_amdgcn_cosf(r);
            }
            const float x0 = bf_lo(qr[c][w]), x1 = bf_hi(qr[c][w]);
            const float y0 = bf_lo(qr[c + 4][w]), y1 = bf_hi(qr[c + 4][w]);
            qr[c][w] = pack_bf16(x0 * cs[0] - y0 * sn[0], x1 * cs[1] - y1 * sn[1]);
            qr[c + 4][w] = pack_bf16(y0 * cs[0] + x0 * sn[0], y1 * cs[1] + x1 * sn[1]);
        }
    swap_halves(qr[0], qr[2]);
    swap_halves(qr[1], qr[3]);
    swap_halves(qr[4], qr[6]);
    swap_halves(qr[5], qr[7]);
}

// ---- Sliding-window band kernel (window <= 128, 8 query heads per KV head).
// One workgroup = the 8 query heads of one KV head (one wave each, two waves per
// SIMD) of one sequence, walking a run of consecutive 32-query blocks.  The 32-key
// K/V tiles of the band live in an LDS ring of kBandSlots slots: a block reads the
// (at most 6) tiles of its window, and each new block stages just the one tile its
// window gains, staged while the block before it computes.  K/V tiles are read
// from HBM about once per run instead of five times per block and head group.
constexpr int kBandSlots = 7;
constexpr int kBandMaxWindow = 128;

template <int NW>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * NW, 64 * NW), amdgpu_waves_per_eu(2, 2)))
void prefill_band_kernel(PrefillArgs a) {
    constexpr int NK = 32, QW = 32, NT = 64 * NW;
    constexpr int VSTR = NK + 8;
    constexpr int K_TILE = NK * KSTR, V_TILE = kDv * VSTR, SLOT = K_TILE + V_TILE;
    static_assert(NT == 512, "staging split: 256 rotating + 512 pass-through + 256 V units");
    __shared__ __attribute__((aligned(16))) uint16_t ring[kBandSlots * SLOT];

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int h2 = lane >> 5, l32 = lane & 31;

    // ---- (sequence b, KV head g, run r of query blocks)
    const int runs = a.band_runs;
    const int r = blockIdx.x % runs, bg = blockIdx.x / runs;
    const int g = bg % a.Hkv, b = bg / a.Hkv;
    const int head = g * NW + w;
    // the head's sink in the exp2 domain, read once by a scalar load (the index made
    // wave-uniform): a vector load waited for at each block's start would also wait
    // for every store and load issued before it
    const float sink_l2 = a.sinks ? a.sinks[__builtin_amdgcn_readfirstlane(head)] * kLog2e : kNegInf;

    int Tq, Tk;
    size_t q_tok0, k_tok0, lse_off;
    int64_t q_pos0, k_pos0;
    if (a.cu_q) {
        const int qs = a.cu_q[b], ks = a.cu_k[b];
        Tq = a.cu_q[b + 1] - qs;
        Tk = a.cu_k[b + 1] - ks;
        q_tok0 = (size_t)qs;
        k_tok0 = (size_t)ks;
        k_pos0 = a.kpos ? a.kpos[b] : 0;
        q_pos0 = k_pos0 + Tk - Tq;
        lse_off = (size_t)qs;
    } else {
        Tq = a.Tq;
        Tk = a.Tk;
        q_tok0 = (size_t)b * a.Tq;
        k_tok0 = (size_t)b * a.Tk;
        q_pos0 = a.q_pos0;
        k_pos0 = a.k_pos0;
        lse_off = (size_t)b * a.Hq * a.Tq;
    }
    const int off = Tk - Tq;                       // query t is key index t + off
    const int nqb = (Tq + QW - 1) / QW;
    const int per = (a.n_qblk + runs - 1) / runs;
    const int qb0 = r * per, qb1 = min(nqb, qb0 + per);
    if (qb0 >= qb1) return;                        // whole workgroup
    const int W = a.window;
    // 32-key tiles of the keys block qb sees: index [32 qb + off - W + 1, last query + off]
    auto tlo = [&](int qb) { const int j = qb * QW + off - W + 1; return j > 0 ? j / NK : 0; };
    auto thi = [&](int qb) { return (min(qb * QW + QW - 1, Tq - 1) + off) / NK; };
    const int t_last = thi(qb1 - 1);

    const size_t krow_stride = (size_t)a.Hkv * kDqk;
    const size_t vrow_stride = (size_t)a.Hkv * kDv;
    const uint16_t *kbase = a.k + k_tok0 * krow_stride + (size_t)g * kDqk;
    const uint16_t *vbase = a.v + k_tok0 * vrow_stride + (size_t)g * kDv;

    // ---- staging of a tile: threads < 256 rotate K piece (row rrow, pairs
    // 4*(tid&7)..+3); every thread moves pass-through chunk 8 + (tid&15) of row
    // tid>>4; threads >= 256 transpose V (key pair u%16, 8-dv chunk u/16, u = tid-256).
    // LDS banks: the rows a half-wave's rotating pieces land in are 4 apart (starts
    // 16 dwords apart for the 400-byte row stride), and lanes whose dv chunk has bit 1
    // set hold their chunk's halves swapped and write its transposed rows in the
    // order d ^ 4, so the four 16-lane groups of a transposed store hit disjoint banks.
    const bool rot_thr = tid < 256;
    const int rgrp = (tid & 255) >> 3;
    const int rrow = (rgrp & 16) | ((rgrp & 3) << 2) | ((rgrp >> 2) & 3), rq = tid & 7;
    const int prow_ = tid >> 4, pch = 8 + (tid & 15);
    const int vu = tid & 255, vkp = vu % 16, vcc = vu / 16;
    const int vsw = (vcc & 2) ? 4 : 0;             // element offset of the half loaded first
    uint64_t my_turn[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) my_turn[e] = a.rt.turn[4 * rq + e];
    struct TileRegs {
        u32x2 rx, ry;
        u32x4 pl;
        u32x4 v[2];
    };
    // unconditional loads of tile jt (rows past Tk re-read the last key: masked, finite)
    auto load_tile = [&](TileRegs &R, int jt) {
        const int j0 = jt * NK, last = Tk - 1 - j0;
        const uint16_t *kt = kbase + (size_t)j0 * krow_stride;
        const uint16_t *vt = vbase + (size_t)j0 * vrow_stride;
        if (rot_thr) {
            const uint16_t *src = kt + (size_t)min(rrow, last) * krow_stride + 4 * rq;
            R.rx = *reinterpret_cast<const u32x2 *>(src);
            R.ry = *reinterpret_cast<const u32x2 *>(src + 32);
        } else {
            const uint16_t *src = vt + 8 * vcc;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const uint16_t *row = src + (size_t)min(2 * vkp + i, last) * vrow_stride;
                const u32x2 h0 = *reinterpret_cast<const u32x2 *>(row + vsw);
                const u32x2 h1 = *reinterpret_cast<const u32x2 *>(row + (4 - vsw));
                R.v[i] = u32x4{h0[0], h0[1], h1[0], h1[1]};
            }
        }
        R.pl = ldg128(kt + (size_t)min(prow_, last) * krow_stride + 8 * pch);
    };
    auto store_tile = [&](const TileRegs &R, int jt) {
        uint16_t *Ks = ring + (jt % kBandSlots) * SLOT;
        uint16_t *Vs = Ks + K_TILE;
        if (rot_thr) {
            const uint64_t pos = (uint64_t)(k_pos0 + (int64_t)jt * NK + rrow);
            u32x2 x = R.rx, y = R.ry;
#pragma unroll
            for (int wd = 0; wd < 2; ++wd) {
                float s0, c0, s1, c1;
                turn_sincos(pos * my_turn[2 * wd], s0, c0);
                turn_sincos(pos * my_turn[2 * wd + 1], s1, c1);
                const float x0 = bf_lo(x[wd]), x1 = bf_hi(x[wd]);
                const float y0 = bf_lo(y[wd]), y1 = bf_hi(y[wd]);
                x[wd] = pack_bf16(x0 * c0 - y0 * s0, x1 * c1 - y1 * s1);
                y[wd] = pack_bf16(y0 * c0 + x0 * s0, y1 * c1 + x1 * s1);
            }
            *reinterpret_cast<u32x2 *>(Ks + rrow * KSTR + 4 * rq) = x;
            *reinterpret_cast<u32x2 *>(Ks + rrow * KSTR + 4 * rq + 32) = y;
        } else {
            // word d >> 1 of R.v holds dv 8 vcc + (d ^ vsw) and its neighbour
            uint16_t *vlo = Vs + (8 * vcc + vsw) * VSTR + 2 * vkp;         // rows of d < 4
            uint16_t *vhi = Vs + (8 * vcc + 4 - vsw) * VSTR + 2 * vkp;     // rows of d >= 4
#pragma unroll
            for (int d = 0; d < 8; ++d) {
                const uint32_t sel = (d & 1) ? 0x07060302u : 0x05040100u;
                const uint32_t wv = __builtin_amdgcn_perm(R.v[1][d >> 1], R.v[0][d >> 1], sel);
                *reinterpret_cast<uint32_t *>((d < 4 ? vlo : vhi) + (d & 3) * VSTR) = wv;
            }
        }
        *reinterpret_cast<u32x4 *>(Ks + prow_ * KSTR + 8 * pch) = R.pl;
    };

    const float cl2 = a.scale_log2;
    const int prow = (l32 & 0x13) | ((l32 & 4) << 1) | ((l32 & 8) >> 1);

    // ---- Two phases per CU.  Waves w and w + 4 share a SIMD; the odd waves ("late")
    // take block n - 1 whole in iteration n, the even waves ("early") finish block
    // n - 1 and then start block n (its Q, RoPE and first tile) before the
    // iteration's barrier, so half the SIMDs run about half a block ahead of the
    // other half (3.5-4.5 % faster than every wave in step).  Iteration n stages
    // tile thi(n), read from iteration n + 1 on; its reads lie in tlo(n - 1) ..
    // thi(n) - 1, so with tile thi(n) at most 7 distinct tiles: the ring's slots.
    const bool early = (w & 1) == 0;
    // first tile of a block's second half (the first half never takes thi)
    auto mid = [&](int qb) { return min(tlo(qb) + 1, thi(qb)); };

    TileRegs R;
    int staged;
    {
        const int t0 = tlo(qb0), tp = thi(qb0) - 1;
        load_tile(R, t0);
        for (int jt = t0; jt <= tp; ++jt) {
            store_tile(R, jt);
            load_tile(R, min(jt + 1, t_last));
        }
        staged = max(tp, t0 - 1);   // R holds tile staged + 1 = thi(qb0)
    }
    __syncthreads();

    u32x4 qr[12];
    float m_run = 0.0f, l_run = 0.0f;
    f32x16 O[4];
    auto begin_block = [&](int qb) {
        const int q0 = qb * QW;
        const int tq = min(q0 + l32, Tq - 1);
        const uint16_t *src = a.q + ((q_tok0 + tq) * a.Hq + head) * kDqk + 96 * h2;
#pragma unroll
        for (int ks = 0; ks < 12; ++ks) qr[ks] = ldg128(src + 8 * ks);
        rope_rotate_block(qr, q_pos0 + q0, l32, h2, a.rt);
        m_run = sink_l2;
        l_run = (a.sinks && h2 == 0) ? 1.0f : 0.0f;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int e = 0; e < 16; ++e) O[mb][e] = 0.0f;
    };

    // S^T of tile jt
    auto qk_tile = [&](int jt) {
        const uint16_t *Ks = ring + (jt % kBandSlots) * SLOT;
        f32x16 S;
#pragma unroll
        for (int e = 0; e < 16; ++e) S[e] = 0.0f;
        {
            const uint16_t *kr0 = Ks + prow * KSTR + 96 * h2;
            u32x4 kf[RING];
#pragma unroll
            for (int i = 0; i < RING; ++i) kf[i] = lds128(kr0 + 8 * i);
#pragma unroll
            for (int i = 0; i < 12; ++i) {
                S = mfma32(kf[i % RING], qr[i], S);
                if (i + RING < 12) kf[i % RING] = lds128(kr0 + 8 * (i + RING));
            }
            // keep RING reads in flight: left alone, the scheduler waits for each
            // fragment right before its MFMA here
            __builtin_amdgcn_sched_group_barrier(0x100, RING, 0);   // LDS reads
#pragma unroll
            for (int i = 0; i < 12 - RING; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, RING, 0);
        }
        return S;
    };
    // mask, online softmax, O^T += V^T P^T of tile jt for block qb
    auto rest_tile = [&](int qb, int jt, f32x16 S) {
        const uint16_t *Ks = ring + (jt % kBandSlots) * SLOT;
        const uint16_t *Vs = Ks + K_TILE;
        const int j0 = jt * NK;
        const int q0 = qb * QW, t = q0 + l32;
        const int qhi = min(q0 + QW - 1, Tq - 1);
        // ---- mask unless every key of the tile is visible to every query of the block
        const bool full = (j0 + NK <= Tk) && (q0 + off - (j0 + NK - 1) >= 0) && (qhi + off - j0 < W);
        if (!full) {
            // Score e holds tile key 16 (e >> 3) + 8 h2 + (e & 7).  Less 8 h2, the
            // keys this lane's query sees form the range [lo, hi]; a key c is in
            // it when c - lo <= hi - lo as unsigned (constants c: no per-key registers).
            const int dd = t + off - j0 - 8 * h2;
            const int hi = min(dd, Tk - j0 - 8 * h2 - 1);
            int lo = max(dd - W + 1, 0);
            uint32_t span = (uint32_t)(hi - lo);
            if (hi < lo) {   // nothing visible
                lo = 0x40000000;
                span = 0;
            }
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int c = 16 * (e >> 3) + (e & 7);
                if ((uint32_t)(c - lo) > span) S[e] = kNegInf;
            }
        }
        // ---- online softmax (exp2 domain), lazy rescale
        float mx = kNegInf;
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, S[e]);
        mx = max_xor32(mx);
        const float mc = mx * cl2;
        const bool need = mc > m_run + 8.0f;
        if (__any(need)) {
            const float alpha = need ? __builtin_amdgcn_exp2f(m_run - mc) : 1.0f;
            if (need) m_run = mc;
            l_run *= alpha;
#pragma unroll
            for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                for (int e = 0; e < 16; ++e) O[mb][e] *= alpha;
        }
        const float mu = (m_run == kNegInf) ? 0.0f : m_run;
        u32x4 P[2];
        float ls[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(S[e], cl2, -mu));
            S[e] = p;
            ls[e & 3] += p;
        }
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int x = 0; x < 4; ++x) P[s][x] = pack_bf16(S[8 * s + 2 * x], S[8 * s + 2 * x + 1]);
        l_run += (ls[0] + ls[1]) + (ls[2] + ls[3]);
        {
            const uint16_t *vr0 = Vs + l32 * VSTR + 8 * h2;
            auto vaddr = [&](int i) { return vr0 + (i >> 1) * 32 * VSTR + 16 * (i & 1); };
            u32x4 vf[RING];
#pragma unroll
            for (int i = 0; i < RING; ++i) vf[i] = lds128(vaddr(i));
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                O[i >> 1] = mfma32(vf[i % RING], P[i & 1], O[i >> 1]);
                if (i + RING < 8) vf[i % RING] = lds128(vaddr(i + RING));
            }
        }
    };
    auto run_tiles = [&](int qb, int ta, int tb) {
        for (int jt = ta; jt <= tb; ++jt) rest_tile(qb, jt, qk_tile(jt));
    };
    // o = v_scale * O / l, bf16
    auto end_block = [&](int qb) {
        const int t = qb * QW + l32;
        const float lt = sum_xor32(l_run);
        if (t < Tq) {
            const float inv = lt > 0.0f ? a.v_scale / lt : 0.0f;
            uint16_t *dst = a.out + ((q_tok0 + t) * a.Hq + head) * kDv;
            store_out_row(O, inv, dst, h2);
            if (a.lse && h2 == 0)
                a.lse[lse_off + (size_t)head * a.lse_hstride + t] = lt > 0.0f ? (m_run + log2f(lt)) * kLn2 : kNegInf;
        }
    };

    for (int n = qb0; n <= qb1; ++n) {
        if (n < qb1 && thi(n) > staged) {   // uniform over the workgroup
            store_tile(R, thi(n));
            staged = thi(n);
            load_tile(R, min(staged + 1, t_last));
        }
        if (early) {
            if (n > qb0) {
                run_tiles(n - 1, mid(n - 1), thi(n - 1));
                end_block(n - 1);
            }
            if (n < qb1) {
                begin_block(n);
                run_tiles(n, tlo(n), mid(n) - 1);
            }
        } else if (n > qb0) {
            begin_block(n - 1);
            run_tiles(n - 1, tlo(n - 1), thi(n - 1));
            end_block(n - 1);
        }
        __syncthreads();   // tile thi(n) is visible; no wave still reads the slot written next
    }
}

static hipError_t launch_band(PrefillArgs a, hipStream_t stream) {
    a.n_qblk = (a.Tq + 31) / 32;
    // about one workgroup per CU: runs of blocks per (sequence, KV head)
    const int pairs = a.B * a.Hkv;
    int runs = (256 + pairs - 1) / pairs;
    if (runs > a.n_qblk) runs = a.n_qblk;
    if (runs < 1) runs = 1;
    a.band_runs = runs;
    const int64_t blocks = (int64_t)pairs * runs;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((prefill_band_kernel<8>), dim3((unsigned)blocks), dim3(512), 0, stream, a);
    return hipGetLastError();
}

template <int NW, int NK>
static hipError_t launch_variant(PrefillArgs a, hipStream_t stream) {
    const int QW = 32;
    const int G = a.Hq / a.Hkv;
    a.n_qblk = (a.Tq + QW - 1) / QW;
    a.n_hgrp = G / NW;
    const int64_t combos = (int64_t)a.B * a.Hkv * a.n_hgrp;
    const int64_t blocks = combos * a.n_qblk;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    a.xcd_remap = ((a.Hkv * a.n_hgrp) % 8 == 0) ? 2 : (combos % 8 == 0) ? 1 : 0;
    hipLaunchKernelGGL((prefill_kernel<NW, NK>), dim3((unsigned)blocks), dim3(64 * NW), 0, stream, a);
    return hipGetLastError();
}

size_t prefill_image_count(int32_t B, int64_t total_k, int32_t Hkv) {
    return (size_t)((total_k + kImgNK - 1) / kImgNK + B) * Hkv;
}

size_t prefill_image_norm_offset(int32_t B, int64_t total_k, int32_t Hkv) {
    return prefill_image_count(B, total_k, Hkv) * kImgTile * sizeof(uint16_t);
}

size_t prefill_image_bytes(int32_t B, int64_t total_k, int32_t Hkv) {
    return prefill_image_norm_offset(B, total_k, Hkv) + prefill_image_count(B, total_k, Hkv) * sizeof(float);
}

static hipError_t launch_image(PrefillArgs a, hipStream_t stream) {
    const int QW = 32, NW = 8;
    const int G = a.Hq / a.Hkv;
    a.n_qblk = (a.Tq + QW - 1) / QW;
    a.n_hgrp = G / NW;
    // one workgroup per tile of the longest sequence (packed: Tk is the total key
    // count, which bounds it; the count of each sequence is only known on the
    // device), capped; workgroups stride over the tiles of their own sequence
    int64_t tiles = ((int64_t)a.Tk + kImgNK - 1) / kImgNK;
    if (a.cu_k && tiles > 4096) tiles = 4096;
    if (tiles > 65535) tiles = 65535;
    if (tiles < 1) tiles = 1;
    hipLaunchKernelGGL(kv_image_kernel, dim3((unsigned)tiles, a.B, a.Hkv), dim3(256), 0, stream, a);
    const int64_t combos = (int64_t)a.B * a.Hkv * a.n_hgrp;
    const int64_t blocks = combos * a.n_qblk;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    a.xcd_remap = ((a.Hkv * a.n_hgrp) % 8 == 0) ? 2 : (combos % 8 == 0) ? 1 : 0;
    hipLaunchKernelGGL((prefill_image_kernel<8>), dim3((unsigned)blocks), dim3(64 * NW), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_prefill(PrefillArgs a, hipStream_t stream) {
    // Global layers given a tile-image workspace: image pass + DMA-staged kernel.
    if (a.kv_img && a.window == 0 && (a.Hq / a.Hkv) % 8 == 0) return launch_image(a, stream);
    // GQA group sizes are multiples of 4 (checked by the caller).  Sliding
    // windows see a short band of keys: the band kernel (8 query heads per KV
    // head, window <= 128), else 4 heads x 32-key tiles, two workgroups per CU.
    // Global prefixes are long: 8 heads share each 64-key tile.
    // The band kernel pays when its workgroups walk runs of blocks and fill the
    // CUs; with fewer 32-query blocks (over sequences and KV heads) than CUs, the
    // per-block kernel's two workgroups per KV head fill twice as many.
    const bool wide = (a.Hq / a.Hkv) % 8 == 0;
    const int64_t qblocks = (int64_t)a.B * a.Hkv * ((a.Tq + 31) / 32);
    if (a.window > 0 && a.window <= kBandMaxWindow && a.Hq == 8 * a.Hkv && qblocks >= 256)
        return launch_band(a, stream);
    if (a.window == 0 && wide) return launch_variant<8, 64>(a, stream);
    return launch_variant<4, 32>(a, stream);
}

}  // namespace mimo
