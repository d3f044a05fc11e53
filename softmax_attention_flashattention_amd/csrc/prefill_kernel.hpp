// prefill_kernel.hpp -- non-causal varlen prefill attention for gfx950.
//
// Computes, per sequence and head, out = softmax(scale * Q K^T) V (the
// operator of the atrex-bench page "attention_forward" #001, Reference
// Implementation) as a tiled online softmax: the full score matrix is never
// formed.
//
// Work decomposition.  One workgroup (4 waves) owns a tile of BM = 128 query
// rows of one (sequence, head); each wave owns 32 of those rows.  The
// workgroup streams the sequence's keys and values in tiles of BN = 64 rows
// through LDS (double-buffered, staged through registers so the next tile's
// global loads are in flight while the current tile is computed).
//
// Both contractions run on 32x32x16 MFMA with fp32 accumulation, computed
// transposed so that each lane owns one query row:
//   S^T[key, query] = K Q^T     A = K tile from LDS, B = Q^T held in VGPRs
//   O^T[d, query]  += V^T P^T   A = V^T read with ds_read_b64_tr_b16, B = P^T
// With that orientation the 32x32 accumulator gives lane l the column
// (query) l % 32 and 16 of the 32 key rows; lanes l and l ^ 32 share a query.
// Row max and row sum are therefore in-lane reductions plus one exchange with
// lane l ^ 32, and P^T is already in the B-operand layout of the second MFMA:
// only a conversion to 16 bits is needed.  The order of keys inside a 16-key
// MFMA step follows the accumulator (keys {0-3, 8-11} in lanes 0-31, keys
// {4-7, 12-15} in lanes 32-63); V^T is read in that same order, which the
// transposed LDS read produces directly from a row-major V tile.
//
// Softmax runs in the base-2 domain: with c = scale * log2(e), the running
// max m is kept for c*s and p = exp2(c*s - m), alpha = exp2(m_old - m_new).
//
// head_dim 72 pads the QK^T contraction to 80 (five k-steps of 16; the K pad
// columns are zero) and the V^T row blocks to 96; column 72 of the V tile
// holds 1.0, so row 72 of O^T accumulates the row sum of the 16-bit P that
// actually multiplied V (the padding does useful work instead of a VALU sum).
#pragma once

#include "device_common.hpp"

namespace attn {

struct PrefillParams {
    const uint16_t *q, *k, *v;
    const int32_t *cu_q, *cu_k;
    uint16_t *out;
    int64_t total_q, total_k;
    int num_heads;
    int num_qtiles;  // ceil(max_seqlen_q / BM)
    int total_work;  // num_seqs * num_heads * num_qtiles
    int per_xcd;     // ceil(total_work / 8)
    float scale_log2e;
};

template <int D> struct PrefillShape;
template <> struct PrefillShape<128> {
    static constexpr int KSTEPS = 8;    // QK^T contraction steps of 16
    static constexpr int DBLK = 4;      // O^T row blocks of 32
    static constexpr int KPITCH = 136;  // K tile row pitch, elements (272 B: 16 lanes hit distinct banks)
    static constexpr int VPITCH = 160;  // V tile row pitch (320 B: 4 rows land 16 banks apart)
    static constexpr int ONES_COL = -1;
};
template <> struct PrefillShape<72> {
    static constexpr int KSTEPS = 5;    // 72 padded to 80
    static constexpr int DBLK = 3;      // 72 padded to 96
    static constexpr int KPITCH = 88;   // 176 B
    static constexpr int VPITCH = 96;   // 192 B: rows 48 banks apart
    static constexpr int ONES_COL = 72;
};

constexpr int kPrefillBM = 128;
constexpr int kPrefillBN = 64;
constexpr int kPrefillThreads = 256;

template <typename T> struct One16;
template <> struct One16<Bf16> { static constexpr uint32_t bits = 0x3F80u; };
template <> struct One16<Fp16> { static constexpr uint32_t bits = 0x3C00u; };

template <int D, typename T>
__global__ __launch_bounds__(kPrefillThreads) __attribute__((amdgpu_waves_per_eu(2)))
void prefill_fwd_kernel(PrefillParams p)
{
    using S = PrefillShape<D>;
    constexpr int BM = kPrefillBM, BN = kPrefillBN;
    constexpr int KP = S::KPITCH, VP = S::VPITCH;
    constexpr int CH = D / 8;                      // 16-byte chunks per row
    constexpr int NCH = BN * CH;                   // chunks per K (or V) tile
    constexpr int PER = (NCH + kPrefillThreads - 1) / kPrefillThreads;

    __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][BN * KP];
    __shared__ __attribute__((aligned(16))) uint16_t v_lds[2][BN * VP];

    // XCD-aware work id: hardware hands consecutive workgroups to the 8 XCDs
    // in turn, so bid -> (bid % 8) * per_xcd + bid / 8 keeps runs of
    // consecutive work items (same head, neighbouring query tiles, hence the
    // same K/V stream) on one XCD and its L2.
    const int bid = blockIdx.x;
    const int w = (bid & 7) * p.per_xcd + (bid >> 3);
    if (w >= p.total_work) return;
    const int qtile = w % p.num_qtiles;
    const int sh = w / p.num_qtiles;
    const int head = sh % p.num_heads;
    const int seq = sh / p.num_heads;

    int64_t qa = p.cu_q[seq], qb = p.cu_q[seq + 1];
    int64_t ka = p.cu_k[seq], kb = p.cu_k[seq + 1];
    qa = qa < 0 ? 0 : (qa > p.total_q ? p.total_q : qa);
    qb = qb < qa ? qa : (qb > p.total_q ? p.total_q : qb);
    ka = ka < 0 ? 0 : (ka > p.total_k ? p.total_k : ka);
    kb = kb < ka ? ka : (kb > p.total_k ? p.total_k : kb);
    const int Sq = static_cast<int>(qb - qa);
    const int Sk = static_cast<int>(kb - ka);
    const int q0 = qtile * BM;
    if (q0 >= Sq) return;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hi = lane >> 5;
    const int64_t rs = static_cast<int64_t>(p.num_heads) * D;   // token row stride
    const uint16_t *kbase_ptr = p.k + ka * rs + head * D;
    const uint16_t *vbase_ptr = p.v + ka * rs + head * D;

    if constexpr (S::ONES_COL >= 0) {
        // constant pad columns of both buffers: K cols 72..79 = 0,
        // V col 72 = 1, V cols 73..95 = 0
        const uint4 z = {0u, 0u, 0u, 0u};
        const uint4 one = {One16<T>::bits, 0u, 0u, 0u};
        for (int i = tid; i < 2 * BN; i += kPrefillThreads) {
            const int buf = i / BN, r = i % BN;
            st16(&k_lds[buf][r * KP + 72], z);
            st16(&v_lds[buf][r * VP + 72], one);
            st16(&v_lds[buf][r * VP + 80], z);
            st16(&v_lds[buf][r * VP + 88], z);
        }
    }

    // Q^T as the B operand of S^T = K Q^T: lane l holds row l % 32 of this
    // wave's 32 queries, elements 16 ks + 8 (l / 32) .. +7.
    s16x8 qreg[S::KSTEPS];
    const int qrow = q0 + 32 * wave + l32;
#pragma unroll
    for (int ks = 0; ks < S::KSTEPS; ++ks) {
        const int d0 = 16 * ks + 8 * hi;
        uint4 v4 = {0u, 0u, 0u, 0u};
        if (qrow < Sq && d0 < D) v4 = ld16(p.q + (qa + qrow) * rs + head * D + d0);
        qreg[ks] = __builtin_bit_cast(s16x8, v4);
    }

    const int ntiles = (Sk + BN - 1) / BN;
    uint4 kst[PER], vst[PER];

    auto load_tile = [&](int t) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int c = tid + i * kPrefillThreads;
            uint4 kz = {0u, 0u, 0u, 0u}, vz = {0u, 0u, 0u, 0u};
            if (c < NCH) {
                const int r = c / CH, col = (c % CH) * 8;
                const int key = t * BN + r;
                if (key < Sk) {
                    kz = ld16(kbase_ptr + key * rs + col);
                    vz = ld16(vbase_ptr + key * rs + col);
                }
            }
            kst[i] = kz;
            vst[i] = vz;
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int c = tid + i * kPrefillThreads;
            if (c < NCH) {
                const int r = c / CH, col = (c % CH) * 8;
                st16(&k_lds[buf][r * KP + col], kst[i]);
                st16(&v_lds[buf][r * VP + col], vst[i]);
            }
        }
    };

    float m_run = -INFINITY;   // running max of c*s for this lane's query
    float l_run = 0.f;         // this lane's partial row sum (its 16 keys of each 32)
    f32x16 oacc[S::DBLK];
#pragma unroll
    for (int db = 0; db < S::DBLK; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;

    if (ntiles > 0) {
        load_tile(0);
        store_tile(0);
    }
    __syncthreads();

    // transposed-read addressing of the V tile (see the header comment)
    const int g16 = lane >> 4;
    const int tr_row = 4 * (g16 >> 1) + ((lane & 15) >> 2);
    const int tr_col = 16 * (g16 & 1) + 4 * (lane & 3);

    for (int t = 0; t < ntiles; ++t) {
        const int buf = t & 1;
        if (t + 1 < ntiles) load_tile(t + 1);

        // ---- S^T = K Q^T for two 32-key blocks
        f32x16 sacc[2];
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[kb2][r] = 0.f;
            const uint16_t *krow = &k_lds[buf][(32 * kb2 + l32) * KP + 8 * hi];
#pragma unroll
            for (int ks = 0; ks < S::KSTEPS; ++ks) {
                const s16x8 a = *reinterpret_cast<const s16x8 *>(krow + 16 * ks);
                sacc[kb2] = T::mfma32(a, qreg[ks], sacc[kb2]);
            }
        }

        // ---- mask keys past the end of the sequence (last tile only)
        const int kbase = t * BN;
        if (kbase + BN > Sk) {
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kbase + 32 * kb2 + 8 * (r >> 2) + 4 * hi + (r & 3);
                    if (key >= Sk) sacc[kb2][r] = -INFINITY;
                }
        }

        // ---- online softmax
        float mx = -INFINITY;
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb2][r]);
        mx = fmaxf(mx, xor_shfl(mx, 32));
        const float m_new = fmaxf(m_run, mx * p.scale_log2e);
        const float alpha = fast_exp2(m_run - m_new);
        m_run = m_new;

        s16x8 pk[4];
        float rowsum = 0.f;
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const float p0 = fast_exp2(__builtin_fmaf(sacc[kb2][r], p.scale_log2e, -m_new));
                const float p1 = fast_exp2(__builtin_fmaf(sacc[kb2][r + 1], p.scale_log2e, -m_new));
                if constexpr (S::ONES_COL < 0) rowsum += p0 + p1;
                const uint32_t pp = pack2<T>(p0, p1);
                const int kc = 2 * kb2 + (r >> 3);
                const int e = r & 7;
                pk[kc][e] = static_cast<short>(pp & 0xffffu);
                pk[kc][e + 1] = static_cast<short>(pp >> 16);
            }
        if constexpr (S::ONES_COL < 0) l_run = l_run * alpha + rowsum;
#pragma unroll
        for (int db = 0; db < S::DBLK; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;

        // ---- O^T += V^T P^T
#pragma unroll
        for (int db = 0; db < S::DBLK; ++db) {
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) {
                const uint16_t *base = &v_lds[buf][(16 * kc + tr_row) * VP + 32 * db + tr_col];
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4 *)(base));
                const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4 *)(base + 8 * VP));
                const s16x8 a = {lo[0], lo[1], lo[2], lo[3], hi4[0], hi4[1], hi4[2], hi4[3]};
                oacc[db] = T::mfma32(a, pk[kc], oacc[db]);
            }
        }

        if (t + 1 < ntiles) store_tile(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: normalise, round to 16 bits, store rows inside the segment
    float l_tot;
    if constexpr (S::ONES_COL < 0) {
        l_tot = l_run + xor_shfl(l_run, 32);
    } else {
        // row 72 of O^T = block 2, register 4, lanes 0..31
        const float lv = oacc[2][4];
        const float other = xor_shfl(lv, 32);
        l_tot = hi ? other : lv;
    }
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (qrow < Sq) {
        uint16_t *orow = p.out + (qa + qrow) * rs + head * D;
#pragma unroll
        for (int db = 0; db < S::DBLK; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int d = 32 * db + 8 * g4 + 4 * hi;
                if (d < D) {
                    uint2 w2;
                    w2.x = pack2<T>(oacc[db][4 * g4 + 0] * inv, oacc[db][4 * g4 + 1] * inv);
                    w2.y = pack2<T>(oacc[db][4 * g4 + 2] * inv, oacc[db][4 * g4 + 3] * inv);
                    *reinterpret_cast<uint2 *>(orow + d) = w2;
                }
            }
    }
}

}  // namespace attn
