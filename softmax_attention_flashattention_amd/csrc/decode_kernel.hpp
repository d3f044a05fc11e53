// decode_kernel.hpp -- paged single-query decode attention for gfx950.
//
// Computes, per sequence s and query head hq, out = softmax(scale * q K^T) V
// over the first seq_lens[s] tokens of the sequence, with K and V read from
// a paged cache through the block table (the operator of the atrex-bench
// page "paged_attention_decode" #024, Reference Implementation and Input
// Generation):
//   token t  -> physical block block_tables[s][t / 16], slot t % 16
//   K cache  [num_blocks, Hkv, D/8, 16, 8]: one (block, kv head) is a
//            contiguous 4 KiB chunk laid out [D/8][16 tokens][8 dims]
//   V cache  [num_blocks, Hkv, D, 16]: one (block, kv head) is a contiguous
//            4 KiB chunk laid out [D][16 tokens]
//   query head hq reads KV head hq / G, G = Hq / Hkv.
//
// The operator is bound by HBM bandwidth, so the kernel is shaped around the
// loads: one wave owns one (sequence, KV head, context partition) and serves
// all G query heads of that KV head from a single read of each K/V chunk.  A
// chunk of four blocks (64 tokens) is read with 32 independent 16-byte loads
// per lane issued back to back; lane l holds, for each block,
//   K: 32 dims (dim groups l/16 + 4c, c = 0..3) of token l % 16
//   V: dims 32c + l/2 (c = 0..3), tokens 8 (l % 2) .. +7.
// Scores need a 4-lane reduction (xor 16, 32); the softmax weights move from
// the token-owning lanes to the dim-owning lanes through LDS.
//
// Split-K: a context longer than one partition is split over several waves;
// each writes (running max m in the log2 domain, sum l, unnormalised output
// o) to the workspace and decode_merge_kernel combines them:
//   M = max_p m_p,  out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p.
#pragma once

#include "device_common.hpp"

namespace attn {

constexpr int kDecodeD = 128;
constexpr int kDecodeBS = 16;
constexpr int kDecodeChunkBlocks = 4;

struct DecodeParams {
    const uint16_t *query, *k_cache, *v_cache;
    const int32_t *block_tables, *seq_lens;
    uint16_t *out;
    float *ws_ml;  // [num_seqs][Hq][num_parts][2]: (m, l)
    float *ws_o;   // [num_seqs][Hq][num_parts][D]
    int64_t num_blocks;
    int num_seqs, Hq, Hkv, G, maxb;
    int part_blocks;  // blocks per partition
    int num_parts;
    float scale_log2e;
};

__device__ __forceinline__ float lo16f_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi16f_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <typename T>
__device__ __forceinline__ float elem16(const uint4 &v, int e) {
    const uint32_t w = (e >> 1) == 0 ? v.x : (e >> 1) == 1 ? v.y : (e >> 1) == 2 ? v.z : v.w;
    return T::to_f32(static_cast<uint16_t>((e & 1) ? (w >> 16) : (w & 0xffffu)));
}

template <typename T, int GMAX>
__global__ __launch_bounds__(64) void decode_partition_kernel(DecodeParams p)
{
    constexpr int D = kDecodeD, BS = kDecodeBS, NB = kDecodeChunkBlocks;
    __shared__ __attribute__((aligned(16))) float q_lds[GMAX][D];
    __shared__ __attribute__((aligned(16))) float p_lds[GMAX][NB][BS];

    const int lane = threadIdx.x;
    int id = blockIdx.x;
    const int part = id % p.num_parts;
    id /= p.num_parts;
    const int hk = id % p.Hkv;
    const int s = id / p.Hkv;
    const int G = p.G;
    const int hq0 = hk * G;

    int L = p.seq_lens[s];
    L = L > p.maxb * BS ? p.maxb * BS : L;
    const int t_begin = part * p.part_blocks * BS;
    const int t_end = L < t_begin + p.part_blocks * BS ? L : t_begin + p.part_blocks * BS;

    if (t_end <= t_begin) {
        // No tokens here.  With one partition the row is final: zeros.  With
        // several, the merge kernel skips partitions past the context.
        if (p.num_parts == 1) {
            for (int g = 0; g < G; ++g) {
                uint16_t *o = p.out + (static_cast<int64_t>(s) * p.Hq + hq0 + g) * D;
                o[lane] = 0;
                o[lane + 64] = 0;
            }
        }
        return;
    }

    // q scaled into the log2 domain, fp32, in LDS
    for (int i = lane; i < G * D; i += 64) {
        const int g = i / D, d = i % D;
        q_lds[g][d] = T::to_f32(p.query[(static_cast<int64_t>(s) * p.Hq + hq0 + g) * D + d]) *
                      p.scale_log2e;
    }
    __syncthreads();

    float m_run[GMAX], l_run[GMAX], acc[GMAX][4];
#pragma unroll
    for (int g = 0; g < GMAX; ++g) {
        m_run[g] = -INFINITY;
        l_run[g] = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[g][c] = 0.f;
    }

    const int blk_begin = t_begin / BS;
    const int blk_end = (t_end + BS - 1) / BS;
    const int32_t *bt_row = p.block_tables + static_cast<int64_t>(s) * p.maxb;
    const int kgrp = lane >> 4;     // K: dim group within a 1 KiB slice
    const int vhalf = lane & 1;     // V: which 8 tokens of the row

    for (int b0 = blk_begin; b0 < blk_end; b0 += NB) {
        uint4 kr[NB][4], vr[NB][4];
        bool ok[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const int jb = b0 + j;
            int64_t phys = -1;
            if (jb < blk_end) phys = bt_row[jb];
            ok[j] = phys >= 0 && phys < p.num_blocks;
            const int64_t base = ok[j] ? (phys * p.Hkv + hk) * (D * BS) : 0;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint4 z = {0u, 0u, 0u, 0u};
                kr[j][c] = ok[j] ? ld16(p.k_cache + base + c * 512 + lane * 8) : z;
                vr[j][c] = ok[j] ? ld16(p.v_cache + base + c * 512 + lane * 8) : z;
            }
        }

        // scores of token (lane % 16) of each block, per query head
        float sc[GMAX][NB];
#pragma unroll
        for (int g = 0; g < GMAX; ++g) {
            if (g < G) {
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    float dot = 0.f;
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const float *qv = &q_lds[g][8 * (4 * c + kgrp)];
#pragma unroll
                        for (int e = 0; e < 8; ++e) dot = __builtin_fmaf(qv[e], elem16<T>(kr[j][c], e), dot);
                    }
                    dot += xor_shfl(dot, 16);
                    dot += xor_shfl(dot, 32);
                    const int tok = (b0 + j) * BS + (lane & 15);
                    sc[g][j] = (ok[j] && tok < t_end) ? dot : -INFINITY;
                }
            }
        }

        // online softmax per query head; weights to LDS for the V pass
#pragma unroll
        for (int g = 0; g < GMAX; ++g) {
            if (g < G) {
                float cm = sc[g][0];
#pragma unroll
                for (int j = 1; j < NB; ++j) cm = fmaxf(cm, sc[g][j]);
#pragma unroll
                for (int sh = 1; sh < 16; sh <<= 1) cm = fmaxf(cm, xor_shfl(cm, sh));
                const float m_new = fmaxf(m_run[g], cm);
                const bool none = m_new == -INFINITY;
                const float alpha = none ? 1.f : fast_exp2(m_run[g] - m_new);
                float ps = 0.f;
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    const float pj = none ? 0.f : fast_exp2(sc[g][j] - m_new);
                    ps += pj;
                    if (lane < 16) p_lds[g][j][lane] = pj;
                }
#pragma unroll
                for (int sh = 1; sh < 16; sh <<= 1) ps += xor_shfl(ps, sh);
                l_run[g] = l_run[g] * alpha + ps;
                m_run[g] = m_new;
#pragma unroll
                for (int c = 0; c < 4; ++c) acc[g][c] *= alpha;
            }
        }
        __syncthreads();

        // acc[g][c] += sum over this lane's 8 tokens of p * V[token][32c + lane/2]
#pragma unroll
        for (int g = 0; g < GMAX; ++g) {
            if (g < G) {
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    const float4 pa = *reinterpret_cast<const float4 *>(&p_lds[g][j][8 * vhalf]);
                    const float4 pb = *reinterpret_cast<const float4 *>(&p_lds[g][j][8 * vhalf + 4]);
                    const float pw[8] = {pa.x, pa.y, pa.z, pa.w, pb.x, pb.y, pb.z, pb.w};
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        float a = acc[g][c];
#pragma unroll
                        for (int e = 0; e < 8; ++e) a = __builtin_fmaf(pw[e], elem16<T>(vr[j][c], e), a);
                        acc[g][c] = a;
                    }
                }
            }
        }
        __syncthreads();
    }

    // lanes l and l ^ 1 hold the two 8-token halves of the same dims
#pragma unroll
    for (int g = 0; g < GMAX; ++g)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[g][c] += xor_shfl(acc[g][c], 1);

    for (int g = 0; g < G && g < GMAX; ++g) {
        const int64_t row = static_cast<int64_t>(s) * p.Hq + hq0 + g;
        if (p.num_parts == 1) {
            const float inv = l_run[g] > 0.f ? 1.f / l_run[g] : 0.f;
            if (vhalf == 0) {
#pragma unroll
                for (int c = 0; c < 4; ++c) p.out[row * D + 32 * c + (lane >> 1)] = T::from_f32(acc[g][c] * inv);
            }
        } else {
            const int64_t slot = row * p.num_parts + part;
            if (vhalf == 0) {
#pragma unroll
                for (int c = 0; c < 4; ++c) p.ws_o[slot * D + 32 * c + (lane >> 1)] = acc[g][c];
            }
            if (lane == 0) {
                p.ws_ml[slot * 2 + 0] = m_run[g];
                p.ws_ml[slot * 2 + 1] = l_run[g];
            }
        }
    }
}

// One wave per (sequence, query head): log-sum-exp merge of the partitions
// that hold part of the context.
template <typename T>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecodeParams p)
{
    constexpr int D = kDecodeD, BS = kDecodeBS;
    const int lane = threadIdx.x;
    const int64_t row = blockIdx.x;  // s * Hq + hq
    const int s = static_cast<int>(row / p.Hq);
    int L = p.seq_lens[s];
    L = L > p.maxb * BS ? p.maxb * BS : L;
    const int pt = p.part_blocks * BS;
    int nparts = L > 0 ? (L + pt - 1) / pt : 0;
    nparts = nparts > p.num_parts ? p.num_parts : nparts;

    float M = -INFINITY;
    for (int i = 0; i < nparts; ++i) M = fmaxf(M, p.ws_ml[(row * p.num_parts + i) * 2]);
    float den = 0.f, o0 = 0.f, o1 = 0.f;
    if (M != -INFINITY) {
        for (int i = 0; i < nparts; ++i) {
            const int64_t slot = row * p.num_parts + i;
            const float m = p.ws_ml[slot * 2];
            const float w = m == -INFINITY ? 0.f : fast_exp2(m - M);
            den += w * p.ws_ml[slot * 2 + 1];
            o0 += w * p.ws_o[slot * D + lane];
            o1 += w * p.ws_o[slot * D + lane + 64];
        }
    }
    const float inv = den > 0.f ? 1.f / den : 0.f;
    p.out[row * D + lane] = T::from_f32(o0 * inv);
    p.out[row * D + lane + 64] = T::from_f32(o1 * inv);
}

}  // namespace attn
