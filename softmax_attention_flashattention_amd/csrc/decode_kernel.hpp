// decode_kernel.hpp -- paged single-query decode attention for gfx950.
//
// Computes, per sequence s and query head hq, out = softmax(scale * q K^T) V
// over the first seq_lens[s] tokens of the sequence, with K and V read from
// a paged cache through the block table (the operator of the atrex-bench
// page "paged_attention_decode" #024, Reference Implementation and Input
// Generation):
//   token t  -> physical block block_tables[s][t / 16], slot t % 16
//   K cache  [num_blocks, Hkv, D/8, 16, 8]: one (block, kv head) is a
//            contiguous chunk laid out [D/8][16 tokens][8 dims]
//   V cache  [num_blocks, Hkv, D, 16]: one (block, kv head) is a contiguous
//            chunk laid out [D][16 tokens]
//   query head hq reads KV head hq / G, G = Hq / Hkv.
//
// The operator is bound by HBM bandwidth, so the kernel is shaped around the
// loads.  A workgroup of four waves owns one (sequence, KV head, context
// partition) and serves all G query heads of that KV head from a single read
// of each K/V chunk.  The partition's blocks are dealt to the waves round
// robin; a wave reads a block's K and V chunks with D/32 + D/32 independent
// 16-byte loads per lane (the next block's loads are issued before the
// current one is used; each K/V chunk is read once, so the loads are
// non-temporal) and keeps its own online softmax.  Lane l holds, for
// each block,
//   K: dims 8 (4 c + l / 16) .. +7 of token l % 16   (c = 0 .. D/32 - 1)
//   V: dim 32 c + l / 2 of tokens 8 (l % 2) .. +7.
// Both dot products run on v_dot2 (two 16-bit products summed into fp32):
// q K^T with the 16-bit query, P V with the weights rounded to the 16-bit
// type (like the P operand of the prefill kernel); the row sum adds up those
// same rounded weights.  Scores need a 4-lane
// reduction (v_permlane16/32_swap) and the block max and sum a 16-lane one
// (DPP), all in VALU; the weights move from the token-owning lanes to the
// dim-owning lanes through LDS.  At the end the four waves' (max, sum, partial output)
// are merged through LDS.
//
// Few workgroups: when sequences x KV heads x partitions would leave compute
// units idle, the G query heads of a KV head are dealt to ngroups
// workgroups of gsub heads each.  Each reads the same K/V chunks (from L2
// after the first), and the per-block softmax chain of a wave is gsub heads
// long instead of G; the outputs are disjoint, so nothing is merged.
//
// Split-K: a context longer than one partition is split over several
// workgroups; each writes (running max m in the log2 domain, sum l,
// unnormalised output o) to the workspace and decode_merge_kernel combines
// them:  M = max_p m_p,  out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p.
#pragma once

#include "device_common.hpp"

namespace attn {

constexpr int kDecodeBS = 16;
constexpr int kDecodeWaves = 4;
constexpr int kDecodeThreads = 64 * kDecodeWaves;

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
    int gsub;         // query heads per workgroup (G when the heads are not dealt out)
    int ngroups;      // workgroups per (sequence, KV head, partition): ceil(G / gsub)
    int on_mfma;      // 1: decode_mfma_kernel (host-side choice, unused by the kernels)
    float scale_log2e;
};

template <typename T, int D, int GMAX>
__global__ __launch_bounds__(kDecodeThreads) void decode_partition_kernel(DecodeParams p)
{
    constexpr int BS = kDecodeBS, NW = kDecodeWaves;
    constexpr int NC = D / 32;          // 16-byte loads per lane per block, for K and for V
    constexpr int CHUNK = D * BS;       // elements of one (block, kv head) chunk
    __shared__ __attribute__((aligned(16))) uint32_t q_lds[GMAX][D / 2];   // 16-bit pairs
    __shared__ __attribute__((aligned(16))) float p_lds[NW][GMAX][BS];
    __shared__ float m_lds[NW][GMAX], l_lds[NW][GMAX], c_lds[NW][GMAX];
    __shared__ __attribute__((aligned(16))) float o_lds[NW][GMAX][D];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int id = blockIdx.x;
    const int part = id % p.num_parts;
    id /= p.num_parts;
    const int gg = id % p.ngroups;
    id /= p.ngroups;
    const int hk = id % p.Hkv;
    const int s = id / p.Hkv;
    // this workgroup's query heads: hq0 .. hq0 + G - 1 (G <= GMAX)
    const int hq0 = hk * p.G + gg * p.gsub;
    const int G = p.G - gg * p.gsub < p.gsub ? p.G - gg * p.gsub : p.gsub;

    int L = p.seq_lens[s];
    L = L > p.maxb * BS ? p.maxb * BS : L;
    const int t_begin = part * p.part_blocks * BS;
    const int t_end = L < t_begin + p.part_blocks * BS ? L : t_begin + p.part_blocks * BS;

    if (t_end <= t_begin) {
        // No tokens here.  With one partition the rows are final: zeros.  With
        // several, the merge kernel skips partitions past the context.
        if (p.num_parts == 1)
            for (int i = tid; i < G * D; i += kDecodeThreads)
                p.out[(static_cast<int64_t>(s) * p.Hq + hq0) * D + i] = 0;
        return;
    }

    float m_run[GMAX], l_run[GMAX], acc[GMAX][NC];
#pragma unroll
    for (int g = 0; g < GMAX; ++g) {
        m_run[g] = -INFINITY;
        l_run[g] = 0.f;
#pragma unroll
        for (int c = 0; c < NC; ++c) acc[g][c] = 0.f;
    }

    const int blk_begin = t_begin / BS;
    const int blk_end = (t_end + BS - 1) / BS;
    const int32_t *bt_row = p.block_tables + static_cast<int64_t>(s) * p.maxb;
    const int kgrp = lane >> 4;        // K: dim group inside a 1 KiB slice
    const int vhalf = lane & 1;        // V: which 8 tokens of a dim row
    const float c2 = p.scale_log2e;

    auto load_block = [&](int jb, uint4 (&kr)[NC], uint4 (&vr)[NC]) -> bool {
        int64_t phys = -1;
        if (jb < blk_end) phys = bt_row[jb];
        const bool ok = phys >= 0 && phys < p.num_blocks;
        const int64_t base = ok ? (phys * p.Hkv + hk) * CHUNK : 0;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const uint4 z = {0u, 0u, 0u, 0u};
            kr[c] = ok ? ld16_stream(p.k_cache + base + c * 512 + lane * 8) : z;
            vr[c] = ok ? ld16_stream(p.v_cache + base + c * 512 + lane * 8) : z;
        }
        return ok;
    };

    // the first block's loads go out before anything else waits
    uint4 kr[NC], vr[NC], kn[NC], vn[NC];
    int jb = blk_begin + wave;
    bool ok = load_block(jb, kr, vr);

    // the G query rows of this KV head, as 16-bit pairs
    {
        const uint32_t *qsrc = reinterpret_cast<const uint32_t *>(
            p.query + (static_cast<int64_t>(s) * p.Hq + hq0) * D);
        for (int i = tid; i < G * D / 2; i += kDecodeThreads) q_lds[i / (D / 2)][i % (D / 2)] = qsrc[i];
    }
    __syncthreads();
    for (; jb < blk_end; jb += NW) {
        const bool ok_next = load_block(jb + NW, kn, vn);   // in flight while this block is used
        const int tok = jb * BS + (lane & 15);
        const bool valid = ok && tok < t_end;

#pragma unroll
        for (int g = 0; g < GMAX; ++g) {
            if (g < G) {
                // score of token lane % 16: partial over this lane's 8 NC dims
                float dot = 0.f;
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    const uint4 qv = *reinterpret_cast<const uint4 *>(&q_lds[g][4 * (4 * c + kgrp)]);
                    dot = T::dot2(kr[c].x, qv.x, dot);
                    dot = T::dot2(kr[c].y, qv.y, dot);
                    dot = T::dot2(kr[c].z, qv.z, dot);
                    dot = T::dot2(kr[c].w, qv.w, dot);
                }
                dot = sum_xor16(dot);
                dot = sum_xor32(dot);
                const float sc = valid ? dot * c2 : -INFINITY;
                // online softmax over the block's 16 tokens (lanes 0..15, replicated)
                const float bm = row16_max(sc);
                const float m_new = fmaxf(m_run[g], bm);
                const bool none = m_new == -INFINITY;
                const float alpha = none ? 1.f : fast_exp2(m_run[g] - m_new);
                // the weight as the 16-bit value that multiplies V, so that
                // the row sum divides out exactly what the product summed
                const float pv = T::to_f32(T::from_f32(none ? 0.f : fast_exp2(sc - m_new)));
                const float ps = row16_sum(pv);
                l_run[g] = l_run[g] * alpha + ps;
                m_run[g] = m_new;
#pragma unroll
                for (int c = 0; c < NC; ++c) acc[g][c] *= alpha;
                if (lane < 16) p_lds[wave][g][lane] = pv;
            }
        }
        // p_lds is written and read by this wave only: LDS operations of one
        // wave complete in order
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int g = 0; g < GMAX; ++g) {
            if (g < G) {
                const float4 pa = *reinterpret_cast<const float4 *>(&p_lds[wave][g][8 * vhalf]);
                const float4 pb = *reinterpret_cast<const float4 *>(&p_lds[wave][g][8 * vhalf + 4]);
                const uint32_t w0 = T::pack2(pa.x, pa.y), w1 = T::pack2(pa.z, pa.w);
                const uint32_t w2 = T::pack2(pb.x, pb.y), w3 = T::pack2(pb.z, pb.w);
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    float a = acc[g][c];
                    a = T::dot2(vr[c].x, w0, a);
                    a = T::dot2(vr[c].y, w1, a);
                    a = T::dot2(vr[c].z, w2, a);
                    a = T::dot2(vr[c].w, w3, a);
                    acc[g][c] = a;
                }
            }
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            kr[c] = kn[c];
            vr[c] = vn[c];
        }
        ok = ok_next;
    }

    // lanes l and l ^ 1 hold the two 8-token halves of the same dims
#pragma unroll
    for (int g = 0; g < GMAX; ++g)
#pragma unroll
        for (int c = 0; c < NC; ++c) acc[g][c] += dpp_mov<kDppXor1>(acc[g][c]);

    // merge the four waves through LDS
#pragma unroll
    for (int g = 0; g < GMAX; ++g) {
        if (g < G) {
            if (lane == 0) {
                m_lds[wave][g] = m_run[g];
                l_lds[wave][g] = l_run[g];
            }
            if (vhalf == 0) {
#pragma unroll
                for (int c = 0; c < NC; ++c) o_lds[wave][g][32 * c + (lane >> 1)] = acc[g][c];
            }
        }
    }
    __syncthreads();
    // per head, once: the waves' weights 2^(m_w - M) (zero for a wave that saw
    // no token), folded with 1 / sum when this partition is the whole context
    if (tid < G) {
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, m_lds[w][tid]);
        float sw[NW], den = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float mw = m_lds[w][tid];
            sw[w] = mw == -INFINITY ? 0.f : fast_exp2(mw - M);
            den += sw[w] * l_lds[w][tid];
        }
        const float f = p.num_parts == 1 ? (den > 0.f ? 1.f / den : 0.f) : 1.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) c_lds[w][tid] = sw[w] * f;
        if (p.num_parts > 1) {
            const int64_t slot = (static_cast<int64_t>(s) * p.Hq + hq0 + tid) * p.num_parts + part;
            p.ws_ml[slot * 2 + 0] = M;
            p.ws_ml[slot * 2 + 1] = den;
        }
    }
    __syncthreads();
    // four dims of one head per thread: the weighted sum of the waves' O
    for (int i = tid; i < G * (D / 4); i += kDecodeThreads) {
        const int g = i / (D / 4), d = 4 * (i % (D / 4));
        f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < NW; ++w) o += c_lds[w][g] * *reinterpret_cast<const f32x4 *>(&o_lds[w][g][d]);
        const int64_t row = static_cast<int64_t>(s) * p.Hq + hq0 + g;
        if (p.num_parts == 1) {
            *reinterpret_cast<uint2 *>(p.out + row * D + d) = uint2{pack2<T>(o[0], o[1]), pack2<T>(o[2], o[3])};
        } else {
            *reinterpret_cast<f32x4 *>(p.ws_o + (row * p.num_parts + part) * D + d) = o;
        }
    }
}

// One wave per (sequence, query head): log-sum-exp merge of the partitions
// that hold part of the context.
template <typename T, int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecodeParams p)
{
    constexpr int BS = kDecodeBS;
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
    float den = 0.f, o[D / 64];
#pragma unroll
    for (int j = 0; j < D / 64; ++j) o[j] = 0.f;
    if (M != -INFINITY) {
        for (int i = 0; i < nparts; ++i) {
            const int64_t slot = row * p.num_parts + i;
            const float m = p.ws_ml[slot * 2];
            const float w = m == -INFINITY ? 0.f : fast_exp2(m - M);
            den += w * p.ws_ml[slot * 2 + 1];
#pragma unroll
            for (int j = 0; j < D / 64; ++j) o[j] += w * p.ws_o[slot * D + lane + 64 * j];
        }
    }
    const float inv = den > 0.f ? 1.f / den : 0.f;
#pragma unroll
    for (int j = 0; j < D / 64; ++j) p.out[row * D + lane + 64 * j] = T::from_f32(o[j] * inv);
}

}  // namespace attn
