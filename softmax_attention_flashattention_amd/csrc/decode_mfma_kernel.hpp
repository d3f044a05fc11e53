// decode_mfma_kernel.hpp -- paged single-query decode for grouped query heads
// on MFMAs, for gfx950.
//
// The operator of decode_kernel.hpp ("paged_attention_decode" #024,
// Reference Implementation): per sequence s and query head hq,
// out = softmax(scale * q K^T) V over the first seq_lens[s] tokens, K and V
// read through the block table from the paged cache (K [blocks, Hkv, D/8, 16,
// 8], V [blocks, Hkv, D, 16]).  With G query heads per KV head, the G x D by
// D x 16 score product and the G x 16 by 16 x D value product of each cache
// block are small matrix products; on VALU dot products their cost grows with
// G until it, not the cache reads, bounds the launch (one sequence block of
// 64 sequences x 2048 tokens x 8 KV heads ran at 5.0 TB/s with one query head
// per KV head and 2.2 TB/s with 16).  Here they run on 16x16x32 MFMAs, the
// query heads padded to 16 columns:
//   S^T[token, g] = K Q^T     A = K rows (16 tokens x 32 dims), B = Q^T
//   O^T[d, g]    += V^T P^T   A = V^T (16 dims x 32 tokens), B = P^T
// Lane l owns query head g = l % 16 (the rows past G are zero and their
// results are dropped) and token / dim group q = l / 16.  The score
// accumulator of a 16-token block holds, in lane (g, q), tokens 4q .. 4q+3
// of head g; the accumulators of two consecutive blocks together are, word
// for word, the B operand of the value product over those 32 tokens, with the
// k slots 8q .. 8q+7 standing for tokens 4q .. 4q+3 of the first block and
// 4q .. 4q+3 of the second.  The V^T operand takes its k slots in the same
// order, so no lane exchange is needed between the two products.  Cache
// reads: K 16 bytes per lane per 32 dims (one 1 KiB run per instruction), V 8
// bytes per lane per block and 16 dims (one 512-byte run).
//
// Each wave takes every fourth pair of blocks of the workgroup's partition
// (every fourth block when there are fewer than eight) and keeps its own
// online softmax per head (base-2 domain, running max
// raised only when a score passes it by more than 2^8: the result is
// shift-invariant); the row sum adds up the 16-bit weights that multiply V.
// The four waves merge through LDS (per head once: the waves' weights and the
// reciprocal of the row sum; then four dims a thread); a split context writes
// (max, sum, unnormalised output) for decode_merge_kernel, as
// decode_partition_kernel does.
#pragma once

#include "decode_kernel.hpp"
#include "device_common.hpp"

namespace attn {

constexpr float kDecodeRescaleThreshold = 8.0f;   // log2 units the running max may lag

// max(v, value of lane l ^ 16) (v_permlane16_swap exchanges rows 0<->1, 2<->3)
__device__ __forceinline__ float max_xor16(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// 8-byte load of data read once (non-temporal)
__device__ __forceinline__ uint2 ld8_stream(const void *p) {
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
    return uint2{v.x, v.y};
}

template <typename T, int D>
__global__ __launch_bounds__(kDecodeThreads) __attribute__((amdgpu_waves_per_eu(D == 128 ? 4 : 2))) void decode_mfma_kernel(DecodeParams p)
{
    constexpr int BS = kDecodeBS, NW = kDecodeWaves;
    constexpr int KS = D / 32;          // 32-dim k-steps of a block's score product
    constexpr int DT = D / 16;          // 16-dim tiles of O^T
    constexpr int CHUNK = D * BS;       // elements of one (block, kv head) chunk
    __shared__ float m_lds[NW][16], l_lds[NW][16], c_lds[NW][16];
    __shared__ __attribute__((aligned(16))) float o_lds[NW][16][D];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane & 15, q = lane >> 4;
    int id = blockIdx.x;
    const int part = id % p.num_parts;
    id /= p.num_parts;
    const int hk = id % p.Hkv;           // one workgroup holds all G query heads (ngroups 1)
    const int s = id / p.Hkv;
    const int G = p.G;
    const int hq0 = hk * G;

    int L = p.seq_lens[s];
    L = L > p.maxb * BS ? p.maxb * BS : L;
    const int t_begin = part * p.part_blocks * BS;
    const int t_end = L < t_begin + p.part_blocks * BS ? L : t_begin + p.part_blocks * BS;
    if (t_end <= t_begin) {
        // no tokens here: final zeros with one partition; with several the
        // merge kernel skips partitions past the context
        if (p.num_parts == 1)
            for (int i = tid; i < G * D; i += kDecodeThreads)
                p.out[(static_cast<int64_t>(s) * p.Hq + hq0) * D + i] = 0;
        return;
    }

    // Q^T of this lane's head as B operands: dims 32 ks + 8 q .. +7
    s16x8 qop[KS];
    {
        const uint16_t *qrow = p.query + (static_cast<int64_t>(s) * p.Hq + hq0 + g) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const uint4 z = {0u, 0u, 0u, 0u};
            qop[ks] = __builtin_bit_cast(s16x8, g < G ? ld16(qrow + 32 * ks + 8 * q) : z);
        }
    }

    const int blk_begin = t_begin / BS;
    const int blk_end = (t_end + BS - 1) / BS;
    // a wave's unit of work: a pair of blocks, or one block (the second half
    // of the value product's k slots then carries zero weights) when the
    // partition has fewer than two blocks per wave, so that all waves work
    const int ub = blk_end - blk_begin >= 2 * NW ? 2 : 1;
    const int nunits = (blk_end - blk_begin + ub - 1) / ub;
    const int32_t *bt_row = p.block_tables + static_cast<int64_t>(s) * p.maxb;
    const float c2 = p.scale_log2e;

    float m_run = -INFINITY;   // running max of c2 * score for head g (log2 domain)
    float l_run = 0.f;         // this lane's part of the row sum
    f32x4 oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int u = wave; u < nunits; u += NW) {
        const int jb0 = blk_begin + ub * u;
        int64_t base[2];
        bool ok[2];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int jb = jb0 + b;
            const int64_t phys = (jb < blk_end && b < ub) ? bt_row[jb] : -1;
            ok[b] = phys >= 0 && phys < p.num_blocks;
            base[b] = ok[b] ? (phys * p.Hkv + hk) * CHUNK : 0;
        }
        // K: token t = lane % 16, dims 32 ks + 8 q .. +7 (chunk 4 ks + q of the
        // [D/8][16][8] block); V: dim 16 dt + lane % 16, tokens 4 q .. 4 q + 3
        // of each block ([D][16] block)
        uint4 kr[2][KS];
        uint2 vr[2][DT];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const uint4 z = {0u, 0u, 0u, 0u};
                kr[b][ks] = ok[b] ? ld16_stream(p.k_cache + base[b] + ((4 * ks + q) * BS + g) * 8) : z;
            }
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const uint2 z = {0u, 0u};
                vr[b][dt] = ok[b] ? ld8_stream(p.v_cache + base[b] + (16 * dt + g) * BS + 4 * q) : z;
            }
        }
        // S^T of both blocks: lane (g, q) gets tokens 4 q .. 4 q + 3 of head g
        f32x4 sc[2];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            sc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) sc[b] = T::mfma16(__builtin_bit_cast(s16x8, kr[b][ks]), qop[ks], sc[b]);
        }
        // scaled scores, tokens past the context (or in a missing block) at -inf
        float mx = -INFINITY;
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tok = (jb0 + b) * BS + 4 * q + r;
                sc[b][r] = (ok[b] && tok < t_end) ? sc[b][r] * c2 : -INFINITY;
                mx = fmaxf(mx, sc[b][r]);
            }
        mx = max_xor16(mx);
        mx = max_halves(mx);   // head g's max over the 32 tokens (every lane of g)
        if (__builtin_amdgcn_ballot_w64(mx > m_run + kDecodeRescaleThreshold) != 0) {
            // some head's max passed the running one by more than the
            // threshold (always on the first pair): raise it, rescale O and l
            const float m_new = mx > m_run + kDecodeRescaleThreshold ? mx : m_run;
            const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m_run - m_new);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
        }
        // weights rounded to the 16-bit type, packed as the B operand of the
        // value product; the row sum adds up the same rounded weights
        uint32_t pw[4];
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const float e0 = m_run == -INFINITY ? 0.f : fast_exp2(sc[b][2 * h] - m_run);
                const float e1 = m_run == -INFINITY ? 0.f : fast_exp2(sc[b][2 * h + 1] - m_run);
                const uint32_t w = pack2<T>(e0, e1);
                pw[2 * b + h] = w;
                l_run = T::sum2(w, l_run);
            }
        const s16x8 pop = __builtin_bit_cast(s16x8, uint4{pw[0], pw[1], pw[2], pw[3]});
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const uint4 a = {vr[0][dt].x, vr[0][dt].y, vr[1][dt].x, vr[1][dt].y};
            oacc[dt] = T::mfma16(__builtin_bit_cast(s16x8, a), pop, oacc[dt]);
        }
    }

    // this wave's (max, sum, O) per head to LDS: the row sum over the four
    // token groups of head g; lane (g, q) holds dims 16 dt + 4 q .. +3
    const float l_tot = sum_xor32(sum_xor16(l_run));
    if (g < G) {   // the padded heads' columns are dropped (skipping them: 7-14% on short contexts)
        if (q == 0) {
            m_lds[wave][g] = m_run;
            l_lds[wave][g] = l_tot;
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
            *reinterpret_cast<f32x4 *>(&o_lds[wave][g][16 * dt + 4 * q]) = oacc[dt];
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
        const int gi = i / (D / 4), d = 4 * (i % (D / 4));
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < NW; ++w) acc += c_lds[w][gi] * *reinterpret_cast<const f32x4 *>(&o_lds[w][gi][d]);
        const int64_t row = static_cast<int64_t>(s) * p.Hq + hq0 + gi;
        if (p.num_parts == 1) {
            *reinterpret_cast<uint2 *>(p.out + row * D + d) = uint2{pack2<T>(acc[0], acc[1]), pack2<T>(acc[2], acc[3])};
        } else {
            *reinterpret_cast<f32x4 *>(p.ws_o + (row * p.num_parts + part) * D + d) = acc;
        }
    }
}

}  // namespace attn
