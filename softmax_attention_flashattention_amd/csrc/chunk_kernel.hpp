// chunk_kernel.hpp -- output step of chunked gated delta-rule linear
// attention on gfx950.
//
// Operator (atrex-bench "chunk_delta_rule_output" #004, Reference
// Implementation): for every batch b, value head hd and chunk c of 64 tokens,
// with query head hq = min(hd / max(H / Hq, 1), Hq - 1),
//   o[i, :]   = exp(g[i]) * q[i, :] h_c               (h_c: 128 x 128 state)
//   a[i, j]   = (q[i] . k[j]) * exp(g[i] - g[j])   if j <= i and g[i] <= g[j]
//               0                                   otherwise
//   out[i, :] = scale * (o[i, :] + sum_j a[i, j]_16 v[j, :])
// where a_16 is a rounded to the 16-bit value type (round to nearest even).
//
// One workgroup of four waves per (b, c, hd); wave w owns chunk rows
// 32 (w % 2) .. + 31 (lane l: row l % 32) and output values
// 64 (w / 2) .. + 63.  All products
// are transposed so that a lane owns a token row, as in the prefill kernel:
//   S^T = K Q^T     (A = K rows j from global, B = Q^T from global)
//   O^T = h^T Q^T   (A = h^T by transposing LDS reads of the staged state)
//   O^T += V^T A^T  (A = V^T by transposing LDS reads of the staged values,
//                    B = a_16^T straight from the S^T accumulator)
// Lane l (hi = l / 32) holds contraction indices 8 hi .. 8 hi + 7 of each
// 16-step for the two Q products (Q and K rows are read as 16 contiguous
// bytes; the state's transposing reads take rows 8 hi + 0..3 and + 4..7);
// for the score product the S^T accumulator gives lane l the keys
// 4 hi + {0..3, 8..11} of each 16, and the value reads follow that order.
// The state h_c (32 KiB) and the chunk's v rows (16 KiB) go global -> LDS by
// direct DMA while S^T is computed; the chunk's 64 gate values are staged in
// LDS for the key-side exponentials.
//
// The operator streams q, k, v, h and out once: it is bound by HBM
// bandwidth (about 51 flop per byte), not by the matrix cores.
#pragma once

#include "device_common.hpp"

namespace attn {

typedef __attribute__((address_space(3))) void chunk_lds_void;

constexpr int kChunk = 64;        // tokens per chunk
constexpr int kChunkDim = 128;    // key_dim = value_dim
constexpr int kChunkWaves = 4;    // 2 row halves x 2 value halves
constexpr int kChunkThreads = 64 * kChunkWaves;

struct ChunkParams {
    const uint16_t *q, *k, *v, *h;
    const float *g;
    uint16_t *out;
    int batch, tokens, num_q_heads, num_heads, num_chunks, per_q;
    float scale;
};

template <typename T>
__global__ __launch_bounds__(kChunkThreads) void chunk_delta_out_kernel(ChunkParams p)
{
    constexpr int D = kChunkDim, C = kChunk;
    constexpr int PITCH = D;   // LDS row pitch (elements); 16-byte chunks XOR-swizzled
    __shared__ __attribute__((aligned(16))) uint16_t h_lds[D * PITCH];   // h_c: [k][v]
    __shared__ __attribute__((aligned(16))) uint16_t v_lds[C * PITCH];   // v rows: [j][v]
    __shared__ __attribute__((aligned(16))) float g_lds[C];

    // block -> work item w = (b, c, hd), value head fastest.  Hardware hands
    // consecutive blocks to the 8 XCDs in turn; the remap keeps runs of
    // consecutive items (the value heads that share one query head's q and k
    // rows) on one XCD's L2.
    const int64_t bid = blockIdx.x, total = gridDim.x;
    const int64_t per_xcd = total / 8;
    const int64_t w = bid < 8 * per_xcd ? (bid & 7) * per_xcd + (bid >> 3) : bid;
    const int hd = static_cast<int>(w % p.num_heads);
    const int64_t bc = w / p.num_heads;
    const int c = static_cast<int>(bc % p.num_chunks);
    const int b = static_cast<int>(bc / p.num_chunks);
    int hq = hd / p.per_q;
    if (hq > p.num_q_heads - 1) hq = p.num_q_heads - 1;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    const int l32 = lane & 31, hi = lane >> 5;
    const int rh = wave_s & 1, vh = wave_s >> 1;   // row half, value half
    constexpr int NDB = 2;                          // value blocks of 32 per wave
    const int t0 = c * C;
    const int n = p.tokens - t0 < C ? p.tokens - t0 : C;   // valid rows of this chunk
    const int64_t tok0 = static_cast<int64_t>(b) * p.tokens + t0;   // flat index of row 0
    const int64_t qrs = static_cast<int64_t>(p.num_q_heads) * D;     // q/k token stride
    const int64_t vrs = static_cast<int64_t>(p.num_heads) * D;       // v/out token stride

    // ---- h_c and the chunk's v rows -> LDS by direct DMA.  Instruction j of
    // wave w fills 4 rows; chunk cc of row R sits at cc ^ 4 (R % 4).
    {
        const int rsub = lane >> 4, pos = lane & 15;
        const uint16_t *hbase = p.h + ((static_cast<int64_t>(b) * p.num_chunks + c) * p.num_heads + hd) * D * D;
        const __amdgpu_buffer_rsrc_t rsh = make_rsrc(hbase, D * D * 2u);
        const __amdgpu_buffer_rsrc_t rsv = make_rsrc(p.v + tok0 * vrs + static_cast<int64_t>(hd) * D,
                                                    static_cast<uint32_t>(n - 1) * static_cast<uint32_t>(vrs * 2) + D * 2u);
        // h: 32 instructions of 4 rows, 8 per wave
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int R = 32 * wave + 4 * j + rsub;
            const uint32_t off = static_cast<uint32_t>(R) * (D * 2u) + 16u * static_cast<uint32_t>(pos ^ (4 * (R & 3)));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsh, (chunk_lds_void *)(h_lds + (32 * wave_s + 4 * j) * PITCH), 16, off, 0, 0, 0);
        }
        // v: 16 instructions of 4 rows, 4 per wave (rows past the chunk's end read as zeros)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int R = 16 * wave + 4 * j + rsub;
            const uint32_t off = static_cast<uint32_t>(R) * static_cast<uint32_t>(vrs * 2) +
                                 16u * static_cast<uint32_t>(pos ^ (4 * (R & 3)));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsv, (chunk_lds_void *)(v_lds + (16 * wave_s + 4 * j) * PITCH), 16, off, 0, 0, 0);
        }
    }
    // gate values of the chunk's tokens (0 past the end; those keys are masked)
    if (wave == 0) {
        const int t = lane;
        g_lds[t] = t < n ? p.g[(tok0 + t) * p.num_heads + hd] : 0.f;
    }

    // ---- Q^T operands of this wave's rows (B of both Q products) and the
    // K operands (A of S^T): contraction indices 16 ks + 8 hi .. + 7
    const int row = 32 * rh + l32;             // this lane's chunk row
    const bool row_ok = row < n;
    s16x8 qreg[8];
    {
        const uint16_t *qrow = p.q + (tok0 + row) * qrs + static_cast<int64_t>(hq) * D + 8 * hi;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            uint4 v4 = {0u, 0u, 0u, 0u};
            if (row_ok) v4 = ld16(qrow + 16 * ks);
            qreg[ks] = __builtin_bit_cast(s16x8, v4);
        }
    }
    // key blocks of 32 that can hold keys j <= row for this wave's rows
    const int nkb = rh + 1;
    f32x16 sacc[2];
    const f32x16 zero = {};
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
        if (kb2 < nkb) {
            const int key = 32 * kb2 + l32;
            const bool key_ok = key < n;
            const uint16_t *krow = p.k + (tok0 + key) * qrs + static_cast<int64_t>(hq) * D + 8 * hi;
            s16x8 kop[8];
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                uint4 v4 = {0u, 0u, 0u, 0u};
                if (key_ok) v4 = ld16(krow + 16 * ks);
                kop[ks] = __builtin_bit_cast(s16x8, v4);
            }
#pragma unroll
            for (int ks = 0; ks < 8; ++ks)
                sacc[kb2] = T::mfma32(kop[ks], qreg[ks], ks == 0 ? zero : sacc[kb2]);
        } else {
            sacc[kb2] = zero;
        }
    }

    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's DMA has landed
    __syncthreads();                      // ... and every wave's, and g_lds

    // ---- gated, masked scores rounded to 16 bits, packed as the B operand
    // of O^T += V^T A^T.  Register r of key block kb2 holds key
    // 32 kb2 + 8 (r / 4) + 4 hi + r % 4 for this lane's row.
    const float gi = g_lds[row];
    uint32_t pw[16];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const int kbase = 32 * kb2 + 8 * r4 + 4 * hi;
            const float4 gj = *reinterpret_cast<const float4 *>(&g_lds[kbase]);
            const float gjs[4] = {gj.x, gj.y, gj.z, gj.w};
            float a[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int key = kbase + e;
                const bool keep = kb2 < nkb && key <= row && gi <= gjs[e];
                a[e] = keep ? sacc[kb2][4 * r4 + e] * fast_exp2((gi - gjs[e]) * kLog2e) : 0.f;
            }
            pw[8 * kb2 + 2 * r4] = T::pack2(a[0], a[1]);
            pw[8 * kb2 + 2 * r4 + 1] = T::pack2(a[2], a[3]);
        }
    }

    // ---- O^T = h_c^T Q^T (4 blocks of 32 values x 8 contraction steps).
    // A transposing read returns, to lane i of each 16, one column of four
    // consecutive rows; lane m of the 16 addresses row m / 4 (of those four)
    // and the four columns 4 (m % 4) .. + 3.  Which four rows each group of
    // 16 lanes starts at, and how far the second read is from the first,
    // decides the contraction order: `first` rows and a `step` apart.
    const int g16 = lane >> 4;
    const int tr_col = 16 * (g16 & 1) + 4 * (lane & 3);
    auto tr_addr = [&](int first_row, int (&a)[4]) {
#pragma unroll
        for (int db = 0; db < 4; ++db)
            a[db] = first_row * PITCH + 8 * ((4 * db + (tr_col >> 3)) ^ (4 * (first_row & 3))) + (tr_col & 7);
    };
    auto trop = [&](const uint16_t *tile, const int (&rd)[4], int step, int row16, int db) {
        const uint16_t *base = tile + 16 * row16 * PITCH + rd[db];
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(base));
        const s16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(base + step * PITCH));
        return s16x8{lo[0], lo[1], lo[2], lo[3], up[0], up[1], up[2], up[3]};
    };
    // state: rows 8 hi + 0..3, then + 4 (the order of Q's 16-byte pieces)
    int rd_h[4], rd_v[4];
    tr_addr(8 * (g16 >> 1) + ((lane & 15) >> 2), rd_h);
    tr_addr(4 * (g16 >> 1) + ((lane & 15) >> 2), rd_v);
    f32x16 oacc[NDB];   // value blocks NDB vh + i
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
        for (int i = 0; i < NDB; ++i)
            oacc[i] = T::mfma32(trop(h_lds, rd_h, 4, ks, NDB * vh + i), qreg[ks], ks == 0 ? zero : oacc[i]);
    const float egi = fast_exp2(gi * kLog2e);
#pragma unroll
    for (int i = 0; i < NDB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[i][r] *= egi;

    // ---- O^T += V^T A^T over the key chunks of 16 this wave's rows can see
    // (value rows 4 hi + 0..3, then + 8: the key order of the accumulator)
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
        if (kc < 2 * nkb) {
            const uint4 w4 = {pw[4 * kc], pw[4 * kc + 1], pw[4 * kc + 2], pw[4 * kc + 3]};
#pragma unroll
            for (int i = 0; i < NDB; ++i)
                oacc[i] = T::mfma32(trop(v_lds, rd_v, 8, kc, NDB * vh + i), __builtin_bit_cast(s16x8, w4), oacc[i]);
        }
    }

    // ---- epilogue: scale, round to 16 bits, store the valid rows
    if (row_ok) {
        uint16_t *orow = p.out + (tok0 + row) * vrs + static_cast<int64_t>(hd) * D;
        const float s = p.scale;
#pragma unroll
        for (int i = 0; i < NDB; ++i)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                uint2 w2;
                w2.x = T::pack2(oacc[i][4 * g4] * s, oacc[i][4 * g4 + 1] * s);
                w2.y = T::pack2(oacc[i][4 * g4 + 2] * s, oacc[i][4 * g4 + 3] * s);
                *reinterpret_cast<uint2 *>(orow + 32 * (NDB * vh + i) + 8 * g4 + 4 * hi) = w2;
            }
    }
}

}  // namespace attn
