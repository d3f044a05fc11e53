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
//   S^T = K Q^T     (A = K rows j, B = Q^T: 16-byte LDS reads of the rows)
//   O^T = h^T Q^T   (A = h^T by transposing LDS reads of the staged state)
//   O^T += V^T A^T  (A = V^T by transposing LDS reads of the staged values,
//                    B = a_16^T straight from the S^T accumulator)
// Lane l (hi = l / 32) holds contraction indices 8 hi .. 8 hi + 7 of each
// 16-step for the two Q products (the state's transposing reads take rows
// 8 hi + 0..3 and + 4..7 to match); for the score product the S^T
// accumulator gives lane l the keys 4 hi + {0..3, 8..11} of each 16, and the
// value reads follow that order.
//
// Every input tile goes global -> LDS by direct DMA, whole rows per
// instruction: the chunk's q and k rows (16 KiB each), then h_c (32 KiB) and
// the v rows (16 KiB), 80 KiB in all (two workgroups per CU).  Loads of one
// row per lane straight into registers touch 32 rows per instruction and
// read far below HBM speed; DMA of whole rows does not.  Each stage waits
// only for the tiles it reads (loads land in issue order).  Gate values
// travel by lane shuffles; the output tile is staged in LDS over the q rows
// and stored as whole 256-byte rows.
//
// The operator streams q, k, v, h and out once: it is bound by HBM
// bandwidth (about 51 flop per byte), not by the matrix cores.
#pragma once

#include "device_common.hpp"

namespace attn {

typedef __attribute__((address_space(3))) void chunk_lds_void;
typedef unsigned int chunk_u32x4 __attribute__((ext_vector_type(4)));
constexpr int kNonTemporal = 2;   // cache-policy bit of buffer loads: streamed, not kept

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
    __shared__ __attribute__((aligned(16))) uint16_t q_lds[C * PITCH];   // q rows [i][k]; then the output tile
    __shared__ __attribute__((aligned(16))) uint16_t k_lds[C * PITCH];   // k rows [j][k]
    __shared__ __attribute__((aligned(16))) uint16_t h_lds[D * PITCH];   // h_c: [k][v]
    __shared__ __attribute__((aligned(16))) uint16_t v_lds[C * PITCH];   // v rows: [j][v]

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

    // Every global read goes through a buffer resource that ends at the
    // chunk's last valid token: rows past the end read as zeros.  Lane t
    // holds the gate value of token t.
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(p.g + tok0 * p.num_heads + hd,
                                                static_cast<uint32_t>((n - 1) * p.num_heads + 1) * 4u);
    const float gval = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rg, lane * p.num_heads * 4, 0, 0));

    // ---- DMA, in the order the stages below need the tiles.  Instruction j
    // of wave w fills rows 4 m .. 4 m + 3, m = 4 j + w, one row per 16 lanes;
    // lane (r, pos) fetches 16-byte chunk pos ^ f(R) of row R = 4 m + r, so
    // LDS chunk position x of row R holds chunk x ^ f(R).  q and k rows,
    // read 16 bytes per lane: f(R) = R % 8; h_c and v rows, read by
    // transposing reads: f(R) = 4 (R % 4).  h_c and v are read once and go
    // non-temporal; the q and k rows stay cached for the other value heads
    // of the same query head.
    {
        const int rsub = lane >> 4, pos = lane & 15;
        const uint32_t qk_bytes = static_cast<uint32_t>((n - 1) * qrs + D) * 2u;
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.q + tok0 * qrs + static_cast<int64_t>(hq) * D, qk_bytes);
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k + tok0 * qrs + static_cast<int64_t>(hq) * D, qk_bytes);
        const uint16_t *hbase = p.h + ((static_cast<int64_t>(b) * p.num_chunks + c) * p.num_heads + hd) * D * D;
        const __amdgpu_buffer_rsrc_t rsh = make_rsrc(hbase, D * D * 2u);
        const __amdgpu_buffer_rsrc_t rsv = make_rsrc(p.v + tok0 * vrs + static_cast<int64_t>(hd) * D,
                                                    static_cast<uint32_t>(n - 1) * static_cast<uint32_t>(vrs * 2) + D * 2u);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int m = 4 * j + wave_s, R = 4 * m + rsub;
            const uint32_t off = static_cast<uint32_t>(R) * static_cast<uint32_t>(qrs * 2) +
                                 16u * static_cast<uint32_t>(pos ^ (R & 7));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (chunk_lds_void *)(q_lds + 4 * m * PITCH), 16, off, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (chunk_lds_void *)(k_lds + 4 * m * PITCH), 16, off, 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int m = 4 * j + wave_s, R = 4 * m + rsub;
            const uint32_t off = static_cast<uint32_t>(R) * (D * 2u) + 16u * static_cast<uint32_t>(pos ^ (4 * (R & 3)));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsh, (chunk_lds_void *)(h_lds + 4 * m * PITCH), 16, off, 0, 0, kNonTemporal);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int m = 4 * j + wave_s, R = 4 * m + rsub;
            const uint32_t off = static_cast<uint32_t>(R) * static_cast<uint32_t>(vrs * 2) +
                                 16u * static_cast<uint32_t>(pos ^ (4 * (R & 3)));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsv, (chunk_lds_void *)(v_lds + 4 * m * PITCH), 16, off, 0, 0, kNonTemporal);
        }
    }
    // a workgroup barrier that waits for no load still in flight; the memory
    // clobber keeps LDS accesses on their side of it
    auto barrier = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    };
    __builtin_amdgcn_s_waitcnt(0x0F7C);   // vmcnt(12): g, q and k have landed (h_c and v in flight)
    barrier();

    // ---- Q^T operands of this wave's rows (B of both Q products) and the
    // K operands (A of S^T): contraction indices 16 ks + 8 hi .. + 7
    const int row = 32 * rh + l32;   // this lane's chunk row
    auto rd16 = [&](const uint16_t *tile, int r, int chunk) {
        return *reinterpret_cast<const s16x8 *>(tile + r * PITCH + 8 * (chunk ^ (r & 7)));
    };
    s16x8 qreg[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qreg[ks] = rd16(q_lds, row, 2 * ks + hi);
    // key blocks of 32 that can hold keys j <= row for this wave's rows
    const int nkb = rh + 1;
    f32x16 sacc[2];
    const f32x16 zero = {};
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
        if (kb2 < nkb) {
            s16x8 kop[8];
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) kop[ks] = rd16(k_lds, 32 * kb2 + l32, 2 * ks + hi);
#pragma unroll
            for (int ks = 0; ks < 8; ++ks)
                sacc[kb2] = T::mfma32(kop[ks], qreg[ks], ks == 0 ? zero : sacc[kb2]);
        } else {
            sacc[kb2] = zero;
        }
    }

    // ---- gated, masked scores rounded to 16 bits, packed as the B operand
    // of O^T += V^T A^T.  Register r of key block kb2 holds key
    // 32 kb2 + 8 (r / 4) + 4 hi + r % 4 for this lane's row.
    const float gi = __shfl(gval, row, 64);
    float gk[2][16];   // gate values of the keys in the accumulator's order
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            gk[kb2][r] = __shfl(gval, 32 * kb2 + 8 * (r >> 2) + 4 * hi + (r & 3), 64);
    uint32_t pw[16];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const int kbase = 32 * kb2 + 8 * r4 + 4 * hi;
            float a[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int key = kbase + e;
                const float gj = gk[kb2][4 * r4 + e];
                const bool keep = kb2 < nkb && key <= row && gi <= gj;
                // computed for every key, then selected: no branch per element
                const float x = sacc[kb2][4 * r4 + e] * fast_exp2(fminf(gi - gj, 0.f) * kLog2e);
                a[e] = keep ? x : 0.f;
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
    // addresses of this wave's value blocks NDB vh + i
    auto tr_addr = [&](int first_row, int (&a)[NDB]) {
#pragma unroll
        for (int i = 0; i < NDB; ++i)
            a[i] = first_row * PITCH + 8 * ((4 * (NDB * vh + i) + (tr_col >> 3)) ^ (4 * (first_row & 3))) + (tr_col & 7);
    };
    auto trop = [&](const uint16_t *tile, const int (&rd)[NDB], int step, int row16, int i) {
        const uint16_t *base = tile + 16 * row16 * PITCH + rd[i];
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(base));
        const s16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(base + step * PITCH));
        return s16x8{lo[0], lo[1], lo[2], lo[3], up[0], up[1], up[2], up[3]};
    };
    // state: rows 8 hi + 0..3, then + 4 (the order of Q's 16-byte pieces)
    int rd_h[NDB], rd_v[NDB];
    tr_addr(8 * (g16 >> 1) + ((lane & 15) >> 2), rd_h);
    tr_addr(4 * (g16 >> 1) + ((lane & 15) >> 2), rd_v);
    __builtin_amdgcn_s_waitcnt(0x0F74);   // vmcnt(4): h_c has landed
    barrier();                            // ... for every wave; q_lds is no longer read
    f32x16 oacc[NDB];   // value blocks NDB vh + i
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
        for (int i = 0; i < NDB; ++i)
            oacc[i] = T::mfma32(trop(h_lds, rd_h, 4, ks, i), qreg[ks], ks == 0 ? zero : oacc[i]);
    const float egi = fast_exp2(gi * kLog2e);
#pragma unroll
    for (int i = 0; i < NDB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[i][r] *= egi;

    // ---- O^T += V^T A^T over the key chunks of 16 this wave's rows can see
    // (value rows 4 hi + 0..3, then + 8: the key order of the accumulator)
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the v rows have landed
    barrier();
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
        if (kc < 2 * nkb) {
            const uint4 w4 = {pw[4 * kc], pw[4 * kc + 1], pw[4 * kc + 2], pw[4 * kc + 3]};
#pragma unroll
            for (int i = 0; i < NDB; ++i)
                oacc[i] = T::mfma32(trop(v_lds, rd_v, 8, kc, i), __builtin_bit_cast(s16x8, w4), oacc[i]);
        }
    }

    // ---- epilogue: scale, round to 16 bits, stage the 64 x 128 output tile
    // in q_lds (16-byte chunk x of row R at x ^ (R % 16)) and store whole
    // rows of the valid tokens, streaming past the caches
    {
        const float s = p.scale;
#pragma unroll
        for (int i = 0; i < NDB; ++i)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                uint2 w2;
                w2.x = T::pack2(oacc[i][4 * g4] * s, oacc[i][4 * g4 + 1] * s);
                w2.y = T::pack2(oacc[i][4 * g4 + 2] * s, oacc[i][4 * g4 + 3] * s);
                const int chunk = 4 * (NDB * vh + i) + g4;
                *reinterpret_cast<uint2 *>(q_lds + row * PITCH + 8 * (chunk ^ (row & 15)) + 4 * hi) = w2;
            }
    }
    barrier();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int R = 16 * wave_s + 4 * j + (lane >> 4), pos = lane & 15;
        const uint4 w4 = *reinterpret_cast<const uint4 *>(q_lds + R * PITCH + 8 * (pos ^ (R & 15)));
        if (R < n)
            __builtin_nontemporal_store(chunk_u32x4{w4.x, w4.y, w4.z, w4.w},
                                        reinterpret_cast<chunk_u32x4 *>(p.out + (tok0 + R) * vrs +
                                                                        static_cast<int64_t>(hd) * D + 8 * pos));
    }
}

}  // namespace attn
