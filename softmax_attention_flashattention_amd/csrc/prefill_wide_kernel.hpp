// prefill_wide_kernel.hpp -- varlen prefill attention, head_dim 128, with
// 64 query rows per wave.
//
// Same operator and same arithmetic as prefill_fwd_kernel (see
// prefill_kernel.hpp for the MFMA orientation, the online softmax and the
// LDS layout); what changes is the work split.  Each wave owns two 32-row
// sub-tiles (A and B) of the workgroup's 256 query rows, so every K and V
// operand read from LDS feeds two MFMAs instead of one: the LDS read traffic
// per flop halves, which is what bounds the 32-row kernel.  The price is
// registers: Q, S and O of two sub-tiles need about 400 per lane, so the
// kernel runs one wave per SIMD (O lives in AGPRs), and all latency hiding
// comes from its own software pipeline:
//   block 1: the 32 MFMAs of S(t+1) for A and B (each K operand read once),
//            interleaved with most of the exponentials of tile t;
//   block 2: the 32 MFMAs of O += V P for tile t (each V operand read once),
//            interleaved with the rest of the exponentials and with the row
//            max of tile t+1;
//   then the (rarely taken) rescale and one barrier.
#pragma once

#include "prefill_kernel.hpp"

namespace attn {

constexpr int kWideWaves = 4;
constexpr int kWideThreads = 64 * kWideWaves;
constexpr int kWideBM = 64 * kWideWaves;   // 256 query rows per workgroup

template <typename T>
__global__ __launch_bounds__(kWideThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void prefill_fwd_wide_kernel(PrefillParams p)
{
    constexpr int D = 128, BN = kPrefillBN, KP = 128, VP = 128;
    constexpr int KSTEPS = 8, DBLK = 4, BM = kWideBM;
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;

    __shared__ __attribute__((aligned(16))) uint16_t k_lds0[BN * KP];
    __shared__ __attribute__((aligned(16))) uint16_t k_lds1[BN * KP];
    __shared__ __attribute__((aligned(16))) uint16_t v_lds0[BN * VP];
    __shared__ __attribute__((aligned(16))) uint16_t v_lds1[BN * VP];
    auto kbuf = [&](auto par) -> uint16_t * {
        if constexpr (decltype(par)::value == 0) return k_lds0; else return k_lds1;
    };
    auto vbuf = [&](auto par) -> uint16_t * {
        if constexpr (decltype(par)::value == 0) return v_lds0; else return v_lds1;
    };

    // work id (as in prefill_fwd_kernel)
    const int bid = blockIdx.x;
    int w, part = 0, nparts = 1;
    if (bid < p.whole_work) {
        w = (bid & 7) * (p.whole_work >> 3) + (bid >> 3);
    } else {
        const int j = bid - p.whole_work;
        nparts = p.split_parts;
        w = p.whole_work + j / nparts;
        part = j % nparts;
    }
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
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    const int l32 = lane & 31, hi = lane >> 5;
    const int64_t rs = static_cast<int64_t>(p.num_heads) * D;
    const uint32_t row_bytes = static_cast<uint32_t>(rs * 2);
    const uint16_t *k_head = p.k + ka * rs + head * D;
    const uint16_t *v_head = p.v + ka * rs + head * D;
    const float c = p.scale_log2e;

    // Q^T operands of the two sub-tiles: rows q0 + 64 wave + 32 sub + l32
    s16x8 qreg[2][KSTEPS];
    int qrow[2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
        qrow[sub] = q0 + 64 * wave + 32 * sub + l32;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            const int d0 = 16 * ks + 8 * hi;
            uint4 v4 = {0u, 0u, 0u, 0u};
            if (qrow[sub] < Sq) v4 = ld16(p.q + (qa + qrow[sub]) * rs + head * D + d0);
            qreg[sub][ks] = __builtin_bit_cast(s16x8, v4);
        }
    }

    // key tiles [t0, t1) of this workgroup
    const int ntiles = (Sk + BN - 1) / BN;
    const int t0 = static_cast<int>((static_cast<int64_t>(part) * ntiles) / nparts);
    const int t1 = static_cast<int>((static_cast<int64_t>(part + 1) * ntiles) / nparts);
    auto tile_bytes = [&](int t) -> uint32_t {
        const int rows = Sk - t * BN < BN ? Sk - t * BN : BN;
        return (rows > 0 && t < t1) ? static_cast<uint32_t>(rows - 1) * row_bytes + D * 2u : 0u;
    };

    // global -> LDS: instruction j of wave w fills rows 16 w + 4 j .. +3;
    // chunk c of row R sits at c ^ (R % 16) for K and c ^ 4 (R % 4) for V
    uint32_t dk_off[4];
    {
        const int rsub = lane >> 4, pos = lane & 15;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int R = 16 * wave + 4 * j + rsub;
            dk_off[j] = static_cast<uint32_t>(R) * row_bytes + 16u * static_cast<uint32_t>(pos ^ (R & 15));
        }
    }
    const uint32_t dv_off = static_cast<uint32_t>(16 * wave + (lane >> 4)) * row_bytes +
                            16u * static_cast<uint32_t>((lane & 15) ^ (4 * ((lane >> 4) & 3)));
    auto load_k = [&](int t, auto par) {
        const __amdgpu_buffer_rsrc_t r = make_rsrc(k_head + static_cast<int64_t>(t) * BN * rs, tile_bytes(t));
#pragma unroll
        for (int j = 0; j < 4; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                r, (lds_void *)(kbuf(par) + (16 * wave_s + 4 * j) * KP), 16, dk_off[j], 0, 0, 0);
    };
    auto load_v = [&](int t, auto par) {
        const __amdgpu_buffer_rsrc_t r = make_rsrc(v_head + static_cast<int64_t>(t) * BN * rs, tile_bytes(t));
#pragma unroll
        for (int j = 0; j < 4; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                r, (lds_void *)(vbuf(par) + (16 * wave_s + 4 * j) * VP), 16, dv_off,
                static_cast<int>(4 * j * row_bytes), 0, 0);
    };
    auto tiles_ready = [&]() {
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
        __syncthreads();
    };

    // operand addressing inside a tile buffer (elements)
    int k_rd[KSTEPS];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) k_rd[ks] = l32 * KP + 8 * ((2 * ks + hi) ^ (l32 & 15));
    const int g16 = lane >> 4;
    const int tr_row = 4 * (g16 >> 1) + ((lane & 15) >> 2);
    const int tr_col = 16 * (g16 & 1) + 4 * (lane & 3);
    int v_rd[DBLK];
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
        v_rd[db] = tr_row * VP + 8 * ((4 * db + (tr_col >> 3)) ^ (4 * (tr_row & 3))) + (tr_col & 7);

    // S^T accumulators: [sub][kb2]
    auto mask_tail = [&](int t, f32x16 (&s)[2][2]) {
        const int kbase = t * BN;
        if (kbase + BN > Sk) {
#pragma unroll
            for (int sub = 0; sub < 2; ++sub)
#pragma unroll
                for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = kbase + 32 * kb2 + 8 * (r >> 2) + 4 * hi + (r & 3);
                        if (key >= Sk) s[sub][kb2][r] = -INFINITY;
                    }
        }
    };

    float m_run[2] = {-INFINITY, -INFINITY};
    float l_run[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
    f32x16 oacc[2][DBLK];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int db = 0; db < DBLK; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[sub][db][r] = 0.f;

    // row max of S(t) for one sub-tile, over value range [vb, ve) of its 32
    auto max_part = [&](const f32x16 (&s)[2], int vb, int ve, float mx) {
#pragma unroll
        for (int v = vb; v < ve; ++v) mx = fmaxf(mx, s[v >> 4][v & 15]);
        return mx;
    };
    auto max_finish = [&](int sub, float mx, bool valid) {
        mx = max_halves(mx);
        const float cand = mx * c;
        const float m_new = valid && cand > m_run[sub] + kRescaleThreshold ? cand : m_run[sub];
        const float alpha = fast_exp2(m_run[sub] - m_new);
        const bool rescale = __builtin_amdgcn_ballot_w64(m_new != m_run[sub]) != 0;
        m_run[sub] = m_new;
        l_run[sub][0] *= alpha;
        l_run[sub][1] *= alpha;
        if (rescale) {
#pragma unroll
            for (int db = 0; db < DBLK; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[sub][db][r] *= alpha;
        }
    };

    // prologue: K(t0), V(t0) in buffer 0, K(t0+1) in buffer 1, S(t0), its max
    f32x16 sa[2][2], sb[2][2];
    const f32x16 zero = {};
    if (t1 > t0) {
        load_k(t0, P0{});
        load_v(t0, P0{});
        load_k(t0 + 1, P1{});
        tiles_ready();
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) {
                const s16x8 a = *reinterpret_cast<const s16x8 *>(k_lds0 + 32 * kb2 * KP + k_rd[ks]);
#pragma unroll
                for (int sub = 0; sub < 2; ++sub)
                    sa[sub][kb2] = T::mfma32(a, qreg[sub][ks], ks == 0 ? zero : sa[sub][kb2]);
            }
        mask_tail(t0, sa);
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) max_finish(sub, max_part(sa[sub], 0, 32, -INFINITY), true);
        __syncthreads();   // K buffer 0 is refilled at the start of the first iteration
    }

    // Exponential pairs of a tile, in the order they are needed by the PV
    // MFMAs (kc-major): item e -> sub (e >> 2) & 1, pair 4 (e >> 3) + (e & 3).
    // Pair pi of a sub-tile covers keys 2 (pi & 7), +1 of 32-key block pi >> 3.
    constexpr int NPAIR = 32;
    constexpr int NA = 20;   // pairs computed alongside the S MFMAs; the rest alongside PV
    constexpr int NS = 2 * KSTEPS * 2;    // S MFMAs per tile, both sub-tiles
    constexpr int NPV = 4 * DBLK * 2;     // PV MFMAs per tile
    constexpr int NLATE = 24;             // PV MFMAs carrying the late pairs

    auto step = [&](int t, auto par, auto npar, f32x16 (&cur)[2][2], f32x16 (&nxt)[2][2], auto masked) {
        load_k(t + 2, par);
        load_v(t + 1, npar);
        __builtin_amdgcn_sched_barrier(0);

        uint32_t pw[2][16];
        auto exp_items = [&](int eb, int ee) {
#pragma unroll
            for (int e = eb; e < ee; ++e) {
                const int sub = (e >> 2) & 1, pi = 4 * (e >> 3) + (e & 3);
                const int kb = pi >> 3, r = 2 * (pi & 7);
                const float p0 = fast_exp2(__builtin_fmaf(cur[sub][kb][r], c, -m_run[sub]));
                const float p1 = fast_exp2(__builtin_fmaf(cur[sub][kb][r + 1], c, -m_run[sub]));
                pw[sub][pi] = pack2<T>(p0, p1);
                // the empty asm keeps each sum in its slice
                l_run[sub][pi & 1] = T::sum2(pw[sub][pi], l_run[sub][pi & 1]);
                asm volatile("" : "+v"(l_run[sub][pi & 1]));
            }
        };

        // block 1: S(t+1) for both sub-tiles; MFMA i -> kb2 = i / 16,
        // ks = (i / 2) % 8, sub = i % 2; K operand read 2 reads (4 MFMAs) ahead
        const uint16_t *kt = kbuf(npar);
        auto kop = [&](int r) {   // read r = kb2 * 8 + ks
            return *reinterpret_cast<const s16x8 *>(kt + 32 * (r >> 3) * KP + k_rd[r & 7]);
        };
        constexpr int KD = 2;
        s16x8 kq[KD + 1];
#pragma unroll
        for (int r = 0; r < KD; ++r) kq[r] = kop(r);
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            const int r = i >> 1, sub = i & 1, kb2 = r >> 3, ks = r & 7;
            if (sub == 0 && r + KD < NS / 2) kq[(r + KD) % (KD + 1)] = kop(r + KD);
            nxt[sub][kb2] = T::mfma32(kq[r % (KD + 1)], qreg[sub][ks], ks == 0 ? zero : nxt[sub][kb2]);
            exp_items((NA * i) / NS, (NA * (i + 1)) / NS);
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (decltype(masked)::value) mask_tail(t + 1, nxt);

        // block 2: O += V P for tile t; MFMA j -> operand o = j / 2
        // (kc = o / 4, db = o % 4), sub = j % 2; V^T read 2 operands ahead
        const uint16_t *vt = vbuf(par);
        auto vop = [&](int o) {
            const uint16_t *base = vt + 16 * (o / DBLK) * VP + v_rd[o % DBLK];
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(base));
            const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(base + 8 * VP));
            return s16x8{lo[0], lo[1], lo[2], lo[3], hi4[0], hi4[1], hi4[2], hi4[3]};
        };
        constexpr int VD = 2;
        s16x8 vq[VD + 1];
#pragma unroll
        for (int o = 0; o < VD; ++o) vq[o] = vop(o);
        float mx[2] = {-INFINITY, -INFINITY};
#pragma unroll
        for (int j = 0; j < NPV; ++j) {
            const int o = j >> 1, sub = j & 1, kc = o / DBLK, db = o % DBLK;
            if (sub == 0 && o + VD < NPV / 2) vq[(o + VD) % (VD + 1)] = vop(o + VD);
            const uint4 w4 = {pw[sub][4 * kc], pw[sub][4 * kc + 1], pw[sub][4 * kc + 2], pw[sub][4 * kc + 3]};
            oacc[sub][db] = T::mfma32(vq[o % (VD + 1)], __builtin_bit_cast(s16x8, w4), oacc[sub][db]);
            if (j < NLATE)
                exp_items(NA + ((NPAIR - NA) * j) / NLATE, NA + ((NPAIR - NA) * (j + 1)) / NLATE);
            // row max of the next tile: sub-tile j % 2, values 2 (j / 2) .. +1
            mx[sub] = max_part(nxt[sub], 2 * (j >> 1), 2 * (j >> 1) + 2, mx[sub]);
            __builtin_amdgcn_sched_barrier(0);
        }
        max_finish(0, mx[0], t + 1 < t1);
        max_finish(1, mx[1], t + 1 < t1);
        tiles_ready();
    };
    using Unmasked = std::false_type;
    using Masked = std::true_type;
    int t = t0;
    for (; t + 3 < t1; t += 2) {
        step(t, P0{}, P1{}, sa, sb, Unmasked{});
        step(t + 1, P1{}, P0{}, sb, sa, Unmasked{});
    }
    if (t < t1) step(t, P0{}, P1{}, sa, sb, Masked{});
    if (t + 1 < t1) step(t + 1, P1{}, P0{}, sb, sa, Masked{});
    if (t + 2 < t1) step(t + 2, P0{}, P1{}, sa, sb, Masked{});

    // epilogue, per sub-tile
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
        const float lr = l_run[sub][0] + l_run[sub][1];
        const float l_tot = lr + swap_halves(lr);
        if (nparts > 1) {
            if (qrow[sub] < Sq) {
                const int64_t slot = static_cast<int64_t>(w - p.whole_work) * nparts + part;
                const int row = 64 * wave + 32 * sub + l32;
                float *o = p.ws_o + (slot * BM + row) * D;
#pragma unroll
                for (int db = 0; db < DBLK; ++db)
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4)
                        *reinterpret_cast<float4 *>(o + 32 * db + 8 * g4 + 4 * hi) =
                            make_float4(oacc[sub][db][4 * g4], oacc[sub][db][4 * g4 + 1],
                                        oacc[sub][db][4 * g4 + 2], oacc[sub][db][4 * g4 + 3]);
                if (hi == 0)
                    *reinterpret_cast<float2 *>(p.ws_ml + (slot * BM + row) * 2) = make_float2(m_run[sub], l_tot);
            }
            continue;
        }
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        if (qrow[sub] < Sq) {
            uint16_t *orow = p.out + (qa + qrow[sub]) * rs + head * D;
#pragma unroll
            for (int db = 0; db < DBLK; ++db)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    uint2 w2;
                    w2.x = pack2<T>(oacc[sub][db][4 * g4 + 0] * inv, oacc[sub][db][4 * g4 + 1] * inv);
                    w2.y = pack2<T>(oacc[sub][db][4 * g4 + 2] * inv, oacc[sub][db][4 * g4 + 3] * inv);
                    *reinterpret_cast<uint2 *>(orow + 32 * db + 8 * g4 + 4 * hi) = w2;
                }
        }
    }
}

}  // namespace attn
