// prefill_split_kernel.hpp -- non-causal varlen prefill attention at head_dim
// 72 for gfx950 on grids of few work items: the waves of a workgroup share 32
// query rows and split the keys among themselves.
//
// Same operator as prefill_kernel.hpp (atrex-bench "attention_forward" #001,
// Reference Implementation): per sequence and head, out = softmax(scale Q K^T) V.
//
// Why a third layout.  The other head_dim-72 kernels give each wave its own
// query rows and walk every key tile of the sequence in turn, a chain of
// roughly a microsecond per tile.  With few work items (short sequences, few
// heads) most compute units idle and the launch lasts as long as one chain.
// Here a workgroup of W waves owns 32 query rows of one (sequence, head); wave
// w walks the w-th of W contiguous ranges of the key tiles with its own online
// softmax, and the W partial results (running max, row sum, unnormalised O)
// are combined by log-sum-exp in LDS at the end of the same launch: the chain
// is W times shorter, and there is no second launch and no workspace.
//
// No tile is shared between waves, so nothing goes through a workgroup-wide
// buffer.  K goes from global memory straight into the registers that are the
// A operand of S^T = K Q^T (lane l: key l % 32, dims 16 ks + 8 (l / 32) ..
// +7).  V goes into registers and from there into the wave's own
// double-buffered LDS tile, from which the transposing reads give V^T.  Both
// are loaded two tiles ahead, through buffer resources that end at the
// sequence's last key (zero extent past the wave's range), so rows past the
// end read as zeros and loads past the range fetch nothing.  A wave's LDS
// accesses execute in program order, so the loop needs no barrier.
//
// The products, the padding (QK^T 72 -> 80 with zero K columns; O^T as two
// 32-row blocks plus a 16-row tail on 16x16x32 MFMAs whose dim 72 is a ones
// column of V, accumulating the row sum of the 16-bit P), the base-2 online
// softmax with its lazy rescale, and the key masking are those of
// prefill_kernel.hpp, with 32-key tiles (one 32x32 S^T block per tile).
#pragma once

#include <type_traits>

#include "device_common.hpp"
#include "prefill_kernel.hpp"

namespace attn {

constexpr int kSplitBQ = 32;     // query rows per workgroup
constexpr int kSplitBN = 32;     // keys per tile
constexpr int kSplitWaves = 4;   // key ranges per workgroup (8 measured slower on every grid tried)
constexpr int split_threads(int waves) { return 64 * waves; }

template <typename T, int W>
__global__ __launch_bounds__(split_threads(W)) __attribute__((amdgpu_waves_per_eu(2)))
void prefill_fwd_split_kernel(PrefillParams p)
{
    constexpr int D = 72, BQ = kSplitBQ, BN = kSplitBN;
    constexpr int KSTEPS = 5;                   // QK^T contraction 72 padded to 80
    constexpr int VP = 96;                      // V tile row pitch (elements)
    constexpr int VT = BN * VP;                 // elements of one V tile
    constexpr int CH = D / 8;                   // 16-byte chunks of a row (9)
    constexpr int NVL = (BN * CH + 63) / 64;    // V loads per lane and tile (5; the last in lanes 0-31)
    constexpr int MP = 76;                      // merge row: 72 dims, the row sum, 16-byte aligned
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;

    // V tiles [buffer][wave][BN][VP]; after the loop the same memory holds
    // the partial results for the merge
    __shared__ __attribute__((aligned(16))) uint16_t v_lds[2 * W * VT];
    static_assert(W * BQ * (MP + 1) * 4 <= 2 * W * VT * 2, "the merge area overlays the V tiles");

    // Work id: one item = 32 query rows of one (sequence, head); runs of
    // consecutive items (the same head's K/V) stay on one XCD, as in the other
    // prefill kernels.
    const int bid = blockIdx.x;
    const int w = bid < p.whole_work ? (bid & 7) * (p.whole_work >> 3) + (bid >> 3) : bid;
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
    const int q0 = qtile * BQ;
    if (q0 >= Sq) return;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    const int l32 = lane & 31, hi = lane >> 5;
    const int g16 = lane >> 4;
    const int64_t rs = static_cast<int64_t>(p.num_heads) * D;   // token row stride (elements)
    const uint32_t row_bytes = static_cast<uint32_t>(rs * 2);
    const uint16_t *k_head = p.k + ka * rs + head * D;
    const uint16_t *v_head = p.v + ka * rs + head * D;
    const float c = p.scale_log2e;

    // this wave's two V tile buffers; pad columns 72..79 set once: 1.0 in
    // column 72 (the row sum), zeros after it (columns 80..95 are never read)
    uint16_t *vb0 = v_lds + (0 * W + wave_s) * VT;
    uint16_t *vb1 = v_lds + (1 * W + wave_s) * VT;
    if (lane < BN) {
        const uint4 one = {T::one_bits, 0u, 0u, 0u};
        st16(vb0 + lane * VP + 72, one);
        st16(vb1 + lane * VP + 72, one);
    }

    // Q^T as the B operand of S^T = K Q^T: lane l holds query row q0 + l % 32,
    // elements 16 ks + 8 (l / 32) .. +7 (zeros past 72 and past the segment)
    s16x8 qreg[KSTEPS];
    const int qrow = q0 + l32;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
        const int d0 = 16 * ks + 8 * hi;
        uint4 v4 = {0u, 0u, 0u, 0u};
        if (qrow < Sq && d0 < D) v4 = ld16(p.q + (qa + qrow) * rs + head * D + d0);
        if (p.negate_q) {   // flip the sign bit of each 16-bit element
            v4.x ^= 0x80008000u;
            v4.y ^= 0x80008000u;
            v4.z ^= 0x80008000u;
            v4.w ^= 0x80008000u;
        }
        qreg[ks] = __builtin_bit_cast(s16x8, v4);
    }

    // ---- this wave's key tiles [ta, tb), n of them
    const int ntiles = (Sk + BN - 1) / BN;
    const int ta = (wave_s * ntiles) / W, tb = ((wave_s + 1) * ntiles) / W;
    const int n = tb - ta;
    // Nothing in a step branches on the lane or on the tile: a branch would
    // split the step into blocks, and the compiler would then sink the
    // softmax work past it, away from the MFMAs it is meant to overlap.
    // Buffer resource of tile t: its rows up to the sequence's last key
    // (tiles t < tb hold at least one), zero extent from tb on.
    auto tile_rsrc = [&](const uint16_t *head_base, int t) __attribute__((always_inline)) {
        int rows = Sk - t * BN;
        rows = rows < BN ? rows : BN;
        rows = rows > 1 ? rows : 1;
        // (the clamp becomes a vector instruction; keep the extent scalar)
        rows = __builtin_amdgcn_readfirstlane(rows);
        const uint32_t valid = static_cast<uint32_t>(t < tb);
        const uint32_t bytes = valid * (static_cast<uint32_t>(rows - 1) * row_bytes + D * 2u);
        return make_rsrc(head_base + static_cast<int64_t>(t) * BN * rs, bytes);
    };
    // K tile t as the five A operands of S^T.  The fifth holds dims 64-71 in
    // lanes 0-31; lanes 32-63 (dims 72-79) read at an offset past any extent
    // (tiles are under 2^31 bytes), which returns zeros and touches nothing.
    const uint32_t k_off = static_cast<uint32_t>(l32) * row_bytes + 16u * static_cast<uint32_t>(hi);
    const uint32_t k_off4 = hi ? 0x80000000u : k_off + 128u;
    auto load_k = [&](int t, s16x8 (&kr)[KSTEPS]) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t r = tile_rsrc(k_head, t);
#pragma unroll
        for (int ks = 0; ks < KSTEPS - 1; ++ks) kr[ks] = __builtin_bit_cast(s16x8, buf_ld16(r, k_off + 32u * ks));
        kr[KSTEPS - 1] = __builtin_bit_cast(s16x8, buf_ld16(r, k_off4));
    };
    // V tile t: 16-byte chunk s = lane + 64 i is chunk s % 9 of row s / 9.
    // The chunks past the tile (s >= 288: lanes 32-63 of load 4) lie past the
    // resource's extent and read as zeros; they are stored into column 80 of
    // rows 0-31, which no operand read touches.
    uint32_t v_goff[NVL];
    int v_soff[NVL];
#pragma unroll
    for (int i = 0; i < NVL; ++i) {
        const int s = lane + 64 * i;
        v_goff[i] = static_cast<uint32_t>(s / CH) * row_bytes + 16u * static_cast<uint32_t>(s % CH);
        v_soff[i] = s < BN * CH ? (s / CH) * VP + 8 * (s % CH) : (s - BN * CH) * VP + 80;
    }
    static_assert(BN * CH + BN >= 64 * NVL && VP >= 88, "the spare chunks land in column 80 of the tile");
    auto load_v = [&](int t, uint4 (&vr)[NVL]) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t r = tile_rsrc(v_head, t);
#pragma unroll
        for (int i = 0; i < NVL; ++i) vr[i] = buf_ld16(r, v_goff[i]);
    };
    auto store_v = [&](uint16_t *vt, const uint4 (&vr)[NVL]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < NVL; ++i) st16(vt + v_soff[i], vr[i]);
    };

    // ---- V^T operands by transposed LDS reads (as in prefill_kernel.hpp):
    // o = 2 kc + db (o < 4) covers keys 16 kc .. +15, dims 32 db .. +31; o = 4
    // is the tail's operand (dims 64-79 over all 32 keys)
    const int tr_row = 4 * (g16 >> 1) + ((lane & 15) >> 2);
    const int tr_col = 16 * (g16 & 1) + 4 * (lane & 3);
    const int v_rd = tr_row * VP + tr_col;
    const int v_rd_tail = (16 * (g16 & 1) + 4 * (g16 >> 1) + ((lane & 15) >> 2)) * VP + 64 + 4 * (lane & 3);
    auto vop = [&](const uint16_t *vt, int o) __attribute__((always_inline)) {
        const uint16_t *base = o < 4 ? vt + 16 * (o >> 1) * VP + 32 * (o & 1) + v_rd : vt + v_rd_tail;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(base));
        const s16x4 h4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(base + 8 * VP));
        return s16x8{lo[0], lo[1], lo[2], lo[3], h4[0], h4[1], h4[2], h4[3]};
    };

    float m_run = -INFINITY;   // running max of c s for this lane's query (log2 domain)
    float m_lim = -INFINITY;   // raw scores above this may need the running max raised
    f32x16 oacc[2];
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
    // O^T tail, dims 64-79: elements 4 h .. 4 h + 3 hold queries 16 h + l % 16,
    // dims 64 + 4 (l / 16) .. +3 (elements 8-15 unused)
    f32x16 otail;
#pragma unroll
    for (int r = 0; r < 16; ++r) otail[r] = 0.f;

    // S^T of one tile: five dependent MFMAs; `slice(ks)` after each
    auto compute_s = [&](const s16x8 (&kr)[KSTEPS], f32x16 &s, auto &&slice) __attribute__((always_inline)) {
        const f32x16 zero = {};
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            s = T::mfma32(kr[ks], qreg[ks], ks == 0 ? zero : s);
            slice(ks);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // keys past the end of the sequence (only in the last tile) get -inf
    auto mask_tail = [&](int t, f32x16 &s) __attribute__((always_inline)) {
        const int kbase = t * BN;
        if (kbase + BN > Sk) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = kbase + 8 * (r >> 2) + 4 * hi + (r & 3);
                if (key >= Sk) s[r] = -INFINITY;
            }
        }
    };
    // exponentials and 16-bit packing of value pairs [pb, pe) of tile t
    // (pair pi = values 2 pi, 2 pi + 1: word pi of P^T)
    auto exp_pairs = [&](const f32x16 &s, uint32_t (&pw)[8], int pb, int pe, int t, auto masked)
        __attribute__((always_inline)) {
#pragma unroll
        for (int pi = pb; pi < pe; ++pi) {
            const int r = 2 * pi;
            float p0 = fast_exp2(__builtin_fmaf(s[r], c, -m_run));
            float p1 = fast_exp2(__builtin_fmaf(s[r + 1], c, -m_run));
            if constexpr (decltype(masked)::value) {
                // keys past the end get weight 0 whatever the scale
                if (t * BN + BN > Sk) {
                    const int key = t * BN + 8 * (r >> 2) + 4 * hi + (r & 3);
                    p0 = key < Sk ? p0 : 0.f;
                    p1 = key + 1 < Sk ? p1 : 0.f;
                }
            }
            pw[pi] = pack2<T>(p0, p1);
        }
    };
    // The running max moves only past the threshold, and then O and the row
    // sums (tail dim 72) are rescaled: a wave-uniform branch, rarely taken
    // after the first tile.
    auto max_finish = [&](float mx) __attribute__((always_inline)) {
        if (__builtin_amdgcn_ballot_w64(mx > m_lim) != 0) {
            mx = max_halves(mx);
            const float cand = mx * c;
            const bool up = cand > m_run + kRescaleThreshold;
            const float m_new = up ? cand : m_run;
            const float alpha = fast_exp2(m_run - m_new);   // 1 in the lanes that keep m
            m_run = m_new;
            // (m_run + threshold) / c, lowered by a relative 2^-16 so that no
            // score the exact test would take fails the cheap one
            const float lim = (m_run + kRescaleThreshold) / c;
            m_lim = lim - fabsf(lim) * 0x1p-16f;
#pragma unroll
            for (int db = 0; db < 2; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
            // the tail's columns are queries l % 16 and 16 + l % 16
            const float a_lo = __shfl(alpha, lane & 15, 64), a_hi = __shfl(alpha, 16 + (lane & 15), 64);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                otail[r] *= a_lo;
                otail[4 + r] *= a_hi;
            }
        }
    };
    // O^T += V^T P^T for one tile: slots 0-3 the 32-row blocks (kc = j / 2,
    // db = j % 2, P words 4 kc .. +3), slots 4-5 the tail for queries 0-15 and
    // 16-31 (B = P regrouped between 16-lane rows, as in prefill_kernel.hpp);
    // `slice(j)` after each
    auto pv = [&](const uint16_t *vt, const uint32_t (&pw)[8], auto &&slice) __attribute__((always_inline)) {
        // operands read two slots ahead: 0 and 1 first, operand j + 2 before slot j
        s16x8 ops[5];
        ops[0] = vop(vt, 0);
        ops[1] = vop(vt, 1);
        uint32_t tb2[2][4];
#pragma unroll
        for (int j = 0; j < 6; ++j) {
            if (j < 3) ops[j + 2] = vop(vt, j + 2);
            if (j < 4) {
                const int kc = j >> 1, db = j & 1;
                const uint4 w4 = {pw[4 * kc], pw[4 * kc + 1], pw[4 * kc + 2], pw[4 * kc + 3]};
                oacc[db] = T::mfma32(ops[j], __builtin_bit_cast(s16x8, w4), oacc[db]);
            } else {
                const int h = j - 4;
                if (!h) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const auto r = __builtin_amdgcn_permlane16_swap(pw[q], pw[4 + q], false, false);
                        tb2[0][q] = r[0];
                        tb2[1][q] = r[1];
                    }
                }
                const uint4 w4 = {tb2[h][0], tb2[h][1], tb2[h][2], tb2[h][3]};
                f32x4 c4 = {otail[4 * h], otail[4 * h + 1], otail[4 * h + 2], otail[4 * h + 3]};
                c4 = T::mfma16(ops[4], __builtin_bit_cast(s16x8, w4), c4);
#pragma unroll
                for (int r = 0; r < 4; ++r) otail[4 * h + r] = c4[r];
            }
            slice(j);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // ---- the loop.  Before step i (tile t = ta + i): S(i) in `cur` (masked,
    // its max folded in), V(i) in LDS buffer i % 2, K(i+1) in kr[(i+1) % 2]
    // and K(i+2) in kr[i % 2] (loading), V(i+1) in vr[(i+1) % 2] and V(i+2)
    // in vr[i % 2] (loading).  Step i: S(i+1) with the exponentials of S(i)
    // between its MFMAs, then the loads of K(i+3) into the registers just
    // read; PV(i) with the row max of S(i+1) between its MFMAs; V(i+1) into
    // LDS buffer (i+1) % 2 (last read by PV(i-1)) and the loads of V(i+3) into
    // its registers.
    s16x8 kr[2][KSTEPS];
    uint4 vr[2][NVL];
    f32x16 sa, sb;
    auto step = [&](int i, auto par, f32x16 &cur, f32x16 &nxt, auto has_next, auto masked)
        __attribute__((always_inline)) {
        constexpr int PA = decltype(par)::value;
        constexpr bool NEXT = decltype(has_next)::value;
        const int t = ta + i;
        uint32_t pw[8];
        if constexpr (NEXT) {
            compute_s(kr[1 - PA], nxt, [&](int ks) __attribute__((always_inline)) {
                exp_pairs(cur, pw, (8 * ks) / KSTEPS, (8 * (ks + 1)) / KSTEPS, t, masked);
            });
            load_k(t + 3, kr[1 - PA]);
            if constexpr (decltype(masked)::value) mask_tail(t + 1, nxt);
        } else {
            exp_pairs(cur, pw, 0, 8, t, masked);
        }
        float mx = -INFINITY;
        pv(PA ? vb1 : vb0, pw, [&](int j) __attribute__((always_inline)) {
            if constexpr (NEXT) {
#pragma unroll
                for (int r = (16 * j) / 6; r < (16 * (j + 1)) / 6; ++r) mx = fmaxf(mx, nxt[r]);
            }
        });
        if constexpr (NEXT) {
            store_v(PA ? vb0 : vb1, vr[1 - PA]);
            load_v(t + 3, vr[1 - PA]);
            max_finish(mx);
        }
    };
    using Unmasked = std::false_type;
    using Masked = std::true_type;
    using Next = std::true_type;
    using Last = std::false_type;
    if (n > 0) {
        load_k(ta, kr[0]);
        load_v(ta, vr[0]);
        load_k(ta + 1, kr[1]);
        load_v(ta + 1, vr[1]);
        compute_s(kr[0], sa, [](int) {});
        load_k(ta + 2, kr[0]);
        store_v(vb0, vr[0]);
        load_v(ta + 2, vr[0]);
        mask_tail(ta, sa);
        float mx = sa[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sa[r]);
        max_finish(mx);   // the first tile always sets the running max
    }
    int i = 0;
    for (; i + 3 < n; i += 2) {   // S(i+1), S(i+2) and the exponentials of S(i), S(i+1): full tiles
        step(i, P0{}, sa, sb, Next{}, Unmasked{});
        step(i + 1, P1{}, sb, sa, Next{}, Unmasked{});
    }
    if (i + 2 < n) {
        step(i, P0{}, sa, sb, Next{}, Masked{});
        step(i + 1, P1{}, sb, sa, Next{}, Masked{});
        step(i + 2, P0{}, sa, sb, Last{}, Masked{});
    } else if (i + 1 < n) {
        step(i, P0{}, sa, sb, Next{}, Masked{});
        step(i + 1, P1{}, sb, sa, Last{}, Masked{});
    } else if (i < n) {
        step(i, P0{}, sa, sb, Last{}, Masked{});
    }

    // ---- merge of the W key ranges by log-sum-exp.  Each wave leaves its
    // running max and its unnormalised O and row sum (rows [wave][query][MP],
    // fp32) in LDS over the V tiles; a wave whose range was empty leaves max
    // -inf and zeros, and weighs nothing.
    __syncthreads();   // every wave is done with its V tiles
    float *mo = reinterpret_cast<float *>(v_lds);
    float *mm = mo + W * BQ * MP;
    {
        float *mine = mo + wave_s * BQ * MP;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4)
                *reinterpret_cast<float4 *>(mine + l32 * MP + 32 * db + 8 * g4 + 4 * hi) =
                    make_float4(oacc[db][4 * g4], oacc[db][4 * g4 + 1], oacc[db][4 * g4 + 2], oacc[db][4 * g4 + 3]);
        const int c0 = lane & 15, c1 = 16 + (lane & 15);
        if (lane < 32) {   // dims 64 + 4 (l / 16) .. +3
            const int dt = 64 + 4 * g16;
            *reinterpret_cast<float4 *>(mine + c0 * MP + dt) = make_float4(otail[0], otail[1], otail[2], otail[3]);
            *reinterpret_cast<float4 *>(mine + c1 * MP + dt) = make_float4(otail[4], otail[5], otail[6], otail[7]);
            mm[wave_s * BQ + lane] = m_run;
        } else if (lane < 48) {   // dim 72: the row sum
            mine[c0 * MP + 72] = otail[0];
            mine[c1 * MP + 72] = otail[4];
        }
    }
    __syncthreads();
    // item e: query row e / 9, dims 8 (e % 9) .. +7
    for (int e = tid; e < BQ * CH; e += split_threads(W)) {
        const int q = e / CH, ch = e % CH;
        if (q0 + q >= Sq) continue;
        float M = -INFINITY;
#pragma unroll
        for (int wv = 0; wv < W; ++wv) M = fmaxf(M, mm[wv * BQ + q]);
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        float den = 0.f;
#pragma unroll
        for (int wv = 0; wv < W; ++wv) {
            const float mw = mm[wv * BQ + q];
            const float a = mw == -INFINITY ? 0.f : fast_exp2(mw - M);
            const float *row = mo + (wv * BQ + q) * MP;
            den += a * row[72];
            const float4 x0 = *reinterpret_cast<const float4 *>(row + 8 * ch);
            const float4 x1 = *reinterpret_cast<const float4 *>(row + 8 * ch + 4);
            acc[0] += a * x0.x;
            acc[1] += a * x0.y;
            acc[2] += a * x0.z;
            acc[3] += a * x0.w;
            acc[4] += a * x1.x;
            acc[5] += a * x1.y;
            acc[6] += a * x1.z;
            acc[7] += a * x1.w;
        }
        const float inv = den > 0.f ? 1.f / den : 0.f;
        const uint4 o = {pack2<T>(acc[0] * inv, acc[1] * inv), pack2<T>(acc[2] * inv, acc[3] * inv),
                         pack2<T>(acc[4] * inv, acc[5] * inv), pack2<T>(acc[6] * inv, acc[7] * inv)};
        st16(p.out + (qa + q0 + q) * rs + head * D + 8 * ch, o);
    }
}

}  // namespace attn
