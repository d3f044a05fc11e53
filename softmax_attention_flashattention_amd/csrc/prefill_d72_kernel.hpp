// prefill_d72_kernel.hpp -- non-causal varlen prefill attention at head_dim
// 72 for gfx950, with 64 query rows per wave.
//
// Same operator as prefill_kernel.hpp (atrex-bench "attention_forward" #001,
// Reference Implementation): per sequence and head, out = softmax(scale Q K^T) V,
// as a tiled online softmax with fp32 accumulation.
//
// Why 64 rows per wave.  Every MFMA of both products takes one operand from
// LDS (a K tile or a V^T block) and the other from registers.  With 32 query
// rows per wave, each 1 KiB operand read feeds one MFMA; at this head_dim the
// reads of a compute unit's 8 waves ask for more than its LDS delivers per
// clock once the matrix cores run near their rate.  Here a wave owns two
// 32-row query blocks, and every K and V^T operand it reads feeds two MFMAs,
// one per block.  Both blocks' Q^T (five k-steps of 16, 72 padded to 80) fit
// in registers, so Q costs no LDS reads at all.
//
// Tiles hold BN = 32 keys.  K rows are padded in LDS to 88 elements (columns
// 72-79 zero: the fifth k-step), V rows to 96 (column 72 holds 1.0, 73-79
// zero); the padding spreads every operand read over distinct banks.  Tiles
// go from global memory straight into LDS (buffer loads with the LDS
// destination bit), one 16-byte slot per lane, lanes on pad slots off.
//
// Products, transposed so a lane owns a query row:
//   S^T[key, q] = K Q^T      A = K rows from LDS, B = Q^T (registers)
//   O^T[d, q]  += V^T P^T    A = V^T by ds_read_b64_tr_b16, B = P^T (registers)
// O^T of a query block is two 32-row blocks (dims 0-63) on 32x32x16 MFMAs and
// a 16-row tail (dims 64-79) on 16x16x32 MFMAs, one per 16 queries over the
// whole 32-key tile; tail row 8 (dim 72, the ones column of V) is the row sum
// of the 16-bit P that multiplied V.  The tail's B operand is P regrouped
// between 16-lane rows by v_permlane16_swap (see pv).
//
// Schedule of a step (K(t+1) and V(t) in LDS): the 10 S MFMAs of tile t+1
// with the DMA of K(t+2) and V(t+1) among them; the 12 PV MFMAs of tile t;
// then the softmax of S(t+1) as one block of VALU work: its row max, a
// raised running max where a cheap per-lane test says some row may have
// passed it by more than 2^8 (rarely after the first tile; O is rescaled
// then), and the exponentials, written over P(t) once the MFMAs have read
// it.  The two waves of a SIMD come from different workgroups, so one's
// VALU block runs beside the other's MFMAs: this order measured 0.8% faster
// than the exponentials spread under the PV MFMAs, and 4-5% faster than
// those pinned there (the head_dim-128 kernel, with more MFMAs per score,
// measured the other way round).
//
// Softmax runs in the base-2 domain with c = |scale| log2(e); a negative
// scale negates Q as it is loaded.  Keys past the end of the sequence get
// weight 0 by selection.
#pragma once

#include <type_traits>

#include "device_common.hpp"
#include "prefill_kernel.hpp"

namespace attn {

constexpr int kD72Waves = 4;
constexpr int kD72Threads = 64 * kD72Waves;
constexpr int kD72BM = 64 * kD72Waves;   // query rows per workgroup
constexpr int kD72BN = 32;               // keys per tile

template <typename T>
__global__ __launch_bounds__(kD72Threads) __attribute__((amdgpu_waves_per_eu(2)))
void prefill_fwd_d72_kernel(PrefillParams p)
{
    constexpr int D = 72, BM = kD72BM, BN = kD72BN, W = kD72Waves;
    constexpr int KP = 88, VP = 96;            // padded row pitch (elements)
    constexpr int KC = KP / 8, VC = VP / 8;    // 16-byte slots per padded row
    constexpr int NKI = (BN * KC + 63) / 64;   // DMA instructions per K tile (6, the last partly)
    constexpr int NVI = (BN * VC + 63) / 64;   // ... per V tile (6)
    constexpr int DJK = (NKI + W - 1) / W, DJV = (NVI + W - 1) / W;
    constexpr int KS = 5;                      // QK^T k-steps of 16 (72 padded to 80)

    __shared__ __attribute__((aligned(16))) uint16_t k_lds0[BN * KP];
    __shared__ __attribute__((aligned(16))) uint16_t k_lds1[BN * KP];
    __shared__ __attribute__((aligned(16))) uint16_t v_lds0[BN * VP];
    __shared__ __attribute__((aligned(16))) uint16_t v_lds1[BN * VP];
    // buffer `par` (0 or 1, wave-uniform) of the double-buffered tiles
    auto kbuf = [&](int par) __attribute__((always_inline)) { return par ? k_lds1 : k_lds0; };
    auto vbuf = [&](int par) __attribute__((always_inline)) { return par ? v_lds1 : v_lds0; };
    auto setprio = [&](auto prio) __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(decltype(prio)::value);
        __builtin_amdgcn_sched_barrier(0);
    };

    // Work id: whole items XCD-remapped, split items as key ranges (as in
    // prefill_fwd_kernel).
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

    int64_t qa = p.cu_q[seq], qb_ = p.cu_q[seq + 1];
    int64_t ka = p.cu_k[seq], kb_ = p.cu_k[seq + 1];
    qa = qa < 0 ? 0 : (qa > p.total_q ? p.total_q : qa);
    qb_ = qb_ < qa ? qa : (qb_ > p.total_q ? p.total_q : qb_);
    ka = ka < 0 ? 0 : (ka > p.total_k ? p.total_k : ka);
    kb_ = kb_ < ka ? ka : (kb_ > p.total_k ? p.total_k : kb_);
    const int Sq = static_cast<int>(qb_ - qa);
    const int Sk = static_cast<int>(kb_ - ka);
    const int q0 = qtile * BM;
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

    // constant pad columns of all four tile buffers (the DMA never writes
    // them): K cols 72..79 = 0, V col 72 = 1, V cols 73..79 = 0
    if (tid < BN) {
        const uint4 z = {0u, 0u, 0u, 0u};
        const uint4 one = {T::one_bits, 0u, 0u, 0u};
        st16(&k_lds0[tid * KP + 72], z);
        st16(&k_lds1[tid * KP + 72], z);
        st16(&v_lds0[tid * VP + 72], one);
        st16(&v_lds1[tid * VP + 72], one);
    }

    // ---- Q^T of both query blocks (rows 64 wave + 32 qb + l32) as MFMA B
    // operands: lane l holds elements 16 ks + 8 (l / 32) .. +7 (72..79: zero)
    s16x8 qreg[2][KS];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const int qrow = q0 + 64 * wave + 32 * qb + l32;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int d0 = 16 * ks + 8 * hi;
            uint4 v4 = {0u, 0u, 0u, 0u};
            if (qrow < Sq && d0 < D) v4 = ld16(p.q + (qa + qrow) * rs + head * D + d0);
            if (p.negate_q) {   // flip the sign bit of each 16-bit element
                v4.x ^= 0x80008000u; v4.y ^= 0x80008000u; v4.z ^= 0x80008000u; v4.w ^= 0x80008000u;
            }
            qreg[qb][ks] = __builtin_bit_cast(s16x8, v4);
        }
    }

    // ---- tile movement.  Buffer resources end at the sequence's last key
    // (zero extent past this workgroup's last tile): rows past the end read as
    // zeros, loads past the last tile fetch nothing.  Every lane's whole byte
    // offset goes in the VGPR offset, which the range check covers.
    const int ntiles = (Sk + BN - 1) / BN;
    const int t0 = static_cast<int>((static_cast<int64_t>(part) * ntiles) / nparts);
    const int t1 = static_cast<int>((static_cast<int64_t>(part + 1) * ntiles) / nparts);
    auto tile_bytes = [&](int t) __attribute__((always_inline)) -> uint32_t {
        const int rows = Sk - t * BN < BN ? Sk - t * BN : BN;
        return (rows > 0 && t < t1) ? static_cast<uint32_t>(rows - 1) * row_bytes + D * 2u : 0u;
    };
    // DMA instruction n of a tile fills the 64 slots 64 n .. 64 n + 63 (1 KiB
    // of LDS); slot s is chunk s % pitch-slots of row s / pitch-slots.  Wave w
    // issues n = W j + w.  Lanes on pad chunks or past the tile stay off.
    auto dma_k_to = [&](const __amdgpu_buffer_rsrc_t &r, uint16_t *buf, int j) __attribute__((always_inline)) {
        const int n = W * j + wave_s;
        const int sl = 64 * n + lane;
        if (n < NKI && sl % KC < D / 8 && sl < BN * KC)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                r, (lds_void *)(buf + 512 * n), 16,
                static_cast<uint32_t>(sl / KC) * row_bytes + 16u * static_cast<uint32_t>(sl % KC), 0, 0, 0);
    };
    auto dma_v_to = [&](const __amdgpu_buffer_rsrc_t &r, uint16_t *buf, int j) __attribute__((always_inline)) {
        const int n = W * j + wave_s;
        const int sl = 64 * n + lane;
        if (n < NVI && sl % VC < D / 8 && sl < BN * VC)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                r, (lds_void *)(buf + 512 * n), 16,
                static_cast<uint32_t>(sl / VC) * row_bytes + 16u * static_cast<uint32_t>(sl % VC), 0, 0, 0);
    };
    auto rsrc_k = [&](int t) __attribute__((always_inline)) { return make_rsrc(k_head + static_cast<int64_t>(t) * BN * rs, tile_bytes(t)); };
    auto rsrc_v = [&](int t) __attribute__((always_inline)) { return make_rsrc(v_head + static_cast<int64_t>(t) * BN * rs, tile_bytes(t)); };

    // ---- operand addressing (elements inside a tile buffer)
    const int k_rd = l32 * KP + 8 * hi;                  // + 16 ks
    const int tr_row = 4 * (g16 >> 1) + ((lane & 15) >> 2);
    const int tr_col = 16 * (g16 & 1) + 4 * (lane & 3);
    const int v_rd = tr_row * VP + tr_col;               // + 16 kc VP + 32 db (+ 8 VP)
    // The tail's A operand (16x16x32: dim 64 + l % 16, the 8 keys of 16-lane
    // row l / 16) by the same transposed reads over columns 64-79: row g takes
    // keys 16 (g % 2) + 4 (g / 2) .. +3 and the same +8, the keys its lanes
    // hold in the tail's B operand.
    const int v_rd_tail = (16 * (g16 & 1) + 4 * (g16 >> 1) + ((lane & 15) >> 2)) * VP + 64 + 4 * (lane & 3);
    auto kop = [&](const uint16_t *kt, int ks) __attribute__((always_inline)) {
        return *reinterpret_cast<const s16x8 *>(kt + k_rd + 16 * ks);
    };
    auto tr8 = [&](const uint16_t *base) __attribute__((always_inline)) {
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(base));
        const s16x4 h4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(base + 8 * VP));
        return s16x8{lo[0], lo[1], lo[2], lo[3], h4[0], h4[1], h4[2], h4[3]};
    };
    // V^T operand of PV slot j: 0-3 the 32-row blocks (kc = j / 2, db = j % 2), 4 the tail
    auto vop = [&](const uint16_t *vt, int j) __attribute__((always_inline)) {
        return j < 4 ? tr8(vt + v_rd + 16 * (j >> 1) * VP + 32 * (j & 1)) : tr8(vt + v_rd_tail);
    };

    float m_run[2] = {-INFINITY, -INFINITY};   // running max of c s per query block (log2 domain)
    float m_lim[2] = {-INFINITY, -INFINITY};   // raw scores above this may need the max raised
    f32x16 oacc[2][2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[qb][db][r] = 0.f;
    // O^T tails, dims 64-79: elements 8 qb + 4 h .. +3 hold the 16x16 block
    // of queries 16 h .. 16 h + 15 of query block qb (lane l: query 16 h +
    // l % 16, dims 64 + 4 (l / 16) .. +3)
    f32x16 otail;
#pragma unroll
    for (int r = 0; r < 16; ++r) otail[r] = 0.f;

    // S^T of one tile for both query blocks; each K operand feeds two MFMAs
    // (`slice(ks)` runs after MFMA pair ks)
    auto compute_s = [&](const uint16_t *kt, f32x16 (&s)[2], auto &&slice) __attribute__((always_inline)) {
        const f32x16 zero = {};
        s16x8 ka = kop(kt, 0), kb = kop(kt, 1);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const s16x8 a = ka;
            ka = kb;
            if (ks + 2 < KS) kb = kop(kt, ks + 2);
            s[0] = T::mfma32(a, qreg[0][ks], ks == 0 ? zero : s[0]);
            s[1] = T::mfma32(a, qreg[1][ks], ks == 0 ? zero : s[1]);
            slice(ks);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // keys past the end of the sequence (only in the last tile) get -inf
    auto mask_tail = [&](int t, f32x16 (&s)[2]) __attribute__((always_inline)) {
        const int kbase = t * BN;
        if (kbase + BN > Sk) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = kbase + 8 * (r >> 2) + 4 * hi + (r & 3);
                if (key >= Sk) {
                    s[0][r] = -INFINITY;
                    s[1][r] = -INFINITY;
                }
            }
        }
    };
    // exponentials and 16-bit packing of pair pi (0..15: block pi >> 3,
    // values 2 (pi & 7), +1) of tile t; the row sums come from the ones column
    auto exp_pair = [&](const f32x16 (&s)[2], uint32_t (&pw)[2][8], int pi, int t, auto masked) __attribute__((always_inline)) {
        const int qb = pi >> 3, r = 2 * (pi & 7);
        float e0 = fast_exp2(__builtin_fmaf(s[qb][r], c, -m_run[qb]));
        float e1 = fast_exp2(__builtin_fmaf(s[qb][r + 1], c, -m_run[qb]));
        if constexpr (decltype(masked)::value) {
            // keys past the end get weight 0 whatever the scale
            const int key = t * BN + 8 * (r >> 2) + 4 * hi + (r & 3);
            e0 = key < Sk ? e0 : 0.f;
            e1 = key + 1 < Sk ? e1 : 0.f;
        }
        pw[qb][pi & 7] = pack2<T>(e0, e1);
    };
    // Raise the running max where some row passed it by more than the
    // threshold, rescaling O.  mx: this lane's max of raw scores of the new
    // tile per query block.  Called for the first tile and when the cheap
    // per-lane test fired somewhere in the wave, before that tile's
    // exponentials.
    auto rescale = [&](const float (&mx)[2]) __attribute__((always_inline)) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const float cand = max_halves(mx[qb]) * c;
            const bool up = cand > m_run[qb] + kRescaleThreshold;
            const float m_new = up ? cand : m_run[qb];
            const float alpha = fast_exp2(m_run[qb] - m_new);   // 1 where m stays
            m_run[qb] = m_new;
            // (m + threshold) / c, lowered by a relative 2^-16 so that no score
            // the exact test would take fails the cheap one
            const float lim = (m_new + kRescaleThreshold) / c;
            m_lim[qb] = lim - fabsf(lim) * 0x1p-16f;
#pragma unroll
            for (int db = 0; db < 2; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[qb][db][r] *= alpha;
            // the tail's columns are queries l % 16 and 16 + l % 16
            const float a_lo = __shfl(alpha, lane & 15, 64), a_hi = __shfl(alpha, 16 + (lane & 15), 64);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                otail[8 * qb + r] *= a_lo;
                otail[8 * qb + 4 + r] *= a_hi;
            }
        }
    };
    auto lane_max1 = [&](const f32x16 (&s)[2], float (&mx)[2], int qb) __attribute__((always_inline)) {
        float a = s[qb][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) a = fmaxf(a, s[qb][r]);
        mx[qb] = a;
    };
    auto needs_rescale = [&](const float (&mx)[2]) __attribute__((always_inline)) {
        return __builtin_amdgcn_ballot_w64(mx[0] > m_lim[0] || mx[1] > m_lim[1]) != 0;
    };
    // O^T += V^T P^T for both query blocks, six slots j of two MFMAs each
    // sharing one V^T operand (read one slot ahead):
    //   j = 0..3: 32-row block db = j % 2, 16-key step kc = j / 2 (P words 4 kc .. +3)
    //   j = 4, 5: the tail for queries 16 (j - 4) .. +15 over all 32 keys.
    // Before slot 4 the P words are regrouped in place for the tail's B
    // operand by one v_permlane16_swap per word pair.  Lane rows 0 and 2 hold
    // queries 0-15 and rows 1 and 3 queries 16-31: words 0-3 (keys of step 0)
    // then hold, for queries 0-15, rows 0 and 2's own step-0 words and in rows
    // 1 and 3 the step-1 words of rows 0 and 2; words 4-7 hold, for queries
    // 16-31, rows 1 and 3's own step-1 words and in rows 0 and 2 the step-0
    // words of rows 1 and 3.  `slice(j)` runs after each slot.
    auto pv = [&](const uint16_t *vt, uint32_t (&pw)[2][8], auto &&slice) __attribute__((always_inline)) {
        s16x8 va = vop(vt, 0);
#pragma unroll
        for (int j = 0; j < 6; ++j) {
            if (j < 4) {
                const s16x8 a = va;
                va = vop(vt, j + 1);   // slot 3 reads the tail's operand, used by slots 4 and 5
                const int kc = j >> 1, db = j & 1;
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) {
                    const uint4 w4 = {pw[qb][4 * kc], pw[qb][4 * kc + 1], pw[qb][4 * kc + 2], pw[qb][4 * kc + 3]};
                    oacc[qb][db] = T::mfma32(a, __builtin_bit_cast(s16x8, w4), oacc[qb][db]);
                }
            } else {
                const int h = j - 4;
                if (h == 0) {
#pragma unroll
                    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const auto r = __builtin_amdgcn_permlane16_swap(pw[qb][i], pw[qb][4 + i], false, false);
                            pw[qb][i] = r[0];
                            pw[qb][4 + i] = r[1];
                        }
                }
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) {
                    const uint4 w4 = {pw[qb][4 * h], pw[qb][4 * h + 1], pw[qb][4 * h + 2], pw[qb][4 * h + 3]};
                    f32x4 c4 = {otail[8 * qb + 4 * h], otail[8 * qb + 4 * h + 1], otail[8 * qb + 4 * h + 2],
                                otail[8 * qb + 4 * h + 3]};
                    c4 = T::mfma16(va, __builtin_bit_cast(s16x8, w4), c4);
#pragma unroll
                    for (int r = 0; r < 4; ++r) otail[8 * qb + 4 * h + r] = c4[r];
                }
            }
            slice(j);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto tiles_ready = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
        __syncthreads();
    };

    uint32_t pw[2][8];
    using Unmasked = std::false_type;
    using Masked = std::true_type;
    // ---- prologue: K(t0), V(t0), K(t0+1) in, S(t0), its max and exponentials
    if (t1 > t0) {
        const __amdgpu_buffer_rsrc_t r0 = rsrc_k(t0), r1 = rsrc_k(t0 + 1), rv = rsrc_v(t0);
#pragma unroll
        for (int j = 0; j < DJK; ++j) dma_k_to(r0, k_lds0, j);
#pragma unroll
        for (int j = 0; j < DJV; ++j) dma_v_to(rv, v_lds0, j);
#pragma unroll
        for (int j = 0; j < DJK; ++j) dma_k_to(r1, k_lds1, j);
        tiles_ready();   // (also publishes the pad columns)
        f32x16 s[2];
        compute_s(k_lds0, s, [](int) {});
        mask_tail(t0, s);
        float mx[2];
        lane_max1(s, mx, 0);
        lane_max1(s, mx, 1);
        rescale(mx);   // the first tile always sets the running max
#pragma unroll
        for (int pi = 0; pi < 16; ++pi) exp_pair(s, pw, pi, t0, Masked{});
        __syncthreads();   // K buffer 0 is refilled during the first step
    }

    // ---- one step: S(t+1) (if has_next), PV(t), then the softmax of
    // S(t+1).  K(t) and V(t) live in buffer par, K(t+1) in npar; this step's
    // DMA brings K(t+2) into par and V(t+1) into npar.  The four tile buffers
    // come in restrict-qualified: the buffer parity is a run-time value, and
    // without this the compiler cannot tell the tiles being read from those
    // the DMA is filling and waits for the DMA before the first V^T read of
    // every step.  Wave priority by phase: PV 2, S 1, the softmax block 0
    // (the two waves of a SIMD come from different workgroups, so the MFMAs
    // of one issue ahead of the other's VALU work).
    auto step_bufs = [&](int t, const uint16_t *__restrict__ k_read, uint16_t *__restrict__ k_fill,
                         const uint16_t *__restrict__ v_read, uint16_t *__restrict__ v_fill, auto has_next,
                         auto masked) __attribute__((always_inline)) {
        constexpr bool NEXT = decltype(has_next)::value;
        f32x16 s[2];
        setprio(std::integral_constant<int, 1>{});
        if constexpr (NEXT) {
            const __amdgpu_buffer_rsrc_t rk = rsrc_k(t + 2), rv = rsrc_v(t + 1);
            // DMA instructions spread over the S MFMA pairs
            compute_s(k_read, s, [&](int ks) {
                if (ks < DJK) dma_k_to(rk, k_fill, ks);
                else if (ks - DJK < DJV) dma_v_to(rv, v_fill, ks - DJK);
            });
            if constexpr (decltype(masked)::value) mask_tail(t + 1, s);
        }
        const uint16_t *vt = v_read;
        setprio(std::integral_constant<int, 2>{});
        if constexpr (!NEXT) {
            pv(vt, pw, [](int) {});
            setprio(std::integral_constant<int, 0>{});
        } else {
            // PV(t), then the softmax of S(t+1): its row max, a raised max
            // where some row passed the threshold, and the exponentials,
            // written over P(t) now that the MFMAs have read it
            pv(vt, pw, [](int) {});
            setprio(std::integral_constant<int, 0>{});
            float mx[2];
            lane_max1(s, mx, 0);
            lane_max1(s, mx, 1);
            if (needs_rescale(mx)) rescale(mx);   // wave-uniform; rare after the first tile
#pragma unroll
            for (int pi = 0; pi < 16; ++pi) exp_pair(s, pw, pi, t + 1, masked);
        }
    };

    auto step = [&](int t, int par, auto has_next, auto masked) __attribute__((always_inline)) {
        step_bufs(t, kbuf(par ^ 1), kbuf(par), vbuf(par), vbuf(par ^ 1), has_next, masked);
    };

    // tiles t0 .. t1-1: S(t+1) is a full tile for t + 2 < t1; the step that
    // computes the last tile's S is peeled (masked), and so is the last PV
    int t = t0;
    for (; t + 2 < t1; ++t) {
        step(t, (t - t0) & 1, std::true_type{}, Unmasked{});
        tiles_ready();
    }
    if (t + 1 < t1) {
        step(t, (t - t0) & 1, std::true_type{}, Masked{});
        tiles_ready();
        ++t;
    }
    if (t < t1) step(t, (t - t0) & 1, std::false_type{}, Masked{});

    // ---- epilogue: normalise, round, store rows inside the segment (or the
    // unnormalised partials of a key range).  Cross-lane values first, with
    // every lane active.
    float l_tot[2], inv_t[2][2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        // the row sum: dim 72 = tail row 8, in lanes 32-47: element 8 qb for
        // query l % 16, element 8 qb + 4 for query 16 + l % 16
        const float l_lo = __shfl(otail[8 * qb], 32 + (l32 & 15), 64);
        const float l_hi = __shfl(otail[8 * qb + 4], 32 + (l32 & 15), 64);
        l_tot[qb] = l32 < 16 ? l_lo : l_hi;
        const float inv = l_tot[qb] > 0.f ? 1.f / l_tot[qb] : 0.f;
        inv_t[qb][0] = __shfl(inv, lane & 15, 64);
        inv_t[qb][1] = __shfl(inv, 16 + (lane & 15), 64);
    }
    const int64_t slot = static_cast<int64_t>(w - p.whole_work) * nparts + part;
    const int dt = 64 + 4 * (g16 & 1);   // the tail dims lanes 0-31 hold
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const int row = 64 * wave + 32 * qb + l32;
        const int qrow = q0 + row;
        if (qrow < Sq) {
            if (nparts > 1) {
                float *o = p.ws_o + (slot * BM + row) * D;
#pragma unroll
                for (int db = 0; db < 2; ++db)
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4) {
                        const int d = 32 * db + 8 * g4 + 4 * hi;
                        *reinterpret_cast<float4 *>(o + d) =
                            make_float4(oacc[qb][db][4 * g4], oacc[qb][db][4 * g4 + 1], oacc[qb][db][4 * g4 + 2],
                                        oacc[qb][db][4 * g4 + 3]);
                    }
                if (hi == 0)
                    *reinterpret_cast<float2 *>(p.ws_ml + (slot * BM + row) * 2) = make_float2(m_run[qb], l_tot[qb]);
            } else {
                const float inv = l_tot[qb] > 0.f ? 1.f / l_tot[qb] : 0.f;
                uint16_t *orow = p.out + (qa + qrow) * rs + head * D;
#pragma unroll
                for (int db = 0; db < 2; ++db)
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4) {
                        const int d = 32 * db + 8 * g4 + 4 * hi;
                        uint2 w2;
                        w2.x = pack2<T>(oacc[qb][db][4 * g4 + 0] * inv, oacc[qb][db][4 * g4 + 1] * inv);
                        w2.y = pack2<T>(oacc[qb][db][4 * g4 + 2] * inv, oacc[qb][db][4 * g4 + 3] * inv);
                        *reinterpret_cast<uint2 *>(orow + d) = w2;
                    }
            }
        }
        // dims 64-71 from the tail: lanes 0-31, 4 dims for each of queries
        // l % 16 and 16 + l % 16 of this block
        if (lane < 32) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int trow = 64 * wave + 32 * qb + 16 * h + (lane & 15);
                if (q0 + trow >= Sq) continue;
                if (nparts > 1) {
                    *reinterpret_cast<float4 *>(p.ws_o + (slot * BM + trow) * D + dt) =
                        make_float4(otail[8 * qb + 4 * h], otail[8 * qb + 4 * h + 1], otail[8 * qb + 4 * h + 2],
                                    otail[8 * qb + 4 * h + 3]);
                } else {
                    const float iv = inv_t[qb][h];
                    uint2 w2;
                    w2.x = pack2<T>(otail[8 * qb + 4 * h] * iv, otail[8 * qb + 4 * h + 1] * iv);
                    w2.y = pack2<T>(otail[8 * qb + 4 * h + 2] * iv, otail[8 * qb + 4 * h + 3] * iv);
                    *reinterpret_cast<uint2 *>(p.out + (qa + q0 + trow) * rs + head * D + dt) = w2;
                }
            }
        }
    }
}

}  // namespace attn
