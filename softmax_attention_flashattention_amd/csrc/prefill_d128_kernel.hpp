// prefill_d128_kernel.hpp -- non-causal varlen prefill attention at head_dim
// 128 for gfx950, with 64 query rows per wave.
//
// Same operator as prefill_kernel.hpp (atrex-bench "attention_forward" #001,
// Reference Implementation): per sequence and head, out = softmax(scale Q K^T) V,
// as a tiled online softmax with fp32 accumulation.
//
// Why 64 rows per wave.  Both products read one MFMA operand from LDS (a K
// tile or a V tile) and take the other from registers (Q^T or P^T).  With 32
// query rows per wave every 1 KiB operand read feeds one 32x32x16 MFMA, and
// the LDS read bandwidth of a compute unit (about 128 bytes per clock), shared
// by the 8 waves, caps the matrix cores well below their rate.  Here a wave
// owns two 32-row query blocks and every K and V^T operand it reads feeds two
// MFMAs, one per block.  A wave's registers then hold O^T for 64 rows (128
// VGPRs) and Q^T for the first block (32 VGPRs); the second block's Q^T is
// kept in LDS and read back as the B operand of its S MFMAs (one read per
// MFMA), which keeps two waves per SIMD.  Per MFMA the wave reads 0.75 KiB of
// operands from LDS instead of 1 KiB, and a workgroup of 4 waves (256 query
// rows) moves each K/V tile into LDS once for twice the rows.
//
// Tiles hold BN = 32 keys.  K and V rows are padded in LDS (136 and 160
// elements) so that every operand read is a fixed base plus an immediate
// offset and no two lanes of a read hit the same bank; the tiles go from
// global memory straight into LDS (buffer loads with the LDS destination
// bit), one 16-byte slot per lane, with the lanes on pad slots switched off.
//
// Products, transposed so a lane owns a query row (as in prefill_kernel.hpp):
//   S^T[key, q] = K Q^T      A = K rows from LDS, B = Q^T (registers / LDS)
//   O^T[d, q]  += V^T P^T    A = V^T by ds_read_b64_tr_b16, B = P^T (registers)
// The 32x32 accumulator gives lane l query l % 32 and 16 of the 32 keys (keys
// {0-3, 8-11, 16-19, 24-27} + 4 (l / 32)); lanes l and l ^ 32 share a query.
//
// Schedule of a step (K(t+1) and V(t) in LDS): the 16 S MFMAs of tile t+1,
// with the DMA of K(t+2) and V(t+1) spread among them; then the 16 PV MFMAs
// of tile t, with the row max of S(t+1) and then its exponentials (P(t+1),
// written in place over P(t) as the MFMAs release its words) riding along.
// The two waves of a SIMD belong to different workgroups, so one's VALU-heavy
// PV phase overlaps the other's MFMA-only S phase.  The running max is raised
// only when a row's new max passes it by more than 2^8 (the result is
// shift-invariant).  P(t+1) is computed with the current max; when a cheap
// per-lane test says some row's max may have risen that far (rarely after
// the first tile), a branch of plain VALU work rescales O and the row sums
// and redoes P(t+1) with the raised max.  Keeping the MFMAs out of that
// branch keeps each accumulator in one register tuple (a second copy of the
// PV MFMAs in a branch made the register allocator split them and spill).
//
// Softmax runs in the base-2 domain with c = |scale| log2(e); a negative
// scale negates Q as it is loaded.  Keys past the end of the sequence get
// weight 0 by selection.  The row sum accumulates the 16-bit P that
// multiplies V (v_dot2 against ones).
#pragma once

#include <type_traits>

#include "device_common.hpp"
#include "prefill_kernel.hpp"

namespace attn {

constexpr int kD128Waves = 4;
constexpr int kD128Threads = 64 * kD128Waves;
constexpr int kD128BM = 64 * kD128Waves;   // query rows per workgroup
constexpr int kD128BN = 32;                // keys per tile

template <typename T>
__global__ __launch_bounds__(kD128Threads) __attribute__((amdgpu_waves_per_eu(2)))
void prefill_fwd_d128_kernel(PrefillParams p)
{
    constexpr int D = 128, BM = kD128BM, BN = kD128BN, W = kD128Waves;
    constexpr int KP = 136, VP = 160;          // padded row pitch (elements)
    constexpr int KC = KP / 8, VC = VP / 8;    // 16-byte slots per padded row
    constexpr int NKI = (BN * KC + 63) / 64;   // DMA instructions per K tile (9)
    constexpr int NVI = (BN * VC + 63) / 64;   // ... per V tile (10)
    constexpr int DJK = (NKI + W - 1) / W, DJV = (NVI + W - 1) / W;

    __shared__ __attribute__((aligned(16))) uint16_t k_lds0[BN * KP];
    __shared__ __attribute__((aligned(16))) uint16_t k_lds1[BN * KP];
    __shared__ __attribute__((aligned(16))) uint16_t v_lds0[BN * VP];
    __shared__ __attribute__((aligned(16))) uint16_t v_lds1[BN * VP];
    // Q^T of each wave's second query block as MFMA B operands: [wave][ks][lane][8]
    __shared__ __attribute__((aligned(16))) uint16_t q_lds[W * 8 * 64 * 8];
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
    const int64_t rs = static_cast<int64_t>(p.num_heads) * D;   // token row stride (elements)
    const uint32_t row_bytes = static_cast<uint32_t>(rs * 2);
    const uint16_t *k_head = p.k + ka * rs + head * D;
    const uint16_t *v_head = p.v + ka * rs + head * D;
    const float c = p.scale_log2e;

    // ---- Q: block 0 (rows 64 wave + l32) in VGPRs, block 1 (rows 64 wave +
    // 32 + l32) in LDS; lane l holds elements 16 ks + 8 (l / 32) .. +7
    s16x8 qreg[8];
    const int qrow0 = q0 + 64 * wave + l32, qrow1 = qrow0 + 32;
    uint16_t *q1_lds = q_lds + (wave * 8 * 64 + lane) * 8;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        const int d0 = 16 * ks + 8 * hi;
        uint4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
        if (qrow0 < Sq) a = ld16(p.q + (qa + qrow0) * rs + head * D + d0);
        if (qrow1 < Sq) b = ld16(p.q + (qa + qrow1) * rs + head * D + d0);
        if (p.negate_q) {   // flip the sign bit of each 16-bit element
            a.x ^= 0x80008000u; a.y ^= 0x80008000u; a.z ^= 0x80008000u; a.w ^= 0x80008000u;
            b.x ^= 0x80008000u; b.y ^= 0x80008000u; b.z ^= 0x80008000u; b.w ^= 0x80008000u;
        }
        qreg[ks] = __builtin_bit_cast(s16x8, a);
        st16(q1_lds + ks * 64 * 8, b);
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
    const int g16 = lane >> 4;
    const int tr_row = 4 * (g16 >> 1) + ((lane & 15) >> 2);
    const int tr_col = 16 * (g16 & 1) + 4 * (lane & 3);
    const int v_rd = tr_row * VP + tr_col;               // + 16 kc VP + 32 db (+ 8 VP)
    auto kop = [&](const uint16_t *kt, int ks) __attribute__((always_inline)) {
        return *reinterpret_cast<const s16x8 *>(kt + k_rd + 16 * ks);
    };
    auto q1op = [&](int ks) __attribute__((always_inline)) { return *reinterpret_cast<const s16x8 *>(q1_lds + ks * 64 * 8); };
    auto vop = [&](const uint16_t *vt, int j) __attribute__((always_inline)) {   // j = 4 kc + db
        const uint16_t *base = vt + v_rd + 16 * (j >> 2) * VP + 32 * (j & 3);
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(base));
        const s16x4 h4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(base + 8 * VP));
        return s16x8{lo[0], lo[1], lo[2], lo[3], h4[0], h4[1], h4[2], h4[3]};
    };

    float m_run[2] = {-INFINITY, -INFINITY};   // running max of c s per query block (log2 domain)
    float m_lim[2] = {-INFINITY, -INFINITY};   // raw scores above this may need the max raised
    float l_run[2] = {0.f, 0.f};
    f32x16 oacc[2][4];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[qb][db][r] = 0.f;

    // S^T of one tile for both query blocks; each K operand feeds two MFMAs
    // (`slice(i)` runs after MFMA pair i)
    auto compute_s = [&](const uint16_t *kt, f32x16 (&s)[2], auto &&slice) __attribute__((always_inline)) {
        const f32x16 zero = {};
        s16x8 ka = kop(kt, 0), qa = q1op(0);
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const s16x8 a = ka, b1 = qa;
            if (ks + 1 < 8) {
                ka = kop(kt, ks + 1);
                qa = q1op(ks + 1);
            }
            s[0] = T::mfma32(a, qreg[ks], ks == 0 ? zero : s[0]);
            s[1] = T::mfma32(a, b1, ks == 0 ? zero : s[1]);
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
    // exponentials, 16-bit packing and row sums of pair pi (0..15: block
    // pi >> 3, values 2 (pi & 7), +1) of tile t
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
        const uint32_t w2 = pack2<T>(e0, e1);
        pw[qb][pi & 7] = w2;
        l_run[qb] = T::sum2(w2, l_run[qb]);
        asm volatile("" : "+v"(l_run[qb]));   // keeps each sum in its slice
    };
    // Raise the running max where some row passed it by more than the
    // threshold, rescaling O and l.  mx: this lane's max of raw scores of the
    // new tile per query block.  Called for the first tile and when the cheap
    // per-lane test fired somewhere in the wave.
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
            l_run[qb] *= alpha;
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[qb][db][r] *= alpha;
        }
    };
    auto lane_max = [&](const f32x16 (&s)[2], float (&mx)[2]) __attribute__((always_inline)) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            float a = s[qb][0];
#pragma unroll
            for (int r = 1; r < 16; ++r) a = fmaxf(a, s[qb][r]);
            mx[qb] = a;
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
    // O^T += V^T P^T for both query blocks, MFMAs j0 .. j1-1 (j = 4 kc + db);
    // each V^T operand (read two ahead) feeds two MFMAs; `slice(j)` after each
    auto pv = [&](const uint16_t *vt, const uint32_t (&pw)[2][8], int j0, int j1, auto &&slice) __attribute__((always_inline)) {
        s16x8 va = vop(vt, j0);
#pragma unroll
        for (int j = j0; j < j1; ++j) {
            const int kc = j >> 2, db = j & 3;
            const s16x8 a = va;
            if (j + 1 < j1) va = vop(vt, j + 1);
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                const uint4 w4 = {pw[qb][4 * kc], pw[qb][4 * kc + 1], pw[qb][4 * kc + 2], pw[qb][4 * kc + 3]};
                oacc[qb][db] = T::mfma32(a, __builtin_bit_cast(s16x8, w4), oacc[qb][db]);
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
        tiles_ready();
        f32x16 s[2];
        compute_s(k_lds0, s, [](int) {});
        mask_tail(t0, s);
        float mx[2];
        lane_max(s, mx);
        rescale(mx);   // the first tile always sets the running max
#pragma unroll
        for (int pi = 0; pi < 16; ++pi) exp_pair(s, pw, pi, t0, Masked{});
        __syncthreads();   // K buffer 0 is refilled during the first step
    }

    // ---- one step: S(t+1) (if has_next), then PV(t) with the softmax of
    // S(t+1) riding along.  K(t) and V(t) live in buffer par, K(t+1) in npar;
    // this step's DMA brings K(t+2) into par and V(t+1) into npar.
    // The four tile buffers of a step come in restrict-qualified: the buffer
    // parity is a run-time value, and without this the compiler cannot tell
    // the tiles being read from those the DMA is filling and waits for the
    // DMA before the first V^T read of every step.  (A loop of two steps with
    // compile-time buffers would do the same, but its register allocation
    // spills.)  Wave priority by phase: S phase 2, PV phase 1, rest 0 (the
    // two waves of a SIMD come from different workgroups and drift apart).
    auto step_bufs = [&](int t, const uint16_t *__restrict__ k_read, uint16_t *__restrict__ k_fill,
                         const uint16_t *__restrict__ v_read, uint16_t *__restrict__ v_fill, auto has_next,
                         auto masked) __attribute__((always_inline)) {
        constexpr bool NEXT = decltype(has_next)::value;
        f32x16 s[2];
        setprio(std::integral_constant<int, 2>{});
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
        setprio(std::integral_constant<int, 1>{});
        if constexpr (!NEXT) {
            pv(vt, pw, 0, 8, [](int) {});
            setprio(std::integral_constant<int, 0>{});
        } else {
            // PV(t) with the softmax of S(t+1) riding along: the row max over
            // the first two MFMA pairs, then the exponentials, at most three
            // pairs under each MFMA pair.  Pairs 0-3 and 8-11 of P(t+1) go in
            // place into the words of P(t) the first four MFMA pairs (keys
            // 0..15) have read; pairs 4-7 and 12-15 go to pn until the last
            // MFMAs have read their words.  (Exponentials left until after the
            // last MFMA cost 9%: this wave then has no MFMA to hide them.)
            float mx[2];
            uint32_t pn[2][4];
            auto into_pn = [&](int pi) __attribute__((always_inline)) {   // pi in 4-7 or 12-15
                uint32_t tmp[2][8];
                exp_pair(s, tmp, pi, t + 1, masked);
                pn[pi >> 3][(pi & 7) - 4] = tmp[pi >> 3][pi & 7];
            };
            bool raise = false;
            float l_keep0 = 0.f, l_keep1 = 0.f;
            pv(vt, pw, 0, 8, [&](int j) __attribute__((always_inline)) {
                switch (j) {
                case 0: lane_max1(s, mx, 0); break;
                case 1:
                    lane_max1(s, mx, 1);
                    raise = needs_rescale(mx);   // wave-uniform; rare after the first tile
                    l_keep0 = l_run[0];
                    l_keep1 = l_run[1];
                    break;
                case 2: into_pn(4); into_pn(12); break;
                case 3: into_pn(5); into_pn(13); break;
                default:   // j = 4..7: the words of keys 0..15 are free
                    exp_pair(s, pw, j - 4, t + 1, masked);
                    exp_pair(s, pw, j + 4, t + 1, masked);
                    into_pn(j < 6 ? j + 2 : j + 8);   // 6, 7, 14, 15
                    break;
                }
            });
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                for (int i = 0; i < 4; ++i) pw[qb][4 + i] = pn[qb][i];
            setprio(std::integral_constant<int, 0>{});
            if (raise) {
                // some row's max rose past the threshold: those exponentials
                // are discarded; rescale O and the row sums kept from before
                // them, and redo P(t+1) with the raised max
                l_run[0] = l_keep0;
                l_run[1] = l_keep1;
                rescale(mx);
#pragma unroll
                for (int pi = 0; pi < 16; ++pi) exp_pair(s, pw, pi, t + 1, masked);
            }
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
    // unnormalised partials of a key range)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const float l_tot = l_run[qb] + swap_halves(l_run[qb]);
        const int row = 64 * wave + 32 * qb + l32;
        const int qrow = q0 + row;
        if (qrow >= Sq) continue;
        if (nparts > 1) {
            const int64_t slot = static_cast<int64_t>(w - p.whole_work) * nparts + part;
            float *o = p.ws_o + (slot * BM + row) * D;
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int d = 32 * db + 8 * g4 + 4 * hi;
                    *reinterpret_cast<float4 *>(o + d) =
                        make_float4(oacc[qb][db][4 * g4], oacc[qb][db][4 * g4 + 1], oacc[qb][db][4 * g4 + 2],
                                    oacc[qb][db][4 * g4 + 3]);
                }
            if (hi == 0)
                *reinterpret_cast<float2 *>(p.ws_ml + (slot * BM + row) * 2) = make_float2(m_run[qb], l_tot);
        } else {
            const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
            uint16_t *orow = p.out + (qa + qrow) * rs + head * D;
#pragma unroll
            for (int db = 0; db < 4; ++db)
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
}

}  // namespace attn
