// prefill_kernel.hpp -- non-causal varlen prefill attention for gfx950 at
// head_dim 72 with 32 query rows per wave, for the grids between those of
// the key-splitting workgroups (prefill_split_kernel.hpp, small grids) and
// those the 64-row kernel of prefill_d72_kernel.hpp runs faster (head_dim 128
// runs prefill_d128_kernel.hpp); also the parameter block and the key-range
// merge kernel that all prefill kernels share.
//
// Computes, per sequence and head, out = softmax(scale * Q K^T) V (the
// operator of the atrex-bench page "attention_forward" #001, Reference
// Implementation) as a tiled online softmax: the full score matrix is never
// formed.
//
// Work decomposition.  One workgroup of WAVES waves owns a tile of BM = 32
// WAVES query rows of one (sequence, head); each wave owns 32 of those rows.
// WAVES is 4 (BM 128), or 8 (BM 256) when the work items fill the device at
// least once: twice the rows then share each K/V tile in LDS, halving the
// tile DMA per flop, the costliest part at this head_dim.  The workgroup
// streams the sequence's keys and values in tiles of BN = 64 rows through
// double-buffered LDS.  The tiles go from global memory straight into LDS
// (buffer loads with the LDS destination bit) as padded rows whose pitch
// spreads the operand reads over the banks, with the DMA lanes that would
// land on pad chunks masked off.
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
// Softmax runs in the base-2 domain: with c = |scale| * log2(e), the running
// max m is kept for c*s and p = exp2(c*s - m), alpha = exp2(m_old - m_new).
// A negative scale is applied by negating Q as it is loaded (exact in 16
// bits), so c >= 0 and the max of the raw scores is the max of c*s.  Keys past
// the end of the sequence get weight 0 by selection, which holds for c = 0
// as well (where c * -inf would be NaN).
//
// The QK^T contraction is padded to 80 (five k-steps of 16; the K pad columns
// are zero).  O^T is two 32-row blocks (dims 0-63) on 32x32x16 MFMAs and a
// 16-row tail (dims 64-79) on 16x16x32 MFMAs; column 72 of the V tile holds
// 1.0, so tail row 8 (dim 72) accumulates the row sum of the 16-bit P that
// actually multiplied V (the padding does useful work instead of a VALU sum).
#pragma once

#include <type_traits>

#include "device_common.hpp"

namespace attn {

struct PrefillParams {
    const uint16_t *q, *k, *v;
    const int32_t *cu_q, *cu_k;
    uint16_t *out;
    int64_t total_q, total_k;
    int num_heads;
    int num_qtiles;   // ceil(max_seqlen_q / BM)
    int total_work;   // work items: num_seqs * num_heads * num_qtiles
    int whole_work;   // items [0, whole_work) run whole; a multiple of 8
    int split_parts;  // items [whole_work, total_work) run as this many key ranges
    float *ws_o;      // split items: [(item - whole_work) * split_parts + part][BM][D], unnormalised O
    float *ws_ml;     // split items: [... same slot ...][BM][2]: running max (log2 domain), row sum
    float scale_log2e;  // |scale| * log2(e)
    int negate_q;       // scale < 0: Q enters the products negated
};

template <int D> struct PrefillShape;
template <> struct PrefillShape<72> {
    static constexpr int KSTEPS = 5;    // 72 padded to 80
    static constexpr int DBLK = 2;      // 32-row O^T blocks (dims 0-63); dims 64-79 form a 16-row tail
    static constexpr int KPITCH = 88;   // 176 B: 16 lanes reading one column hit distinct banks
    static constexpr int VPITCH = 96;   // 192 B: rows 48 banks apart
    static constexpr int ONES_COL = 72;
};

constexpr int kPrefillBN = 64;
// Workgroup size: WAVES (4 or 8) waves of 32 query rows each (BM = 32 WAVES rows).
constexpr int prefill_bm(int waves) { return 32 * waves; }
constexpr int prefill_threads(int waves) { return 64 * waves; }

// Rescaling threshold (log2 units) of the lazy online softmax: the running
// max is raised, and O, l rescaled, only when some row's new max exceeds it by
// more than this; otherwise p = exp2(c s - m) may reach 2^8, harmless in fp32
// and in the 16-bit P operand (the result is shift-invariant).
constexpr float kRescaleThreshold = 8.0f;

typedef __attribute__((address_space(3))) void lds_void;

template <int D, typename T, int WAVES>
__global__ __launch_bounds__(prefill_threads(WAVES)) __attribute__((amdgpu_waves_per_eu(2)))
void prefill_fwd_kernel(PrefillParams p)
{
    constexpr int kPrefillThreads = prefill_threads(WAVES);
    using S = PrefillShape<D>;
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    constexpr int BM = prefill_bm(WAVES), BN = kPrefillBN;
    constexpr int KP = S::KPITCH, VP = S::VPITCH;
    constexpr int CH = D / 8;                      // 16-byte chunks per row

    // one array per buffer, so that the compiler can tell the buffers apart
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

    // Work id.  Hardware hands consecutive workgroups to the 8 XCDs in turn,
    // so for the whole items bid -> (bid % 8) * (whole_work / 8) + bid / 8
    // keeps runs of consecutive items (same head, neighbouring query tiles,
    // hence the same K/V stream) on one XCD and its L2.  The items left for
    // the last, partly filled wave of workgroups are split into key ranges
    // (`split_parts` workgroups each) so that they fill it.
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
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);   // the same value, in an SGPR
    const int l32 = lane & 31, hi = lane >> 5;
    const int64_t rs = static_cast<int64_t>(p.num_heads) * D;   // token row stride, elements
    const uint32_t row_bytes = static_cast<uint32_t>(rs * 2);
    const uint16_t *k_head = p.k + ka * rs + head * D;
    const uint16_t *v_head = p.v + ka * rs + head * D;
    const float c = p.scale_log2e;

    {
        // constant pad columns of both buffers: K cols 72..79 = 0,
        // V col 72 = 1, V cols 73..95 = 0
        static_assert(S::ONES_COL == 72 && KP >= 80 && VP >= 96, "pad columns");
        const uint4 z = {0u, 0u, 0u, 0u};
        const uint4 one = {T::one_bits, 0u, 0u, 0u};
        for (int r = tid; r < BN; r += kPrefillThreads) {
            st16(&k_lds0[r * KP + 72], z);
            st16(&k_lds1[r * KP + 72], z);
            st16(&v_lds0[r * VP + 72], one);
            st16(&v_lds0[r * VP + 80], z);
            st16(&v_lds0[r * VP + 88], z);
            st16(&v_lds1[r * VP + 72], one);
            st16(&v_lds1[r * VP + 80], z);
            st16(&v_lds1[r * VP + 88], z);
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
        if (p.negate_q) {   // flip the sign bit of each 16-bit element
            v4.x ^= 0x80008000u;
            v4.y ^= 0x80008000u;
            v4.z ^= 0x80008000u;
            v4.w ^= 0x80008000u;
        }
        qreg[ks] = __builtin_bit_cast(s16x8, v4);
    }

    // ---- tile movement.  Each tile gets its own buffer resource whose extent
    // ends at the sequence's last key (zero past the last tile), so rows past
    // the end read as zeros and loads past the last tile fetch nothing.
    // this workgroup's key tiles [t0, t1)
    const int ntiles = (Sk + BN - 1) / BN;
    const int t0 = static_cast<int>((static_cast<int64_t>(part) * ntiles) / nparts);
    const int t1 = static_cast<int>((static_cast<int64_t>(part + 1) * ntiles) / nparts);
    auto tile_bytes = [&](int t) -> uint32_t {
        const int rows = Sk - t * BN < BN ? Sk - t * BN : BN;
        return (rows > 0 && t < t1) ? static_cast<uint32_t>(rows - 1) * row_bytes + D * 2u : 0u;
    };

    // Direct path.  A DMA instruction fills 1 KiB of LDS (lane i -> bytes
    // 16 i .. 16 i + 15), each lane from its own global address.  The padded
    // tile (KP or VP elements a row) is BN KP / 512 instructions; instruction
    // n = WAVES j + w covers the 16-byte slots 64 n .. 64 n + 63 of the tile,
    // slot s being chunk s % (pitch / 8) of row s / (pitch / 8); lanes on the
    // pad chunks (>= 9) are masked off, so the constant pad columns set up
    // above stay as they are.
    constexpr int NKI = BN * KP / 512, NVI = BN * VP / 512;   // DMA instructions per tile
    constexpr int DJK = (NKI + WAVES - 1) / WAVES;            // ... per wave (at most)
    constexpr int DJV = (NVI + WAVES - 1) / WAVES;
    // The whole byte offset of every lane goes in the VGPR offset: the
    // buffer range check covers that offset only (not the scalar one), so
    // this is what turns rows past the sequence's last key into zeros.
    uint32_t dk_off[4] = {0u, 0u, 0u, 0u};
    uint32_t dv_off[4] = {0u, 0u, 0u, 0u};
    bool dk_act[4] = {false, false, false, false}, dv_act[4] = {false, false, false, false};
    {
        constexpr int KC = KP / 8, VC = VP / 8;   // 16-byte slots per padded row
        static_assert(DJK <= 4 && DJV <= 4, "offset arrays");
#pragma unroll
        for (int j = 0; j < DJK; ++j) {
            const int s = 64 * (WAVES * j + wave) + lane;
            dk_off[j] = static_cast<uint32_t>(s / KC) * row_bytes + 16u * static_cast<uint32_t>(s % KC);
            dk_act[j] = s % KC < CH;
        }
#pragma unroll
        for (int j = 0; j < DJV; ++j) {
            const int s = 64 * (WAVES * j + wave) + lane;
            dv_off[j] = static_cast<uint32_t>(s / VC) * row_bytes + 16u * static_cast<uint32_t>(s % VC);
            dv_act[j] = s % VC < CH;
        }
    }

    // one DMA instruction (number j of this wave) of a K or V tile
    auto dma_k = [&](const __amdgpu_buffer_rsrc_t &r, auto par, int j) {
        const int n = WAVES * j + wave_s;
        if (n < NKI && dk_act[j])
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(kbuf(par) + 512 * n), 16, dk_off[j], 0, 0, 0);
    };
    auto dma_v = [&](const __amdgpu_buffer_rsrc_t &r, auto par, int j) {
        const int n = WAVES * j + wave_s;
        if (n < NVI && dv_act[j])
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(vbuf(par) + 512 * n), 16, dv_off[j], 0, 0, 0);
    };
    auto load_k = [&](int t, auto par) {
        const __amdgpu_buffer_rsrc_t r = make_rsrc(k_head + static_cast<int64_t>(t) * BN * rs, tile_bytes(t));
#pragma unroll
        for (int j = 0; j < DJK; ++j) dma_k(r, par, j);
    };
    auto load_v = [&](int t, auto par) {
        const __amdgpu_buffer_rsrc_t r = make_rsrc(v_head + static_cast<int64_t>(t) * BN * rs, tile_bytes(t));
#pragma unroll
        for (int j = 0; j < DJV; ++j) dma_v(r, par, j);
    };
    // all tile data of this iteration in LDS and visible to every wave
    auto tiles_ready = [&]() {
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
        __syncthreads();
    };

    // ---- operand addressing (element offsets inside a tile buffer)
    // K rows for S^T: row 32 kb2 + l32, chunk 2 ks + hi
    int k_rd[S::KSTEPS];
#pragma unroll
    for (int ks = 0; ks < S::KSTEPS; ++ks) k_rd[ks] = l32 * KP + 16 * ks + 8 * hi;
    // V^T by transposed reads: row 16 kc + tr_row (+8), column 32 db + tr_col
    const int g16 = lane >> 4;
    const int tr_row = 4 * (g16 >> 1) + ((lane & 15) >> 2);
    const int tr_col = 16 * (g16 & 1) + 4 * (lane & 3);
    int v_rd[S::DBLK];
#pragma unroll
    for (int db = 0; db < S::DBLK; ++db) v_rd[db] = tr_row * VP + 32 * db + tr_col;
    // The tail's A operand (16x16x32: dim 64 + l % 16, keys of group l / 16
    // of a 32-key chunk) by the same transposed reads over columns 64-79:
    // group g takes keys 16 (g % 2) + 4 (g / 2) .. +3 and the same +8, the
    // keys its lanes hold in the tail's B operand (the regrouped P in pv).
    const int v_rd_tail = (16 * (g16 & 1) + 4 * (g16 >> 1) + ((lane & 15) >> 2)) * VP + 64 + 4 * (lane & 3);

    // S^T = K Q^T for the two 32-key blocks of a tile
    auto compute_s = [&](auto par, f32x16 (&sacc)[2]) {
        const f32x16 zero = {};
        const uint16_t *kt = kbuf(par);
#pragma unroll
        for (int ks = 0; ks < S::KSTEPS; ++ks)
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2) {
                const s16x8 a = *reinterpret_cast<const s16x8 *>(kt + 32 * kb2 * KP + k_rd[ks]);
                sacc[kb2] = T::mfma32(a, qreg[ks], ks == 0 ? zero : sacc[kb2]);
            }
    };
    // keys past the end of the sequence (only in the last tile) get -inf
    auto mask_tail = [&](int t, f32x16 (&sacc)[2]) {
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
    };

    float m_run = -INFINITY;   // running max of c*s for this lane's query (log2 domain)
    float m_lim = -INFINITY;   // raw scores above this may need the running max raised
    f32x16 oacc[S::DBLK];
#pragma unroll
    for (int db = 0; db < S::DBLK; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
    // O^T tail, dims 64-79: elements 4 h .. 4 h + 3 of otail hold the 16x16
    // block of queries 16 h .. 16 h + 15 (lane l: query 16 h + l % 16, dims
    // 64 + 4 (l / 16) .. +3); elements 8-15 are unused (two separate 4-wide
    // accumulators made the register allocator copy every accumulator between
    // the loop's two step bodies)
    f32x16 otail;
#pragma unroll
    for (int r = 0; r < 16; ++r) otail[r] = 0.f;

    // O^T += V^T P^T over the tile's two 32-key chunks m.  Per chunk: the
    // 32-row blocks take 16-key steps kc = 2m, 2m + 1 (P words 4 kc .. +3 as
    // their B operand); the tail takes the whole chunk in one 16x16x32 MFMA
    // per 16 queries (half the MFMA work of a third 32-row block).  The
    // tail's B operand (P^T of 16 queries, 8 keys in each 16-lane row) is
    // the same P regrouped by one v_permlane16_swap per word pair.  Lane rows
    // 0 and 2 hold queries 0-15 and rows 1 and 3 queries 16-31; for queries
    // 0-15, rows 0 and 2 keep their step-2m words and rows 1 and 3 take the
    // step-(2m+1) words of rows 0 and 2; for queries 16-31, rows 1 and 3 keep
    // their step-(2m+1) words and rows 0 and 2 take the step-2m words of rows
    // 1 and 3.  Order per chunk (consecutive MFMAs independent): big(2m, 0),
    // big(2m, 1), big(2m+1, 0), big(2m+1, 1), tail(queries 0-15),
    // tail(queries 16-31); the swap goes in place once the chunk's big MFMAs
    // have read its words.  Between the MFMAs runs `slice(j)`, a piece of
    // VALU work (the row max of the next tile).
    auto pv = [&](auto par, const uint32_t (&pw)[16], auto &&slice) {
        constexpr int NPV = 12;   // MFMA slots j: 6 per chunk
        constexpr int NOP = 10;   // V^T operands o: per chunk 4 big (o % 5 < 4) and the tail's
        constexpr int PD = 3;     // operands read this many ahead
        const uint16_t *vt = vbuf(par);
        auto vop = [&](int o) {
            const int m = o / 5, oo = o % 5;
            const uint16_t *base = oo < 4 ? vt + 16 * (2 * m + oo / 2) * VP + v_rd[oo % 2]
                                          : vt + 32 * m * VP + v_rd_tail;
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(base));
            const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(base + 8 * VP));
            return s16x8{lo[0], lo[1], lo[2], lo[3], hi4[0], hi4[1], hi4[2], hi4[3]};
        };
        // the operand of slot j (slots 4 and 5 of a chunk share the tail's)
        auto op_of = [](int j) { return 5 * (j / 6) + (j % 6 < 4 ? j % 6 : 4); };
        s16x8 a[PD + 1];
#pragma unroll
        for (int o = 0; o < PD; ++o) a[o] = vop(o);
        uint32_t tb[2][4];
#pragma unroll
        for (int j = 0; j < NPV; ++j) {
            const int m = j / 6, jj = j % 6;
            // read ahead up to operand op_of(j) + PD (the ring slot it takes
            // was last used PD + 1 operands back)
            const int o_lo = j == 0 ? PD : op_of(j - 1) + PD + 1;
            const int o_hi = op_of(j) + PD + 1 < NOP ? op_of(j) + PD + 1 : NOP;
#pragma unroll
            for (int o = o_lo; o < o_hi; ++o) a[o % (PD + 1)] = vop(o);
            const s16x8 &av = a[op_of(j) % (PD + 1)];
            if (jj >= 4) {
                const int h = jj - 4;
                if (!h) {
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        const auto r = __builtin_amdgcn_permlane16_swap(pw[8 * m + w], pw[8 * m + 4 + w], false, false);
                        tb[0][w] = r[0];
                        tb[1][w] = r[1];
                    }
                }
                const uint4 w4 = {tb[h][0], tb[h][1], tb[h][2], tb[h][3]};
                f32x4 c4 = {otail[4 * h], otail[4 * h + 1], otail[4 * h + 2], otail[4 * h + 3]};
                c4 = T::mfma16(av, __builtin_bit_cast(s16x8, w4), c4);
#pragma unroll
                for (int r = 0; r < 4; ++r) otail[4 * h + r] = c4[r];
            } else {
                const int kc = 2 * m + jj / 2, db = jj % 2;
                const uint4 w4 = {pw[4 * kc], pw[4 * kc + 1], pw[4 * kc + 2], pw[4 * kc + 3]};
                oacc[db] = T::mfma32(av, __builtin_bit_cast(s16x8, w4), oacc[db]);
            }
            slice(j);
        }
    };

    // Row max of a masked S^T tile, taken before the tile's exponentials: the
    // running max moves only past the threshold (and only when `valid`), and
    // then O and l are rescaled (a wave-uniform branch that is rarely taken
    // after the first tile).
    auto max_part = [&](const f32x16 (&sacc)[2], int j, int nparts, float mx) {
        // values j * 32 / nparts .. (j + 1) * 32 / nparts - 1 of this lane
#pragma unroll
        for (int v = (32 * j) / nparts; v < (32 * (j + 1)) / nparts; ++v)
            mx = fmaxf(mx, sacc[v >> 4][v & 15]);
        return mx;
    };
    auto max_finish = [&](float mx, bool valid) {
        // a cheap, conservative test of this lane's half row against the
        // raw-score limit first; the exact test below decides
        if (valid && __builtin_amdgcn_ballot_w64(mx > m_lim) != 0) {   // wave-uniform; rare after the first tile
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
            for (int db = 0; db < S::DBLK; ++db)
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

    // Software pipeline: iteration t computes S for tile t+1 (MFMA) while it
    // runs the exponentials of tile t (VALU), then O += V_t P_t, then the row
    // max of tile t+1.  K runs one tile ahead of V in the LDS double buffers;
    // tile t+2 of K and t+1 of V are in flight from global memory during the
    // iteration.  Past the last tile the buffer resources have zero extent, so
    // those loads fetch nothing and return zeros; the extra S block of the
    // last iteration is discarded.
    f32x16 sa[2], sb[2];
    constexpr int KD = 3;   // K operands read this many MFMAs ahead
    s16x8 kq_pre[KD];       // the first KD K operands of a step, read before it starts
    auto kop_at = [&](const uint16_t *kt, int i) {
        return *reinterpret_cast<const s16x8 *>(kt + 32 * (i & 1) * KP + k_rd[i >> 1]);
    };
    if (t1 > t0) {
        load_k(t0, P0{});
        load_v(t0, P0{});
        load_k(t0 + 1, P1{});
        tiles_ready();
        compute_s(P0{}, sa);
        mask_tail(t0, sa);
        max_finish(max_part(sa, 0, 1, -INFINITY), true);
        __syncthreads();   // K buffer 0 is refilled at the start of the first iteration
#pragma unroll
        for (int i = 0; i < KD; ++i) kq_pre[i] = kop_at(k_lds1, i);
    }

    constexpr int NS = 2 * S::KSTEPS;   // S MFMAs per tile (two 32-key blocks)
    // par = (t - t0) % 2: K(t) and V(t) live in buffer par, K(t+1) in buffer 1 - par
    // masked: whether S(t+1) may be the partial last tile (a branch; kept out
    // of the main loop so that the exponentials are not moved past it)
    auto step = [&](int t, auto par, auto npar, const f32x16 (&cur)[2], f32x16 (&nxt)[2], auto masked) {
        // K(t+2) goes to the buffer K(t) left, V(t+1) to the one V(t-1) left.
        // Direct DMA: the instructions spread over the S MFMAs (issued in
        // one burst they stall the wave at issue).
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(k_head + static_cast<int64_t>(t + 2) * BN * rs, tile_bytes(t + 2));
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(v_head + static_cast<int64_t>(t + 1) * BN * rs, tile_bytes(t + 1));
        // DMA instruction n of this wave's DJK + DJV goes after S MFMA
        // floor(n NS / (DJK + DJV))
        auto dma_slot = [&](int mfma) {
            constexpr int ND = DJK + DJV;
#pragma unroll
            for (int n = 0; n < ND; ++n) {
                if ((n * NS) / ND == mfma) {
                    if (n < DJK) dma_k(rk, par, n); else dma_v(rv, npar, n - DJK);
                }
            }
        };
        __builtin_amdgcn_sched_barrier(0);
        // Wave priority by phase: the two workgroups sharing a SIMD drift
        // apart, so one wave is often in its S phase (MFMAs plus most of the
        // exponentials) while the other is in its PV phase or at the barrier.
        // Issuing the S phase first, then PV, then the rest measured 1-2%
        // faster than equal priorities.
        __builtin_amdgcn_s_setprio(2);
        __builtin_amdgcn_sched_barrier(0);

        // The NS MFMAs of S(t+1) = K(t+1) Q^T, in the order ks outer, kb2
        // inner (two independent accumulator chains), each K operand read KD
        // MFMAs ahead.  Between consecutive MFMAs sits a slice of the softmax
        // of tile t: exponentials and 16-bit packing of its 16 value pairs
        // (the row sums come from the ones column of V).
        const uint16_t *kt = kbuf(npar);
        auto kop = [&](int i) { return kop_at(kt, i); };
        s16x8 kq[KD + 1];
#pragma unroll
        for (int i = 0; i < KD; ++i) kq[i] = kq_pre[i];   // read during the previous step
        const f32x16 zero = {};
        uint32_t pw[16];
        // exponentials and 16-bit packing of value pairs [pb, pe)
        // of tile t (pair pi = keys 2 (pi & 7), +1 of 32-key block pi >> 3)
        auto exp_pairs = [&](int pb, int pe) {
#pragma unroll
            for (int pi = pb; pi < pe; ++pi) {
                const int kb = pi >> 3, r = 2 * (pi & 7);
                float p0 = fast_exp2(__builtin_fmaf(cur[kb][r], c, -m_run));
                float p1 = fast_exp2(__builtin_fmaf(cur[kb][r + 1], c, -m_run));
                if constexpr (decltype(masked)::value) {
                    // tile t may be the partial last one (peeled steps only):
                    // keys past the end get weight 0 whatever the scale
                    if (t * BN + BN > Sk) {
                        const int key = t * BN + 32 * kb + 8 * (r >> 2) + 4 * hi + (r & 3);
                        p0 = key < Sk ? p0 : 0.f;
                        p1 = key + 1 < Sk ? p1 : 0.f;
                    }
                }
                pw[pi] = pack2<T>(p0, p1);
            }
        };
        // The VALU work of a tile is spread over all its MFMAs: pairs
        // 0 .. NA-1 ride along the NS S MFMAs, the last 16 - NA along the
        // first PV MFMAs (before the MFMAs that use them), and the row max of
        // the next tile along all PV MFMAs.
        constexpr int NA = 10;  // one pair per S MFMA: 0.6% faster than 8 and 6 (interleaved A/B)
        constexpr int NPV = 12;   // PV MFMA slots
        constexpr int NB = 6;     // PV MFMAs carrying the late pairs (chunk 1 starts at slot 6)
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            const int ks = i >> 1, kb2 = i & 1;
            if (i + KD < NS) kq[(i + KD) % (KD + 1)] = kop(i + KD);
            nxt[kb2] = T::mfma32(kq[i % (KD + 1)], qreg[ks], ks == 0 ? zero : nxt[kb2]);
            dma_slot(i);
            exp_pairs((NA * i) / NS, (NA * (i + 1)) / NS);
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (decltype(masked)::value) mask_tail(t + 1, nxt);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(1);
        __builtin_amdgcn_sched_barrier(0);
        float mx = -INFINITY;
        // The end-of-step barrier sits before the last BAR_AT PV MFMAs: by
        // then every V(t) operand read has been issued (PD ahead), so once
        // they have landed and this wave's tile DMA is complete, all waves
        // may hand the buffers over.  The first KD operands of K(t+2), which
        // the next step starts with, are then read while those MFMAs run.
        constexpr int BAR_AT = 3;
        // (pv issues its last V^T read, operand 9, at slot 6)
        static_assert(NPV - BAR_AT >= 6, "the barrier must follow the last V^T operand read");
        pv(par, pw, [&](int j) {
            if (j < NB) exp_pairs(NA + ((16 - NA) * j) / NB, NA + ((16 - NA) * (j + 1)) / NB);
            mx = max_part(nxt, j, NPV, mx);
            __builtin_amdgcn_sched_barrier(0);
            if (j == NPV - BAR_AT) {
                __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
                __syncthreads();
                __builtin_amdgcn_sched_barrier(0);
                const uint16_t *kn = kbuf(par);    // K(t+2), complete and visible now
#pragma unroll
                for (int i = 0; i < KD; ++i) kq_pre[i] = kop_at(kn, i);
                __builtin_amdgcn_sched_barrier(0);
            }
        });
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);
        max_finish(mx, t + 1 < t1);
    };
    using Unmasked = std::false_type;
    using Masked = std::true_type;
    int t = t0;
    for (; t + 3 < t1; t += 2) {                // S(t+1), S(t+2) are full tiles
        step(t, P0{}, P1{}, sa, sb, Unmasked{});
        step(t + 1, P1{}, P0{}, sb, sa, Unmasked{});
    }
    if (t < t1) step(t, P0{}, P1{}, sa, sb, Masked{});
    if (t + 1 < t1) step(t + 1, P1{}, P0{}, sb, sa, Masked{});
    if (t + 2 < t1) step(t + 2, P0{}, P1{}, sa, sb, Masked{});

    // ---- epilogue: normalise, round to 16 bits, store rows inside the segment
    // the row sum: dim 72 = tail row 8, in lanes 32-47: otail element 0 for
    // query l % 16, element 4 for query 16 + l % 16
    const float l_lo = __shfl(otail[0], 32 + (l32 & 15), 64);
    const float l_hi = __shfl(otail[4], 32 + (l32 & 15), 64);
    const float l_tot = l32 < 16 ? l_lo : l_hi;
    // dims 64-71 of the tail: lanes 0-31, 4 dims (64 + 4 (l / 16)) for each of
    // queries c0 = l % 16 and c1 = 16 + l % 16 of this wave
    const int c0 = lane & 15, c1 = 16 + (lane & 15), dt = 64 + 4 * (g16 & 1);
    if (nparts > 1) {
        // a key range of a split item: unnormalised O^T, running max and row
        // sum to the workspace; prefill_merge_kernel combines the ranges
        if (qrow < Sq) {
            const int64_t slot = static_cast<int64_t>(w - p.whole_work) * nparts + part;
            const int row = 32 * wave + l32;
            float *o = p.ws_o + (slot * BM + row) * D;
#pragma unroll
            for (int db = 0; db < S::DBLK; ++db)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int d = 32 * db + 8 * g4 + 4 * hi;
                    if (d < D)
                        *reinterpret_cast<float4 *>(o + d) =
                            make_float4(oacc[db][4 * g4], oacc[db][4 * g4 + 1], oacc[db][4 * g4 + 2],
                                        oacc[db][4 * g4 + 3]);
                }
            if (hi == 0) *reinterpret_cast<float2 *>(p.ws_ml + (slot * BM + row) * 2) = make_float2(m_run, l_tot);
        }
        if (lane < 32) {
            const int64_t slot = static_cast<int64_t>(w - p.whole_work) * nparts + part;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int row = 32 * wave + (h ? c1 : c0);
                if (q0 + row < Sq)
                    *reinterpret_cast<float4 *>(p.ws_o + (slot * BM + row) * D + dt) =
                        make_float4(otail[4 * h], otail[4 * h + 1], otail[4 * h + 2], otail[4 * h + 3]);
            }
        }
        return;
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
    const float inv0 = __shfl(inv, c0, 64), inv1 = __shfl(inv, c1, 64);
    if (lane < 32) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int q = q0 + 32 * wave + (h ? c1 : c0);
            const float iv = h ? inv1 : inv0;
            if (q < Sq) {
                uint2 w2;
                w2.x = pack2<T>(otail[4 * h] * iv, otail[4 * h + 1] * iv);
                w2.y = pack2<T>(otail[4 * h + 2] * iv, otail[4 * h + 3] * iv);
                *reinterpret_cast<uint2 *>(p.out + (qa + q) * rs + head * D + dt) = w2;
            }
        }
    }
}

// Log-sum-exp merge of the key ranges of the split work items.  Each thread
// owns four consecutive output values of one row of one item and walks the
// item's ranges; consecutive threads own consecutive values, so every
// partial-row load is contiguous across the wave.  kMergeBlocks<D, BM>
// workgroups of kMergeThreads per item.
constexpr int kMergeThreads = 256;
template <int D, int BM> constexpr int merge_blocks() { return (BM * (D / 4) + kMergeThreads - 1) / kMergeThreads; }

template <int D, int BM, typename T>
__global__ __launch_bounds__(kMergeThreads) void prefill_merge_kernel(PrefillParams p)
{
    constexpr int C4 = D / 4;   // float4 columns per row
    constexpr int NB = merge_blocks<D, BM>();
    const int item = blockIdx.x / NB;
    const int e = (blockIdx.x % NB) * kMergeThreads + threadIdx.x;
    if (e >= BM * C4) return;
    const int row = e / C4, c4 = e % C4;
    const int w = p.whole_work + item;
    if (w >= p.total_work) return;
    const int qtile = w % p.num_qtiles;
    const int sh = w / p.num_qtiles;
    const int head = sh % p.num_heads;
    const int seq = sh / p.num_heads;
    int64_t qa = p.cu_q[seq], qb = p.cu_q[seq + 1];
    qa = qa < 0 ? 0 : (qa > p.total_q ? p.total_q : qa);
    qb = qb < qa ? qa : (qb > p.total_q ? p.total_q : qb);
    const int Sq = static_cast<int>(qb - qa);
    const int q = qtile * BM + row;
    if (q >= Sq) return;
    const int P = p.split_parts;
    const int64_t slot0 = static_cast<int64_t>(item) * P;

    float M = -INFINITY;
    for (int i = 0; i < P; ++i) M = fmaxf(M, p.ws_ml[((slot0 + i) * BM + row) * 2]);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float den = 0.f;
    for (int i = 0; i < P; ++i) {
        const float2 ml = *reinterpret_cast<const float2 *>(p.ws_ml + ((slot0 + i) * BM + row) * 2);
        const float wi = (M == -INFINITY || ml.x == -INFINITY) ? 0.f : fast_exp2(ml.x - M);
        den += wi * ml.y;
        const float4 v = *reinterpret_cast<const float4 *>(p.ws_o + ((slot0 + i) * BM + row) * D + 4 * c4);
        acc.x += wi * v.x;
        acc.y += wi * v.y;
        acc.z += wi * v.z;
        acc.w += wi * v.w;
    }
    const float inv = den > 0.f ? 1.f / den : 0.f;
    const int64_t rs = static_cast<int64_t>(p.num_heads) * D;
    uint16_t *orow = p.out + (qa + q) * rs + head * D + 4 * c4;
    *reinterpret_cast<uint2 *>(orow) = make_uint2(pack2<T>(acc.x * inv, acc.y * inv), pack2<T>(acc.z * inv, acc.w * inv));
}

}  // namespace attn
