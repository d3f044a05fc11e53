// attn_api.hip -- the C ABI of libattn (declared in include/attn.h):
// host-side argument validation, kernel selection and launch.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "attn.h"
#include "chunk_kernel.hpp"
#include "decode_kernel.hpp"
#include "decode_mfma_kernel.hpp"
#include "prefill_d128_kernel.hpp"
#include "prefill_d72_kernel.hpp"
#include "prefill_kernel.hpp"
#include "prefill_split_kernel.hpp"

// Device-side scratch of attn_paged_decode_noalloc: the per-partition
// (max, sum) pairs and partial outputs of a split context, laid out as the
// caller workspace of attn_paged_decode.  Every GPU the library runs on holds
// its own copy until the process ends.  In host code `scratch` names a host
// stand-in, not device memory: its device address comes from
// hipGetSymbolAddress, looked up once per device (scratch_address below).
static __device__ __align__(256) unsigned char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kDefaultPartitionTokens = 512;
constexpr int kMinAutoPartitionTokens = 128;

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int launch_status() { return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP; }

template <int D, typename T, int W>
int launch_prefill(const attn::PrefillParams &p, int64_t grid, hipStream_t stream)
{
    constexpr int BM = attn::prefill_bm(W);
    hipLaunchKernelGGL((attn::prefill_fwd_kernel<D, T, W>), dim3(static_cast<unsigned>(grid)),
                       dim3(attn::prefill_threads(W)), 0, stream, p);
    int rc = launch_status();
    if (rc != ATTN_OK || p.split_parts == 1 || p.total_work == p.whole_work) return rc;
    hipLaunchKernelGGL((attn::prefill_merge_kernel<D, BM, T>),
                       dim3(static_cast<unsigned>((p.total_work - p.whole_work) * attn::merge_blocks<D, BM>())),
                       dim3(attn::kMergeThreads), 0, stream, p);
    return launch_status();
}

template <typename T>
int launch_prefill_d72(const attn::PrefillParams &p, int64_t grid, hipStream_t stream)
{
    hipLaunchKernelGGL((attn::prefill_fwd_d72_kernel<T>), dim3(static_cast<unsigned>(grid)),
                       dim3(attn::kD72Threads), 0, stream, p);
    int rc = launch_status();
    if (rc != ATTN_OK || p.split_parts == 1 || p.total_work == p.whole_work) return rc;
    hipLaunchKernelGGL((attn::prefill_merge_kernel<72, attn::kD72BM, T>),
                       dim3(static_cast<unsigned>((p.total_work - p.whole_work) *
                                                  attn::merge_blocks<72, attn::kD72BM>())),
                       dim3(attn::kMergeThreads), 0, stream, p);
    return launch_status();
}

template <typename T>
int launch_prefill_d128(const attn::PrefillParams &p, int64_t grid, hipStream_t stream)
{
    hipLaunchKernelGGL((attn::prefill_fwd_d128_kernel<T>), dim3(static_cast<unsigned>(grid)),
                       dim3(attn::kD128Threads), 0, stream, p);
    int rc = launch_status();
    if (rc != ATTN_OK || p.split_parts == 1 || p.total_work == p.whole_work) return rc;
    hipLaunchKernelGGL((attn::prefill_merge_kernel<128, attn::kD128BM, T>),
                       dim3(static_cast<unsigned>((p.total_work - p.whole_work) *
                                                  attn::merge_blocks<128, attn::kD128BM>())),
                       dim3(attn::kMergeThreads), 0, stream, p);
    return launch_status();
}

template <typename T, int W>
int launch_prefill_split(const attn::PrefillParams &p, int64_t grid, hipStream_t stream)
{
    hipLaunchKernelGGL((attn::prefill_fwd_split_kernel<T, W>), dim3(static_cast<unsigned>(grid)),
                       dim3(attn::split_threads(W)), 0, stream, p);
    return launch_status();
}

// Work items that fit the device at once: compute units x resident
// workgroups per unit of `kernel` (0 when the runtime cannot tell).
template <typename K>
int kernel_slots(int dev, K kernel, int threads)
{
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0);
    return e == hipSuccess ? cus * per_cu : 0;
}

// What the launch plans need to know of a device, queried once per device
// (the answers are fixed for the process; the queries cost host time on
// every call otherwise).  All zero when there is no current device.
struct DeviceShape {
    int cus = 0;        // compute units
    int slots_d128 = 0, slots_d72 = 0, slots_32x8 = 0, slots_32x4 = 0, slots_split = 0;
};
constexpr int kMaxShapeDevices = 64;
std::once_flag g_shape_once[kMaxShapeDevices];
DeviceShape g_shape[kMaxShapeDevices];

const DeviceShape &device_shape()
{
    static const DeviceShape none;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxShapeDevices) return none;
    std::call_once(g_shape_once[dev], [dev] {
        DeviceShape d;
        if (hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) d.cus = 0;
        d.slots_d128 = kernel_slots(dev, attn::prefill_fwd_d128_kernel<attn::Bf16>, attn::kD128Threads);
        d.slots_d72 = kernel_slots(dev, attn::prefill_fwd_d72_kernel<attn::Bf16>, attn::kD72Threads);
        d.slots_32x8 = kernel_slots(dev, attn::prefill_fwd_kernel<72, attn::Bf16, 8>, attn::prefill_threads(8));
        d.slots_32x4 = kernel_slots(dev, attn::prefill_fwd_kernel<72, attn::Bf16, 4>, attn::prefill_threads(4));
        d.slots_split = kernel_slots(dev, attn::prefill_fwd_split_kernel<attn::Bf16, attn::kSplitWaves>,
                                     attn::split_threads(attn::kSplitWaves));
        g_shape[dev] = d;
    });
    return g_shape[dev];
}

// The kernel for a call, and the resulting work items and slots.  head_dim
// 128 runs prefill_fwd_d128_kernel (4 waves of 64 query rows, 256 rows per
// item).  head_dim 72 runs prefill_fwd_split_kernel (32 query rows per item,
// the keys split over 4 waves) when those items all fit the device at once
// and max_seqlen_q <= kSplitMaxRows (at most 64 key tiles per wave): on such
// grids the other kernels' serial walk over the key tiles bounds the launch.
// Graph-replayed against the kernels chosen before, on 31 grids of 1-128
// heads and 64-8192 tokens: 1.1-1.9x faster with up to half the slots
// filled, 0.98-1.4x with up to all of them, 0.6-0.93x beyond (each wave
// then streams its own K/V tiles for only 32 rows, and the L2 bandwidth
// bounds it).  Otherwise prefill_fwd_d72_kernel (4 waves of 64 rows) runs
// when its items fill every slot at least once or the sequences are long
// (max_seqlen_q >= kD72LongRows: measured 2-6% faster on 8184, 15476 and
// 24952 tokens x 4 heads, 5-8% slower on 4100 x 4 and 3844 x 16); other
// grids run prefill_fwd_kernel with 8 waves of 32 rows (256 rows per item,
// one workgroup per CU) when those items fill the device, else with 4 waves
// (128 rows): the shorter Shapes rows ran up to 30% slower on fewer, longer
// items.
enum PrefillKind { kPrefill32x4, kPrefill32x8, kPrefillD72, kPrefillD128, kPrefillSplit };
constexpr int64_t kD72LongRows = 6144;
constexpr int64_t kSplitMaxRows = 8192;
bool is_split(PrefillKind k) { return k == kPrefillSplit; }
struct PrefillShapeChoice {
    PrefillKind kind = kPrefill32x4;
    int bm = 128, slots = 0;
    int64_t qtiles = 0, work = 0;
};

PrefillShapeChoice choose_prefill(int64_t num_seqs, int64_t max_seqlen_q, int64_t num_heads, int head_dim)
{
    PrefillShapeChoice c;
    const DeviceShape &ds = device_shape();
    const int64_t work256 = num_seqs * num_heads * ((max_seqlen_q + 255) / 256);
    const int64_t work32 = num_seqs * num_heads * ((max_seqlen_q + attn::kSplitBQ - 1) / attn::kSplitBQ);
    if (head_dim == 72 && ds.slots_split > 0 && work32 <= ds.slots_split && max_seqlen_q <= kSplitMaxRows) {
        c.kind = kPrefillSplit;
        c.slots = ds.slots_split;
        c.bm = attn::kSplitBQ;
    } else if (head_dim == 72) {
        const int slots64 = ds.slots_d72;
        const int slots8 = ds.slots_32x8;
        if (slots64 > 0 && (work256 >= slots64 || max_seqlen_q >= kD72LongRows)) {
            c.kind = kPrefillD72;
            c.slots = slots64;
            c.bm = attn::kD72BM;
        } else if (slots8 > 0 && work256 >= slots8) {
            c.kind = kPrefill32x8;
            c.slots = slots8;
            c.bm = attn::prefill_bm(8);
        } else {
            c.slots = ds.slots_32x4;
            c.bm = attn::prefill_bm(4);
        }
    } else {
        c.kind = kPrefillD128;
        c.slots = ds.slots_d128;
        c.bm = attn::kD128BM;
    }
    c.qtiles = (max_seqlen_q + c.bm - 1) / c.bm;
    c.work = num_seqs * num_heads * c.qtiles;
    return c;
}

// How the work items are launched.  When the last wave of workgroups would
// be at most half full, its items are split into key ranges (at most 8) that
// fill it, and a merge kernel combines the ranges; when it would be more than
// half full, its items are split into the number of ranges that finishes
// them soonest, if that saves a quarter of an item's time or more.
struct PrefillPlan {
    int64_t work = 0, whole = 0, parts = 1, grid = 0;
    size_t ws_o_bytes = 0, ws_bytes = 0;
};

PrefillPlan plan_prefill(int64_t work, int slots, int bm, int head_dim, int64_t key_tiles)
{
    PrefillPlan pl;
    pl.work = work;
    const int64_t full = slots > 0 ? work / slots : 0;
    const int64_t rest = slots > 0 ? work % slots : 0;
    if (full >= 1 && rest > 0 && 2 * rest <= slots) {
        pl.parts = slots / rest < 8 ? slots / rest : 8;
        pl.whole = (full * slots) / 8 * 8;
    } else if (full == 0 && work > 0 && 2 * work <= slots) {
        // fewer items than half the device holds: split every item into
        // ranges of at least four key tiles, when there are 16 or more
        // (key_tiles estimates the keys per sequence from the query length;
        // below that the merge costs more than the split gains)
        int64_t parts = slots / work < 8 ? slots / work : 8;
        if (parts > key_tiles / 4) parts = key_tiles / 4;
        if (key_tiles >= 16 && parts >= 2) {
            pl.parts = parts;
            pl.whole = 0;
        }
    } else if (rest > 0 && key_tiles >= 32) {
        // the last wave is more than half full: split its items into p
        // ranges of at least 16 key tiles, with p chosen to minimise the
        // tail's time ceil(tail p / slots) / p (in units of one whole item),
        // and only when that saves at least a quarter of the unsplit time.
        // (Shorter ranges lose more to writing and merging the fp32 partial
        // results of a tail this large than the split gains.)
        const int64_t whole = (full * slots) / 8 * 8;
        const int64_t tail = work - whole;
        int64_t best_p = 1, best_waves = (tail + slots - 1) / slots;   // time: best_waves / best_p items
        const int64_t pmax = key_tiles / 16 < 8 ? key_tiles / 16 : 8;
        for (int64_t p = 2; p <= pmax; ++p) {
            const int64_t waves = (tail * p + slots - 1) / slots;
            if (waves * best_p < best_waves * p) {
                best_p = p;
                best_waves = waves;
            }
        }
        const int64_t base_waves = (tail + slots - 1) / slots;   // unsplit: base_waves / 1
        if (best_p > 1 && 4 * best_waves <= 3 * best_p * base_waves) {
            pl.parts = best_p;
            pl.whole = whole;
        }
    }
    if (pl.parts < 2) {
        pl.parts = 1;
        pl.whole = work / 8 * 8;
    }
    pl.grid = pl.whole + (work - pl.whole) * pl.parts;
    if (pl.parts > 1) {
        const size_t slots_ws = static_cast<size_t>(work - pl.whole) * pl.parts * bm;
        pl.ws_o_bytes = (slots_ws * head_dim * sizeof(float) + 255) / 256 * 256;
        pl.ws_bytes = pl.ws_o_bytes + slots_ws * 2 * sizeof(float);
    }
    return pl;
}

template <typename T, int D, int GMAX>
int launch_decode(const attn::DecodeParams &p, int64_t grid, hipStream_t stream)
{
    hipLaunchKernelGGL((attn::decode_partition_kernel<T, D, GMAX>), dim3(static_cast<unsigned>(grid)),
                       dim3(attn::kDecodeThreads), 0, stream, p);
    int rc = launch_status();
    if (rc != ATTN_OK || p.num_parts == 1) return rc;
    hipLaunchKernelGGL((attn::decode_merge_kernel<T, D>),
                       dim3(static_cast<unsigned>(static_cast<int64_t>(p.num_seqs) * p.Hq)), dim3(64), 0,
                       stream, p);
    return launch_status();
}

// Grouped query heads held by one workgroup: the products on MFMAs
template <typename T, int D>
int launch_decode_mfma(const attn::DecodeParams &p, int64_t grid, hipStream_t stream)
{
    hipLaunchKernelGGL((attn::decode_mfma_kernel<T, D>), dim3(static_cast<unsigned>(grid)),
                       dim3(attn::kDecodeThreads), 0, stream, p);
    int rc = launch_status();
    if (rc != ATTN_OK || p.num_parts == 1) return rc;
    hipLaunchKernelGGL((attn::decode_merge_kernel<T, D>),
                       dim3(static_cast<unsigned>(static_cast<int64_t>(p.num_seqs) * p.Hq)), dim3(64), 0,
                       stream, p);
    return launch_status();
}

template <typename T, int D>
int dispatch_decode_g(const attn::DecodeParams &p, int64_t grid, hipStream_t stream)
{
    if (p.on_mfma) return launch_decode_mfma<T, D>(p, grid, stream);
    if (p.gsub <= 1) return launch_decode<T, D, 1>(p, grid, stream);
    if (p.gsub <= 2) return launch_decode<T, D, 2>(p, grid, stream);
    if (p.gsub <= 4) return launch_decode<T, D, 4>(p, grid, stream);
    if (p.gsub <= 8) return launch_decode<T, D, 8>(p, grid, stream);
    return launch_decode<T, D, 16>(p, grid, stream);
}

template <typename T>
int dispatch_decode(const attn::DecodeParams &p, int head_size, int64_t grid, hipStream_t stream)
{
    return head_size == 128 ? dispatch_decode_g<T, 128>(p, grid, stream)
                            : dispatch_decode_g<T, 256>(p, grid, stream);
}

// Compute units of the current device (256 when the runtime cannot tell).
int device_cus()
{
    const int cus = device_shape().cus;
    return cus > 0 ? cus : 256;
}

// Tokens per context partition.  Left to the library (partition_size 0):
// kDefaultPartitionTokens, halved down to kMinAutoPartitionTokens while the
// workgroups (sequence x KV head x partition) would leave compute units
// without one.  Few long contexts then spread over the device (graph
// replayed: 1 sequence x 2 KV heads x 1024 tokens 29.4 -> 13.3 us, 4 x 8 x
// 2048 23.1 -> 16.6 us, 1 x 1 x 4096 32.2 -> 20.2 us); shorter partitions
// (one block per wave) were slower on most of the small rows measured,
// their merge and per-workgroup start costing more than they spread.
int partition_tokens(int64_t num_seqs, int64_t num_kv_heads, int64_t max_blocks_per_seq,
                     int32_t block_size, int32_t partition_size)
{
    if (partition_size > 0) return partition_size;
    const int64_t cus = device_cus();
    const int64_t ctx = max_blocks_per_seq * block_size;
    int pt = kDefaultPartitionTokens;
    while (pt > kMinAutoPartitionTokens && num_seqs * num_kv_heads * ((ctx + pt - 1) / pt) < cus) pt /= 2;
    return pt;
}

int partitions(int32_t num_seqs, int32_t num_kv_heads, int32_t max_blocks_per_seq, int32_t block_size,
               int32_t partition_size, int *part_blocks)
{
    if (num_seqs < 0 || num_kv_heads <= 0 || max_blocks_per_seq < 0 || block_size <= 0 || partition_size < 0)
        return -ATTN_ERR_INVALID_ARG;
    if (partition_size % block_size) return -ATTN_ERR_INVALID_ARG;
    const int pt = partition_tokens(num_seqs, num_kv_heads, max_blocks_per_seq, block_size, partition_size);
    int pb = pt / block_size;
    if (pb < 1) pb = 1;
    if (part_blocks) *part_blocks = pb;
    if (max_blocks_per_seq == 0) return 1;
    return (max_blocks_per_seq + pb - 1) / pb;
}

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void *g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// The device address of the current device's copy of `scratch`.
int scratch_address(void **ptr)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return ATTN_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return ATTN_ERR_UNSUPPORTED;
    std::call_once(g_scratch_once[dev], [dev] {
        void *p = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = p;
    });
    if (g_scratch_err[dev] != hipSuccess || !g_scratch_ptr[dev]) return ATTN_ERR_HIP;
    *ptr = g_scratch_ptr[dev];
    return ATTN_OK;
}

}  // namespace

extern "C" {

const char *attn_status_string(int32_t status)
{
    switch (status) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_ERR_INVALID_ARG: return "ATTN_ERR_INVALID_ARG";
    case ATTN_ERR_UNSUPPORTED: return "ATTN_ERR_UNSUPPORTED";
    case ATTN_ERR_WORKSPACE: return "ATTN_ERR_WORKSPACE";
    case ATTN_ERR_HIP: return "ATTN_ERR_HIP";
    default: return "ATTN_ERR_UNKNOWN";
    }
}

size_t attn_varlen_fwd_workspace_size(int32_t num_seqs, int32_t max_seqlen_q, int32_t num_heads,
                                      int32_t head_dim)
{
    if (num_seqs <= 0 || max_seqlen_q <= 0 || num_heads <= 0) return 0;
    if (head_dim != 72 && head_dim != 128) return 0;
    const PrefillShapeChoice c = choose_prefill(num_seqs, max_seqlen_q, num_heads, head_dim);
    if (is_split(c.kind)) return 0;
    const int64_t key_tiles = (static_cast<int64_t>(max_seqlen_q) + attn::kPrefillBN - 1) / attn::kPrefillBN;
    return plan_prefill(c.work, c.slots, c.bm, head_dim, key_tiles).ws_bytes;
}

static int attn_varlen_fwd_impl(const void *q, const void *k, const void *v, const int32_t *cu_seqlens_q,
                                const int32_t *cu_seqlens_k, int32_t num_seqs, int32_t max_seqlen_q,
                                int64_t total_q, int64_t total_k, int32_t num_heads, int32_t head_dim,
                                float scale, int32_t dtype, void *workspace, size_t workspace_bytes,
                                void *out, void *stream)
{
    if (num_seqs < 0 || max_seqlen_q < 0 || total_q < 0 || total_k < 0 || num_heads <= 0 ||
        head_dim <= 0)
        return ATTN_ERR_INVALID_ARG;
    if (dtype != ATTN_DTYPE_BF16 && dtype != ATTN_DTYPE_FP16) return ATTN_ERR_INVALID_ARG;
    if (!std::isfinite(scale)) return ATTN_ERR_INVALID_ARG;
    if (head_dim != 72 && head_dim != 128) return ATTN_ERR_UNSUPPORTED;
    // the kernel addresses a key tile with 32-bit byte offsets
    if (static_cast<int64_t>(num_heads) * head_dim * 2 * attn::kPrefillBN > UINT32_MAX)
        return ATTN_ERR_INVALID_ARG;
    if (num_seqs == 0 || max_seqlen_q == 0 || total_q == 0) return ATTN_OK;
    if (!q || !cu_seqlens_q || !cu_seqlens_k || !out) return ATTN_ERR_INVALID_ARG;
    if ((!k || !v) && total_k > 0) return ATTN_ERR_INVALID_ARG;   // k, v may be empty
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
        !aligned(cu_seqlens_q, 4) || !aligned(cu_seqlens_k, 4) || !aligned(workspace, 256))
        return ATTN_ERR_INVALID_ARG;

    // (work items at 128 rows bound the count for either workgroup size)
    const int64_t work128 = static_cast<int64_t>(num_seqs) * num_heads * ((max_seqlen_q + 127) / 128);
    if (work128 > INT32_MAX / 8) return ATTN_ERR_INVALID_ARG;
    const PrefillShapeChoice c = choose_prefill(num_seqs, max_seqlen_q, num_heads, head_dim);
    const int bm = c.bm;
    const int64_t qtiles = c.qtiles;
    const int64_t work = c.work;
    const int64_t key_tiles = (static_cast<int64_t>(max_seqlen_q) + attn::kPrefillBN - 1) / attn::kPrefillBN;
    PrefillPlan pl;
    if (is_split(c.kind)) {
        // items of 32 query rows, all run whole (their waves split the keys)
        pl.work = work;
        pl.whole = work / 8 * 8;
        pl.grid = work;
    } else {
        pl = plan_prefill(work, c.slots, bm, head_dim, key_tiles);
        if (pl.parts > 1 && (!workspace || workspace_bytes < pl.ws_bytes))
            pl = plan_prefill(work, 0, bm, head_dim, key_tiles);    // no room for the split: run items whole
    }

    attn::PrefillParams p;
    p.q = static_cast<const uint16_t *>(q);
    p.k = static_cast<const uint16_t *>(k);
    p.v = static_cast<const uint16_t *>(v);
    p.cu_q = cu_seqlens_q;
    p.cu_k = cu_seqlens_k;
    p.out = static_cast<uint16_t *>(out);
    p.total_q = total_q;
    p.total_k = total_k;
    p.num_heads = num_heads;
    p.num_qtiles = static_cast<int>(qtiles);
    p.total_work = static_cast<int>(work);
    p.whole_work = static_cast<int>(pl.whole);
    p.split_parts = static_cast<int>(pl.parts);
    p.ws_o = pl.parts > 1 ? static_cast<float *>(workspace) : nullptr;
    p.ws_ml = pl.parts > 1 ? reinterpret_cast<float *>(static_cast<char *>(workspace) + pl.ws_o_bytes) : nullptr;
    p.scale_log2e = std::fabs(scale) * attn::kLog2e;
    p.negate_q = scale < 0.f ? 1 : 0;
    hipStream_t s = static_cast<hipStream_t>(stream);

    const bool bf = dtype == ATTN_DTYPE_BF16;
    switch (c.kind) {
    case kPrefillSplit:
        return bf ? launch_prefill_split<attn::Bf16, attn::kSplitWaves>(p, pl.grid, s)
                  : launch_prefill_split<attn::Fp16, attn::kSplitWaves>(p, pl.grid, s);
    case kPrefillD128:
        return bf ? launch_prefill_d128<attn::Bf16>(p, pl.grid, s) : launch_prefill_d128<attn::Fp16>(p, pl.grid, s);
    case kPrefillD72:
        return bf ? launch_prefill_d72<attn::Bf16>(p, pl.grid, s) : launch_prefill_d72<attn::Fp16>(p, pl.grid, s);
    case kPrefill32x8:
        return bf ? launch_prefill<72, attn::Bf16, 8>(p, pl.grid, s) : launch_prefill<72, attn::Fp16, 8>(p, pl.grid, s);
    default:
        return bf ? launch_prefill<72, attn::Bf16, 4>(p, pl.grid, s) : launch_prefill<72, attn::Fp16, 4>(p, pl.grid, s);
    }
}

int32_t attn_paged_decode_num_partitions(int32_t num_seqs, int32_t num_kv_heads, int32_t max_blocks_per_seq,
                                         int32_t block_size, int32_t partition_size)
{
    return partitions(num_seqs, num_kv_heads, max_blocks_per_seq, block_size, partition_size, nullptr);
}

size_t attn_paged_decode_workspace_size(int32_t num_seqs, int32_t num_query_heads, int32_t num_kv_heads,
                                        int32_t head_size, int32_t max_blocks_per_seq, int32_t block_size,
                                        int32_t partition_size)
{
    if (num_seqs < 0 || num_query_heads <= 0 || head_size <= 0) return 0;
    const int np = partitions(num_seqs, num_kv_heads, max_blocks_per_seq, block_size, partition_size, nullptr);
    if (np <= 1) return 0;
    const size_t rows = static_cast<size_t>(num_seqs) * num_query_heads * np;
    const size_t ml = (rows * 2 * sizeof(float) + 255) / 256 * 256;
    return ml + rows * static_cast<size_t>(head_size) * sizeof(float);
}

}  // extern "C"

namespace {

// Argument checks of a paged-decode call, before anything touches the device.
int check_decode_args(const void *query, const void *k_cache, const void *v_cache,
                      const int32_t *block_tables, const int32_t *seq_lens, int32_t num_seqs,
                      int32_t num_query_heads, int32_t num_kv_heads, int32_t head_size,
                      int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks, float scale,
                      int32_t dtype, int32_t partition_size, const void *out)
{
    if (num_seqs < 0 || num_query_heads <= 0 || num_kv_heads <= 0 || head_size <= 0 ||
        block_size <= 0 || max_blocks_per_seq < 0 || num_blocks < 0 || partition_size < 0)
        return ATTN_ERR_INVALID_ARG;
    if (dtype != ATTN_DTYPE_BF16 && dtype != ATTN_DTYPE_FP16) return ATTN_ERR_INVALID_ARG;
    if (!std::isfinite(scale)) return ATTN_ERR_INVALID_ARG;
    if (num_query_heads % num_kv_heads) return ATTN_ERR_INVALID_ARG;
    if (head_size % 8) return ATTN_ERR_INVALID_ARG;
    if (partition_size % block_size) return ATTN_ERR_INVALID_ARG;
    if ((head_size != 128 && head_size != 256) || block_size != attn::kDecodeBS) return ATTN_ERR_UNSUPPORTED;
    const int G = num_query_heads / num_kv_heads;
    if (G > 16) return ATTN_ERR_UNSUPPORTED;
    if (num_seqs == 0) return ATTN_OK;
    if (!query || !k_cache || !v_cache || !seq_lens || !out) return ATTN_ERR_INVALID_ARG;
    if (!block_tables && max_blocks_per_seq > 0) return ATTN_ERR_INVALID_ARG;
    if (!aligned(query, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
        !aligned(block_tables, 4) || !aligned(seq_lens, 4))
        return ATTN_ERR_INVALID_ARG;
    return ATTN_OK;
}

// The launches of a checked paged-decode call with a workspace of at least
// attn_paged_decode_workspace_size bytes (or none, when that size is 0).
int launch_paged_decode(const void *query, const void *k_cache, const void *v_cache,
                        const int32_t *block_tables, const int32_t *seq_lens, int32_t num_seqs,
                        int32_t num_query_heads, int32_t num_kv_heads, int32_t head_size,
                        int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks,
                        float scale, int32_t dtype, int32_t partition_size, void *workspace,
                        size_t workspace_bytes, void *out, void *stream)
{
    const int G = num_query_heads / num_kv_heads;
    int part_blocks = 1;
    const int np = partitions(num_seqs, num_kv_heads, max_blocks_per_seq, block_size, partition_size,
                              &part_blocks);
    if (np < 1) return ATTN_ERR_INVALID_ARG;
    const int64_t units = static_cast<int64_t>(num_seqs) * num_kv_heads * np;
    if (units > INT32_MAX || static_cast<int64_t>(num_seqs) * num_query_heads > INT32_MAX)
        return ATTN_ERR_INVALID_ARG;
    // Fewer (sequence, KV head, partition) units than compute units: deal
    // the G query heads of each out to up to cus / units workgroups, one
    // head each where there is room (graph replayed, 1 sequence x 16/2 heads
    // x 128 tokens at head_size 256: 13.1 -> 4.9 us; 4 x 32/4 x 128: 9.5 ->
    // 4.1 us; at least 2 heads per workgroup, or at most 4 workgroups per
    // unit, were slower on every small row measured).
    int ngroups = 1;
    const int cus = device_cus();
    if (G > 1 && units > 0 && units < cus) {
        const int64_t room = cus / units;
        ngroups = static_cast<int>(room < G ? room : G);
    }
    const int gsub = (G + ngroups - 1) / ngroups;
    ngroups = (G + gsub - 1) / gsub;
    const int64_t grid = units * ngroups;
    // One workgroup per KV head holding two or more query heads (no head
    // dealing): the score and value products on MFMAs (decode_mfma_kernel).
    // Graph-replayed against the VALU dot-product kernel on device-filling
    // grids, it ran faster or level at every shape measured: 16 query heads
    // per KV head 1.8x at 64 tokens and 2.1x at 2048; 4 heads 12-16% over
    // 48-100 tokens; 2 heads 2-10% over 16-200 tokens; at head_size 256, 2-4
    // heads 6-17%, 16 heads 3x.  With one query head per KV head only where a
    // workgroup walks 8 blocks or more (3% at 128 tokens, 5% at head_size
    // 256 over 1024; over 64 tokens the VALU kernel is 1-2% ahead, 12% at
    // head_size 256).
    const int walk_blocks = part_blocks < max_blocks_per_seq ? part_blocks : max_blocks_per_seq;
    const bool on_mfma = ngroups == 1 && (G >= 2 || walk_blocks >= 8);

    attn::DecodeParams p;
    p.query = static_cast<const uint16_t *>(query);
    p.k_cache = static_cast<const uint16_t *>(k_cache);
    p.v_cache = static_cast<const uint16_t *>(v_cache);
    p.block_tables = block_tables;
    p.seq_lens = seq_lens;
    p.out = static_cast<uint16_t *>(out);
    p.ws_ml = nullptr;
    p.ws_o = nullptr;
    if (np > 1) {
        const size_t need = attn_paged_decode_workspace_size(num_seqs, num_query_heads, num_kv_heads,
                                                             head_size, max_blocks_per_seq, block_size,
                                                             partition_size);
        if (!workspace || workspace_bytes < need || !aligned(workspace, 256)) return ATTN_ERR_WORKSPACE;
        const size_t rows = static_cast<size_t>(num_seqs) * num_query_heads * np;
        const size_t ml = (rows * 2 * sizeof(float) + 255) / 256 * 256;
        p.ws_ml = static_cast<float *>(workspace);
        p.ws_o = reinterpret_cast<float *>(static_cast<char *>(workspace) + ml);
    }
    p.num_blocks = num_blocks;
    p.num_seqs = num_seqs;
    p.Hq = num_query_heads;
    p.Hkv = num_kv_heads;
    p.G = G;
    p.maxb = max_blocks_per_seq;
    p.part_blocks = part_blocks;
    p.num_parts = np;
    p.gsub = gsub;
    p.ngroups = ngroups;
    p.on_mfma = on_mfma ? 1 : 0;
    p.scale_log2e = scale * attn::kLog2e;
    hipStream_t s = static_cast<hipStream_t>(stream);
    return dtype == ATTN_DTYPE_BF16 ? dispatch_decode<attn::Bf16>(p, head_size, grid, s)
                                    : dispatch_decode<attn::Fp16>(p, head_size, grid, s);
}

}  // namespace

extern "C" {

static int attn_paged_decode_impl(const void *query, const void *k_cache, const void *v_cache,
                                  const int32_t *block_tables, const int32_t *seq_lens, int32_t num_seqs,
                                  int32_t num_query_heads, int32_t num_kv_heads, int32_t head_size,
                                  int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks,
                                  float scale, int32_t dtype, int32_t partition_size, void *workspace,
                                  size_t workspace_bytes, void *out, void *stream)
{
    const int rc = check_decode_args(query, k_cache, v_cache, block_tables, seq_lens, num_seqs,
                                     num_query_heads, num_kv_heads, head_size, block_size,
                                     max_blocks_per_seq, num_blocks, scale, dtype, partition_size, out);
    if (rc != ATTN_OK || num_seqs == 0) return rc;
    return launch_paged_decode(query, k_cache, v_cache, block_tables, seq_lens, num_seqs,
                               num_query_heads, num_kv_heads, head_size, block_size,
                               max_blocks_per_seq, num_blocks, scale, dtype, partition_size,
                               workspace, workspace_bytes, out, stream);
}

static int attn_paged_decode_noalloc_impl(const void *query, const void *k_cache, const void *v_cache,
                                          const int32_t *block_tables, const int32_t *seq_lens,
                                          int32_t num_seqs, int32_t num_query_heads, int32_t num_kv_heads,
                                          int32_t head_size, int32_t block_size, int32_t max_blocks_per_seq,
                                          int64_t num_blocks, float scale, int32_t dtype,
                                          int32_t partition_size, void *out, void *stream)
{
    const int rc = check_decode_args(query, k_cache, v_cache, block_tables, seq_lens, num_seqs,
                                     num_query_heads, num_kv_heads, head_size, block_size,
                                     max_blocks_per_seq, num_blocks, scale, dtype, partition_size, out);
    if (rc != ATTN_OK) return rc;
    const size_t need = attn_paged_decode_workspace_size(num_seqs, num_query_heads, num_kv_heads, head_size,
                                                         max_blocks_per_seq, block_size, partition_size);
    if (need > ATTN_NOALLOC_SCRATCH_BYTES) return ATTN_ERR_WORKSPACE;
    // set-up on the first call on a device (also when no split needs it)
    void *ws = nullptr;
    const int src = scratch_address(&ws);
    if (src != ATTN_OK) return src;
    if (num_seqs == 0) return ATTN_OK;
    return launch_paged_decode(query, k_cache, v_cache, block_tables, seq_lens, num_seqs,
                               num_query_heads, num_kv_heads, head_size, block_size,
                               max_blocks_per_seq, num_blocks, scale, dtype, partition_size,
                               need > 0 ? ws : nullptr, need > 0 ? ATTN_NOALLOC_SCRATCH_BYTES : 0,
                               out, stream);
}

static int attn_chunk_delta_out_impl(const void *q, const void *k, const void *v, const void *h,
                                     const float *g, int32_t batch, int32_t tokens, int32_t num_q_heads,
                                     int32_t num_heads, int32_t key_dim, int32_t value_dim,
                                     int32_t chunk_size, float scale, int32_t dtype, void *out, void *stream)
{
    if (batch < 0 || tokens < 0 || num_q_heads <= 0 || num_heads <= 0 || key_dim <= 0 ||
        value_dim <= 0 || chunk_size <= 0)
        return ATTN_ERR_INVALID_ARG;
    if (dtype != ATTN_DTYPE_BF16 && dtype != ATTN_DTYPE_FP16) return ATTN_ERR_INVALID_ARG;
    if (!std::isfinite(scale)) return ATTN_ERR_INVALID_ARG;
    if (key_dim != attn::kChunkDim || value_dim != attn::kChunkDim || chunk_size != attn::kChunk)
        return ATTN_ERR_UNSUPPORTED;
    if (batch == 0 || tokens == 0) return ATTN_OK;
    if (!q || !k || !v || !h || !g || !out) return ATTN_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(h, 16) || !aligned(out, 16) ||
        !aligned(g, 4))
        return ATTN_ERR_INVALID_ARG;
    const int64_t num_chunks = (static_cast<int64_t>(tokens) + chunk_size - 1) / chunk_size;
    const int64_t grid = static_cast<int64_t>(batch) * num_chunks * num_heads;
    // the kernel's buffer offsets are 32-bit: one chunk of q, k or v rows must
    // span less than 2 GiB
    const int64_t v_span = static_cast<int64_t>(chunk_size) * num_heads * value_dim * 2;
    const int64_t qk_span = static_cast<int64_t>(chunk_size) * num_q_heads * key_dim * 2;
    if (grid > INT32_MAX || v_span > INT32_MAX || qk_span > INT32_MAX) return ATTN_ERR_INVALID_ARG;

    attn::ChunkParams p;
    p.q = static_cast<const uint16_t *>(q);
    p.k = static_cast<const uint16_t *>(k);
    p.v = static_cast<const uint16_t *>(v);
    p.h = static_cast<const uint16_t *>(h);
    p.g = g;
    p.out = static_cast<uint16_t *>(out);
    p.batch = batch;
    p.tokens = tokens;
    p.num_q_heads = num_q_heads;
    p.num_heads = num_heads;
    p.num_chunks = static_cast<int>(num_chunks);
    p.per_q = num_heads / num_q_heads > 1 ? num_heads / num_q_heads : 1;
    p.scale = scale;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (dtype == ATTN_DTYPE_BF16)
        hipLaunchKernelGGL((attn::chunk_delta_out_kernel<attn::Bf16>), dim3(static_cast<unsigned>(grid)),
                           dim3(attn::kChunkThreads), 0, s, p);
    else
        hipLaunchKernelGGL((attn::chunk_delta_out_kernel<attn::Fp16>), dim3(static_cast<unsigned>(grid)),
                           dim3(attn::kChunkThreads), 0, s, p);
    return launch_status();
}


// The entry points proper: the implementations above return attn_status values as int.
attn_status attn_varlen_fwd(const void *q, const void *k, const void *v, const int32_t *cu_seqlens_q,
                            const int32_t *cu_seqlens_k, int32_t num_seqs, int32_t max_seqlen_q,
                            int64_t total_q, int64_t total_k, int32_t num_heads, int32_t head_dim,
                            float scale, int32_t dtype, void *workspace, size_t workspace_bytes, void *out,
                            void *stream)
{
    return static_cast<attn_status>(attn_varlen_fwd_impl(q, k, v, cu_seqlens_q, cu_seqlens_k, num_seqs,
                                                         max_seqlen_q, total_q, total_k, num_heads,
                                                         head_dim, scale, dtype, workspace, workspace_bytes,
                                                         out, stream));
}

attn_status attn_paged_decode(const void *query, const void *k_cache, const void *v_cache,
                              const int32_t *block_tables, const int32_t *seq_lens, int32_t num_seqs,
                              int32_t num_query_heads, int32_t num_kv_heads, int32_t head_size,
                              int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks,
                              float scale, int32_t dtype, int32_t partition_size, void *workspace,
                              size_t workspace_bytes, void *out, void *stream)
{
    return static_cast<attn_status>(attn_paged_decode_impl(query, k_cache, v_cache, block_tables, seq_lens,
                                                           num_seqs, num_query_heads, num_kv_heads,
                                                           head_size, block_size, max_blocks_per_seq,
                                                           num_blocks, scale, dtype, partition_size,
                                                           workspace, workspace_bytes, out, stream));
}

attn_status attn_paged_decode_noalloc(const void *query, const void *k_cache, const void *v_cache,
                                      const int32_t *block_tables, const int32_t *seq_lens,
                                      int32_t num_seqs, int32_t num_query_heads, int32_t num_kv_heads,
                                      int32_t head_size, int32_t block_size, int32_t max_blocks_per_seq,
                                      int64_t num_blocks, float scale, int32_t dtype,
                                      int32_t partition_size, void *out, void *stream)
{
    return static_cast<attn_status>(attn_paged_decode_noalloc_impl(query, k_cache, v_cache, block_tables,
                                                                   seq_lens, num_seqs, num_query_heads,
                                                                   num_kv_heads, head_size, block_size,
                                                                   max_blocks_per_seq, num_blocks, scale,
                                                                   dtype, partition_size, out, stream));
}

attn_status attn_chunk_delta_out(const void *q, const void *k, const void *v, const void *h, const float *g,
                                 int32_t batch, int32_t tokens, int32_t num_q_heads, int32_t num_heads,
                                 int32_t key_dim, int32_t value_dim, int32_t chunk_size, float scale,
                                 int32_t dtype, void *out, void *stream)
{
    return static_cast<attn_status>(attn_chunk_delta_out_impl(q, k, v, h, g, batch, tokens, num_q_heads,
                                                              num_heads, key_dim, value_dim, chunk_size,
                                                              scale, dtype, out, stream));
}

}  // extern "C"
