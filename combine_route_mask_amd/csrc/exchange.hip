// gfx950 kernels of the expert-parallel exchange between P virtual ranks
// that share one GPU: dispatch (routing mask + dedup, per-destination
// wave-ballot scan, 16-byte row scatter with invalid-slot markers) and
// combine (fp32 gather-reduce of the per-rank expert outputs, BF16 or via
// an FP8 landing plane).
//
// Contract (FlashInfer "NVLinkTwoSidedAlltoAll" dispatch/combine, FlashInfer
// "NVLinkOneSidedConfig" lamport paragraph for the slot rule
// q = src * tokens_per_rank + t, vLLM "device_communicators.all2all"
// FlashInferNVLinkTwoSidedManager for the invalid expert id): see moe_ep.h.
//
// Every kernel is a byte mover bounded by HBM bandwidth; nothing here is a
// contraction, so no matrix cores are used.  Rows move as 16-byte vectors
// (global_load/store_dwordx4); a workgroup reads a token row once and
// writes it to every destination in its mask.
#include <algorithm>
#include <mutex>

#include "formats.h"
#include "memory_ops.h"
#include "moe_ep_internal.h"

// Tuning knobs (compile-time; defaults are the measured best on MI355X).
// Launches whose row stores total at most this many bytes write them
// through L2 (write-through stores); larger ones store non-temporally.  At
// the end of a kernel every L2 writes back its dirty lines before the next
// kernel may start, a cost of ~2 us that write-through stores avoid; per
// byte they are slower than non-temporal ones (1-3% on long rows, ~25% on
// rows of a few KB), so they pay only where that flush is a sizeable part of
// the launch.
#ifndef MOE_EP_WT_BYTES
#define MOE_EP_WT_BYTES (256ll << 20)
#endif
// 16-byte vectors per thread in a dispatch row chunk, for payload rows of at
// least MOE_EP_DISPATCH_LONG_ROW bytes and for shorter ones (short rows split
// into more, smaller chunks so more workgroups share a step's few rows).
#ifndef MOE_EP_DISPATCH_VPT_LONG
#define MOE_EP_DISPATCH_VPT_LONG 4
#endif
#ifndef MOE_EP_DISPATCH_VPT_SHORT
#define MOE_EP_DISPATCH_VPT_SHORT 1
#endif
#ifndef MOE_EP_DISPATCH_LONG_ROW
#define MOE_EP_DISPATCH_LONG_ROW 8192
#endif
// Short rows longer than one chunk (4 KB) in launches too large to prefetch
// (below) take this many vectors per thread instead: a row of up to 8 KB
// per workgroup, so each token's mask is built once.  EP64 DeepSeekFp8
// dispatch (7 KB rows, same buffers) 481 -> 429 us; the prefetching MXFP8
// dispatch keeps 1 (2 there: +7%).  Rows of one chunk keep 1: the split is
// the same, and with 1 KB of extra payload loaded beside the row the EP64
// NVFP4 dispatch took 298 us with 2 against 291 with 1 (without extras
// 216 / 220 us).
#ifndef MOE_EP_DISPATCH_VPT_MID
#define MOE_EP_DISPATCH_VPT_MID 2
#endif
// Dispatches of at most this many (token, row chunk) items, eight rounds of
// resident workgroups, load each row before its token's mask.
#ifndef MOE_EP_PREFETCH_ITEMS
#define MOE_EP_PREFETCH_ITEMS 16384
#endif
#ifndef MOE_EP_SCATTER_GRID
#define MOE_EP_SCATTER_GRID 131072 // most payload-scatter workgroups of a dispatch launch
#endif
// BF16 combine shapes: (16-byte vectors per thread, ranks loaded at once)
// for outputs below MOE_EP_COMBINE_LARGE_BYTES and for larger ones.  Output
// rows are not read again within a step, so they never stay in the caches:
// written through for outputs of at most MOE_EP_WT_BYTES, non-temporal
// above.  Large outputs: one vector per thread of 128-thread workgroups (a
// 7168-wide row in seven 2 KB pieces) and four ranks in flight, one item per
// workgroup; on the EP64 workload (same buffers) 713 us against 749 us for
// four vectors per thread in 256-thread workgroups: each workgroup's output
// store is one 2 KB piece, so the combine's writes reach HBM as a denser
// front among its reads (64 / 448 / 896 threads: 756 / 744 / 729 us).
#ifndef MOE_EP_COMBINE_SMALL
#define MOE_EP_COMBINE_SMALL 1, 8
#endif
#ifndef MOE_EP_COMBINE_LARGE
#define MOE_EP_COMBINE_LARGE 1, 4
#endif
// Threads per workgroup of the small-output shape: at H = 7168 a row is
// 896 16-byte vectors, seven chunks of 128 with no idle lanes (256-thread
// workgroups leave half of every fourth one idle).  Measured on the EP8
// step against 256 / 448 / 64 threads: 22.5 against 23.0 / 23.0 / 22.6 us.
#ifndef MOE_EP_COMBINE_SMALL_BLOCK
#define MOE_EP_COMBINE_SMALL_BLOCK 128
#endif
#ifndef MOE_EP_COMBINE_LARGE_BLOCK
#define MOE_EP_COMBINE_LARGE_BLOCK 128 // threads per workgroup of the large-output shape
#endif
// Most workgroups of a BF16 combine launch: up to this many items each
// workgroup runs one item (its token's route mask in one scalar load), above
// it they loop.  The EP64 combine has 229376 items.
#ifndef MOE_EP_COMBINE_GRID_CAP
#define MOE_EP_COMBINE_GRID_CAP (1ll << 22)
#endif
#ifndef MOE_EP_FP8_GATHER
#define MOE_EP_FP8_GATHER 2 // ranks per round in the FP8 combine kernels
#endif
#ifndef MOE_EP_COMBINE_LARGE_BYTES
#define MOE_EP_COMBINE_LARGE_BYTES (128ll << 20)
#endif

namespace moe_ep {
namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short v2i16 __attribute__((ext_vector_type(2)));

// 256-slot chunks per step of a destination's scan.  At EP64 each scan
// block walks 32768 slots, and its latency-bound steps reach past the short
// NVFP4 dispatch's payload scatter (a build without the scan role is 5%
// faster there).  Same buffers: 4 -> NVFP4 dispatch 230.5 us, 2 -> 238.2,
// 8 -> 232.2; EP8, EP64 BF16 and MXFP8 dispatches unchanged.
#ifndef MOE_EP_SCAN_UNROLL
#define MOE_EP_SCAN_UNROLL 4
#endif
constexpr int kScanUnroll = MOE_EP_SCAN_UNROLL; // 256-slot chunks per scan step
constexpr int kWaves = kBlock / 64;
constexpr int kPlaneSlots = kBlock;     // slots per id-plane item (one per thread)
constexpr int kPlaneGroup = 8;          // destinations per id-plane item
constexpr int64_t kGridCap = 256 * 8 * 64; // most workgroups of a launch (64 rounds of the chip)

// Runs item(w) for the launch's items w < items.  ONE: the grid has one
// workgroup per item, so a workgroup runs its item and ends; otherwise
// workgroups loop over the items with the grid's stride.  With no loop, an
// item's first loads (a token's ids or route mask) precede every store
// of the kernel, so the compiler may fetch a uniform one with a scalar load,
// which it cannot do inside a loop whose earlier passes store (EP8 BF16
// combine 11.4 -> 10.9 us).
template <bool ONE, typename F>
__device__ __forceinline__ void for_each_item(int64_t items, F &&item)
{
    if constexpr (ONE) {
        if ((int64_t)blockIdx.x < items)
            item((int64_t)blockIdx.x);
    } else {
        for (int64_t w = blockIdx.x; w < items; w += gridDim.x)
            item(w);
    }
}

// A 16-byte row store: write-through (WT) or non-temporal.
template <bool WT>
__device__ __forceinline__ void store_row16(void *p, u32x4 v)
{
    if constexpr (WT)
        store16_wt(p, v);
    else
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(p));
}

// Bit of the rank owning expert id (experts are owned in contiguous blocks
// of epr), or 0 for an id outside [0, E).
__device__ __forceinline__ uint64_t owner_bit(const DispatchArgs &a, int id)
{
    if ((unsigned)id >= (unsigned)a.E)
        return 0ull;
    const unsigned r = a.epr_shift >= 0 ? (unsigned)id >> a.epr_shift : (unsigned)id / (unsigned)a.epr;
    return 1ull << r;
}

// Destination-rank mask of token q: bit r set when one of its k ids is an
// expert of rank r and rank r takes part in the step.  OR-ing the bits
// deduplicates tokens with several experts on one rank.  KQ > 0: the
// k = 4*KQ ids are read as KQ 16-byte vectors; KQ == 0: any k, all loads of
// the first 16 ids issued together.
template <int KQ>
__device__ __forceinline__ uint64_t route_mask(const DispatchArgs &a, int64_t q)
{
    const int32_t *__restrict__ idrow = a.ids + q * a.k;
    uint64_t m = 0;
    if constexpr (KQ > 0) {
        u32x4 v[KQ];
#pragma unroll
        for (int j = 0; j < KQ; ++j)
            v[j] = reinterpret_cast<const u32x4 *>(idrow)[j];
#pragma unroll
        for (int j = 0; j < KQ; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                m |= owner_bit(a, (int)v[j][e]);
    } else if (a.k <= 16) {
        int32_t id[16];
#pragma unroll
        for (int j = 0; j < 16; ++j)
            id[j] = j < a.k ? idrow[j] : -1;
#pragma unroll
        for (int j = 0; j < 16; ++j)
            m |= owner_bit(a, id[j]);
    } else {
        for (int j = 0; j < a.k; ++j)
            m |= owner_bit(a, idrow[j]);
    }
    return m & a.active; // masked-off ranks receive nothing
}

// Count of set bits of 'bits' in lanes below this one (v_mbcnt).
__device__ __forceinline__ int lanes_below(uint64_t bits)
{
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bits >> 32),
                                          __builtin_amdgcn_mbcnt_lo((uint32_t)bits, 0u));
}

// Copy one short row (a scale row) to every rank in mask, rank r's copy at
// dst0 + r * stride, one word W (16, 4 or 1 bytes) per thread access.
template <typename W>
__device__ __forceinline__ void copy_row_words(const uint8_t *src, int64_t nbytes, uint64_t mask,
                                               uint8_t *dst0, int64_t stride)
{
    const int64_t n = nbytes / (int64_t)sizeof(W);
    for (int64_t i = threadIdx.x; i < n; i += kBlock) {
        const W v = reinterpret_cast<const W *>(src)[i];
        uint64_t m = mask;
        while (m) {
            const int r = __builtin_ctzll(m);
            m &= m - 1;
            reinterpret_cast<W *>(dst0 + (int64_t)r * stride)[i] = v;
        }
    }
}

// copy_row_words with the widest word the row's size and alignment allow.
__device__ __forceinline__ void copy_row_any(const uint8_t *src, int64_t nbytes, uint64_t mask,
                                             uint8_t *dst0, int64_t stride)
{
    const uint64_t align = (uint64_t)(uintptr_t)src | (uint64_t)(uintptr_t)dst0 |
                           (uint64_t)stride | (uint64_t)nbytes;
    if ((align & 15) == 0)
        copy_row_words<uint4>(src, nbytes, mask, dst0, stride);
    else if ((align & 3) == 0)
        copy_row_words<uint32_t>(src, nbytes, mask, dst0, stride);
    else
        copy_row_words<uint8_t>(src, nbytes, mask, dst0, stride);
}

// Receive bookkeeping of destination rank r (and, when given, the EPLB
// statistics all-gather into its region): walks every source slot q in
// ascending order, kBlock * kScanUnroll slots per step (kScanUnroll per
// lane, all id rows loaded before any is tested); a wave ballot marks the
// slots whose token goes to r, v_mbcnt gives each one its rank inside the
// wave, and the per-wave totals in LDS give the step's exclusive prefix.  Produces the ascending
// list of valid slots, the per-source counts and their exclusive prefix
// (src_offsets[P] = rows received).
template <int KQ>
__device__ void scan_destination(const DispatchArgs &a, int r)
{
    __shared__ int wave_tot[kScanUnroll][kWaves];
    __shared__ int src_off[MOE_EP_MAX_RANKS + 1];
    if (!((a.active >> r) & 1u)) // a masked-off rank's region is left alone
        return;
    if (a.eplb) {
        // EPLB statistics all-gather: row s of rank r's [P][n] matrix is
        // live rank s's statistics
        int32_t *dst = reinterpret_cast<int32_t *>(a.ws + (int64_t)r * a.region + a.off_eplb);
        const int64_t nst = (int64_t)a.P * a.n_eplb;
        for (int64_t i = threadIdx.x; i < nst; i += kBlock)
            if ((a.active >> (i / a.n_eplb)) & 1u)
                dst[i] = a.eplb[i];
    }
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint8_t *region = a.ws + (int64_t)r * a.region;
    int32_t *slots = reinterpret_cast<int32_t *>(region + a.off_slots);
    const int64_t S = (int64_t)a.P * a.T;
    const uint64_t rbit = 1ull << r;
    const uint32_t lo = (uint32_t)(r * a.epr); // rank r owns experts [lo, lo + epr)
    int base = 0;
    for (int64_t c0 = 0; c0 < S; c0 += kBlock * kScanUnroll) {
        bool live[kScanUnroll];
        int src[kScanUnroll], tok[kScanUnroll];
#pragma unroll
        for (int u = 0; u < kScanUnroll; ++u) {
            const int64_t q = c0 + u * kBlock + tid;
            live[u] = false;
            src[u] = 0;
            tok[u] = -1;
            if (q < S) {
                const int s = (int)(q / a.T);
                const int t = (int)(q - (int64_t)s * a.T);
                src[u] = s;
                tok[u] = t;
                live[u] = t < a.n[s];
            }
        }
        int bit[kScanUnroll];
        if constexpr (KQ > 0) {
            u32x4 v[kScanUnroll][KQ];
            const u32x4 none = {~0u, ~0u, ~0u, ~0u}; // ids that no rank owns
#pragma unroll
            for (int u = 0; u < kScanUnroll; ++u)
#pragma unroll
                for (int j = 0; j < KQ; ++j)
                    v[u][j] = live[u] ? reinterpret_cast<const u32x4 *>(
                                            a.ids + (c0 + u * kBlock + tid) * a.k)[j]
                                      : none;
#pragma unroll
            for (int u = 0; u < kScanUnroll; ++u) {
                bool hit = false;
#pragma unroll
                for (int j = 0; j < KQ; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        hit |= v[u][j][e] - lo < (uint32_t)a.epr;
                bit[u] = live[u] && hit;
            }
        } else {
#pragma unroll
            for (int u = 0; u < kScanUnroll; ++u)
                bit[u] = live[u] && (route_mask<0>(a, c0 + u * kBlock + tid) & rbit);
        }
        uint64_t bal[kScanUnroll];
#pragma unroll
        for (int u = 0; u < kScanUnroll; ++u)
            bal[u] = __ballot(bit[u]);
        if (lane == 0) {
#pragma unroll
            for (int u = 0; u < kScanUnroll; ++u)
                wave_tot[u][wave] = __popcll(bal[u]);
        }
        __syncthreads();
        int running = base;
#pragma unroll
        for (int u = 0; u < kScanUnroll; ++u) {
            int mine = 0;
            for (int w = 0; w < kWaves; ++w) {
                if (w == wave)
                    mine = running;
                running += wave_tot[u][w];
            }
            const int pos = mine + lanes_below(bal[u]);
            if (bit[u])
                slots[pos] = (int32_t)(c0 + u * kBlock + tid);
            if (tok[u] == 0)
                src_off[src[u]] = pos;
        }
        base = running;
        __syncthreads();
    }
    if (tid == 0)
        src_off[a.P] = base;
    __syncthreads();
    int32_t *counts = reinterpret_cast<int32_t *>(region + a.off_counts);
    int32_t *offs = reinterpret_cast<int32_t *>(region + a.off_src_offsets);
    for (int i = tid; i <= a.P; i += kBlock) {
        offs[i] = src_off[i];
        if (i < a.P)
            counts[i] = src_off[i + 1] - src_off[i];
    }
}

// Id and weight planes of destinations [r0, r1) for slots
// [c*kPlaneSlots, ...), in two phases.  First each lane computes one slot's
// destination mask into LDS (the items of the first destination group also
// store every token's mask in its source rank's region, for combine).  Then
// the block walks the chunk's id rows in 16-byte units (KQ > 0) or words,
// each unit read once (only for tokens that go somewhere) and stored to
// every live destination of the group: a slot whose token goes to r gets
// the token's ids and weights, every other slot k copies of invalid_id.
// Consecutive lanes write consecutive units.
template <int KQ>
__device__ void write_id_planes(const DispatchArgs &a, int r0, int r1, int64_t c)
{
    __shared__ uint64_t smask[kPlaneSlots];
    const int64_t S = (int64_t)a.P * a.T;
    const int64_t q0 = c * kPlaneSlots;
    const int nslot = (int)min<int64_t>(kPlaneSlots, S - q0);
    if ((int)threadIdx.x < nslot) {
        const int64_t q = q0 + threadIdx.x;
        const int s = (int)(q / a.T);
        const int t = (int)(q - (int64_t)s * a.T);
        const uint64_t mask = t < a.n[s] ? route_mask<KQ>(a, q) : 0ull;
        smask[threadIdx.x] = mask;
        if (r0 == 0 && ((a.active >> s) & 1u))
            *reinterpret_cast<uint64_t *>(a.ws + (int64_t)s * a.region + a.off_masks +
                                          (int64_t)t * 8) = mask;
    }
    __syncthreads();
    if constexpr (KQ > 0) {
        const u32x4 *__restrict__ ids_in = reinterpret_cast<const u32x4 *>(a.ids) + q0 * KQ;
        const u32x4 *__restrict__ w_in =
            a.weights ? reinterpret_cast<const u32x4 *>(a.weights) + q0 * KQ : nullptr;
        const uint32_t inv = (uint32_t)a.invalid_id;
        const u32x4 marker = {inv, inv, inv, inv};
        const int nunits = nslot * KQ;
        for (int e = threadIdx.x; e < nunits; e += kBlock) {
            const uint64_t mk = smask[e / KQ];
            const u32x4 idv = mk ? ids_in[e] : marker;
            const u32x4 wv = (mk && w_in) ? w_in[e] : marker;
            for (int r = r0; r < r1; ++r) {
                if (!((a.active >> r) & 1u))
                    continue;
                uint8_t *reg = a.ws + (int64_t)r * a.region;
                const bool go = (mk >> r) & 1u;
                reinterpret_cast<u32x4 *>(reg + a.off_ids)[q0 * KQ + e] = go ? idv : marker;
                if (go && w_in)
                    reinterpret_cast<u32x4 *>(reg + a.off_weights)[q0 * KQ + e] = wv;
            }
        }
    } else {
        const int32_t *__restrict__ ids_in = a.ids + q0 * a.k;
        const float *__restrict__ w_in = a.weights ? a.weights + q0 * a.k : nullptr;
        const int nwords = nslot * a.k;
        for (int e = threadIdx.x; e < nwords; e += kBlock) {
            const uint64_t mk = smask[e / a.k];
            const int32_t idv = mk ? ids_in[e] : a.invalid_id;
            const float wv = (mk && w_in) ? w_in[e] : 0.0f;
            for (int r = r0; r < r1; ++r) {
                if (!((a.active >> r) & 1u))
                    continue;
                uint8_t *reg = a.ws + (int64_t)r * a.region;
                const bool go = (mk >> r) & 1u;
                reinterpret_cast<int32_t *>(reg + a.off_ids)[q0 * a.k + e] = go ? idv : a.invalid_id;
                if (go && w_in)
                    reinterpret_cast<float *>(reg + a.off_weights)[q0 * a.k + e] = wv;
            }
        }
    }
    __syncthreads(); // smask is reused by the block's next item
}

// True when a side row (scale or extra bytes) of nbytes per token can travel
// with chunk 0's payload loads: one aligned 16-byte word per lane, at most
// kBlock words.
__host__ __device__ __forceinline__ bool side_row_fits(const uint8_t *src, int64_t nbytes, int64_t plane_off,
                                              int64_t region)
{
    return nbytes && (nbytes >> 4) <= kBlock &&
           (((uint64_t)(uintptr_t)src | (uint64_t)nbytes | (uint64_t)plane_off | (uint64_t)region) & 15) == 0;
}

// Chunk c of token q's payload row (DV 16-byte vectors per thread, lane
// strided), read once and stored to every destination in the token's mask;
// chunk 0 also carries the scale row and the extra payload row (each loaded
// with the payload vectors when it is at most 256 aligned 16-byte words,
// else copied after them).  PF: the
// row loads go out before the id loads of the mask, so the two latencies
// overlap (a row whose token goes nowhere is then read for nothing); that
// pays in steps of few workgroups and costs in large ones.  WT: payload rows
// are stored write-through, else non-temporally (scale rows always the
// latter).  XF: the launch's extra rows fit side_row_fits (a separate
// instance, as the fused path costs registers where there are none).
template <int KQ, int DV, bool PF, bool WT, bool XF>
__device__ void scatter_chunk(const DispatchArgs &a, int64_t q, int64_t c)
{
    const int s = (int)(q / a.T);
    const int t = (int)(q - (int64_t)s * a.T);
    if (t >= a.n[s])
        return;
    uint64_t mask = 0;
    if (!PF) {
        mask = route_mask<KQ>(a, q);
        if (!mask)
            return;
    }
    const int64_t nvec = a.row_bytes >> 4;
    const int64_t i0 = c * (kBlock * DV) + threadIdx.x;
    const uint8_t *src = a.payload + q * a.row_bytes;
    uint8_t *dst0 = a.ws + a.off_payload + q * a.row_bytes;
    u32x4 v[DV];
#pragma unroll
    for (int u = 0; u < DV; ++u)
        if (i0 + u * kBlock < nvec)
            v[u] = *reinterpret_cast<const u32x4 *>(src + (i0 + u * kBlock) * 16);
    const bool sc_vec = c == 0 && side_row_fits(a.scales, a.srow_bytes, a.off_scales, a.region);
    const bool x_vec = XF && c == 0;
    const bool sc_lane = sc_vec && (int64_t)threadIdx.x < (a.srow_bytes >> 4);
    const bool x_lane = x_vec && (int64_t)threadIdx.x < (a.xrow_bytes >> 4);
    u32x4 sv = {0u, 0u, 0u, 0u}, xv = {0u, 0u, 0u, 0u};
    if (sc_lane)
        sv = *reinterpret_cast<const u32x4 *>(a.scales + q * a.srow_bytes + threadIdx.x * 16);
    if constexpr (XF)
        if (x_lane)
            xv = *reinterpret_cast<const u32x4 *>(a.extra + q * a.xrow_bytes + threadIdx.x * 16);
    if (PF) {
        mask = route_mask<KQ>(a, q);
        if (!mask)
            return;
    }
    uint64_t m = mask;
    while (m) {
        const int r = __builtin_ctzll(m);
        m &= m - 1;
        uint8_t *d = dst0 + (int64_t)r * a.region;
#pragma unroll
        for (int u = 0; u < DV; ++u)
            if (i0 + u * kBlock < nvec)
                store_row16<WT>(d + (i0 + u * kBlock) * 16, v[u]);
        if (sc_lane)
            store_row16<false>(a.ws + a.off_scales + (int64_t)r * a.region + q * a.srow_bytes + threadIdx.x * 16, sv);
        if constexpr (XF)
            if (x_lane)
                store_row16<false>(a.ws + a.off_extra + (int64_t)r * a.region + q * a.xrow_bytes + threadIdx.x * 16,
                                   xv);
    }
    if (c == 0 && a.srow_bytes && !sc_vec)
        copy_row_any(a.scales + q * a.srow_bytes, a.srow_bytes, mask,
                     a.ws + a.off_scales + q * a.srow_bytes, a.region);
    if (c == 0 && a.xrow_bytes && !x_vec)
        copy_row_any(a.extra + q * a.xrow_bytes, a.xrow_bytes, mask,
                     a.ws + a.off_extra + q * a.xrow_bytes, a.region);
}

// One launch, three block roles touching disjoint memory:
//   [0, P)                    receive bookkeeping of destination r
//   [P, P + plane_blocks)     id / weight planes, (destination group, slot chunk) items
//   [P + plane_blocks, grid)  payload scatter, (token, row chunk) items
// except in launches of long rows that do not prefetch, where the id-plane
// blocks come last (EP64 BF16 dispatch -2%; in prefetching launches the
// id-plane work then trails the short payload scatter: EP8 / MXFP8 +12%).
// The last two roles loop over their items when there are more items than
// blocks.  KQ: id rows of k = 4*KQ ids read as 16-byte vectors (0: any k);
// DV: 16-byte vectors per thread in a payload row chunk; PF: row loads
// before the mask, WT: write-through payload stores, XF: extra rows loaded
// with the payload (scatter_chunk).
template <int KQ, int DV, bool PF, bool WT, bool XF>
__global__ __launch_bounds__(kBlock) void dispatch_kernel(DispatchArgs a, int64_t nplane,
                                                          int64_t plane_blocks, int64_t nchunk)
{
    const int64_t b = blockIdx.x;
    if (b < a.P) {
        scan_destination<KQ>(a, (int)b);
        return;
    }
    constexpr bool plane_last = !PF && DV == MOE_EP_DISPATCH_VPT_LONG;
    const int64_t npay = (int64_t)gridDim.x - a.P - plane_blocks; // payload blocks
    const int64_t plane0 = plane_last ? a.P + npay : a.P;         // first id-plane block
    if (b >= plane0 && b < plane0 + plane_blocks) {
        const int ngroups = (a.P + kPlaneGroup - 1) / kPlaneGroup;
        for (int64_t w = b - plane0; w < (int64_t)ngroups * nplane; w += plane_blocks) {
            const int g = (int)(w / nplane);
            write_id_planes<KQ>(a, g * kPlaneGroup, min(a.P, (g + 1) * kPlaneGroup), w % nplane);
        }
        return;
    }
    const int64_t S = (int64_t)a.P * a.T;
    const int64_t first = plane_last ? a.P : a.P + plane_blocks; // first payload block
    // A prefetching launch has a workgroup for every payload item.  With long
    // rows each one runs its item without a loop, so the token's ids come in
    // one scalar load (EP8 dispatch -1%); short rows keep the loop (the
    // one-item form cost the MXFP8 dispatch 2-3%).
    static_assert(MOE_EP_PREFETCH_ITEMS <= MOE_EP_SCATTER_GRID && MOE_EP_PREFETCH_ITEMS <= kGridCap,
                  "prefetching launches need one workgroup per item");
    constexpr bool one = PF && DV == MOE_EP_DISPATCH_VPT_LONG;
    if constexpr (one) {
        const int64_t w = b - first;
        if (w < S * nchunk)
            scatter_chunk<KQ, DV, PF, WT, XF>(a, w / nchunk, w % nchunk);
        return;
    }
    for (int64_t w = b - first; w < S * nchunk; w += npay)
        scatter_chunk<KQ, DV, PF, WT, XF>(a, w / nchunk, w % nchunk);
}

__device__ __forceinline__ void add_bf16x8(float (&acc)[8], u32x4 v)
{
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        float lo, hi;
        unpack_bf16x2(v[e], lo, hi);
        acc[2 * e] += lo;
        acc[2 * e + 1] += hi;
    }
}

// BF16 combine: item (token q = s*T + t, row chunk c of BS*VPT vectors,
// BS threads per workgroup); each thread owns
// VPT 16-byte vectors (8 bf16 each) of the output row and sums, in fp32 and
// ascending rank order, those vectors of row q of every rank in the token's
// mask.  Expert-output rows are read once (non-temporal loads); the loads
// of up to G ranks are issued before any is consumed.
template <int BS, int VPT, int G, bool WT>
__device__ __forceinline__ void combine_bf16_item(const CombineArgs &a, int64_t w, int64_t nchunk)
{
    const int64_t S = (int64_t)a.P * a.T;
    const int64_t rank_bytes = S * a.H * 2;
    const int64_t nvec = a.H >> 3;
    const int64_t q = w / nchunk, c = w % nchunk;
    const int s = (int)(q / a.T);
    const int t = (int)(q - (int64_t)s * a.T);
    const int64_t i0 = c * (BS * VPT) + threadIdx.x;
    if (t >= a.n[s] || i0 >= nvec)
        return;
    const uint64_t mask = *reinterpret_cast<const uint64_t *>(
        a.ws + (int64_t)s * a.region + a.off_masks + (int64_t)t * 8);
    const uint8_t *src = reinterpret_cast<const uint8_t *>(a.eo) + q * a.H * 2 + i0 * 16;
    bool in[VPT];
#pragma unroll
    for (int u = 0; u < VPT; ++u)
        in[u] = i0 + u * BS < nvec;
    float acc[VPT][8];
#pragma unroll
    for (int u = 0; u < VPT; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            acc[u][e] = 0.0f;
    uint64_t m = mask;
    while (m) {
        int r[G];
        int cnt = 0;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            r[g] = 0;
            if (m) {
                r[g] = __builtin_ctzll(m);
                m &= m - 1;
                cnt = g + 1;
            }
        }
        u32x4 v[G][VPT];
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int u = 0; u < VPT; ++u)
                if (g < cnt && in[u])
                    v[g][u] = load16_nt(src + (int64_t)r[g] * rank_bytes + u * BS * 16);
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int u = 0; u < VPT; ++u)
                if (g < cnt && in[u])
                    add_bf16x8(acc[u], v[g][u]);
    }
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
        if (!in[u])
            continue;
        u32x4 o;
        o[0] = pack_bf16x2(acc[u][0], acc[u][1]);
        o[1] = pack_bf16x2(acc[u][2], acc[u][3]);
        o[2] = pack_bf16x2(acc[u][4], acc[u][5]);
        o[3] = pack_bf16x2(acc[u][6], acc[u][7]);
        store_row16<WT>(a.out + q * a.H + (i0 + u * BS) * 8, o);
    }
}

template <int BS, int VPT, int G, bool WT, bool ONE>
__global__ __launch_bounds__(BS) void combine_bf16_kernel(CombineArgs a, int64_t nchunk)
{
    for_each_item<ONE>((int64_t)a.P * a.T * nchunk,
                       [&](int64_t w) { combine_bf16_item<BS, VPT, G, WT>(a, w, nchunk); });
}

// e4m3 codes (two words, element 0 in the lowest byte) and e8m0 scale code
// of one 8-element quarter of a 32-element block; the block's four quarters
// sit in four consecutive lanes (lane & ~3 .. lane | 3), which exchange
// their amax.  A block holding a NaN or an infinity gets scale 0xFF and
// codes 0x7F.  All lanes of the wave must call this together (shuffles).
__device__ __forceinline__ void quantise8(u32x4 x, uint32_t &c0, uint32_t &c1, uint32_t &scale_code)
{
    uint32_t amax = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        amax = max(amax, x[e] & 0x7FFFu);
        amax = max(amax, (x[e] >> 16) & 0x7FFFu);
    }
    amax = max(amax, (uint32_t)__shfl_xor((int)amax, 1));
    amax = max(amax, (uint32_t)__shfl_xor((int)amax, 2));
    if (amax >= 0x7F80u) {
        scale_code = 0xFFu;
        c0 = c1 = 0x7F7F7F7Fu;
        return;
    }
    const int ex = fp8_block_exponent(amax);
    scale_code = (uint32_t)(ex + 127);
    // v_cvt_scalef32_pk_fp8_f32 converts x / scale to e4m3 (round to nearest
    // even) for two values, first operand in the lower byte, into the low or
    // high half of a word.  With scale = 2^ex every |x / scale| is within
    // 448, so no saturation is reached; its results equal those of scaling
    // by 2^-ex first and then converting, for every bf16 value and exponent.
    const float scale = __builtin_amdgcn_ldexpf(1.0f, ex);
    uint32_t c[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const uint32_t w0 = x[2 * j], w1 = x[2 * j + 1];
        v2i16 p = {0, 0};
        p = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(p, __uint_as_float(w0 << 16),
                                                     __uint_as_float(w0 & 0xFFFF0000u), scale, false);
        p = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(p, __uint_as_float(w1 << 16),
                                                     __uint_as_float(w1 & 0xFFFF0000u), scale, true);
        c[j] = __builtin_bit_cast(uint32_t, p);
    }
    c0 = c[0];
    c1 = c[1];
}

// FP8 combine, sending side: item (token q = s*T + t, chunk c of BS * 16
// elements, BS threads per workgroup).  Every rank r that holds the token
// quantises its row q (e4m3fn, one e8m0 scale per 32 elements) into source
// rank s's landing plane at slot r*T + t; the rows of up to G ranks are
// loaded before any is quantised.
// Each lane owns 8 elements in each half of the chunk (elements
// c*BS*16 + h*BS*8 + lane*8 ..), so every load instruction of a wave covers
// 1 KB of a row without gaps; four lanes share a block.  WT: the codes are
// stored write-through (launches with few landing bytes), else cached.
template <int BS, int G, bool WT>
__device__ __forceinline__ void fp8_quant_item(const CombineArgs &a, int64_t w, int64_t nchunk)
{
    const int64_t S = (int64_t)a.P * a.T;
    const int64_t rank_bytes = S * a.H * 2;
    const int64_t q = w / nchunk, c = w % nchunk;
    const int s = (int)(q / a.T);
    const int t = (int)(q - (int64_t)s * a.T);
    if (t >= a.n[s])
        return;
    int64_t e[2];
    bool act[2]; // H % 32 == 0: the four lanes of a block agree
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        e[h] = c * (BS * 16) + h * (BS * 8) + threadIdx.x * 8;
        act[h] = e[h] < a.H;
    }
    const uint64_t mask = *reinterpret_cast<const uint64_t *>(a.ws + (int64_t)s * a.region + a.off_masks +
                                                              (int64_t)t * 8);
    uint8_t *land = a.land + (int64_t)s * a.land_stride;
    const uint8_t *src = reinterpret_cast<const uint8_t *>(a.eo) + q * a.H * 2;
    uint64_t m = mask;
    while (m) {
        int r[G];
        int cnt = 0;
#pragma unroll
        for (int u = 0; u < G; ++u) {
            r[u] = 0;
            if (m) {
                r[u] = __builtin_ctzll(m);
                m &= m - 1;
                cnt = u + 1;
            }
        }
        u32x4 x[G][2];
#pragma unroll
        for (int u = 0; u < G; ++u)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                x[u][h] = (act[h] && u < cnt) ? load16_nt(src + (int64_t)r[u] * rank_bytes + e[h] * 2)
                                              : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int u = 0; u < G; ++u) {
            if (u >= cnt)
                break;
            const int64_t slot = (int64_t)r[u] * a.T + t;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                uint32_t c0, c1, sc;
                quantise8(x[u][h], c0, c1, sc);
                if (act[h]) {
                    if constexpr (WT)
                        store8_wt(land + a.off_land_codes + slot * a.H + e[h], u32x2{c0, c1});
                    else
                        *reinterpret_cast<u32x2 *>(land + a.off_land_codes + slot * a.H + e[h]) =
                            u32x2{c0, c1};
                    if ((threadIdx.x & 3) == 0)
                        land[a.off_land_scales + slot * (a.H >> 5) + (e[h] >> 5)] = (uint8_t)sc;
                }
            }
        }
    }
}

// Looping over items (no one-item launches): on the MXFP8 workload the
// one-item form made both FP8 kernels 1-3% slower.
template <int BS, int G, bool WT>
__global__ __launch_bounds__(BS) void combine_fp8_quant_kernel(CombineArgs a, int64_t nchunk)
{
    for_each_item<false>((int64_t)a.P * a.T * nchunk,
                         [&](int64_t w) { fp8_quant_item<BS, G, WT>(a, w, nchunk); });
}

// FP8 combine, receiving side: item (token q = s*T + t, chunk c of BS * 16
// elements, the quantising side's lane layout).  Each lane dequantises its
// 8 elements in each half of the chunk from the landing rows r*T + t of every
// rank r in the token's mask (codes of up to G ranks loaded at once), sums
// them in fp32 in ascending rank order, rounds to bf16 and stores the output
// non-temporally (it is not read again in the step).
template <int BS, int G>
__device__ __forceinline__ void fp8_gather_item(const CombineArgs &a, int64_t w, int64_t nchunk)
{
    const int64_t q = w / nchunk, c = w % nchunk;
    const int s = (int)(q / a.T);
    const int t = (int)(q - (int64_t)s * a.T);
    int64_t e[2];
    bool act[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        e[h] = c * (BS * 16) + h * (BS * 8) + threadIdx.x * 8;
        act[h] = e[h] < a.H;
    }
    if (t >= a.n[s] || !act[0])
        return;
    const uint64_t mask = *reinterpret_cast<const uint64_t *>(a.ws + (int64_t)s * a.region + a.off_masks +
                                                              (int64_t)t * 8);
    const uint8_t *land = a.land + (int64_t)s * a.land_stride;
    float acc[2][8];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < 8; ++j)
            acc[h][j] = 0.0f;
    uint64_t m = mask;
    while (m) {
        int r[G];
        int cnt = 0;
#pragma unroll
        for (int u = 0; u < G; ++u) {
            r[u] = 0;
            if (m) {
                r[u] = __builtin_ctzll(m);
                m &= m - 1;
                cnt = u + 1;
            }
        }
        u32x2 cv[G][2];
        uint32_t sc[G][2];
#pragma unroll
        for (int u = 0; u < G; ++u) {
            if (u < cnt) {
                const int64_t slot = (int64_t)r[u] * a.T + t;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    if (act[h]) {
                        cv[u][h] = __builtin_nontemporal_load(
                            reinterpret_cast<const u32x2 *>(land + a.off_land_codes + slot * a.H + e[h]));
                        sc[u][h] = land[a.off_land_scales + slot * (a.H >> 5) + (e[h] >> 5)];
                    }
                }
            }
        }
#pragma unroll
        for (int u = 0; u < G; ++u) {
            if (u >= cnt)
                break;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                if (!act[h])
                    continue;
                if (sc[u][h] == 0xFFu) {
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        acc[h][j] = __uint_as_float(0x7FC00000u);
                    continue;
                }
                // v_cvt_scalef32_pk_f32_fp8 decodes two codes (low byte
                // first) and multiplies them by the scale 2^(sc - 127),
                // exactly, subnormal scales included
                const float scale = __builtin_amdgcn_ldexpf(1.0f, (int)sc[u][h] - 127);
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const f32x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((int)cv[u][h][j], scale, false);
                    const f32x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((int)cv[u][h][j], scale, true);
                    acc[h][4 * j] += lo[0];
                    acc[h][4 * j + 1] += lo[1];
                    acc[h][4 * j + 2] += hi[0];
                    acc[h][4 * j + 3] += hi[1];
                }
            }
        }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        if (!act[h])
            continue;
        u32x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            o[j] = pack_bf16x2(acc[h][2 * j], acc[h][2 * j + 1]);
        store_row16<false>(a.out + q * a.H + e[h], o);
    }
}

template <int BS, int G>
__global__ __launch_bounds__(BS) void combine_fp8_gather_kernel(CombineArgs a, int64_t nchunk)
{
    for_each_item<false>((int64_t)a.P * a.T * nchunk,
                         [&](int64_t w) { fp8_gather_item<BS, G>(a, w, nchunk); });
}

// Grid of nitems workgroups capped at 64 rounds of the chip (256 CUs x 8
// resident workgroups); kernels loop over the rest.
inline int64_t grid_for(int64_t nitems)
{
    return nitems < 1 ? 1 : (nitems < kGridCap ? nitems : kGridCap);
}

inline int64_t ceil_div(int64_t x, int64_t y) { return (x + y - 1) / y; }

} // namespace

template <int KQ, int DV, bool PF, bool WT>
static void launch_dispatch_xf(const DispatchArgs &a, bool xf, dim3 g, int64_t nplane, int64_t plane_blocks,
                               int64_t nchunk, hipStream_t s)
{
    if (xf)
        hipLaunchKernelGGL((dispatch_kernel<KQ, DV, PF, WT, true>), g, dim3(kBlock), 0, s, a, nplane,
                           plane_blocks, nchunk);
    else
        hipLaunchKernelGGL((dispatch_kernel<KQ, DV, PF, WT, false>), g, dim3(kBlock), 0, s, a, nplane,
                           plane_blocks, nchunk);
}

template <int KQ>
static hipError_t launch_dispatch_kq(const DispatchArgs &a, hipStream_t s)
{
    const int64_t S = (int64_t)a.P * a.T;
    const int64_t nplane = ceil_div(S, kPlaneSlots);
    int64_t plane_blocks = grid_for(ceil_div(a.P, kPlaneGroup) * nplane);
    const bool long_rows = a.row_bytes >= MOE_EP_DISPATCH_LONG_ROW;
    const int dv = long_rows ? MOE_EP_DISPATCH_VPT_LONG : MOE_EP_DISPATCH_VPT_SHORT;
    int64_t nchunk = ceil_div(a.row_bytes >> 4, (int64_t)kBlock * dv);
    const bool pf = S * nchunk <= MOE_EP_PREFETCH_ITEMS;
    const bool mid = !long_rows && !pf && nchunk > 1; // short rows of several chunks, large launch
    if (mid)
        nchunk = ceil_div(a.row_bytes >> 4, (int64_t)kBlock * MOE_EP_DISPATCH_VPT_MID);
    int64_t N = 0;
    for (int i = 0; i < a.P; ++i)
        N += a.n[i];
    // Short-row launches that do not prefetch run their id-plane blocks
    // first.  When the id planes are a small share of the launch's bytes,
    // fewer such blocks (each looping over several items) leave the early
    // slots to the payload scatter: EP64 NVFP4 dispatch -6% with 128 or 64
    // blocks instead of 1024; with 32 the id planes become the straggler.
    if (!pf && !long_rows) {
        const int64_t plane_bytes = S * a.P * 4 * a.k;
        const int64_t payload_bytes = N * std::min(a.P, a.k) * (a.row_bytes + a.srow_bytes);
        if (plane_bytes * 10 < payload_bytes)
            plane_blocks = std::min<int64_t>(plane_blocks, 128);
    }
    const int64_t grid =
        a.P + plane_blocks + std::min<int64_t>(grid_for(S * nchunk), MOE_EP_SCATTER_GRID);
    // write-through payload stores: long rows only, and a bound on the
    // payload bytes written (each token goes to at most min(P, k) ranks)
    const bool wt = long_rows && N * std::min(a.P, a.k) * a.row_bytes <= MOE_EP_WT_BYTES;
    // extra rows that fit one word per lane travel with the payload loads
    const bool xf = side_row_fits(a.extra, a.xrow_bytes, a.off_extra, a.region);
    const dim3 g((unsigned)grid);
    constexpr int L = MOE_EP_DISPATCH_VPT_LONG, Sh = MOE_EP_DISPATCH_VPT_SHORT, Md = MOE_EP_DISPATCH_VPT_MID;
    if (long_rows && pf && wt)
        launch_dispatch_xf<KQ, L, true, true>(a, xf, g, nplane, plane_blocks, nchunk, s);
    else if (long_rows && pf)
        launch_dispatch_xf<KQ, L, true, false>(a, xf, g, nplane, plane_blocks, nchunk, s);
    else if (long_rows && wt)
        launch_dispatch_xf<KQ, L, false, true>(a, xf, g, nplane, plane_blocks, nchunk, s);
    else if (long_rows)
        launch_dispatch_xf<KQ, L, false, false>(a, xf, g, nplane, plane_blocks, nchunk, s);
    else if (pf)
        launch_dispatch_xf<KQ, Sh, true, false>(a, xf, g, nplane, plane_blocks, nchunk, s);
    else if (mid)
        launch_dispatch_xf<KQ, Md, false, false>(a, xf, g, nplane, plane_blocks, nchunk, s);
    else
        launch_dispatch_xf<KQ, Sh, false, false>(a, xf, g, nplane, plane_blocks, nchunk, s);
    return hipGetLastError();
}

hipError_t launch_dispatch(const DispatchArgs &a, hipStream_t s)
{
    // id rows of 4, 8 or 16 ids with 16-byte aligned id / weight planes move
    // as 16-byte vectors; anything else takes the word path
    const bool al = ((uintptr_t)a.ids & 15) == 0 && ((uintptr_t)a.weights & 15) == 0;
    if (al && a.k == 8)
        return launch_dispatch_kq<2>(a, s);
    if (al && a.k == 4)
        return launch_dispatch_kq<1>(a, s);
    if (al && a.k == 16)
        return launch_dispatch_kq<4>(a, s);
    return launch_dispatch_kq<0>(a, s);
}

template <int BS, int VPT, int G, bool WT>
static hipError_t launch_combine_shape(const CombineArgs &a, hipStream_t s)
{
    const int64_t nchunk = ceil_div((int64_t)a.H >> 3, BS * VPT);
    const int64_t items = (int64_t)a.P * a.T * nchunk;
    const dim3 grid((unsigned)std::max<int64_t>(1, std::min<int64_t>(items, MOE_EP_COMBINE_GRID_CAP)));
    if ((int64_t)grid.x == items)
        hipLaunchKernelGGL((combine_bf16_kernel<BS, VPT, G, WT, true>), grid, dim3(BS), 0, s, a, nchunk);
    else
        hipLaunchKernelGGL((combine_bf16_kernel<BS, VPT, G, WT, false>), grid, dim3(BS), 0, s, a, nchunk);
    return hipGetLastError();
}

hipError_t launch_combine_bf16(const CombineArgs &a, hipStream_t s)
{
    const int64_t out_bytes = (int64_t)a.P * a.T * a.H * 2;
    const bool wt = out_bytes <= MOE_EP_WT_BYTES;
    if (out_bytes >= MOE_EP_COMBINE_LARGE_BYTES)
        return wt ? launch_combine_shape<MOE_EP_COMBINE_LARGE_BLOCK, MOE_EP_COMBINE_LARGE, true>(a, s)
                  : launch_combine_shape<MOE_EP_COMBINE_LARGE_BLOCK, MOE_EP_COMBINE_LARGE, false>(a, s);
    return wt ? launch_combine_shape<MOE_EP_COMBINE_SMALL_BLOCK, MOE_EP_COMBINE_SMALL, true>(a, s)
              : launch_combine_shape<MOE_EP_COMBINE_SMALL_BLOCK, MOE_EP_COMBINE_SMALL, false>(a, s);
}

template <int BS>
static hipError_t launch_combine_fp8_bs(const CombineArgs &a, hipStream_t s)
{
    const int64_t nchunk = ceil_div((int64_t)a.H >> 4, BS);
    const dim3 grid((unsigned)grid_for((int64_t)a.P * a.T * nchunk));
    // the quantise pass writes at most P landing rows per token; the landing
    // codes are written through L2 when that bound is small
    int64_t N = 0;
    for (int i = 0; i < a.P; ++i)
        N += a.n[i];
    const int64_t land_row = (int64_t)a.H + (a.H >> 5);
    if (N * a.P * land_row <= MOE_EP_WT_BYTES)
        hipLaunchKernelGGL((combine_fp8_quant_kernel<BS, MOE_EP_FP8_GATHER, true>), grid, dim3(BS), 0, s, a,
                           nchunk);
    else
        hipLaunchKernelGGL((combine_fp8_quant_kernel<BS, MOE_EP_FP8_GATHER, false>), grid, dim3(BS), 0, s, a,
                           nchunk);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL((combine_fp8_gather_kernel<BS, MOE_EP_FP8_GATHER>), grid, dim3(BS), 0, s, a, nchunk);
    return hipGetLastError();
}

// Workgroup size of the FP8 combine kernels: a workgroup covers BS * 16
// elements of a row, so pick the size that cuts the row into whole chunks
// (H = 7168: one chunk of 448 threads; 256-thread chunks leave half of the
// second one idle).  MXFP8 workload, FP8 combine with 448 / 64 / 128 / 256
// threads: 66.8 / 67.5 / 70.3 / 69.7 us.
hipError_t launch_combine_fp8(const CombineArgs &a, hipStream_t s)
{
    const int64_t units = a.H >> 4; // 16-element units of a row (H % 32 == 0)
    if (units % 448 == 0)
        return launch_combine_fp8_bs<448>(a, s);
    if (units % 256 == 0)
        return launch_combine_fp8_bs<256>(a, s);
    if (units % 64 == 0)
        return launch_combine_fp8_bs<64>(a, s);
    return launch_combine_fp8_bs<256>(a, s);
}

// The library's staging array for callers that cannot allocate: the FP8
// combine landing planes of moe_ep_combine_noalloc.  File scope, so every
// GPU the library runs on holds one copy from module load until the process
// ends.  In host code its name is a host-side stand-in, not a device
// address: kernels get the address static_scratch() looked up.
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices]; // per device, looked up once with that device current
} // namespace

hipError_t static_scratch(void **ptr)
{
    *ptr = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

} // namespace moe_ep
