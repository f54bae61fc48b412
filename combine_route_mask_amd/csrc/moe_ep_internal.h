// Kernel argument blocks and launchers shared by the host library and the
// gfx950 kernels.  Kernel arguments are passed by value (a few hundred
// bytes), so one launch needs no device-side descriptor.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_ep.h"

namespace moe_ep {

constexpr int kBlock = 256;          // threads per workgroup (4 wave64)
constexpr int kMaxPlanes = 8;

// Byte offsets of one rank's planes inside its workspace region.
struct Layout {
    int64_t region;                  // size_per_rank
    int64_t payload, scales, extra, ids, weights, slots, counts, src_offsets, masks, eplb;
    int64_t land_codes, land_scales; // FP8 combine landing plane, -1 if absent
    int64_t row_bytes, srow_bytes, xrow_bytes; // payload / scale / extra row bytes
    int64_t total;                   // bytes needed per region
};

struct DispatchArgs {
    const uint8_t *payload;          // [P][T][row_bytes]
    const uint8_t *scales;           // [P][T][srow_bytes] or null
    const uint8_t *extra;            // [P][T][xrow_bytes] or null
    const int32_t *eplb;             // [P][n_eplb] or null
    const int32_t *ids;              // [P][T][k]
    const float *weights;            // [P][T][k] or null
    uint8_t *ws;                     // region r at ws + r * region
    int64_t region;
    int64_t off_payload, off_scales, off_extra, off_ids, off_weights, off_slots, off_counts,
        off_src_offsets, off_masks, off_eplb;
    int64_t row_bytes, srow_bytes, xrow_bytes;
    int32_t P, T, k, E, epr, invalid_id, n_eplb;
    int32_t epr_shift;               // log2(epr) when epr is a power of two, else -1
    uint64_t active;                 // bit r: rank r takes part in the step
    int32_t n[MOE_EP_MAX_RANKS];     // local token counts (0 for masked-off ranks)
};

struct CombineArgs {
    const uint16_t *eo;              // [P][P*T][H] bf16
    uint16_t *out;                   // [P][T][H] bf16
    uint8_t *ws;                     // token masks of source s at ws + s * region + off_masks
    int64_t region, off_masks;
    uint8_t *land;                   // FP8 landing planes of source s at land + s * land_stride
    int64_t land_stride, off_land_codes, off_land_scales;
    int32_t P, T, H;
    int32_t n[MOE_EP_MAX_RANKS];
};

struct AgPlane {
    const uint8_t *in;
    int64_t in_stride;
    uint8_t *out;
    int64_t out_stride;
    int64_t row_bytes;
};

struct AllGatherArgs {
    AgPlane pl[kMaxPlanes];
    int32_t nplanes, P;
    int32_t off[MOE_EP_MAX_RANKS + 1]; // exclusive prefix of sizes
};

struct ReduceScatterArgs {
    const uint16_t *in;              // rank q at in + q * in_stride (elements)
    int64_t in_stride;
    uint16_t *out;                   // rank r at out + r * out_stride (elements)
    int64_t out_stride;
    int32_t P, H;
    int32_t off[MOE_EP_MAX_RANKS + 1];
};

hipError_t launch_dispatch(const DispatchArgs &a, hipStream_t s);
hipError_t launch_combine_bf16(const CombineArgs &a, hipStream_t s);
hipError_t launch_combine_fp8(const CombineArgs &a, hipStream_t s);
hipError_t launch_allgatherv(const AllGatherArgs &a, int64_t rows, hipStream_t s);

// Bytes of the library's static staging array (one per GPU): the FP8
// combine landing planes of the combine entry point that allocates nothing.
constexpr int64_t kStaticScratchBytes = MOE_EP_STATIC_SCRATCH_BYTES;
// Device address of the current device's staging array (looked up once per
// device and kept); hipSuccess or the lookup's error.
hipError_t static_scratch(void **ptr);
hipError_t launch_reduce_scatterv(const ReduceScatterArgs &a, int64_t rows, hipStream_t s);

} // namespace moe_ep
