// gfx950 kernels of the all-gatherv / reduce-scatterv exchange (vLLM
// "device_communicators.all2all", AgRsAll2AllManager: dispatch gathers
// [hidden, topk_weights, topk_ids] from every rank along dim 0 with
// per-rank sizes; combine reduce-scatters the hidden rows with the same
// sizes) between P virtual ranks on one GPU.
//
// All-gatherv: one workgroup per global row j of the concatenation reads
// the row once and writes it to all P ranks.  Reduce-scatterv: one
// workgroup per piece of row j reads that piece of every rank's partial,
// sums in fp32 and writes it to the owning rank's row.
#include "formats.h"
#include "moe_ep_internal.h"

namespace moe_ep {
namespace {

// Rank whose segment [off[q], off[q+1]) holds global row j (empty segments
// are skipped).  Uniform across the workgroup.
__device__ __forceinline__ int segment_of(const int32_t *off, int P, int64_t j)
{
    int q = 0;
    while (q + 1 < P && off[q + 1] <= j)
        ++q;
    return q;
}

// Read one row once (two words of type W per thread per pass) and write it
// to all P ranks: rank r's copy at dst0 + r * stride.
template <typename W>
__device__ __forceinline__ void bcast_words(const uint8_t *src, int64_t nbytes, int P, uint8_t *dst0,
                                            int64_t stride)
{
    const int64_t n = nbytes / (int64_t)sizeof(W);
    const W *s = reinterpret_cast<const W *>(src);
    for (int64_t i0 = threadIdx.x; i0 < n; i0 += 2 * kBlock) {
        const int64_t i1 = i0 + kBlock;
        const bool p1 = i1 < n;
        const W v0 = s[i0];
        const W v1 = p1 ? s[i1] : v0;
        for (int r = 0; r < P; ++r) {
            W *d = reinterpret_cast<W *>(dst0 + (int64_t)r * stride);
            d[i0] = v0;
            if (p1)
                d[i1] = v1;
        }
    }
}

__global__ __launch_bounds__(kBlock) void allgatherv_kernel(AllGatherArgs a, int64_t rows)
{
    for (int64_t j = blockIdx.x; j < rows; j += gridDim.x) {
        const int q = segment_of(a.off, a.P, j);
        const int64_t i = j - a.off[q];
        for (int p = 0; p < a.nplanes; ++p) {
            const AgPlane &pl = a.pl[p];
            const uint8_t *src = pl.in + (int64_t)q * pl.in_stride + i * pl.row_bytes;
            uint8_t *dst0 = pl.out + j * pl.row_bytes;
            const uint64_t align = (uint64_t)(uintptr_t)pl.in | (uint64_t)(uintptr_t)pl.out |
                                   (uint64_t)pl.in_stride | (uint64_t)pl.out_stride |
                                   (uint64_t)pl.row_bytes;
            if ((align & 15) == 0)
                bcast_words<uint4>(src, pl.row_bytes, a.P, dst0, pl.out_stride);
            else if ((align & 3) == 0)
                bcast_words<uint32_t>(src, pl.row_bytes, a.P, dst0, pl.out_stride);
            else
                bcast_words<uint8_t>(src, pl.row_bytes, a.P, dst0, pl.out_stride);
        }
    }
}

// Ranks whose rows a reduce-scatterv lane loads at once.  P16 AgRs workload,
// same buffers, three buffer placements: 16 and 8 within 0.4% of each other
// (168.7-169.9 us), 4 the same; two vectors per lane instead of one +2-3%.
#ifndef MOE_EP_RS_GATHER
#define MOE_EP_RS_GATHER 16
#endif
#ifndef MOE_EP_RS_VPT
#define MOE_EP_RS_VPT 1    // 16-byte vectors per lane per row chunk
#endif
// Threads per reduce-scatterv workgroup.  Each item is then one 1 KB piece
// of a row (one vector per lane), so a workgroup's single store follows its
// loads at once and the stores reach HBM as a dense front among the reads
// (as in the BF16 combine).  P16 AgRs workload, same buffers, two
// processes: 64 -> 166.0-166.3 us, 128 -> 167.0, 256 -> 170.8-171.6;
// 128 threads with 8 ranks in flight 169.8-170.1.
#ifndef MOE_EP_RS_BLOCK
#define MOE_EP_RS_BLOCK 64
#endif

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Item (global row j, chunk c of BS * VPT vectors): each lane owns VPT
// 16-byte vectors of the output row and sums, in fp32 and ascending rank
// order, those vectors of row j of every rank's partial, with the loads of G
// ranks in flight at once; the owner of row j keeps the bf16 result.
template <int BS, int VPT, int G>
__global__ __launch_bounds__(BS) void reduce_scatterv_kernel(ReduceScatterArgs a, int64_t rows,
                                                             int64_t nchunk)
{
    const int64_t nvec = a.H >> 3;
    for (int64_t w = blockIdx.x; w < rows * nchunk; w += gridDim.x) {
        const int64_t j = w / nchunk, c = w % nchunk;
        const int64_t i0 = c * (BS * VPT) + threadIdx.x;
        if (i0 >= nvec)
            continue;
        const int r = segment_of(a.off, a.P, j);
        const int64_t i = j - a.off[r];
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
        for (int q0 = 0; q0 < a.P; q0 += G) {
            u32x4 v[G][VPT];
#pragma unroll
            for (int g = 0; g < G; ++g)
#pragma unroll
                for (int u = 0; u < VPT; ++u)
                    if (q0 + g < a.P && in[u])
                        v[g][u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(
                            a.in + (int64_t)(q0 + g) * a.in_stride + j * a.H + (i0 + u * BS) * 8));
#pragma unroll
            for (int g = 0; g < G; ++g)
#pragma unroll
                for (int u = 0; u < VPT; ++u)
                    if (q0 + g < a.P && in[u]) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            float lo, hi;
                            unpack_bf16x2(v[g][u][e], lo, hi);
                            acc[u][2 * e] += lo;
                            acc[u][2 * e + 1] += hi;
                        }
                    }
        }
#pragma unroll
        for (int u = 0; u < VPT; ++u) {
            if (!in[u])
                continue;
            u32x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                o[e] = pack_bf16x2(acc[u][2 * e], acc[u][2 * e + 1]);
            // the output is not read again here: keep it out of the caches
            __builtin_nontemporal_store(o, reinterpret_cast<u32x4 *>(a.out + (int64_t)r * a.out_stride +
                                                                    i * a.H + (i0 + u * BS) * 8));
        }
    }
}

inline unsigned grid_for(int64_t nitems)
{
    const int64_t cap = 256 * 8 * 64;
    return (unsigned)(nitems < 1 ? 1 : (nitems < cap ? nitems : cap));
}

} // namespace

hipError_t launch_allgatherv(const AllGatherArgs &a, int64_t rows, hipStream_t s)
{
    hipLaunchKernelGGL(allgatherv_kernel, dim3(grid_for(rows)), dim3(kBlock), 0, s, a, rows);
    return hipGetLastError();
}

hipError_t launch_reduce_scatterv(const ReduceScatterArgs &a, int64_t rows, hipStream_t s)
{
    constexpr int BS = MOE_EP_RS_BLOCK;
    const int64_t nchunk = ((a.H >> 3) + BS * MOE_EP_RS_VPT - 1) / (BS * MOE_EP_RS_VPT);
    hipLaunchKernelGGL((reduce_scatterv_kernel<BS, MOE_EP_RS_VPT, MOE_EP_RS_GATHER>),
                       dim3(grid_for(rows * nchunk)), dim3(BS), 0, s, a, rows, nchunk);
    return hipGetLastError();
}

} // namespace moe_ep
