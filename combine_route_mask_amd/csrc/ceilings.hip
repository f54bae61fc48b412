// Reference kernels for the benchmark: the simplest code that moves the
// exchange's bytes in the exchange's access patterns, with no routing logic,
// bookkeeping or id planes.  Run on the very buffers the exchange kernels use,
// they show what the memory system gives those patterns on that allocation
// (the same kernel runs at different speeds on different allocations of one
// size).  Measurement only: the exchange never calls them.
//
//   ceil_scatter   token-major row scatter: workgroup q reads token row q once
//                  and stores it at slot q of every region in its destination
//                  mask (the dispatch's payload traffic)
//   ceil_gather    gather-sum: one 2 KB piece of output row q per workgroup,
//                  the sum of that piece of row q of every plane in the mask
//                  (the BF16 combine's traffic); with store = 0 the sum is
//                  kept only when it matches a fixed pattern, so the output
//                  traffic disappears and the reads remain
//   (both skip a token whose mask is empty: it is neither read nor written)
//   ceil_fill      grid-stride write of a whole buffer
//   ceil_read      grid-stride read of a whole buffer
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void scatter_kernel(const uint8_t *src, int64_t row, const uint64_t *masks,
                                                      uint64_t live, int64_t ntok, uint8_t *base, int64_t region)
{
    const int64_t q = blockIdx.x;
    if (q >= ntok)
        return;
    const uint64_t mask = masks[q] & live; // regions that exist
    if (!mask)
        return; // a token that goes nowhere is not read
    const int64_t nvec = row >> 4;
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int64_t i = threadIdx.x + u * 256;
        if (i < nvec)
            v[u] = reinterpret_cast<const u32x4 *>(src + q * row)[i];
    }
    uint64_t m = mask;
    while (m) {
        const int r = __builtin_ctzll(m);
        m &= m - 1;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t i = threadIdx.x + u * 256;
            if (i < nvec)
                __builtin_nontemporal_store(v[u], reinterpret_cast<u32x4 *>(base + r * region + q * row) + i);
        }
    }
}

template <bool STORE>
__global__ __launch_bounds__(128) void gather_kernel(const uint8_t *planes, int64_t plane_bytes,
                                                     const uint64_t *masks, uint64_t live, int64_t ntok, int64_t row,
                                                     uint8_t *out)
{
    const int64_t nvec = row >> 4;
    const int64_t npiece = (nvec + 127) / 128;
    const int64_t q = blockIdx.x / npiece, c = blockIdx.x % npiece;
    const int64_t i = c * 128 + threadIdx.x;
    uint64_t m = q < ntok ? masks[q] & live : 0; // planes that exist
    if (!m || i >= nvec)
        return; // an empty mask: the row is neither read nor written
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        acc[e] = 0.0f;
    while (m) {
        int r[4];
        int cnt = 0;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            r[g] = 0;
            if (m) {
                r[g] = __builtin_ctzll(m);
                m &= m - 1;
                cnt = g + 1;
            }
        }
        u32x4 v[4];
#pragma unroll
        for (int g = 0; g < 4; ++g)
            if (g < cnt)
                v[g] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(planes + r[g] * plane_bytes +
                                                                                   q * row) + i);
#pragma unroll
        for (int g = 0; g < 4; ++g)
            if (g < cnt)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    acc[2 * e] += __uint_as_float(v[g][e] << 16);
                    acc[2 * e + 1] += __uint_as_float(v[g][e] & 0xFFFF0000u);
                }
    }
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        o[e] = (__float_as_uint(acc[2 * e]) >> 16) | (__float_as_uint(acc[2 * e + 1]) & 0xFFFF0000u);
    if (STORE)
        __builtin_nontemporal_store(o, reinterpret_cast<u32x4 *>(out + q * row) + i);
    else if (o[0] == 0x12345678u && o[1] == 0x9ABCDEF0u && o[2] == 0x0F1E2D3Cu)
        reinterpret_cast<u32x4 *>(out)[0] = o;
}

__global__ __launch_bounds__(256) void fill_kernel(uint8_t *p, int64_t nvec)
{
    const u32x4 v = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nvec; i += (int64_t)gridDim.x * 256)
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(p) + i);
}

__global__ __launch_bounds__(256) void read_kernel(const uint8_t *p, int64_t nvec, uint32_t *sink)
{
    uint32_t a = 0;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nvec; i += (int64_t)gridDim.x * 256) {
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p) + i);
        a ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    if (a == 0x12345678u)
        sink[blockIdx.x] = a;
}

constexpr int kSweepGrid = 256 * 8 * 8; // workgroups of the sweeps (grid-stride)

} // namespace

namespace {
uint64_t low_bits(int n) { return n >= 64 ? ~0ull : ((1ull << n) - 1); }
} // namespace

// Each call checks its sizes against what the caller says the buffers hold
// (src / planes / out / base bytes) and returns -1 before launching anything
// when an access would fall outside them; mask bits at or above the number
// of regions / planes are ignored.  Else the launch status (0 = ok).
extern "C" int ceil_scatter(const void *src, int64_t src_bytes, int64_t row, const uint64_t *masks, int64_t ntok,
                            int32_t nregions, void *base, int64_t region, int64_t base_bytes, void *stream)
{
    if (!src || !masks || !base || row <= 0 || row % 16 || row > 4 * 256 * 16 || ntok < 1 || nregions < 1 ||
        nregions > 64 || ntok > INT32_MAX || ntok * row > src_bytes || (nregions - 1) * region + ntok * row > base_bytes)
        return -1;
    hipLaunchKernelGGL(scatter_kernel, dim3((unsigned)ntok), dim3(256), 0, (hipStream_t)stream,
                       (const uint8_t *)src, row, masks, low_bits(nregions), ntok, (uint8_t *)base, region);
    return (int)hipGetLastError();
}

extern "C" int ceil_gather(const void *planes, int64_t plane_bytes, int32_t nplanes, const uint64_t *masks,
                           int64_t ntok, int64_t row, void *out, int64_t out_bytes, int32_t store, void *stream)
{
    if (!planes || !masks || !out || row <= 0 || row % 16 || ntok < 1 || nplanes < 1 || nplanes > 64 ||
        ntok * row > plane_bytes || ntok * row > out_bytes)
        return -1;
    const int64_t npiece = ((row >> 4) + 127) / 128;
    if (ntok * npiece > INT32_MAX)
        return -1;
    const dim3 grid((unsigned)(ntok * npiece));
    if (store)
        hipLaunchKernelGGL(gather_kernel<true>, grid, dim3(128), 0, (hipStream_t)stream, (const uint8_t *)planes,
                           plane_bytes, masks, low_bits(nplanes), ntok, row, (uint8_t *)out);
    else
        hipLaunchKernelGGL(gather_kernel<false>, grid, dim3(128), 0, (hipStream_t)stream, (const uint8_t *)planes,
                           plane_bytes, masks, low_bits(nplanes), ntok, row, (uint8_t *)out);
    return (int)hipGetLastError();
}

extern "C" int ceil_fill(void *p, int64_t nbytes, void *stream)
{
    if (!p || nbytes < 16)
        return -1;
    hipLaunchKernelGGL(fill_kernel, dim3(kSweepGrid), dim3(256), 0, (hipStream_t)stream, (uint8_t *)p, nbytes >> 4);
    return (int)hipGetLastError();
}

extern "C" int ceil_read(const void *p, int64_t nbytes, uint32_t *sink, int64_t sink_words, void *stream)
{
    if (!p || !sink || nbytes < 16 || sink_words < kSweepGrid)
        return -1;
    hipLaunchKernelGGL(read_kernel, dim3(kSweepGrid), dim3(256), 0, (hipStream_t)stream, (const uint8_t *)p,
                       nbytes >> 4, sink);
    return (int)hipGetLastError();
}
