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
#include "formats.h"
#include "moe_ep_internal.h"

namespace moe_ep {
namespace {

constexpr int kVpt = 4;        // 16-byte vectors per thread per pass (combine)
constexpr int kScanUnroll = 4; // 256-slot chunks per scan step
constexpr int kWaves = kBlock / 64;

// Destination-rank mask of one token: bit r set when one of its k ids is an
// expert of rank r (experts e / epr == r).  OR-ing the bits deduplicates
// tokens with several experts on one rank; ids outside [0, E) set nothing.
__device__ __forceinline__ uint64_t route_mask(const int32_t *idrow, int k, int E, int epr)
{
    uint64_t m = 0;
    for (int j = 0; j < k; ++j) {
        const int id = idrow[j];
        if (id >= 0 && id < E)
            m |= 1ull << (unsigned)(id / epr);
    }
    return m;
}

// Count of set bits of 'bits' in lanes below this one (v_mbcnt).
__device__ __forceinline__ int lanes_below(uint64_t bits)
{
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bits >> 32),
                                          __builtin_amdgcn_mbcnt_lo((uint32_t)bits, 0u));
}

// Copy one row of nbytes (multiple of 16, 16-byte aligned) to every rank in
// mask: rank r's copy at dst0 + r * stride.  The row is read once into
// registers, four 16-byte vectors per thread per pass (kBlock * 64 bytes),
// then stored once per destination rank.
__device__ __forceinline__ void copy_row_x16(const uint8_t *src, int64_t nbytes, uint64_t mask,
                                             uint8_t *dst0, int64_t stride)
{
    const int64_t nvec = nbytes >> 4;
    const uint4 *s4 = reinterpret_cast<const uint4 *>(src);
    for (int64_t b = threadIdx.x; b < nvec; b += 4 * kBlock) {
        const int64_t i0 = b, i1 = b + kBlock, i2 = b + 2 * kBlock, i3 = b + 3 * kBlock;
        const bool p1 = i1 < nvec, p2 = i2 < nvec, p3 = i3 < nvec;
        const uint4 zero = {0u, 0u, 0u, 0u};
        const uint4 v0 = s4[i0];
        const uint4 v1 = p1 ? s4[i1] : zero;
        const uint4 v2 = p2 ? s4[i2] : zero;
        const uint4 v3 = p3 ? s4[i3] : zero;
        uint64_t m = mask;
        while (m) {
            const int r = __builtin_ctzll(m);
            m &= m - 1;
            uint4 *d4 = reinterpret_cast<uint4 *>(dst0 + (int64_t)r * stride);
            d4[i0] = v0;
            if (p1)
                d4[i1] = v1;
            if (p2)
                d4[i2] = v2;
            if (p3)
                d4[i3] = v3;
        }
    }
}

// Same for short rows of any size, word by word (W = uint32_t or uint8_t).
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

__device__ __forceinline__ void copy_row_any(const uint8_t *src, int64_t nbytes, uint64_t mask,
                                             uint8_t *dst0, int64_t stride)
{
    const uint64_t align = (uint64_t)(uintptr_t)src | (uint64_t)(uintptr_t)dst0 |
                           (uint64_t)stride | (uint64_t)nbytes;
    if ((align & 15) == 0)
        copy_row_x16(src, nbytes, mask, dst0, stride);
    else if ((align & 3) == 0)
        copy_row_words<uint32_t>(src, nbytes, mask, dst0, stride);
    else
        copy_row_words<uint8_t>(src, nbytes, mask, dst0, stride);
}

// Receive bookkeeping of destination rank r: walks every source slot q in
// ascending order, 1024 slots per step; a wave ballot marks the slots whose
// token goes to r, v_mbcnt gives each one its rank inside the wave, and the
// per-wave totals in LDS give the step's exclusive prefix.  Produces the
// ascending list of valid slots, the per-source counts and their exclusive
// prefix (src_offsets[P] = rows received).
__device__ void scan_destination(const DispatchArgs &a, int r)
{
    __shared__ int wave_tot[kScanUnroll][kWaves];
    __shared__ int src_off[MOE_EP_MAX_RANKS + 1];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint8_t *region = a.ws + (int64_t)r * a.region;
    int32_t *slots = reinterpret_cast<int32_t *>(region + a.off_slots);
    const int64_t S = (int64_t)a.P * a.T;
    int base = 0;
    for (int64_t c0 = 0; c0 < S; c0 += kBlock * kScanUnroll) {
        int bit[kScanUnroll], src[kScanUnroll], tok[kScanUnroll];
#pragma unroll
        for (int u = 0; u < kScanUnroll; ++u) {
            const int64_t q = c0 + u * kBlock + tid;
            bit[u] = 0;
            src[u] = 0;
            tok[u] = -1;
            if (q < S) {
                const int s = (int)(q / a.T);
                const int t = (int)(q - (int64_t)s * a.T);
                src[u] = s;
                tok[u] = t;
                if (t < a.n[s])
                    bit[u] = (int)((route_mask(a.ids + q * a.k, a.k, a.E, a.epr) >> r) & 1u);
            }
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

// One source slot q = s*T + t: compute the token's destination mask, store
// it for combine, write ids/weights (or invalid-id markers) to all P
// destinations, then read the payload and scale rows once and write them
// to every destination in the mask.
__device__ void scatter_token(const DispatchArgs &a, int64_t q)
{
    const int s = (int)(q / a.T);
    const int t = (int)(q - (int64_t)s * a.T);
    const bool live = t < a.n[s];
    const int32_t *idrow = a.ids + q * a.k;
    const uint64_t mask = live ? route_mask(idrow, a.k, a.E, a.epr) : 0ull;
    if (threadIdx.x == 0)
        *reinterpret_cast<uint64_t *>(a.ws + (int64_t)s * a.region + a.off_masks + (int64_t)t * 8) =
            mask;
    for (int i = threadIdx.x; i < a.P * a.k; i += kBlock) {
        const int r = i / a.k, j = i - r * a.k;
        uint8_t *reg = a.ws + (int64_t)r * a.region;
        int32_t id = a.invalid_id;
        if ((mask >> r) & 1u) {
            id = idrow[j];
            if (a.weights)
                reinterpret_cast<float *>(reg + a.off_weights)[q * a.k + j] = a.weights[q * a.k + j];
        }
        reinterpret_cast<int32_t *>(reg + a.off_ids)[q * a.k + j] = id;
    }
    if (!mask)
        return;
    copy_row_x16(a.payload + q * a.row_bytes, a.row_bytes, mask,
                 a.ws + a.off_payload + q * a.row_bytes, a.region);
    if (a.srow_bytes)
        copy_row_any(a.scales + q * a.srow_bytes, a.srow_bytes, mask,
                     a.ws + a.off_scales + q * a.srow_bytes, a.region);
}

// Blocks [0, P) do the receive bookkeeping of one destination each; the
// rest walk the source slots.  The two roles touch disjoint memory.
__global__ __launch_bounds__(kBlock) void dispatch_kernel(DispatchArgs a)
{
    if ((int)blockIdx.x < a.P) {
        scan_destination(a, (int)blockIdx.x);
        return;
    }
    const int64_t S = (int64_t)a.P * a.T;
    const int64_t stride = (int64_t)gridDim.x - a.P;
    for (int64_t q = (int64_t)blockIdx.x - a.P; q < S; q += stride)
        scatter_token(a, q);
}

// BF16 combine: source token (s, t) sums, in fp32 and ascending rank order,
// row q = s*T + t of every rank in its mask, then rounds to bf16.
__global__ __launch_bounds__(kBlock) void combine_bf16_kernel(CombineArgs a)
{
    const int64_t S = (int64_t)a.P * a.T;
    const int64_t rank_stride = S * a.H; // elements
    const int64_t nvec = a.H >> 3;       // 8 bf16 per 16 bytes
    for (int64_t q = blockIdx.x; q < S; q += gridDim.x) {
        const int s = (int)(q / a.T);
        const int t = (int)(q - (int64_t)s * a.T);
        if (t >= a.n[s])
            continue;
        const uint64_t mask = *reinterpret_cast<const uint64_t *>(
            a.ws + (int64_t)s * a.region + a.off_masks + (int64_t)t * 8);
        for (int64_t b = 0; b < nvec; b += kBlock * kVpt) {
            float acc[kVpt][8];
#pragma unroll
            for (int u = 0; u < kVpt; ++u)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    acc[u][e] = 0.0f;
            uint64_t m = mask;
            while (m) {
                const int r = __builtin_ctzll(m);
                m &= m - 1;
                const uint4 *src = reinterpret_cast<const uint4 *>(a.eo + r * rank_stride + q * a.H);
                uint4 v[kVpt];
#pragma unroll
                for (int u = 0; u < kVpt; ++u) {
                    const int64_t i = b + u * kBlock + threadIdx.x;
                    if (i < nvec)
                        v[u] = src[i];
                }
#pragma unroll
                for (int u = 0; u < kVpt; ++u) {
                    const int64_t i = b + u * kBlock + threadIdx.x;
                    if (i < nvec) {
                        const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            float lo, hi;
                            unpack_bf16x2(w[e], lo, hi);
                            acc[u][2 * e] += lo;
                            acc[u][2 * e + 1] += hi;
                        }
                    }
                }
            }
            uint4 *dst = reinterpret_cast<uint4 *>(a.out + q * a.H);
#pragma unroll
            for (int u = 0; u < kVpt; ++u) {
                const int64_t i = b + u * kBlock + threadIdx.x;
                if (i < nvec) {
                    uint4 o;
                    o.x = pack_bf16x2(acc[u][0], acc[u][1]);
                    o.y = pack_bf16x2(acc[u][2], acc[u][3]);
                    o.z = pack_bf16x2(acc[u][4], acc[u][5]);
                    o.w = pack_bf16x2(acc[u][6], acc[u][7]);
                    dst[i] = o;
                }
            }
        }
    }
}

// x * 2^-e for a bf16 bit pattern x, exactly, as an fp32 value that is
// either normal or a signed zero (a zero stands for any |x * 2^-e| below
// 2^-10, which the e4m3 rounding sends to zero anyway).  Integer exponent
// arithmetic only, so no denormal mode can change the result.
__device__ __forceinline__ float scale_pow2(uint32_t xb, int e)
{
    const uint32_t sign = (xb & 0x8000u) << 16;
    const int eb = (int)((xb >> 7) & 0xFFu);
    const uint32_t mant = xb & 0x7Fu;
    if (eb == 0) {                       // bf16 zero or subnormal: mant * 2^-133
        if (mant == 0 || e >= -116)      // then |x * 2^-e| < 2^7 * 2^-133 * 2^116 = 2^-10
            return __uint_as_float(sign);
        const float f = (float)mant * __uint_as_float((uint32_t)(-133 - e + 127) << 23);
        return __uint_as_float(sign | __float_as_uint(f));
    }
    const int ev = eb - e;
    if (ev <= 0)
        return __uint_as_float(sign);
    return __uint_as_float(sign | ((uint32_t)ev << 23) | (mant << 16));
}

// FP8 combine, sending side: every rank r that holds token (s, t) quantises
// its row q = s*T + t (e4m3fn, one e8m0 scale per 32 elements) into source
// rank s's landing plane at slot r*T + t.  A thread handles 16 elements;
// two neighbouring lanes share a 32-element block and its amax.
__global__ __launch_bounds__(kBlock) void combine_fp8_quant_kernel(CombineArgs a)
{
    const int64_t S = (int64_t)a.P * a.T;
    const int64_t rank_stride = S * a.H;
    const int64_t ngroups = a.H >> 4;
    for (int64_t q = blockIdx.x; q < S; q += gridDim.x) {
        const int s = (int)(q / a.T);
        const int t = (int)(q - (int64_t)s * a.T);
        if (t >= a.n[s])
            continue;
        uint8_t *land = a.ws + (int64_t)s * a.region;
        const uint64_t mask = *reinterpret_cast<const uint64_t *>(land + a.off_masks + (int64_t)t * 8);
        uint64_t m = mask;
        while (m) {
            const int r = __builtin_ctzll(m);
            m &= m - 1;
            const uint4 *src = reinterpret_cast<const uint4 *>(a.eo + r * rank_stride + q * a.H);
            const int64_t slot = (int64_t)r * a.T + t;
            uint4 *codes = reinterpret_cast<uint4 *>(land + a.off_land_codes + slot * a.H);
            uint8_t *scales = land + a.off_land_scales + slot * (a.H >> 5);
            for (int64_t g0 = 0; g0 < ngroups; g0 += kBlock) {
                const int64_t g = g0 + threadIdx.x;
                const bool act = g < ngroups; // ngroups even: lane pairs agree
                uint4 x0 = {0, 0, 0, 0}, x1 = {0, 0, 0, 0};
                if (act) {
                    x0 = src[2 * g];
                    x1 = src[2 * g + 1];
                }
                const uint32_t w[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
                uint32_t amax = 0;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    amax = max(amax, w[e] & 0x7FFFu);
                    amax = max(amax, (w[e] >> 16) & 0x7FFFu);
                }
                amax = max(amax, (uint32_t)__shfl_xor((int)amax, 1));
                if (!act)
                    continue;
                uint32_t c[16];
                uint32_t scale_code;
                if (amax >= 0x7F80u) {   // a NaN or an infinity in the block
                    scale_code = 0xFFu;
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        c[e] = 0x7Fu;
                } else {
                    const int ex = fp8_block_exponent(amax);
                    scale_code = (uint32_t)(ex + 127);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        c[2 * e] = f32_to_e4m3(scale_pow2(w[e] & 0xFFFFu, ex));
                        c[2 * e + 1] = f32_to_e4m3(scale_pow2(w[e] >> 16, ex));
                    }
                }
                uint4 o;
                o.x = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
                o.y = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
                o.z = c[8] | (c[9] << 8) | (c[10] << 16) | (c[11] << 24);
                o.w = c[12] | (c[13] << 8) | (c[14] << 16) | (c[15] << 24);
                codes[g] = o;
                if ((g & 1) == 0)
                    scales[g >> 1] = (uint8_t)scale_code;
            }
        }
    }
}

// FP8 combine, receiving side: source token (s, t) dequantises the landing
// rows r*T + t of every rank r in its mask, sums them in fp32 (ascending r)
// and rounds to bf16.
__global__ __launch_bounds__(kBlock) void combine_fp8_gather_kernel(CombineArgs a)
{
    const int64_t S = (int64_t)a.P * a.T;
    const int64_t ngroups = a.H >> 4;
    for (int64_t q = blockIdx.x; q < S; q += gridDim.x) {
        const int s = (int)(q / a.T);
        const int t = (int)(q - (int64_t)s * a.T);
        if (t >= a.n[s])
            continue;
        const uint8_t *land = a.ws + (int64_t)s * a.region;
        const uint64_t mask = *reinterpret_cast<const uint64_t *>(land + a.off_masks + (int64_t)t * 8);
        uint4 *dst = reinterpret_cast<uint4 *>(a.out + q * a.H);
        for (int64_t g0 = 0; g0 < ngroups; g0 += kBlock) {
            const int64_t g = g0 + threadIdx.x;
            if (g >= ngroups)
                break;
            float acc[16];
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[e] = 0.0f;
            uint64_t m = mask;
            while (m) {
                const int r = __builtin_ctzll(m);
                m &= m - 1;
                const int64_t slot = (int64_t)r * a.T + t;
                const uint4 cv = reinterpret_cast<const uint4 *>(land + a.off_land_codes + slot * a.H)[g];
                const uint32_t sc = land[a.off_land_scales + slot * (a.H >> 5) + (g >> 1)];
                const uint32_t cw[4] = {cv.x, cv.y, cv.z, cv.w};
                if (sc == 0xFFu) {
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        acc[e] = __uint_as_float(0x7FC00000u);
                    continue;
                }
                const int ex = (int)sc - 127;
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const uint32_t code = (cw[e >> 2] >> (8 * (e & 3))) & 0xFFu;
                    acc[e] += __builtin_amdgcn_ldexpf(e4m3_to_f32(code), ex);
                }
            }
            uint4 o0, o1;
            o0.x = pack_bf16x2(acc[0], acc[1]);
            o0.y = pack_bf16x2(acc[2], acc[3]);
            o0.z = pack_bf16x2(acc[4], acc[5]);
            o0.w = pack_bf16x2(acc[6], acc[7]);
            o1.x = pack_bf16x2(acc[8], acc[9]);
            o1.y = pack_bf16x2(acc[10], acc[11]);
            o1.z = pack_bf16x2(acc[12], acc[13]);
            o1.w = pack_bf16x2(acc[14], acc[15]);
            dst[2 * g] = o0;
            dst[2 * g + 1] = o1;
        }
    }
}

// Grid of nitems workgroups capped at a whole number of waves of the chip
// (256 CUs x 8 workgroups); kernels loop over the rest.
inline unsigned grid_for(int64_t nitems)
{
    const int64_t cap = 256 * 8 * 64;
    return (unsigned)(nitems < 1 ? 1 : (nitems < cap ? nitems : cap));
}

} // namespace

hipError_t launch_dispatch(const DispatchArgs &a, hipStream_t s)
{
    const int64_t S = (int64_t)a.P * a.T;
    hipLaunchKernelGGL(dispatch_kernel, dim3(a.P + grid_for(S)), dim3(kBlock), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_combine_bf16(const CombineArgs &a, hipStream_t s)
{
    hipLaunchKernelGGL(combine_bf16_kernel, dim3(grid_for((int64_t)a.P * a.T)), dim3(kBlock), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_combine_fp8(const CombineArgs &a, hipStream_t s)
{
    const dim3 grid(grid_for((int64_t)a.P * a.T));
    hipLaunchKernelGGL(combine_fp8_quant_kernel, grid, dim3(kBlock), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(combine_fp8_gather_kernel, grid, dim3(kBlock), 0, s, a);
    return hipGetLastError();
}

} // namespace moe_ep
