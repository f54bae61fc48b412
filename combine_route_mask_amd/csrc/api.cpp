// Host side of the C ABI declared in moe_ep.h: argument validation, the
// per-rank workspace layout, handle state and kernel launches.  Every check
// runs before the first launch, so a call either launches all its kernels
// or none.
#include <hip/hip_runtime.h>

#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <unordered_set>

#include "moe_ep.h"
#include "moe_ep_internal.h"

using namespace moe_ep;

struct moe_ep_handle {
    moe_ep_params p;
    uint8_t *ws;
    Layout lay;
    uint8_t *scratch;                 // the static staging array on the handle's device
    bool dispatched;
    int32_t T;                        // step size of the last dispatch
    int32_t n[MOE_EP_MAX_RANKS];      // token counts of the last dispatch
};

namespace {

thread_local std::string g_err;

// Handles created and not yet destroyed.  Looking a pointer up here (rather
// than reading through it) keeps destroy idempotent and lets every entry
// point reject stale handles without touching freed memory.
std::mutex g_handles_mu;
std::unordered_set<const moe_ep_handle *> g_handles;

int fail(int code, const std::string &msg)
{
    g_err = msg;
    return code;
}

int ok()
{
    g_err.clear();
    return MOE_EP_OK;
}

int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }

int64_t payload_row_bytes(const moe_ep_params &p)
{
    switch (p.dispatch_format) {
    case MOE_EP_FMT_BF16: return 2 * (int64_t)p.hidden_size;
    case MOE_EP_FMT_MXFP8: return p.hidden_size;
    case MOE_EP_FMT_NVFP4: return p.hidden_size / 2;
    case MOE_EP_FMT_DEEPSEEK_FP8: return p.hidden_size;
    default: return -1;
    }
}

int64_t scale_row_bytes(const moe_ep_params &p)
{
    switch (p.dispatch_format) {
    case MOE_EP_FMT_BF16: return 0;
    case MOE_EP_FMT_MXFP8: return p.hidden_size / 32;
    case MOE_EP_FMT_NVFP4: return p.hidden_size / 16;
    case MOE_EP_FMT_DEEPSEEK_FP8: return (p.hidden_size / 128) * 4;
    default: return -1;
    }
}

// Validates the parameters; on success fills the region layout.
int check_params(const moe_ep_params *pp, Layout *lay)
{
    if (!pp)
        return fail(MOE_EP_ERR_INVALID_ARG, "params is NULL");
    const moe_ep_params &p = *pp;
    if (p.ep_size < 1 || p.ep_size > MOE_EP_MAX_RANKS)
        return fail(MOE_EP_ERR_INVALID_ARG, "ep_size must be in [1, 64]");
    if (p.num_experts < 1 || p.num_experts % 4 != 0)
        return fail(MOE_EP_ERR_INVALID_ARG, "num_experts must be a positive multiple of 4");
    if (p.num_experts % p.ep_size != 0)
        return fail(MOE_EP_ERR_INVALID_ARG, "num_experts must be a multiple of ep_size");
    if (p.top_k < 1 || p.top_k > MOE_EP_MAX_TOP_K)
        return fail(MOE_EP_ERR_INVALID_ARG, "top_k must be in [1, 64]");
    if (p.max_tokens_per_rank < 1)
        return fail(MOE_EP_ERR_INVALID_ARG, "max_tokens_per_rank must be >= 1");
    if ((int64_t)p.ep_size * p.max_tokens_per_rank > (int64_t)INT32_MAX)
        return fail(MOE_EP_ERR_CAPACITY, "ep_size * max_tokens_per_rank exceeds 2^31 - 1 slots");
    if (p.hidden_size < 1)
        return fail(MOE_EP_ERR_INVALID_ARG, "hidden_size must be >= 1");
    if (p.has_weights != 0 && p.has_weights != 1)
        return fail(MOE_EP_ERR_INVALID_ARG, "has_weights must be 0 or 1");
    if (p.combine_format != MOE_EP_COMBINE_BF16 && p.combine_format != MOE_EP_COMBINE_FP8)
        return fail(MOE_EP_ERR_UNSUPPORTED, "unknown combine_format");
    const int64_t row = payload_row_bytes(p), srow = scale_row_bytes(p);
    if (row < 0)
        return fail(MOE_EP_ERR_UNSUPPORTED, "unknown dispatch_format");
    if (p.dispatch_format == MOE_EP_FMT_BF16 && p.hidden_size % 8 != 0)
        return fail(MOE_EP_ERR_INVALID_ARG,
                    "a BF16 payload row must be a whole number of 16-byte units (hidden_size % 8 == 0)");
    if (p.dispatch_format != MOE_EP_FMT_BF16 && p.hidden_size % 32 != 0)
        return fail(MOE_EP_ERR_INVALID_ARG,
                    "MXFP8 / NVFP4 payloads need hidden_size % 32 == 0 (16-byte rows, whole scale blocks)");
    if (p.dispatch_format == MOE_EP_FMT_DEEPSEEK_FP8 && p.hidden_size % 128 != 0)
        return fail(MOE_EP_ERR_INVALID_ARG, "DeepSeekFp8 payloads need hidden_size % 128 == 0");
    if (p.extra_payload_bytes_per_token < 0)
        return fail(MOE_EP_ERR_INVALID_ARG, "extra_payload_bytes_per_token may not be negative");
    // statistics of at most every expert (NVLinkTwoSidedAlltoAll class
    // paragraph: EPLB statistics cover all num_experts experts)
    if (p.eplb_stats_num_experts < 0 || p.eplb_stats_num_experts > p.num_experts)
        return fail(MOE_EP_ERR_INVALID_ARG, "eplb_stats_num_experts must be in [0, num_experts]");
    if (p.hidden_size % 8 != 0)
        return fail(MOE_EP_ERR_INVALID_ARG, "combine rows need hidden_size % 8 == 0");
    if (p.combine_format == MOE_EP_COMBINE_FP8 && p.hidden_size % 32 != 0)
        return fail(MOE_EP_ERR_INVALID_ARG, "FP8 combine needs hidden_size % 32 == 0");

    const int64_t S = (int64_t)p.ep_size * p.max_tokens_per_rank; // slots per region
    const int64_t k = p.top_k;
    // Every plane is the slot count times a per-slot byte count; capping a
    // region at 2^46 bytes keeps all of them, the region offsets of 64 ranks
    // and the kernels' byte products far from int64 overflow.
    const int64_t per_slot = row + srow + p.extra_payload_bytes_per_token + 8 * k + 4 +
                             (p.combine_format == MOE_EP_COMBINE_FP8 ? p.hidden_size + p.hidden_size / 32 : 0);
    if (per_slot > (1ll << 46) / S)
        return fail(MOE_EP_ERR_CAPACITY, "a workspace region would exceed 2^46 bytes (64 TiB)");
    Layout L;
    std::memset(&L, 0, sizeof L);
    int64_t off = 0;
    auto take = [&](int64_t bytes) {
        const int64_t at = off;
        off = align256(off + bytes);
        return at;
    };
    L.row_bytes = row;
    L.srow_bytes = srow;
    L.xrow_bytes = p.extra_payload_bytes_per_token;
    L.payload = take(S * row);
    L.scales = take(S * srow);
    L.extra = take(S * L.xrow_bytes);
    L.ids = take(S * k * 4);
    L.weights = take(p.has_weights ? S * k * 4 : 0);
    L.slots = take(S * 4);
    L.counts = take((int64_t)p.ep_size * 4);
    L.src_offsets = take((int64_t)(p.ep_size + 1) * 4);
    L.masks = take((int64_t)p.max_tokens_per_rank * 8);
    L.eplb = take((int64_t)p.ep_size * p.eplb_stats_num_experts * 4);
    if (p.combine_format == MOE_EP_COMBINE_FP8) {
        L.land_codes = take(S * p.hidden_size);
        L.land_scales = take(S * (p.hidden_size / 32));
    } else {
        L.land_codes = L.land_scales = -1;
    }
    L.total = off;
    L.region = off;
    if (lay)
        *lay = L;
    return MOE_EP_OK;
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

bool live_handle(const moe_ep_handle *h)
{
    std::lock_guard<std::mutex> lk(g_handles_mu);
    return h && g_handles.count(h) != 0;
}

} // namespace

extern "C" {

int moe_ep_is_supported(void)
{
    int dev = 0, count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || count < 1) {
        (void)hipGetLastError();
        return 0;
    }
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    return std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
}

size_t moe_ep_workspace_bytes(const moe_ep_params *params)
{
    Layout L;
    if (check_params(params, &L) != MOE_EP_OK)
        return 0;
    ok();
    return (size_t)L.total;
}

int moe_ep_create(const moe_ep_params *params, void *workspace, size_t size_per_rank,
                  moe_ep_handle **out)
{
    if (!out)
        return fail(MOE_EP_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    Layout L;
    int rc = check_params(params, &L);
    if (rc != MOE_EP_OK)
        return rc;
    if (!workspace)
        return fail(MOE_EP_ERR_INVALID_ARG, "workspace is NULL");
    if (!aligned(workspace, 256))
        return fail(MOE_EP_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    if (size_per_rank % 256 != 0)
        return fail(MOE_EP_ERR_INVALID_ARG, "size_per_rank must be a multiple of 256");
    if ((int64_t)size_per_rank < L.total)
        return fail(MOE_EP_ERR_CAPACITY, "size_per_rank is below moe_ep_workspace_bytes(params)");
    if (!moe_ep_is_supported())
        return fail(MOE_EP_ERR_UNSUPPORTED, "no gfx950 (MI355X) device is current");
    // the current device's staging array (once per device, kept)
    void *scratch = nullptr;
    hipError_t e = static_scratch(&scratch);
    if (e != hipSuccess)
        return fail(MOE_EP_ERR_HIP, std::string("static staging array lookup failed: ") + hipGetErrorString(e));
    moe_ep_handle *h = new (std::nothrow) moe_ep_handle;
    if (!h)
        return fail(MOE_EP_ERR_INVALID_ARG, "out of host memory");
    std::memset(h, 0, sizeof *h);
    h->p = *params;
    h->ws = static_cast<uint8_t *>(workspace);
    h->lay = L;
    h->lay.region = (int64_t)size_per_rank;
    h->scratch = static_cast<uint8_t *>(scratch);
    {
        std::lock_guard<std::mutex> lk(g_handles_mu);
        g_handles.insert(h);
    }
    *out = h;
    return ok();
}

int moe_ep_dispatch(moe_ep_handle *h, const void *hidden, const void *scales,
                    const void *extra_payload, const int32_t *eplb_local_stats,
                    const int32_t *topk_ids, const float *topk_weights,
                    const int32_t *num_tokens, int32_t runtime_max_tokens_per_rank,
                    const uint64_t *active_rank_mask, void *stream, moe_ep_dispatch_views *views)
{
    if (!live_handle(h))
        return fail(MOE_EP_ERR_INVALID_ARG, "invalid or destroyed handle");
    const moe_ep_params &p = h->p;
    const int32_t T = runtime_max_tokens_per_rank <= 0 ? p.max_tokens_per_rank
                                                       : runtime_max_tokens_per_rank;
    if (T > p.max_tokens_per_rank)
        return fail(MOE_EP_ERR_CAPACITY,
                    "runtime_max_tokens_per_rank exceeds max_tokens_per_rank");
    if (!hidden || !aligned(hidden, 16))
        return fail(MOE_EP_ERR_INVALID_ARG, "hidden must be a 16-byte aligned device pointer");
    if (!topk_ids || !aligned(topk_ids, 4))
        return fail(MOE_EP_ERR_INVALID_ARG, "topk_ids must be a 4-byte aligned device pointer");
    if (p.has_weights && (!topk_weights || !aligned(topk_weights, 4)))
        return fail(MOE_EP_ERR_INVALID_ARG, "topk_weights is required (has_weights = 1)");
    if (!p.has_weights && topk_weights)
        return fail(MOE_EP_ERR_INVALID_ARG,
                    "topk_weights given but the handle was created with has_weights = 0");
    const bool want_scales = h->lay.srow_bytes > 0;
    if (want_scales && !scales)
        return fail(MOE_EP_ERR_INVALID_ARG, "this dispatch format needs a scale row per token");
    if (!want_scales && scales)
        return fail(MOE_EP_ERR_INVALID_ARG, "BF16 dispatch takes no scales");
    if (extra_payload && h->lay.xrow_bytes == 0)
        return fail(MOE_EP_ERR_INVALID_ARG,
                    "extra_payload given but extra_payload_bytes_per_token is 0");
    if (eplb_local_stats && p.eplb_stats_num_experts == 0)
        return fail(MOE_EP_ERR_INVALID_ARG, "eplb_local_stats given but eplb_stats_num_experts is 0");
    if (eplb_local_stats && !aligned(eplb_local_stats, 4))
        return fail(MOE_EP_ERR_INVALID_ARG, "eplb_local_stats must be 4-byte aligned");
    if (!num_tokens)
        return fail(MOE_EP_ERR_INVALID_ARG, "num_tokens is NULL");
    for (int s = 0; s < p.ep_size; ++s)
        if (num_tokens[s] < 0 || num_tokens[s] > T)
            return fail(MOE_EP_ERR_INVALID_ARG,
                        "num_tokens[" + std::to_string(s) + "] must be in [0, T]");
    const uint64_t all = p.ep_size == 64 ? ~0ull : ((1ull << p.ep_size) - 1);
    const uint64_t active = active_rank_mask ? *active_rank_mask : all;
    if (active & ~all)
        return fail(MOE_EP_ERR_INVALID_ARG, "active_rank_mask has bits set at or above ep_size");

    DispatchArgs a;
    std::memset(&a, 0, sizeof a);
    a.payload = static_cast<const uint8_t *>(hidden);
    a.scales = static_cast<const uint8_t *>(scales);
    a.extra = static_cast<const uint8_t *>(extra_payload);
    a.eplb = eplb_local_stats;
    a.ids = topk_ids;
    a.weights = p.has_weights ? topk_weights : nullptr;
    a.ws = h->ws;
    a.region = h->lay.region;
    a.off_payload = h->lay.payload;
    a.off_scales = h->lay.scales;
    a.off_extra = h->lay.extra;
    a.off_eplb = h->lay.eplb;
    a.xrow_bytes = extra_payload ? h->lay.xrow_bytes : 0;
    a.n_eplb = p.eplb_stats_num_experts;
    a.off_ids = h->lay.ids;
    a.off_weights = h->lay.weights;
    a.off_slots = h->lay.slots;
    a.off_counts = h->lay.counts;
    a.off_src_offsets = h->lay.src_offsets;
    a.off_masks = h->lay.masks;
    a.row_bytes = h->lay.row_bytes;
    a.srow_bytes = h->lay.srow_bytes;
    a.P = p.ep_size;
    a.T = T;
    a.k = p.top_k;
    a.E = p.num_experts;
    a.epr = p.num_experts / p.ep_size;
    a.epr_shift = -1;
    for (int sh = 0; sh < 31; ++sh)
        if ((1 << sh) == a.epr)
            a.epr_shift = sh;
    a.invalid_id = p.invalid_expert_id;
    a.active = active;
    for (int s = 0; s < p.ep_size; ++s)
        a.n[s] = ((active >> s) & 1u) ? num_tokens[s] : 0; // masked-off ranks send nothing

    hipError_t e = launch_dispatch(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(MOE_EP_ERR_HIP, std::string("dispatch launch failed: ") + hipGetErrorString(e));
    h->dispatched = true;
    h->T = T;
    for (int s = 0; s < p.ep_size; ++s)
        h->n[s] = a.n[s];
    if (views) {
        views->tokens_per_rank = T;
        views->ep_size = p.ep_size;
        views->region_bytes = h->lay.region;
        views->payload_offset = h->lay.payload;
        views->payload_row_bytes = h->lay.row_bytes;
        views->scales_offset = h->lay.scales;
        views->scale_row_bytes = h->lay.srow_bytes;
        views->ids_offset = h->lay.ids;
        views->weights_offset = h->lay.weights;
        views->slots_offset = h->lay.slots;
        views->counts_offset = h->lay.counts;
        views->src_offsets_offset = h->lay.src_offsets;
        views->combine_payload_offset = h->lay.land_codes;
        views->combine_scales_offset = h->lay.land_scales;
        views->extra_offset = h->lay.extra;
        views->extra_row_bytes = h->lay.xrow_bytes;
        views->eplb_offset = eplb_local_stats ? h->lay.eplb : -1;
        views->eplb_num_experts = p.eplb_stats_num_experts;
    }
    return ok();
}

} // extern "C"

namespace {

// Combine of the last dispatch.  static_land: the FP8 landing planes live
// in the library's static staging array (codes [P][P*T][H], then scales
// [P][P*T][H/32], one block per source rank) instead of the workspace.
int run_combine(moe_ep_handle *h, const void *expert_output, void *output, void *stream, bool static_land)
{
    if (!live_handle(h))
        return fail(MOE_EP_ERR_INVALID_ARG, "invalid or destroyed handle");
    if (!h->dispatched)
        return fail(MOE_EP_ERR_BAD_STATE, "combine called before any dispatch on this handle");
    if (!expert_output || !aligned(expert_output, 16))
        return fail(MOE_EP_ERR_INVALID_ARG, "expert_output must be a 16-byte aligned device pointer");
    if (!output || !aligned(output, 16))
        return fail(MOE_EP_ERR_INVALID_ARG, "output must be a 16-byte aligned device pointer");
    const moe_ep_params &p = h->p;
    const bool fp8 = p.combine_format == MOE_EP_COMBINE_FP8;
    CombineArgs a;
    std::memset(&a, 0, sizeof a);
    a.eo = static_cast<const uint16_t *>(expert_output);
    a.out = static_cast<uint16_t *>(output);
    a.ws = h->ws;
    a.region = h->lay.region;
    a.off_masks = h->lay.masks;
    a.land = h->ws;
    a.land_stride = h->lay.region;
    a.off_land_codes = h->lay.land_codes;
    a.off_land_scales = h->lay.land_scales;
    a.P = p.ep_size;
    a.T = h->T;
    a.H = p.hidden_size;
    if (static_land && fp8) {
        const int64_t slots = (int64_t)a.P * a.T;
        const int64_t codes = slots * a.H, scales = slots * (a.H / 32);
        const int64_t stride = align256(codes + scales);
        if (stride > kStaticScratchBytes / a.P)
            return fail(MOE_EP_ERR_CAPACITY,
                        "FP8 landing planes of this step need " + std::to_string(stride * a.P) +
                            " bytes; the static staging array holds " + std::to_string(kStaticScratchBytes));
        a.land = h->scratch;
        a.land_stride = stride;
        a.off_land_codes = 0;
        a.off_land_scales = codes;
    }
    for (int s = 0; s < p.ep_size; ++s)
        a.n[s] = h->n[s];
    hipError_t e = fp8 ? launch_combine_fp8(a, static_cast<hipStream_t>(stream))
                       : launch_combine_bf16(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(MOE_EP_ERR_HIP, std::string("combine launch failed: ") + hipGetErrorString(e));
    return ok();
}

} // namespace

extern "C" {

int moe_ep_combine(moe_ep_handle *h, const void *expert_output, void *output, void *stream)
{
    return run_combine(h, expert_output, output, stream, false);
}

int moe_ep_combine_noalloc(moe_ep_handle *h, const void *expert_output, void *output, void *stream)
{
    return run_combine(h, expert_output, output, stream, true);
}

int moe_ep_destroy(moe_ep_handle *h)
{
    if (!h)
        return ok();
    bool was_live;
    {
        std::lock_guard<std::mutex> lk(g_handles_mu);
        was_live = g_handles.erase(h) != 0;
    }
    if (was_live)
        delete h;
    return ok();
}

int moe_ep_allgatherv(int32_t ep_size, const int32_t *sizes, int32_t num_planes,
                      const moe_ep_plane *planes, void *stream)
{
    if (ep_size < 1 || ep_size > MOE_EP_MAX_RANKS)
        return fail(MOE_EP_ERR_INVALID_ARG, "ep_size must be in [1, 64]");
    if (!sizes)
        return fail(MOE_EP_ERR_INVALID_ARG, "sizes is NULL");
    if (num_planes < 1 || num_planes > kMaxPlanes)
        return fail(MOE_EP_ERR_INVALID_ARG, "num_planes must be in [1, 8]");
    if (!planes)
        return fail(MOE_EP_ERR_INVALID_ARG, "planes is NULL");
    AllGatherArgs a;
    std::memset(&a, 0, sizeof a);
    a.P = ep_size;
    a.nplanes = num_planes;
    int64_t total = 0;
    for (int q = 0; q < ep_size; ++q) {
        if (sizes[q] < 0)
            return fail(MOE_EP_ERR_INVALID_ARG, "sizes must be >= 0");
        a.off[q] = (int32_t)total;
        total += sizes[q];
        if (total > INT32_MAX)
            return fail(MOE_EP_ERR_CAPACITY, "sum(sizes) exceeds 2^31 - 1");
    }
    a.off[ep_size] = (int32_t)total;
    for (int p = 0; p < num_planes; ++p) {
        const moe_ep_plane &pl = planes[p];
        if (!pl.in || !pl.out || pl.row_bytes <= 0 || pl.in_rank_stride < 0 || pl.out_rank_stride < 0)
            return fail(MOE_EP_ERR_INVALID_ARG, "plane " + std::to_string(p) + " is malformed");
        a.pl[p].in = static_cast<const uint8_t *>(pl.in);
        a.pl[p].in_stride = pl.in_rank_stride;
        a.pl[p].out = static_cast<uint8_t *>(pl.out);
        a.pl[p].out_stride = pl.out_rank_stride;
        a.pl[p].row_bytes = pl.row_bytes;
    }
    if (total == 0)
        return ok();
    hipError_t e = launch_allgatherv(a, total, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(MOE_EP_ERR_HIP, std::string("allgatherv launch failed: ") + hipGetErrorString(e));
    return ok();
}

int moe_ep_reduce_scatterv(int32_t ep_size, const int32_t *sizes, int32_t hidden_size,
                           const void *in, int64_t in_rank_stride, void *out,
                           int64_t out_rank_stride, void *stream)
{
    if (ep_size < 1 || ep_size > MOE_EP_MAX_RANKS)
        return fail(MOE_EP_ERR_INVALID_ARG, "ep_size must be in [1, 64]");
    if (!sizes)
        return fail(MOE_EP_ERR_INVALID_ARG, "sizes is NULL");
    if (hidden_size < 1 || hidden_size % 8 != 0)
        return fail(MOE_EP_ERR_INVALID_ARG, "hidden_size must be a positive multiple of 8");
    if (!in || !out || !aligned(in, 16) || !aligned(out, 16))
        return fail(MOE_EP_ERR_INVALID_ARG, "in / out must be 16-byte aligned device pointers");
    if (in_rank_stride < 0 || out_rank_stride < 0 || in_rank_stride % 16 || out_rank_stride % 16)
        return fail(MOE_EP_ERR_INVALID_ARG, "rank strides must be non-negative multiples of 16 bytes");
    ReduceScatterArgs a;
    std::memset(&a, 0, sizeof a);
    a.P = ep_size;
    a.H = hidden_size;
    int64_t total = 0;
    for (int q = 0; q < ep_size; ++q) {
        if (sizes[q] < 0)
            return fail(MOE_EP_ERR_INVALID_ARG, "sizes must be >= 0");
        a.off[q] = (int32_t)total;
        total += sizes[q];
        if (total > INT32_MAX)
            return fail(MOE_EP_ERR_CAPACITY, "sum(sizes) exceeds 2^31 - 1");
    }
    a.off[ep_size] = (int32_t)total;
    a.in = static_cast<const uint16_t *>(in);
    a.in_stride = in_rank_stride / 2;
    a.out = static_cast<uint16_t *>(out);
    a.out_stride = out_rank_stride / 2;
    if (total == 0)
        return ok();
    hipError_t e = launch_reduce_scatterv(a, total, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(MOE_EP_ERR_HIP,
                    std::string("reduce_scatterv launch failed: ") + hipGetErrorString(e));
    return ok();
}

const char *moe_ep_last_error(void) { return g_err.c_str(); }

} // extern "C"
