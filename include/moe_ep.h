/*
 * moe_ep.h -- C ABI of the MI355X (gfx950) MoE expert-parallel exchange.
 *
 * One call covers all P *virtual* EP ranks that share one GPU's HBM: every
 * per-rank tensor of the exchange is stacked over ranks, and every rank
 * owns one region of a [P][size_per_rank] workspace (the workspace shape of
 * FlashInfer's moe_a2a_dispatch, "workspace" parameter).
 *
 * Semantics follow these documentation pages:
 *  - FlashInfer "flashinfer.moe_ep.NVLinkTwoSidedAlltoAll": dispatch()
 *    delivers every token to each rank that holds one of its chosen
 *    experts, together with the token's top-k ids, top-k weights and scale
 *    row; combine() adds up, over ranks, each token's expert outputs
 *    (each rank having weighted them and summed over its own experts); destroy() is
 *    idempotent; is_platform_supported() performs no collective work.
 *  - FlashInfer "flashinfer.moe_ep.NVLinkOneSidedConfig", lamport
 *    paragraph: token t of rank src lands in slot src * tokens_per_rank + t
 *    of a receiving rank, where tokens_per_rank equals the step's
 *    runtime_max_tokens_per_rank; BF16, MXFP8 and NVFP4 dispatch formats;
 *    at most 64 EP ranks.  First options paragraph: with
 *    use_low_precision_combine the combine moves its rows as FP8 values.
 *    cft paragraph: a payload row's size is a whole number of 16-byte
 *    units.
 *  - FlashInfer "flashinfer.comm.moe_a2a_dispatch": runtime_max_tokens_per_rank
 *    may not exceed the capacity given at initialisation; the outputs are
 *    views into the workspace, one per payload, and the workspace offset
 *    that the combine of the same step will use.
 *  - vLLM "device_communicators.all2all", FlashInferNVLinkTwoSidedManager:
 *    MoEEpCommParams(num_experts, top_k, max_tokens_per_rank, hidden_size,
 *    invalid_expert_id=num_experts); a received row without a token is
 *    marked with expert id invalid_expert_id, an id outside every rank's
 *    range.
 *  - vLLM "device_communicators.all2all", AgRsAll2AllManager: dispatch is
 *    all_gatherv of [hidden, topk_weights, topk_ids] along dim 0 with
 *    per-rank sizes; combine is reduce_scatterv of the hidden rows with
 *    the same sizes (combine_into_output: into a caller buffer).
 *
 * Readings taken where the pages are silent:
 *  - expert e lives on rank e / (E / P) (contiguous blocks; E % P == 0);
 *    ids outside [0, E) route nowhere but are still forwarded;
 *  - a token reaches a rank once however many of its experts live there;
 *  - every receive slot without a token carries invalid_expert_id in all
 *    k id entries after each dispatch (its payload, scale and weight bytes
 *    are left as they were);
 *  - combine sums in fp32 and rounds to bf16 to nearest-even;
 *  - the FP8 combine payload is OCP e4m3fn with one e8m0 scale per 32
 *    elements, the scale being the smallest power of two keeping the
 *    block's magnitudes within 448 (no saturation ever happens).
 *
 * Ownership: the caller owns every buffer (workspace, inputs, outputs).
 * The library allocates no device memory.  A handle keeps the last
 * dispatch's step size and per-rank token counts; combine uses them.
 * Handles are not thread-safe.  All launches go to the caller's stream,
 * in stream order, with no host synchronisation, and may be captured into
 * a HIP graph: the host-side arguments of a call (per-rank token counts,
 * the step size, the active rank mask, buffer pointers) are fixed into the
 * captured launches, so a graph replays exactly the calls it captured and
 * must be captured again when they change.
 *
 * Errors: every entry point validates all arguments before launching
 * anything (no partial launches) and returns one of the MOE_EP_* codes
 * below; moe_ep_last_error() gives a message for the calling thread.
 */
#ifndef MOE_EP_H
#define MOE_EP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_EP_OK 0
#define MOE_EP_ERR_INVALID_ARG (-1) /* bad argument or shape             */
#define MOE_EP_ERR_UNSUPPORTED (-2) /* no gfx950 device / format         */
#define MOE_EP_ERR_BAD_STATE (-3)   /* e.g. combine before any dispatch  */
#define MOE_EP_ERR_CAPACITY (-4)    /* workspace or step too large       */
#define MOE_EP_ERR_HIP (-5)         /* a HIP runtime call failed         */

#define MOE_EP_MAX_RANKS 64         /* one 64-bit destination mask word  */
#define MOE_EP_MAX_TOP_K 64

/* Dispatch payload formats (NVLinkOneSidedConfig, lamport paragraph). */
#define MOE_EP_FMT_BF16 0  /* row = 2H bytes, no scale row               */
#define MOE_EP_FMT_MXFP8 1 /* row = H e4m3 bytes, scale row = H/32 e8m0  */
#define MOE_EP_FMT_NVFP4 2 /* row = H/2 packed e2m1, scale row = H/16 e4m3 */
#define MOE_EP_FMT_DEEPSEEK_FP8 3 /* row = H e4m3, scale row = H/128 fp32 (1x128 blocks) */

/* Combine payload formats. */
#define MOE_EP_COMBINE_BF16 0
#define MOE_EP_COMBINE_FP8 1 /* e4m3fn + e8m0 per 32 on the wire */

/* Exchange parameters (vLLM MoEEpCommParams + NVLinkOneSidedConfig). */
typedef struct moe_ep_params {
    int32_t ep_size;             /* P, 1..64                                   */
    int32_t num_experts;         /* E, E % 4 == 0 and E % P == 0               */
    int32_t top_k;               /* k, 1..64                                   */
    int32_t max_tokens_per_rank; /* capacity C >= 1                            */
    int32_t hidden_size;         /* H: BF16 H % 8 == 0; MXFP8/NVFP4/FP8 combine H % 32 == 0 */
    int32_t dispatch_format;     /* MOE_EP_FMT_*                               */
    int32_t combine_format;      /* MOE_EP_COMBINE_*                           */
    int32_t has_weights;         /* 1: top-k weights travel with tokens        */
    int32_t invalid_expert_id;   /* id written to empty slots (usually E)      */
    int32_t extra_payload_bytes_per_token; /* >= 0: room for extra bytes per token */
    int32_t eplb_stats_num_experts; /* n in [0, num_experts] of the EPLB statistics
                                       all-gather (0: none)                        */
} moe_ep_params;

/* Where a dispatch's receive planes live.  Plane X of rank r starts at
 * workspace + r * region_bytes + X_offset; slot q of that plane at
 * X_offset + q * (row bytes of X).  q = src * tokens_per_rank + t.
 * Views stay valid until the next dispatch on the handle. */
typedef struct moe_ep_dispatch_views {
    int32_t tokens_per_rank;     /* T of this step                            */
    int32_t ep_size;             /* P                                         */
    int64_t region_bytes;        /* size_per_rank                             */
    int64_t payload_offset;      /* [P*T][payload_row_bytes] token rows       */
    int64_t payload_row_bytes;
    int64_t scales_offset;       /* [P*T][scale_row_bytes] (0 bytes if none)  */
    int64_t scale_row_bytes;
    int64_t ids_offset;          /* [P*T][k] int32 global expert ids          */
    int64_t weights_offset;      /* [P*T][k] fp32 (meaningful if has_weights) */
    int64_t slots_offset;        /* [P*T] int32: valid q ascending, first recv_total entries */
    int64_t counts_offset;       /* [P] int32 rows received from each source  */
    int64_t src_offsets_offset;  /* [P+1] int32 exclusive prefix of counts; [P] = recv_total */
    int64_t combine_payload_offset; /* FP8 combine landing codes [P*T][H], or -1 */
    int64_t combine_scales_offset;  /* FP8 combine landing scales [P*T][H/32], or -1 */
    int64_t extra_offset;        /* [P*T][extra_row_bytes] extra per-token bytes */
    int64_t extra_row_bytes;     /* extra_payload_bytes_per_token (0: none)   */
    int64_t eplb_offset;         /* [P][n] int32 gathered statistics (row s = rank s),
                                    -1 when this dispatch carried none        */
    int64_t eplb_num_experts;    /* n                                         */
} moe_ep_dispatch_views;

typedef struct moe_ep_handle moe_ep_handle;

/* 1 when the current HIP device is a gfx950 GPU, else 0.  Collective-free
 * (NVLinkTwoSidedAlltoAll.is_platform_supported). */
int moe_ep_is_supported(void);

/* size_per_rank of the [ep_size, size_per_rank] workspace
 * (moe_a2a_dispatch, workspace parameter; NVLinkOneSidedConfig, first
 * options paragraph: the dispatch workspace holds each token's activations
 * in the dispatch format plus its routing, extra_payload_bytes_per_token
 * more bytes per token and the EPLB statistics): bytes of one rank's
 * region for these parameters, every plane 256-byte aligned.  0 when the
 * parameters are invalid (see moe_ep_last_error), including a region above
 * 2^46 bytes or more than 2^31 - 1 slots (ep_size * max_tokens_per_rank),
 * which moe_ep_create rejects with MOE_EP_ERR_CAPACITY.  Host-only, no
 * device work. */
size_t moe_ep_workspace_bytes(const moe_ep_params *params);

/* Create a handle (NVLinkOneSidedConfig, first paragraph: a communication
 * is made by create_communication with the exchange's parameters and
 * backend options; vLLM FlashInferNVLinkTwoSidedManager: MoEEpCommParams)
 * over a caller-owned device workspace of P regions of size_per_rank bytes
 * each (region r at workspace + r * size_per_rank, size_per_rank >=
 * moe_ep_workspace_bytes and a multiple of 256, workspace 256-byte
 * aligned).  The workspace needs no initialisation; the handle keeps host
 * state only.  Errors: MOE_EP_ERR_INVALID_ARG (bad parameters, NULL or
 * misaligned workspace), MOE_EP_ERR_CAPACITY (region too small or too
 * large), MOE_EP_ERR_UNSUPPORTED (no gfx950 device current). */
int moe_ep_create(const moe_ep_params *params, void *workspace, size_t size_per_rank,
                  moe_ep_handle **out);

/*
 * Dispatch (NVLinkTwoSidedAlltoAll.dispatch / moe_a2a_dispatch).
 *  hidden            device [P][T][payload_row_bytes], 16-byte aligned;
 *                    row t of rank s is token t of rank s
 *  scales            device [P][T][scale_row_bytes]; required for MXFP8 /
 *                    NVFP4 / DeepSeekFp8, must be NULL for BF16
 *  extra_payload     device [P][T][extra_payload_bytes_per_token] or NULL:
 *                    more bytes per token, forwarded like the scale row
 *                    (NVLinkOneSidedConfig, extra_payload_bytes_per_token)
 *  eplb_local_stats  device [P][eplb_stats_num_experts] int32 or NULL: each
 *                    rank's per-expert counters for load balancing; every live rank receives
 *                    the [P][n] matrix (row s = rank s's statistics) in its
 *                    region (moe_a2a_dispatch, eplb_local_stats ->
 *                    eplb_gathered_stats)
 *  topk_ids          device [P][T][k] int32 global expert ids
 *  topk_weights      device [P][T][k] fp32; required iff has_weights
 *  num_tokens        host [P]: local_num_tokens n_s, 0 <= n_s <= T
 *  runtime_max_tokens_per_rank  T (the step's tokens_per_rank); <= 0
 *                    means the capacity; T <= capacity
 *  active_rank_mask  host, one word (NULL = every rank): bit r set when
 *                    rank r takes part in the step (moe_a2a_dispatch,
 *                    active_rank_mask).  A masked-off rank neither sends
 *                    nor receives: tokens routed to it are dropped, nothing
 *                    is written into its region, and the following combine
 *                    produces no rows for it.  Bits >= P must be clear.
 *  views             out (may be NULL): where the receive planes are
 * Rows t >= n_s of the inputs are never read.  Writes, for every rank r and
 * slot q = s*T + t: the token's payload row, scale row, k ids and k weights
 * when t < n_s and r owns one of its experts; otherwise k copies of
 * invalid_expert_id in the ids plane.  Also per-destination counts, source
 * offsets and the ascending list of valid slots.
 */
int moe_ep_dispatch(moe_ep_handle *h, const void *hidden, const void *scales,
                    const void *extra_payload, const int32_t *eplb_local_stats,
                    const int32_t *topk_ids, const float *topk_weights,
                    const int32_t *num_tokens, int32_t runtime_max_tokens_per_rank,
                    const uint64_t *active_rank_mask, void *stream,
                    moe_ep_dispatch_views *views);

/*
 * Combine (NVLinkTwoSidedAlltoAll.combine) of the last dispatch (and of
 * its active rank mask).
 *  expert_output  device [P][P*T][H] bf16: rank r's row for slot q at
 *                 (r*P*T + q)*H; only slots that received a token are read
 *  output         device [P][T][H] bf16: row t of rank s receives the sum
 *                 over ranks r that got token (s, t) of expert_output[r][s*T+t]
 *                 (fp32 accumulation from +0 in ascending rank order, RNE to
 *                 bf16); rows t >= n_s untouched
 * With MOE_EP_COMBINE_FP8 each sending rank first quantises its rows into
 * the source rank's landing plane (e4m3fn + e8m0 per 32), and the sum is
 * taken over the dequantised rows.
 */
int moe_ep_combine(moe_ep_handle *h, const void *expert_output, void *output, void *stream);

/*
 * moe_ep_combine for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid it): the
 * same combine of the last dispatch, with the same arguments and result,
 * but an FP8 combine stages its landing planes (e4m3 codes [P][P*T][H],
 * then e8m0 scales [P][P*T][H/32], per source rank) in the library's own
 * static device array of MOE_EP_STATIC_SCRATCH_BYTES instead of the
 * workspace; a BF16 combine stages nothing and runs as moe_ep_combine.
 * Allocates nothing (no hipMalloc, no allocating library call).
 *  - MOE_EP_ERR_CAPACITY when the step's landing planes,
 *    P * round_up_256(P*T*(H + H/32)) bytes for the last dispatch's T,
 *    exceed the array (e.g. P = 8, H = 7168 fits up to T = 128);
 *  - each GPU holds one array from library load until the process ends,
 *    shared by every call on that GPU; it keeps the last call's contents
 *    and needs no clearing (every landing row a call reads, it writes
 *    first), so calls on one GPU that overlap in time (other streams, other
 *    threads) race on it;
 *  - the workspace's landing-plane views (combine_payload_offset) are not
 *    written by this call.
 */
#define MOE_EP_STATIC_SCRATCH_BYTES (64ll << 20)
int moe_ep_combine_noalloc(moe_ep_handle *h, const void *expert_output, void *output, void *stream);

/* Release the handle.  Idempotent and NULL-safe; frees no caller memory. */
int moe_ep_destroy(moe_ep_handle *h);

/* One plane of an all-gatherv: rank q's sizes[q] input rows start at
 * in + q * in_rank_stride; rank r's gathered [sum(sizes)][row_bytes]
 * output starts at out + r * out_rank_stride. */
typedef struct moe_ep_plane {
    const void *in;
    int64_t in_rank_stride;      /* bytes */
    void *out;
    int64_t out_rank_stride;     /* bytes */
    int64_t row_bytes;           /* > 0 */
} moe_ep_plane;

/*
 * all_gatherv along dim 0 (AgRsAll2AllManager.dispatch): every rank r
 * receives, for every plane, the concatenation in rank order of each rank
 * q's first sizes[q] rows.  sizes: host [P], >= 0; 1 <= num_planes <= 8.
 */
int moe_ep_allgatherv(int32_t ep_size, const int32_t *sizes, int32_t num_planes,
                      const moe_ep_plane *planes, void *stream);

/*
 * reduce_scatterv along dim 0 (AgRsAll2AllManager.combine /
 * combine_into_output): rank q's full-length bf16 partial [sum(sizes)][H]
 * starts at in + q * in_rank_stride (bytes); rank r's result
 * [sizes[r]][H] at out + r * out_rank_stride (bytes) is the fp32 sum over
 * q (from +0, ascending q) of rows off_r .. off_r + sizes[r] - 1
 * (off_r = sum of sizes[q < r]), rounded to bf16 (RNE).
 */
int moe_ep_reduce_scatterv(int32_t ep_size, const int32_t *sizes, int32_t hidden_size,
                           const void *in, int64_t in_rank_stride, void *out,
                           int64_t out_rank_stride, void *stream);

/* Message of the calling thread's last failed call ("" if none). */
const char *moe_ep_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_EP_H */
