/*
 * A plain C program that drives the exchange through its C ABI alone
 * (include/moe_ep.h, libmoe_ep.so), on device buffers from hipMalloc: one
 * dispatch and one BF16 combine of a small step (P = 4 ranks, 16 experts,
 * top-2, up to 16 tokens per rank, hidden 256).
 *
 * Between the two it plays the experts on the host from what the dispatch
 * returned: every rank r, for every receive slot that holds a token, returns
 * the token's row times the sum of the top-k weights of the token's experts
 * that live on r (an identity expert; the row, ids and weights are read
 * back from r's receive planes, slots without a token get NaN rows).  The
 * combine then sums over ranks (FlashInfer NVLinkTwoSidedAlltoAll,
 * combine(): each rank's output already weighted and reduced over its own
 * experts), so every token must come back as its row times the sum of all
 * its top-k weights, within the bf16 rounding of the expert rows and of the
 * result.  Rows past each rank's token count must stay as they were.
 *
 * Then the all-gatherv / reduce-scatterv pair (vLLM AgRsAll2AllManager:
 * dispatch gathers the hidden rows and top-k ids of every rank along dim 0
 * with per-rank sizes, combine reduce-scatters hidden rows with the same
 * sizes) on the same token rows, sizes n[s]: every rank must receive the
 * concatenation of all ranks' rows and ids byte for byte, and with rank q's
 * partial set to (q + 1) times the gathered rows, rank r's result must be,
 * bit for bit, the fp32 sum over q in ascending order of those partials,
 * rounded to bf16.
 *
 * Prints "ok" and exits 0 when every check holds; exits 1 on a failed
 * check, 2 when no gfx950 device is current, 3 when a call fails.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "moe_ep.h"

enum { P = 4, E = 16, K = 2, T = 16, H = 256 };

static uint64_t lcg = 0x9E3779B97F4A7C15ull;

static uint32_t next_u32(void)
{
    lcg = lcg * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(lcg >> 32);
}

/* uniform in [0, 1) */
static float next_unit(void) { return (float)(next_u32() >> 8) * (1.0f / 16777216.0f); }

static float bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* round to nearest even (finite inputs) */
static uint16_t f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

#define CHECK_HIP(x)                                                                          \
    do {                                                                                      \
        if ((x) != hipSuccess) {                                                              \
            fprintf(stderr, "HIP call failed at line %d: %s\n", __LINE__, #x);                \
            return 3;                                                                         \
        }                                                                                     \
    } while (0)

#define CHECK_EP(x)                                                                           \
    do {                                                                                      \
        if ((x) != MOE_EP_OK) {                                                               \
            fprintf(stderr, "exchange call failed at line %d: %s\n", __LINE__, moe_ep_last_error()); \
            return 3;                                                                         \
        }                                                                                     \
    } while (0)

int main(void)
{
    if (!moe_ep_is_supported()) {
        fprintf(stderr, "no gfx950 device is current\n");
        return 2;
    }
    const int S = P * T; /* slots per region */
    moe_ep_params prm;
    memset(&prm, 0, sizeof prm);
    prm.ep_size = P;
    prm.num_experts = E;
    prm.top_k = K;
    prm.max_tokens_per_rank = T;
    prm.hidden_size = H;
    prm.dispatch_format = MOE_EP_FMT_BF16;
    prm.combine_format = MOE_EP_COMBINE_BF16;
    prm.has_weights = 1;
    prm.invalid_expert_id = E;
    const size_t region = moe_ep_workspace_bytes(&prm);
    if (region == 0) {
        fprintf(stderr, "workspace size: %s\n", moe_ep_last_error());
        return 3;
    }

    /* host inputs: rank s has n[s] tokens; rows in [-1, 1), two distinct
       experts per token, weights in [0.1, 1) */
    int32_t n[P];
    static uint16_t hidden[P][T][H];
    static int32_t ids[P][T][K];
    static float wts[P][T][K];
    for (int s = 0; s < P; ++s) {
        n[s] = T - 3 * s;
        for (int t = 0; t < T; ++t) {
            for (int h = 0; h < H; ++h)
                hidden[s][t][h] = f32_to_bf16(2.0f * next_unit() - 1.0f);
            ids[s][t][0] = (int32_t)(next_u32() % E);
            do {
                ids[s][t][1] = (int32_t)(next_u32() % E);
            } while (ids[s][t][1] == ids[s][t][0]);
            for (int j = 0; j < K; ++j)
                wts[s][t][j] = 0.1f + 0.9f * next_unit();
        }
    }

    void *d_ws, *d_hidden, *d_ids, *d_wts, *d_eo, *d_out;
    CHECK_HIP(hipMalloc(&d_ws, (size_t)P * region));
    CHECK_HIP(hipMalloc(&d_hidden, sizeof hidden));
    CHECK_HIP(hipMalloc(&d_ids, sizeof ids));
    CHECK_HIP(hipMalloc(&d_wts, sizeof wts));
    CHECK_HIP(hipMalloc(&d_eo, (size_t)P * S * H * 2));
    CHECK_HIP(hipMalloc(&d_out, (size_t)P * T * H * 2));
    CHECK_HIP(hipMemcpy(d_hidden, hidden, sizeof hidden, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_ids, ids, sizeof ids, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_wts, wts, sizeof wts, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemset(d_out, 0x5A, (size_t)P * T * H * 2));

    moe_ep_handle *ex = NULL;
    CHECK_EP(moe_ep_create(&prm, d_ws, region, &ex));
    moe_ep_dispatch_views v;
    CHECK_EP(moe_ep_dispatch(ex, d_hidden, NULL, NULL, NULL, (const int32_t *)d_ids, (const float *)d_wts, n, T,
                             NULL, NULL, &v));
    CHECK_HIP(hipDeviceSynchronize());

    /* the experts, on the host, from every rank's receive planes */
    uint8_t *ws = (uint8_t *)malloc((size_t)P * region);
    uint16_t *eo = (uint16_t *)malloc((size_t)P * S * H * 2);
    if (!ws || !eo)
        return 3;
    CHECK_HIP(hipMemcpy(ws, d_ws, (size_t)P * region, hipMemcpyDeviceToHost));
    const int epr = E / P;
    int received = 0;
    for (int r = 0; r < P; ++r) {
        const uint8_t *reg = ws + (size_t)r * v.region_bytes;
        for (int q = 0; q < S; ++q) {
            const int32_t *qid = (const int32_t *)(reg + v.ids_offset) + (size_t)q * K;
            const float *qw = (const float *)(reg + v.weights_offset) + (size_t)q * K;
            const uint16_t *row = (const uint16_t *)(reg + v.payload_offset + (size_t)q * v.payload_row_bytes);
            uint16_t *o = eo + ((size_t)r * S + q) * H;
            float wr = 0.0f;
            int mine = 0;
            for (int j = 0; j < K; ++j)
                if (qid[j] >= r * epr && qid[j] < (r + 1) * epr) {
                    wr += qw[j];
                    mine = 1;
                }
            if (!mine) { /* no token in this slot: must never be read */
                for (int h = 0; h < H; ++h)
                    o[h] = 0x7FC0;
                continue;
            }
            ++received;
            for (int h = 0; h < H; ++h)
                o[h] = f32_to_bf16(bf16_to_f32(row[h]) * wr);
        }
    }
    CHECK_HIP(hipMemcpy(d_eo, eo, (size_t)P * S * H * 2, hipMemcpyHostToDevice));
    CHECK_EP(moe_ep_combine(ex, d_eo, d_out, NULL));
    static uint16_t out[P][T][H];
    CHECK_HIP(hipMemcpy(out, d_out, sizeof out, hipMemcpyDeviceToHost));

    /* y = x * (w_0 + w_1): each expert row carries one bf16 rounding of
       x * w_r (relative 2^-9), the fp32 sum over ranks is exact enough,
       and y one more bf16 rounding (2^-9); 2^-7 covers both */
    int bad = 0, tokens = 0;
    for (int s = 0; s < P; ++s)
        for (int t = 0; t < T; ++t)
            for (int h = 0; h < H; ++h) {
                const uint16_t y = out[s][t][h];
                if (t >= n[s]) {
                    bad += y != 0x5A5A;
                    continue;
                }
                const double x = bf16_to_f32(hidden[s][t][h]);
                const double w = (double)wts[s][t][0] + (double)wts[s][t][1];
                const double yf = bf16_to_f32(y);
                if (!(fabs(yf - x * w) <= (0.0078125 + 0.000030517578125) * fabs(x) * w))
                    ++bad;
                tokens += h == 0;
            }
    CHECK_EP(moe_ep_destroy(ex));

    /* all-gatherv of the hidden rows and the ids, sizes n[s] */
    int32_t off[P + 1];
    off[0] = 0;
    for (int s = 0; s < P; ++s)
        off[s + 1] = off[s] + n[s];
    const int R = off[P];
    void *d_gh, *d_gi, *d_part, *d_rs;
    CHECK_HIP(hipMalloc(&d_gh, (size_t)P * R * H * 2));
    CHECK_HIP(hipMalloc(&d_gi, (size_t)P * R * K * 4));
    CHECK_HIP(hipMalloc(&d_part, (size_t)P * R * H * 2));
    CHECK_HIP(hipMalloc(&d_rs, (size_t)P * T * H * 2));
    moe_ep_plane planes[2] = {
        {d_hidden, (int64_t)T * H * 2, d_gh, (int64_t)R * H * 2, (int64_t)H * 2},
        {d_ids, (int64_t)T * K * 4, d_gi, (int64_t)R * K * 4, (int64_t)K * 4},
    };
    CHECK_EP(moe_ep_allgatherv(P, n, 2, planes, NULL));
    uint16_t *gh = (uint16_t *)malloc((size_t)P * R * H * 2);
    int32_t *gi = (int32_t *)malloc((size_t)P * R * K * 4);
    uint16_t *part = (uint16_t *)malloc((size_t)P * R * H * 2);
    static uint16_t rs[P][T][H];
    if (!gh || !gi || !part)
        return 3;
    CHECK_HIP(hipMemcpy(gh, d_gh, (size_t)P * R * H * 2, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(gi, d_gi, (size_t)P * R * K * 4, hipMemcpyDeviceToHost));
    for (int r = 0; r < P; ++r)
        for (int s = 0; s < P; ++s)
            for (int t = 0; t < n[s]; ++t) {
                const size_t j = (size_t)r * R + off[s] + t;
                bad += memcmp(gh + j * H, hidden[s][t], (size_t)H * 2) != 0;
                bad += memcmp(gi + j * K, ids[s][t], (size_t)K * 4) != 0;
            }
    const int gather_bad = bad;

    /* reduce-scatterv: rank q's partial is (q + 1) times the gathered rows */
    for (int q = 0; q < P; ++q)
        for (size_t e = 0; e < (size_t)R * H; ++e)
            part[(size_t)q * R * H + e] = f32_to_bf16((float)(q + 1) * bf16_to_f32(gh[e]));
    CHECK_HIP(hipMemcpy(d_part, part, (size_t)P * R * H * 2, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemset(d_rs, 0x5A, (size_t)P * T * H * 2));
    CHECK_EP(moe_ep_reduce_scatterv(P, n, H, d_part, (int64_t)R * H * 2, d_rs, (int64_t)T * H * 2, NULL));
    CHECK_HIP(hipMemcpy(rs, d_rs, sizeof rs, hipMemcpyDeviceToHost));
    for (int r = 0; r < P; ++r)
        for (int t = 0; t < T; ++t)
            for (int h = 0; h < H; ++h) {
                if (t >= n[r]) {
                    bad += rs[r][t][h] != 0x5A5A;
                    continue;
                }
                float acc = 0.0f;
                for (int q = 0; q < P; ++q)
                    acc += bf16_to_f32(part[((size_t)q * R + off[r] + t) * H + h]);
                bad += rs[r][t][h] != f32_to_bf16(acc);
            }
    (void)hipFree(d_gh);
    (void)hipFree(d_gi);
    (void)hipFree(d_part);
    (void)hipFree(d_rs);
    free(gh);
    free(gi);
    free(part);
    (void)hipFree(d_ws);
    (void)hipFree(d_hidden);
    (void)hipFree(d_ids);
    (void)hipFree(d_wts);
    (void)hipFree(d_eo);
    (void)hipFree(d_out);
    free(ws);
    free(eo);
    if (bad) {
        fprintf(stderr, "%d checks failed (%d in the all-gatherv)\n", bad, gather_bad);
        return 1;
    }
    printf("ok: %d tokens, %d (token, rank) rows, every token back as its row times its weight sum; "
           "%d rows gathered to %d ranks and reduce-scattered bit-exact\n",
           tokens, received, R, P);
    return 0;
}
