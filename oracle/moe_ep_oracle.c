/*
 * CPU oracle of the MoE expert-parallel dispatch / combine exchange and of
 * its all-gatherv / reduce-scatterv variant.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  The product path (the
 * HIP library) never calls it and shares no code with it.
 *
 * Plain, slow, single-threaded C.  Every result is written out from its
 * definition.  Every sum over ranks is taken twice: in single precision
 * (float), adding the terms one by one in ascending rank order starting
 * from +0 -- the fp32 reference the combine's tolerance is stated against,
 * and the value the bf16 results are rounded from -- and in double
 * precision, which holds every sum of bf16 or e4m3 terms exactly and
 * serves the error-bound checks.
 *
 * Sources (FlashInfer and vLLM API documentation pages):
 *  - FlashInfer "flashinfer.moe_ep.NVLinkTwoSidedAlltoAll", dispatch():
 *    a token is delivered to every rank holding one of its chosen experts,
 *    and its global top-k ids, top-k weights and scale row go along with it
 *    in the same slot.
 *  - FlashInfer "flashinfer.moe_ep.NVLinkOneSidedConfig", lamport
 *    paragraph: token t of rank src occupies slot src * tokens_per_rank + t
 *    of a receiving rank, with tokens_per_rank equal to the step's
 *    runtime_max_tokens_per_rank.
 *  - vLLM "device_communicators.all2all", FlashInferNVLinkTwoSidedManager
 *    (MoEEpCommParams(invalid_expert_id=num_experts)): a received slot
 *    beyond the sending rank's token count is marked with expert id
 *    num_experts, outside every rank's range.
 *  - FlashInfer "NVLinkTwoSidedAlltoAll", combine(): each token's expert
 *    outputs, which each rank has weighted and summed over its own experts,
 *    summed over ranks into a [local_num_tokens, hidden] result.
 *  - FlashInfer "NVLinkOneSidedConfig", first options paragraph:
 *    with use_low_precision_combine the combine moves its rows as FP8
 *    values.
 *  - vLLM "device_communicators.all2all", AgRsAll2AllManager.dispatch /
 *    combine: all_gatherv of [hidden, topk_weights, topk_ids] over ranks
 *    in rank order, and reduce_scatterv of the hidden rows by the same
 *    per-rank sizes.
 *
 * Readings taken where the pages are silent (each one is listed with its
 * reason in the design notes of the repository):
 *  - expert e is owned by rank e / (E/P) (contiguous blocks, E % P == 0);
 *    ids outside [0, E) are owned by no rank;
 *  - a token goes to a rank once, however many of its experts live there;
 *  - every slot that receives no row carries invalid_id in all k id
 *    entries, not only the slots past a source's token count;
 *  - sums over ranks are fp32, in ascending rank order from +0;
 *  - output rounding is round-to-nearest-even to bf16;
 *  - extra per-token payload bytes (FlashInfer "NVLinkOneSidedConfig",
 *    options paragraph, extra_payload_bytes_per_token) travel with the
 *    token like its scale row;
 *  - EPLB statistics (same paragraph, eplb_stats_num_experts; FlashInfer
 *    "moe_a2a_dispatch", eplb_local_stats / eplb_gathered_stats): row r of
 *    the gathered [ep_size, n] matrix holds rank r's statistics;
 *  - active rank mask (FlashInfer "flashinfer.comm.moe_a2a_dispatch",
 *    active_rank_mask parameter: a token bound for a rank whose bit is
 *    clear never reaches it): with every virtual rank in one call, a
 *    masked-off rank
 *    neither sends nor receives; nothing is written into its receive
 *    planes and combine produces no rows for it;
 *  - the FP8 combine payload is OCP e4m3fn with one power-of-two (e8m0)
 *    scale per 32 elements, the scale being the smallest power of two
 *    that keeps the block's largest magnitude within 448.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* number formats                                                      */
/* ------------------------------------------------------------------ */

double orc_bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round x to the nearest value on a grid of 'sig' significant bits whose
 * smallest normal exponent is emin: returns the integer significand r
 * (in units of 2^(E - sig + 1)) and the exponent E through *E_out.
 * Ties go to the even significand (rint in the default rounding mode). */
static double round_sig(double a, int sig, int emin, int *E_out)
{
    int e2;
    frexp(a, &e2);               /* a = f * 2^e2, f in [0.5, 1) */
    int E = e2 - 1;              /* a = g * 2^E, g in [1, 2) */
    if (E < emin)
        E = emin;                /* subnormal range keeps the smallest quantum */
    double quantum = ldexp(1.0, E - (sig - 1));
    double r = rint(a / quantum);
    if (r >= ldexp(1.0, sig)) {  /* rounded up into the next binade */
        E += 1;
        r = ldexp(1.0, sig - 1);
    }
    *E_out = E;
    return r;
}

uint16_t orc_double_to_bf16(double x)
{
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    if (isnan(x))
        return (uint16_t)(sign | 0x7FC0u);
    double a = fabs(x);
    if (isinf(a))
        return (uint16_t)(sign | 0x7F80u);
    if (a == 0.0)
        return sign;
    int E;
    double r = round_sig(a, 8, -126, &E);
    if (E > 127)
        return (uint16_t)(sign | 0x7F80u);
    if (r < 128.0)               /* subnormal: exponent field 0 */
        return (uint16_t)(sign | (uint16_t)r);
    return (uint16_t)(sign | (uint16_t)((E + 127) << 7) | (uint16_t)(r - 128.0));
}

/* OCP FP8 E4M3FN: bias 7, no infinities, S.1111.111 is NaN, max 448. */
double orc_e4m3_to_double(uint8_t c)
{
    int s = c >> 7, ef = (c >> 3) & 15, m = c & 7;
    double v;
    if (ef == 15 && m == 7)
        return NAN;
    if (ef == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(1.0 + m / 8.0, ef - 7);
    return s ? -v : v;
}

uint8_t orc_double_to_e4m3(double x)
{
    uint8_t sign = signbit(x) ? 0x80u : 0u;
    if (isnan(x))
        return (uint8_t)(sign | 0x7Fu);
    double a = fabs(x);
    if (a == 0.0)
        return sign;
    int E;
    double r = round_sig(a, 4, -6, &E);
    if (r < 8.0)                 /* subnormal */
        return (uint8_t)(sign | (uint8_t)r);
    int ef = E + 7;
    int m = (int)r - 8;
    if (ef > 15 || (ef == 15 && m == 7))
        return (uint8_t)(sign | 0x7Fu); /* beyond 448: no saturation, NaN */
    return (uint8_t)(sign | (uint8_t)(ef << 3) | (uint8_t)m);
}

/* Smallest e in [-127, 127] with amax <= 448 * 2^e; -127 for amax == 0. */
int orc_fp8_block_exponent(double amax)
{
    int e = -127;
    while (e < 127 && amax > ldexp(448.0, e))
        e++;
    return e;
}

/* Quantise one row of H bf16 values (H % 32 == 0) to e4m3 codes plus one
 * e8m0 scale (exponent + 127) per 32 elements.  A block holding a NaN or
 * an infinity gets scale 0xFF (NaN) and all codes 0x7F. */
void orc_fp8_quantize_row(int H, const uint16_t *x, uint8_t *codes, uint8_t *scales)
{
    for (int b = 0; b < H / 32; ++b) {
        double amax = 0.0;
        int finite = 1;
        for (int i = 0; i < 32; ++i) {
            double v = orc_bf16_to_double(x[b * 32 + i]);
            if (!isfinite(v))
                finite = 0;
            else if (fabs(v) > amax)
                amax = fabs(v);
        }
        if (!finite) {
            scales[b] = 0xFF;
            for (int i = 0; i < 32; ++i)
                codes[b * 32 + i] = 0x7F;
            continue;
        }
        int e = orc_fp8_block_exponent(amax);
        scales[b] = (uint8_t)(e + 127);
        for (int i = 0; i < 32; ++i) {
            double v = orc_bf16_to_double(x[b * 32 + i]);
            codes[b * 32 + i] = orc_double_to_e4m3(ldexp(v, -e));
        }
    }
}

double orc_fp8_dequant(uint8_t code, uint8_t scale)
{
    if (scale == 0xFF)
        return NAN;
    return ldexp(orc_e4m3_to_double(code), (int)scale - 127);
}

/* ------------------------------------------------------------------ */
/* routing                                                             */
/* ------------------------------------------------------------------ */

/* Rank owning expert id, or -1 when the id names no expert. */
int orc_owner(int32_t id, int E, int P)
{
    if (id < 0 || id >= E)
        return -1;
    return id / (E / P);
}

/* 1 when some selected expert of the token lives on rank r. */
int orc_token_goes_to(const int32_t *ids_row, int k, int E, int P, int r)
{
    for (int j = 0; j < k; ++j)
        if (orc_owner(ids_row[j], E, P) == r)
            return 1;
    return 0;
}

/* 1 when rank r takes part in the step (bit r of the active mask). */
static int live(uint64_t active, int r)
{
    return (int)((active >> r) & 1u);
}

/* ------------------------------------------------------------------ */
/* dispatch                                                            */
/* ------------------------------------------------------------------ */

/*
 * Receive planes of destination ranks r in [r0, r1).
 *
 * Inputs are stacked over source ranks: payload [P][T][row_bytes],
 * scales [P][T][srow_bytes] (or NULL), extra [P][T][xrow_bytes] (or
 * NULL), ids [P][T][k], weights [P][T][k] (or NULL), counts [P] (n_s <= T).  Slot q = s * T + t of destination r
 * is valid when t < n_s and r owns one of the token's experts; it then
 * holds the token's payload bytes, scale bytes, all k ids unchanged and
 * all k weights.  Other slots hold invalid_id in every id entry; their
 * payload, scale and weight entries are not defined (left untouched).
 *
 * Outputs, indexed by (r - r0): recv_payload [.][P*T][row_bytes],
 * recv_scales [.][P*T][srow_bytes], recv_extra [.][P*T][xrow_bytes],
 * recv_ids [.][P*T][k],
 * recv_weights [.][P*T][k], recv_valid [.][P*T] (1/0),
 * recv_counts [.][P] (rows received from each source),
 * recv_slots [.][P*T] (valid slots in ascending order, then -1).
 * Any output pointer except recv_ids may be NULL.  Ranks whose bit in
 * active is clear neither send nor receive: their outputs are left
 * untouched, and their tokens reach no rank.
 */
void orc_dispatch(int P, int T, int k, int E, int32_t invalid_id, uint64_t active,
                  const int32_t *counts,
                  const uint8_t *payload, int64_t row_bytes,
                  const uint8_t *scales, int64_t srow_bytes,
                  const uint8_t *extra, int64_t xrow_bytes,
                  const int32_t *ids, const float *weights,
                  int r0, int r1,
                  uint8_t *recv_payload, uint8_t *recv_scales, uint8_t *recv_extra,
                  int32_t *recv_ids, float *recv_weights,
                  uint8_t *recv_valid, int32_t *recv_counts,
                  int32_t *recv_slots)
{
    int64_t slots = (int64_t)P * T;
    for (int r = r0; r < r1; ++r) {
        int64_t ro = r - r0;
        int64_t nslot = 0;
        if (!live(active, r))
            continue;
        for (int s = 0; s < P; ++s) {
            int32_t from_s = 0;
            for (int t = 0; t < T; ++t) {
                int64_t q = (int64_t)s * T + t;
                const int32_t *id_row = ids + ((int64_t)s * T + t) * k;
                int valid = live(active, s) && t < counts[s] && orc_token_goes_to(id_row, k, E, P, r);
                int32_t *out_ids = recv_ids + (ro * slots + q) * k;
                if (recv_valid)
                    recv_valid[ro * slots + q] = (uint8_t)valid;
                if (!valid) {
                    for (int j = 0; j < k; ++j)
                        out_ids[j] = invalid_id;
                    continue;
                }
                from_s++;
                if (recv_slots)
                    recv_slots[ro * slots + nslot] = (int32_t)q;
                nslot++;
                for (int j = 0; j < k; ++j)
                    out_ids[j] = id_row[j];
                if (recv_payload)
                    memcpy(recv_payload + (ro * slots + q) * row_bytes,
                           payload + ((int64_t)s * T + t) * row_bytes, (size_t)row_bytes);
                if (recv_scales && scales && srow_bytes > 0)
                    memcpy(recv_scales + (ro * slots + q) * srow_bytes,
                           scales + ((int64_t)s * T + t) * srow_bytes, (size_t)srow_bytes);
                if (recv_extra && extra && xrow_bytes > 0)
                    memcpy(recv_extra + (ro * slots + q) * xrow_bytes,
                           extra + ((int64_t)s * T + t) * xrow_bytes, (size_t)xrow_bytes);
                if (recv_weights && weights)
                    for (int j = 0; j < k; ++j)
                        recv_weights[(ro * slots + q) * k + j] = weights[((int64_t)s * T + t) * k + j];
            }
            if (recv_counts)
                recv_counts[ro * P + s] = from_s;
        }
        if (recv_slots)
            for (int64_t i = nslot; i < slots; ++i)
                recv_slots[ro * slots + i] = -1;
    }
}

/*
 * EPLB statistics all-gathered during dispatch, as seen by rank r:
 * out [P][n] receives row s = stats [P][n] row s for every rank s taking
 * part; rows of masked-off ranks, and all of out when r itself is masked
 * off, are left untouched.
 */
void orc_eplb_allgather(int P, int n, uint64_t active, const int32_t *stats, int r, int32_t *out)
{
    if (!live(active, r))
        return;
    for (int s = 0; s < P; ++s) {
        if (!live(active, s))
            continue;
        for (int i = 0; i < n; ++i)
            out[(int64_t)s * n + i] = stats[(int64_t)s * n + i];
    }
}

/* ------------------------------------------------------------------ */
/* combine                                                             */
/* ------------------------------------------------------------------ */

/*
 * One token's BF16 combine.  Rank r's row for this token's slot is
 * eo_row0 + r * rank_stride (elements): whatever that rank's expert
 * computation wrote there, read only when the token was sent to r.  ref[H]
 * is the fp32 sum over ranks r that own one of the token's experts, added
 * in ascending r starting from +0; exact[H] is the same sum in double
 * (exact for up to 2^20 bf16 terms); y[H] is ref rounded to bf16.  A token
 * sent nowhere gives +0.  Ranks whose bit in active is clear contribute
 * nothing.
 */
void orc_combine_token_bf16(int P, int H, int k, int E, uint64_t active, const int32_t *ids_row,
                            const uint16_t *eo_row0, int64_t rank_stride,
                            float *ref, double *exact, uint16_t *y)
{
    for (int h = 0; h < H; ++h) {
        ref[h] = 0.0f;
        exact[h] = 0.0;
    }
    for (int r = 0; r < P; ++r) {
        if (!live(active, r) || !orc_token_goes_to(ids_row, k, E, P, r))
            continue;
        const uint16_t *row = eo_row0 + (int64_t)r * rank_stride;
        for (int h = 0; h < H; ++h) {
            double v = orc_bf16_to_double(row[h]);
            ref[h] = ref[h] + (float)v;
            exact[h] += v;
        }
    }
    for (int h = 0; h < H; ++h)
        y[h] = orc_double_to_bf16((double)ref[h]);
}

/*
 * BF16 combine for source ranks s in [s0, s1).  eo holds every rank's
 * expert output for slots slot0 .. slot0 + nslot - 1 ([P][nslot][H]; the
 * whole tensor [P][P*T][H] when slot0 = 0 and nslot = P*T); the slots of
 * the sources s0 .. s1-1 must lie in that range.  ref / exact / y are
 * [s1-s0][T][H]; rows t >= n_s are left untouched (the result holds
 * local_num_tokens rows), and so are all rows of a source whose bit in
 * active is clear.
 */
void orc_combine_bf16(int P, int T, int H, int k, int E, uint64_t active, const int32_t *counts,
                      const int32_t *ids, const uint16_t *eo, int64_t slot0, int64_t nslot,
                      int s0, int s1, float *ref, double *exact, uint16_t *y)
{
    for (int s = s0; s < s1; ++s)
        for (int t = 0; live(active, s) && t < counts[s]; ++t) {
            int64_t q = (int64_t)s * T + t;
            int64_t o = ((int64_t)(s - s0) * T + t) * H;
            orc_combine_token_bf16(P, H, k, E, active, ids + q * k, eo + (q - slot0) * H, nslot * H,
                                   ref + o, exact + o, y + o);
        }
}

/*
 * One token's FP8 combine.  Each owning rank r quantises its row
 * (eo_row0 + r * rank_stride) into codes[r] / scales[r] ([P][H] and
 * [P][H/32]); the token's result is the fp32 sum of the dequantised rows,
 * added in ascending r from +0 (ref_q), rounded to bf16 (y); exact_q is
 * the same sum in double.  Rows of ranks the token was not sent to are
 * left untouched in codes / scales.
 */
void orc_combine_token_fp8(int P, int H, int k, int E, uint64_t active, const int32_t *ids_row,
                           const uint16_t *eo_row0, int64_t rank_stride, uint8_t *codes,
                           uint8_t *scales, float *ref_q, double *exact_q, uint16_t *y)
{
    for (int h = 0; h < H; ++h) {
        ref_q[h] = 0.0f;
        exact_q[h] = 0.0;
    }
    for (int r = 0; r < P; ++r) {
        if (!live(active, r) || !orc_token_goes_to(ids_row, k, E, P, r))
            continue;
        uint8_t *c = codes + (int64_t)r * H;
        uint8_t *sc = scales + (int64_t)r * (H / 32);
        orc_fp8_quantize_row(H, eo_row0 + (int64_t)r * rank_stride, c, sc);
        for (int h = 0; h < H; ++h) {
            double v = orc_fp8_dequant(c[h], sc[h / 32]);
            ref_q[h] = ref_q[h] + (float)v;
            exact_q[h] += v;
        }
    }
    for (int h = 0; h < H; ++h)
        y[h] = orc_double_to_bf16((double)ref_q[h]);
}

/*
 * FP8 combine for source ranks s in [s0, s1); eo as for orc_combine_bf16.
 * The quantised rows a source rank s receives land, one per sending rank
 * r, at slot r * T + t of s's landing planes: land_codes [s1-s0][P*T][H],
 * land_scales [s1-s0][P*T][H/32] (slots with no row are untouched).
 * ref_q / exact_q / y are [s1-s0][T][H].
 */
void orc_combine_fp8(int P, int T, int H, int k, int E, uint64_t active, const int32_t *counts,
                     const int32_t *ids, const uint16_t *eo, int64_t slot0, int64_t nslot,
                     int s0, int s1, uint8_t *land_codes, uint8_t *land_scales, float *ref_q,
                     double *exact_q, uint16_t *y,
                     uint8_t *scratch_codes /* [P][H] */, uint8_t *scratch_scales /* [P][H/32] */)
{
    int64_t slots = (int64_t)P * T;
    for (int s = s0; s < s1; ++s)
        for (int t = 0; live(active, s) && t < counts[s]; ++t) {
            int64_t q = (int64_t)s * T + t;
            int64_t o = ((int64_t)(s - s0) * T + t) * H;
            orc_combine_token_fp8(P, H, k, E, active, ids + q * k, eo + (q - slot0) * H, nslot * H,
                                  scratch_codes, scratch_scales, ref_q + o, exact_q + o, y + o);
            for (int r = 0; r < P; ++r) {
                if (!live(active, r) || !orc_token_goes_to(ids + q * k, k, E, P, r))
                    continue;
                int64_t land = (int64_t)(s - s0) * slots + (int64_t)r * T + t;
                memcpy(land_codes + land * H, scratch_codes + (int64_t)r * H, (size_t)H);
                memcpy(land_scales + land * (H / 32), scratch_scales + (int64_t)r * (H / 32),
                       (size_t)(H / 32));
            }
        }
}

/* ------------------------------------------------------------------ */
/* all-gatherv / reduce-scatterv                                       */
/* ------------------------------------------------------------------ */

/*
 * all_gatherv along dim 0: every rank receives the concatenation, in
 * rank order, of each rank q's first sizes[q] rows.  in [P][in_rows][row_bytes]
 * (rank q's rows start at q * in_rows); out [sum(sizes)][row_bytes] is the
 * one result every rank holds.
 */
void orc_allgatherv(int P, const int32_t *sizes, int64_t row_bytes,
                    const uint8_t *in, int64_t in_rows, uint8_t *out)
{
    int64_t o = 0;
    for (int q = 0; q < P; ++q)
        for (int32_t i = 0; i < sizes[q]; ++i) {
            memcpy(out + o * row_bytes, in + ((int64_t)q * in_rows + i) * row_bytes,
                   (size_t)row_bytes);
            o++;
        }
}

/*
 * reduce_scatterv along dim 0 for rank r: in [P][sum(sizes)][H] bf16 is
 * every rank's full-length partial; rank r keeps rows off_r .. off_r +
 * sizes[r] - 1 summed over ranks, off_r being the sum of sizes[q] for
 * q < r.  ref is the fp32 sum (ascending q, from +0), exact the same sum
 * in double, out = ref rounded to bf16; all three are [sizes[r]][H].
 */
void orc_reduce_scatterv(int P, const int32_t *sizes, int H, const uint16_t *in,
                         int r, float *ref, double *exact, uint16_t *out)
{
    int64_t total = 0, off = 0;
    for (int q = 0; q < P; ++q) {
        if (q < r)
            off += sizes[q];
        total += sizes[q];
    }
    for (int32_t i = 0; i < sizes[r]; ++i)
        for (int h = 0; h < H; ++h) {
            float acc = 0.0f;
            double ex = 0.0;
            for (int q = 0; q < P; ++q) {
                double v = orc_bf16_to_double(in[((int64_t)q * total + off + i) * H + h]);
                acc = acc + (float)v;
                ex += v;
            }
            ref[(int64_t)i * H + h] = acc;
            exact[(int64_t)i * H + h] = ex;
            out[(int64_t)i * H + h] = orc_double_to_bf16((double)acc);
        }
}
