/*
 * CPU oracle for the MoE expert-parallel layout / dispatch / combine path.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library. It shares no code with the GPU path
 * and must never be used as a fallback for it.
 *
 * Plain, single-threaded loops that write out the definitions:
 *
 *  - layout: from the get_dispatch_layout API page (sgl-kernel-npu deep_ep
 *    docs), sections "Parameters" and "Return Values": topk_idx is int64
 *    [num_tokens, num_topk]; num_tokens_per_rank is int32 [num_ranks], how
 *    many tokens go to each rank; num_tokens_per_expert is int32
 *    [num_experts], how many token slots land on each expert;
 *    is_token_in_rank is bool [num_tokens, num_ranks]. Section "Notes": the
 *    expert count is a multiple of the rank count.
 *  - expert -> rank map: DeepEP legacy test analysis page, low-latency
 *    per-expert check excerpt: local expert i of rank r has global id
 *    r * num_local_experts + i, i.e. contiguous blocks, rank(e) = e / L.
 *  - a topk_idx entry of -1 marks an unselected slot: DeepEP Python interface
 *    notes ("4 Python接口"), section "Dispatch API", input parameter topk_idx.
 *  - expert_alignment: same section; per-expert receive counts are rounded up
 *    to a multiple of it (default 1).
 *  - dispatch moves each token's row to the receivers of its selected experts
 *    (same page, opening paragraph of "Dispatch API"); this oracle's receive
 *    buffer holds one contiguous segment per expert, segments in ascending
 *    expert id (so rank-major, local-expert-minor, like the low-latency
 *    packed per-local-expert buffers), rows inside a segment in ascending
 *    (token, slot) order. recv_src_idx maps a received row back to its token,
 *    the role the handle's receive-index tensor plays on the legacy test
 *    analysis page ("legacy.py" handle excerpt).
 *  - combine: legacy test analysis page, low-latency combine check excerpt:
 *    the combined row is x scaled by the sum of the token's weights with
 *    unselected (-1) slots masked to 0; for general expert outputs y that is
 *    out[t] = sum over selected k of w[t,k] * y[row of (t,k)].
 *    The sum is formed in double: each product of an fp32 weight and a bf16
 *    value is exact in double, and the sum of at most 16 of them is within
 *    about 2^-49 of the terms' magnitude, far below bf16 spacing (2^-8
 *    relative). It is then rounded once to the nearest bf16, ties to even.
 *
 * Where the pages are silent the readings are:
 *  - a slot counts once per slot, so a token that repeats an expert sends two
 *    rows to it (the second ordered after the first);
 *  - num_tokens_per_rank counts distinct tokens (column sums of
 *    is_token_in_rank);
 *  - the row order inside a segment is ascending (token, slot);
 *  - padding rows (alignment) and rows past the data carry recv_src_idx = -1
 *    and their contents are unspecified;
 *  - num_tokens = 0 is allowed and gives all-zero counts.
 *
 * Status: 0 ok, -1 invalid argument (size or index out of range), -2 capacity
 * too small.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL -1
#define ORACLE_ECAPACITY -2

/* Checks of the sizes named on the get_dispatch_layout API page:
 * num_topk in [1,16], num_experts in [1,512], num_ranks at most 384,
 * num_experts divisible by num_ranks; every topk_idx entry in [-1, E). */
static int check_routing(const int64_t* idx, int64_t T, int K, int E, int R) {
    if (T < 0 || K < 1 || K > 16 || E < 1 || E > 512 || R < 1 || R > 384 || E % R != 0) return ORACLE_EINVAL;
    for (int64_t i = 0; i < T * (int64_t)K; ++i)
        if (idx[i] < -1 || idx[i] >= E) return ORACLE_EINVAL;
    return ORACLE_OK;
}

int oracle_layout(const int64_t* topk_idx, int64_t T, int K, int E, int R,
                  int32_t* num_tokens_per_rank, int32_t* num_tokens_per_expert, uint8_t* is_token_in_rank) {
    int rc = check_routing(topk_idx, T, K, E, R);
    if (rc) return rc;
    int L = E / R;
    for (int e = 0; e < E; ++e) num_tokens_per_expert[e] = 0;
    for (int64_t i = 0; i < T * (int64_t)R; ++i) is_token_in_rank[i] = 0;
    for (int64_t t = 0; t < T; ++t) {
        for (int k = 0; k < K; ++k) {
            int64_t e = topk_idx[t * K + k];
            if (e < 0) continue;
            num_tokens_per_expert[e] += 1;
            is_token_in_rank[t * R + e / L] = 1;
        }
    }
    for (int r = 0; r < R; ++r) {
        int32_t n = 0;
        for (int64_t t = 0; t < T; ++t) n += is_token_in_rank[t * R + r];
        num_tokens_per_rank[r] = n;
    }
    return ORACLE_OK;
}

/* Rows a receive buffer needs for any routing of this size: every slot
 * selected plus the worst alignment padding of every expert. */
int64_t oracle_capacity(int64_t T, int K, int E, int A) {
    return T * (int64_t)K + (int64_t)E * (int64_t)(A - 1);
}

/* Dispatch: expert_offset [E+1], dst_row [T,K], recv_src_idx [cap], and,
 * when recv_x is non-NULL, the received rows [cap, H] (bf16 bit patterns).
 * x may be NULL when recv_x is NULL. */
int oracle_dispatch(const uint16_t* x, int64_t T, int64_t H, const int64_t* topk_idx, int K, int E, int R, int A,
                    int32_t* expert_offset, int32_t* dst_row, int32_t* recv_src_idx, int64_t cap, uint16_t* recv_x) {
    int rc = check_routing(topk_idx, T, K, E, R);
    if (rc) return rc;
    if (A < 1 || H < 0) return ORACLE_EINVAL;
    if (cap < oracle_capacity(T, K, E, A)) return ORACLE_ECAPACITY;

    /* received rows per expert, one per selected slot */
    int64_t* cnt = (int64_t*)calloc((size_t)E, sizeof(int64_t));
    int64_t* fill = (int64_t*)calloc((size_t)E, sizeof(int64_t));
    for (int64_t t = 0; t < T; ++t)
        for (int k = 0; k < K; ++k)
            if (topk_idx[t * K + k] >= 0) cnt[topk_idx[t * K + k]] += 1;

    /* segment of expert e starts after the aligned sizes of experts 0..e-1 */
    expert_offset[0] = 0;
    for (int e = 0; e < E; ++e) {
        int64_t aligned = (cnt[e] + A - 1) / A * A;
        expert_offset[e + 1] = (int32_t)(expert_offset[e] + aligned);
    }

    for (int64_t r = 0; r < cap; ++r) recv_src_idx[r] = -1;
    for (int e = 0; e < E; ++e) fill[e] = expert_offset[e];

    /* walk the slots in ascending (token, slot) order; each takes the next
     * free row of its expert's segment */
    for (int64_t t = 0; t < T; ++t) {
        for (int k = 0; k < K; ++k) {
            int64_t e = topk_idx[t * K + k];
            if (e < 0) {
                dst_row[t * K + k] = -1;
                continue;
            }
            int64_t row = fill[e];
            fill[e] += 1;
            dst_row[t * K + k] = (int32_t)row;
            recv_src_idx[row] = (int32_t)t;
            if (recv_x)
                for (int64_t h = 0; h < H; ++h) recv_x[row * H + h] = x[t * H + h];
        }
    }
    free(cnt);
    free(fill);
    return ORACLE_OK;
}

static double bf16_bits_to_double(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Nearest bf16 to v, ties to even, as a bit pattern. bf16 has 8 exponent bits
 * (bias 127) and 7 stored fraction bits: in the binade [2^p, 2^(p+1)) with
 * p >= -126 its values are spaced 2^(p-7); below 2^-126 (subnormals) they are
 * spaced 2^-133. The largest finite value is (2 - 2^-7) * 2^127; anything that
 * rounds to 2^128 or beyond is infinity. */
uint16_t oracle_bf16_round(double v) {
    if (isnan(v)) return 0x7FC0;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (a == 0.0) return sign;
    if (isinf(a)) return sign | 0x7F80;
    int e2;
    frexp(a, &e2);      /* a = m * 2^e2, m in [0.5, 1): a in [2^(e2-1), 2^e2) */
    int p = e2 - 1;     /* binade exponent */
    if (p < -126) p = -126;
    double q = ldexp(1.0, p - 7);           /* spacing of bf16 values here */
    double n = nearbyint(a / q);            /* a/q is exact; round to nearest, ties even */
    double r = n * q;
    if (r >= 0x1.0p128) return sign | 0x7F80;
    float f = (float)r;                     /* exact: r is a bf16 value */
    uint32_t u;
    memcpy(&u, &f, 4);
    return sign | (uint16_t)(u >> 16);
}

/* Combine: out[t] = bf16( sum over k with dst_row[t,k] >= 0 of
 * w[t,k] * y[dst_row[t,k]] ), summed in double in ascending k from +0.
 * y has `rows` rows of H bf16 values. A token with no selected slot gives +0. */
int oracle_combine(const uint16_t* y, int64_t rows, int64_t H, const int32_t* dst_row, const float* w,
                   int64_t T, int K, uint16_t* out) {
    if (T < 0 || K < 1 || H < 0 || rows < 0) return ORACLE_EINVAL;
    for (int64_t i = 0; i < T * (int64_t)K; ++i)
        if (dst_row[i] < -1 || dst_row[i] >= rows) return ORACLE_EINVAL;
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t h = 0; h < H; ++h) {
            double acc = 0.0;
            for (int k = 0; k < K; ++k) {
                int32_t row = dst_row[t * K + k];
                if (row < 0) continue;
                acc += (double)w[t * K + k] * bf16_bits_to_double(y[(int64_t)row * H + h]);
            }
            out[t * H + h] = oracle_bf16_round(acc);
        }
    }
    return ORACLE_OK;
}

/* ---------------------------------------------------------------------------
 * Rank-granular ("normal mode") dispatch and combine.
 *
 * DeepEP legacy test analysis page: the normal-mode dispatch call site returns
 * recv_x, recv_topk_idx, recv_topk_weights, the per-expert receive counts and
 * a handle; check_data walks the received rows rank by rank through the
 * receive prefix sums and expects every row of rank i's range to come from a
 * token routed to rank i; the normal-mode combine call adds bias = (bias_0,
 * bias_1) and returns combined_x and combined_topk_weights, and its check
 * divides (combined_x - bias_0 - bias_1) by is_token_in_rank.sum(1) to get x
 * back. DeepEP Python interface notes, "Dispatch API": recv_topk_idx
 * [num_recv, num_topk] int64 and recv_topk_weights [num_recv, num_topk]
 * float accompany recv_x, with -1 for a slot without an expert here; the
 * per-expert counts are aligned to expert_alignment.
 *
 * Readings: a token is received once by every rank that is_token_in_rank
 * flags for it; rank r's rows form one segment, segments in rank order, rows
 * in ascending token order; in a received row, slot k keeps its expert as a
 * rank-local id (e - r*L) and its weight when the expert is on rank r, else
 * -1 and 0; rows past the data carry src -1, ids -1, weights 0; the
 * per-expert receive counts are the layout's counts rounded up to
 * expert_alignment. topk_idx / topk_weights may be absent (NULL), as in the
 * pages' dispatch calls without top-k; then no recv_topk_* is produced.
 * --------------------------------------------------------------------------- */

/* A token reaches at most min(K, R) ranks, so T * min(K, R) rows hold any
 * routing (the num_worst_tokens bound of the Dispatch API notes). */
int64_t oracle_normal_capacity(int64_t T, int K, int R) { return T * (int64_t)(K < R ? K : R); }

int oracle_dispatch_normal(const uint16_t* x, int64_t T, int64_t H, const uint8_t* is_token_in_rank,
                           const int32_t* num_tokens_per_expert, const int64_t* topk_idx, const float* topk_weights,
                           int K, int E, int R, int A, int64_t cap, int32_t* rank_offset, int32_t* send_row,
                           int32_t* recv_src_idx, int64_t* recv_topk_idx, float* recv_topk_weights,
                           int32_t* num_recv_tokens_per_expert, uint16_t* recv_x) {
    if (T < 0 || K < 1 || K > 16 || E < 1 || E > 512 || R < 1 || R > 384 || E % R != 0) return ORACLE_EINVAL;
    if (A < 1 || H < 0 || cap < 0) return ORACLE_EINVAL;
    if (topk_idx) {
        int rc = check_routing(topk_idx, T, K, E, R);
        if (rc) return rc;
    }
    int L = E / R;

    /* rows per rank: the tokens flagged for it */
    int64_t total = 0;
    rank_offset[0] = 0;
    for (int r = 0; r < R; ++r) {
        int64_t c = 0;
        for (int64_t t = 0; t < T; ++t) c += is_token_in_rank[t * R + r] != 0;
        total += c;
        rank_offset[r + 1] = (int32_t)total;
    }
    if (total > cap) return ORACLE_ECAPACITY;
    if (num_tokens_per_expert)
        for (int e = 0; e < E; ++e)
            num_recv_tokens_per_expert[e] = (num_tokens_per_expert[e] + A - 1) / A * A;

    for (int64_t row = 0; row < cap; ++row) {
        recv_src_idx[row] = -1;
        if (topk_idx)
            for (int k = 0; k < K; ++k) {
                recv_topk_idx[row * K + k] = -1;
                recv_topk_weights[row * K + k] = 0.0f;
            }
    }
    /* each rank takes its flagged tokens in ascending order */
    for (int r = 0; r < R; ++r) {
        int64_t row = rank_offset[r];
        for (int64_t t = 0; t < T; ++t) {
            if (!is_token_in_rank[t * R + r]) {
                send_row[t * R + r] = -1;
                continue;
            }
            send_row[t * R + r] = (int32_t)row;
            recv_src_idx[row] = (int32_t)t;
            if (topk_idx)
                for (int k = 0; k < K; ++k) {
                    int64_t e = topk_idx[t * K + k];
                    if (e >= 0 && e / L == r) {
                        recv_topk_idx[row * K + k] = e - (int64_t)r * L;
                        recv_topk_weights[row * K + k] = topk_weights[t * K + k];
                    }
                }
            if (recv_x)
                for (int64_t h = 0; h < H; ++h) recv_x[row * H + h] = x[t * H + h];
            row += 1;
        }
    }
    return ORACLE_OK;
}

/* Normal-mode combine: out[t] = bf16( sum over ranks r that received t of
 * y[send_row[t,r]] + bias_0[t] + bias_1[t] ) (biases optional, NULL = none),
 * summed in double and rounded once; combined_topk_weights[t,k] = sum over
 * those rows of recv_topk_weights[row, k]. */
int oracle_combine_normal(const uint16_t* y, int64_t rows, int64_t H, const int32_t* send_row,
                          const float* recv_topk_weights, const uint16_t* bias0, const uint16_t* bias1, int64_t T,
                          int K, int R, uint16_t* out, float* combined_topk_weights) {
    if (T < 0 || K < 1 || R < 1 || H < 0 || rows < 0) return ORACLE_EINVAL;
    for (int64_t i = 0; i < T * (int64_t)R; ++i)
        if (send_row[i] < -1 || send_row[i] >= rows) return ORACLE_EINVAL;
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t h = 0; h < H; ++h) {
            double acc = 0.0;
            for (int r = 0; r < R; ++r) {
                int32_t row = send_row[t * R + r];
                if (row >= 0) acc += bf16_bits_to_double(y[(int64_t)row * H + h]);
            }
            if (bias0) acc += bf16_bits_to_double(bias0[t * H + h]);
            if (bias1) acc += bf16_bits_to_double(bias1[t * H + h]);
            out[t * H + h] = oracle_bf16_round(acc);
        }
        for (int k = 0; k < K; ++k) {
            double wsum = 0.0;
            for (int r = 0; r < R; ++r) {
                int32_t row = send_row[t * R + r];
                if (row >= 0) wsum += recv_topk_weights[(int64_t)row * K + k];
            }
            combined_topk_weights[t * K + k] = (float)wsum;
        }
    }
    return ORACLE_OK;
}

/* ---------------------------------------------------------------------------
 * FP8 payload: per-token cast to OCP e4m3fn with one scale per 128 channels,
 * and the cast back to bf16.
 *
 * Pages: DeepEP Python interface notes, "Dispatch API": x may be the tuple
 * (x_e4m3 float8_e4m3fn [T, H], x_scales float [T, H/128]) with H divisible
 * by 128, and recv_x is then such a tuple too. DeepEP legacy test analysis
 * page, test data excerpt: per_token_cast_to_fp8 turns a bf16 x into that
 * tuple (its scales may be stored column-major), per_token_cast_back restores
 * bf16; the low-latency dispatch has round_scale and use_ue8m0 options.
 *
 * The pages do not print the cast itself. Reading taken: for each token and
 * each block of 128 channels, amax = max |x| over the block, floored at 1e-4
 * so that a block of zeros keeps a positive scale.
 *   scale format 0 (fp32):      s = amax / 448, codes e4m3(x * (448 / amax)),
 *                               so the block's largest magnitude maps to 448,
 *                               the largest finite e4m3fn value;
 *   scale format 1 (round_scale): s = 2^k, the smallest power of two with
 *                               s >= amax / 448, codes e4m3(x * 2^-k);
 *   scale format 2 (UE8M0):     as format 1, the scale stored as the byte
 *                               k + 127 (an unsigned 8-bit exponent).
 * Cast back: bf16(e4m3 value * s), the product in fp32.
 * Every step is fp32 arithmetic (the 8-bit codes are decided in fp32):
 * 448 / amax and amax / 448 are correctly rounded fp32 divisions, x times the
 * multiplier one fp32 product, clamped to [-448, 448] before encoding.
 *
 * e4m3fn (OCP 8-bit floating point specification, E4M3): 1 sign bit, 4
 * exponent bits with bias 7, 3 fraction bits. Exponent field e in 1..15 gives
 * (1 + f/8) * 2^(e-7), except e = 15, f = 7, which is NaN; so the largest
 * finite value is 1.75 * 2^8 = 448. Exponent field 0 gives subnormals
 * f/8 * 2^-6. There are no infinities. Rounding is to nearest, ties to even.
 * Scales are written row-major [T, H/128].
 * --------------------------------------------------------------------------- */

#define ORACLE_E4M3_MAX 448.0

/* Nearest e4m3fn code to v (ties to even); |v| above 448 saturates to 448. */
uint8_t oracle_e4m3_encode(float v) {
    uint8_t sign = signbit(v) ? 0x80 : 0;
    double a = fabs((double)v);
    if (isnan(v)) return 0x7F;
    if (a > ORACLE_E4M3_MAX) a = ORACLE_E4M3_MAX;
    if (a == 0.0) return sign;
    int e2;
    frexp(a, &e2); /* a in [2^(e2-1), 2^e2) */
    int p = e2 - 1;
    if (p < -6) p = -6;                /* below 2^-6 the spacing is that of subnormals */
    double q = ldexp(1.0, p - 3);      /* spacing of e4m3 values in this binade */
    double r = nearbyint(a / q) * q;   /* a/q is exact; round to nearest, ties even */
    if (r == 0.0) return sign;
    frexp(r, &e2);                     /* r may have moved up to the next binade */
    p = e2 - 1;
    if (p < -6) return sign | (uint8_t)(r / ldexp(1.0, -9)); /* subnormal: f = r / 2^-9 */
    int frac = (int)(r / ldexp(1.0, p - 3)) - 8;              /* r = (8 + f) * 2^(p-3) */
    return sign | (uint8_t)((p + 7) << 3) | (uint8_t)frac;
}

float oracle_e4m3_decode(uint8_t c) {
    int e = (c >> 3) & 15, f = c & 7;
    if (e == 15 && f == 7) return NAN;
    double m = (e == 0) ? ldexp((double)f, -9) : ldexp((double)(8 + f), e - 10);
    return (float)((c & 0x80) ? -m : m);
}

static float bf16_bits_to_float(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* Smallest k with 2^k >= s (s > 0, finite). */
static int ceil_log2f(float s) {
    int e;
    float m = frexpf(s, &e); /* s = m * 2^e, m in [0.5, 1) */
    return (m == 0.5f) ? e - 1 : e;
}

int oracle_cast_to_fp8(const uint16_t* x, int64_t T, int64_t H, int scale_format, uint8_t* q, void* scales) {
    if (T < 0 || H < 0 || H % 128 != 0 || scale_format < 0 || scale_format > 2) return ORACLE_EINVAL;
    int64_t nb = H / 128;
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t b = 0; b < nb; ++b) {
            const uint16_t* xb = x + t * H + b * 128;
            float amax = 0.0f;
            for (int j = 0; j < 128; ++j) amax = fmaxf(amax, fabsf(bf16_bits_to_float(xb[j])));
            if (amax < 1e-4f) amax = 1e-4f;
            float mul;
            if (scale_format == 0) {
                mul = 448.0f / amax;
                ((float*)scales)[t * nb + b] = amax / 448.0f;
            } else {
                int k = ceil_log2f(amax / 448.0f);
                mul = ldexpf(1.0f, -k);
                if (scale_format == 1)
                    ((float*)scales)[t * nb + b] = ldexpf(1.0f, k);
                else
                    ((uint8_t*)scales)[t * nb + b] = (uint8_t)(k + 127);
            }
            for (int j = 0; j < 128; ++j) {
                float v = bf16_bits_to_float(xb[j]) * mul;
                if (v > 448.0f) v = 448.0f;
                if (v < -448.0f) v = -448.0f;
                q[t * H + b * 128 + j] = oracle_e4m3_encode(v);
            }
        }
    }
    return ORACLE_OK;
}

int oracle_cast_back(const uint8_t* q, const void* scales, int64_t T, int64_t H, int scale_format, uint16_t* out) {
    if (T < 0 || H < 0 || H % 128 != 0 || scale_format < 0 || scale_format > 2) return ORACLE_EINVAL;
    int64_t nb = H / 128;
    for (int64_t t = 0; t < T; ++t)
        for (int64_t b = 0; b < nb; ++b) {
            float s = (scale_format == 2) ? ldexpf(1.0f, (int)((const uint8_t*)scales)[t * nb + b] - 127)
                                          : ((const float*)scales)[t * nb + b];
            for (int j = 0; j < 128; ++j) {
                int64_t i = t * H + b * 128 + j;
                float v = oracle_e4m3_decode(q[i]) * s;
                out[i] = oracle_bf16_round((double)v);
            }
        }
    return ORACLE_OK;
}

/* ---------------------------------------------------------------------------
 * Fixed-capacity packed layout (the low-latency dispatch's receive buffers).
 *
 * DeepEP legacy test analysis page, low-latency dispatch call and per-expert
 * check: packed_recv_x holds one fixed-size buffer per local expert,
 * packed_recv_count[i] is the number of valid rows of expert i and equals the
 * number of selected slots naming that expert, and the handle carries
 * recv_src_info per expert (here the source token of each valid row).
 * DeepEP Python interface notes, "Dispatch API", num_worst_tokens: a receive
 * size fixed in advance avoids a host synchronisation.
 *
 * Readings: every expert owns rows [e*cap, (e+1)*cap) of a [E*cap, H] buffer;
 * its valid rows come first, in ascending (token, slot) order as in the
 * expert-granular dispatch; a slot whose rank inside its expert is >= cap is
 * dropped (dst_row -1, not counted); rows past an expert's count have
 * recv_src_info -1 and unspecified contents. With a single source the
 * layout range per (expert, source) is (0, count), so it is not produced.
 * cumulative_recv_stats (optional) accumulates packed_recv_count, as the
 * pages' cumulative_local_expert_recv_stats does.
 * --------------------------------------------------------------------------- */
int oracle_dispatch_packed(const uint16_t* x, int64_t T, int64_t H, const int64_t* topk_idx, int K, int E, int R,
                           int64_t cap, int32_t* packed_recv_count, int32_t* recv_src_info, int32_t* dst_row,
                           int32_t* cumulative_recv_stats, uint16_t* packed_recv_x) {
    int rc = check_routing(topk_idx, T, K, E, R);
    if (rc) return rc;
    if (cap < 0 || H < 0) return ORACLE_EINVAL;
    for (int e = 0; e < E; ++e) packed_recv_count[e] = 0;
    for (int64_t r = 0; r < (int64_t)E * cap; ++r) recv_src_info[r] = -1;
    for (int64_t t = 0; t < T; ++t) {
        for (int k = 0; k < K; ++k) {
            int64_t e = topk_idx[t * K + k];
            dst_row[t * K + k] = -1;
            if (e < 0 || packed_recv_count[e] >= cap) continue;
            int64_t row = e * cap + packed_recv_count[e];
            packed_recv_count[e] += 1;
            dst_row[t * K + k] = (int32_t)row;
            recv_src_info[row] = (int32_t)t;
            if (packed_recv_x)
                for (int64_t h = 0; h < H; ++h) packed_recv_x[row * H + h] = x[t * H + h];
        }
    }
    if (cumulative_recv_stats)
        for (int e = 0; e < E; ++e) cumulative_recv_stats[e] += packed_recv_count[e];
    return ORACLE_OK;
}
