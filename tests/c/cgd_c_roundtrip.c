/* A plain C program that uses libcgd through include/cgd.h alone: the HIP
 * runtime for device memory and a stream, no Python and no torch. Test
 * infrastructure, not part of the library: tests/test_gpu_c_program.py
 * builds it with gcc and runs it. Inputs come from the seeded generator
 * (libsynth); every output is checked against the CPU oracle (liboracle):
 * layout, handle and received rows bit for bit (expert-granular, also with
 * the FP8 cast on dispatch, and rank-granular in bf16 and with the FP8
 * cast), the combine within
 * 1e-2 of the sum of its terms' magnitudes with > 99 % of values
 * bit-identical. Exit status 0 and a last line "ok" when every check passes. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "cgd.h"

/* generator and oracle entry points (exported by libsynth / liboracle) */
uint64_t synth_stream_key(uint64_t seed, uint64_t salt, uint64_t stream);
int synth_topk_uniform(uint64_t key, int64_t T, int K, int E, int64_t* out);
void synth_normal_bf16(uint64_t key, int64_t offset, int64_t n, uint16_t* out);
void synth_softmax_weights(uint64_t key, int64_t T, int K, float* out);
int oracle_layout(const int64_t* topk_idx, int64_t T, int K, int E, int R, int32_t* num_tokens_per_rank,
                  int32_t* num_tokens_per_expert, uint8_t* is_token_in_rank);
int64_t oracle_capacity(int64_t T, int K, int E, int A);
int oracle_dispatch(const uint16_t* x, int64_t T, int64_t H, const int64_t* topk_idx, int K, int E, int R, int A,
                    int32_t* expert_offset, int32_t* dst_row, int32_t* recv_src_idx, int64_t cap, uint16_t* recv_x);
int oracle_combine(const uint16_t* y, int64_t rows, int64_t H, const int32_t* dst_row, const float* w, int64_t T,
                   int K, uint16_t* out);
int64_t oracle_normal_capacity(int64_t T, int K, int R);
int oracle_dispatch_normal(const uint16_t* x, int64_t T, int64_t H, const uint8_t* is_token_in_rank,
                           const int32_t* num_tokens_per_expert, const int64_t* topk_idx, const float* topk_weights,
                           int K, int E, int R, int A, int64_t cap, int32_t* rank_offset, int32_t* send_row,
                           int32_t* recv_src_idx, int64_t* recv_topk_idx, float* recv_topk_weights,
                           int32_t* num_recv_tokens_per_expert, uint16_t* recv_x);
int oracle_cast_to_fp8(const uint16_t* x, int64_t T, int64_t H, int scale_format, uint8_t* q, void* scales);

static int failures = 0;

#define HIP_OK(call)                                                                     \
    do {                                                                                 \
        hipError_t e_ = (call);                                                          \
        if (e_ != hipSuccess) {                                                          \
            fprintf(stderr, "%s:%d: %s: %s\n", __FILE__, __LINE__, #call, hipGetErrorString(e_)); \
            exit(2);                                                                     \
        }                                                                                \
    } while (0)

#define CGD_OK_(call)                                                                    \
    do {                                                                                 \
        int s_ = (call);                                                                 \
        if (s_ != CGD_OK) {                                                              \
            fprintf(stderr, "%s:%d: %s returned %d: %s\n", __FILE__, __LINE__, #call, s_, cgd_last_error()); \
            exit(3);                                                                     \
        }                                                                                \
    } while (0)

static void expect(int cond, const char* what, const char* name) {
    if (!cond) {
        fprintf(stderr, "[%s] mismatch: %s\n", name, what);
        ++failures;
    }
}

static void* dev_alloc(size_t bytes) {
    void* p = NULL;
    HIP_OK(hipMalloc(&p, bytes ? bytes : 1));
    return p;
}

static void* dev_copy(const void* host, size_t bytes) {
    void* p = dev_alloc(bytes);
    if (bytes) HIP_OK(hipMemcpy(p, host, bytes, hipMemcpyHostToDevice));
    return p;
}

static void* host_copy(const void* dev, size_t bytes) {
    void* p = malloc(bytes ? bytes : 1);
    if (bytes) HIP_OK(hipMemcpy(p, dev, bytes, hipMemcpyDeviceToHost));
    return p;
}

static double bf16_value(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static void run_case(const char* name, int64_t T, int K, int E, int R, int H, int A, uint64_t seed,
                     hipStream_t stream) {
    printf("[%s] T=%lld K=%d E=%d R=%d H=%d alignment=%d\n", name, (long long)T, K, E, R, H, A);
    fflush(stdout);
    const int64_t TK = T * K;
    int64_t* idx = malloc(sizeof(int64_t) * (size_t)TK);
    uint16_t* x = malloc(sizeof(uint16_t) * (size_t)(T * H));
    float* w = malloc(sizeof(float) * (size_t)TK);
    if (synth_topk_uniform(synth_stream_key(seed, 91, 2), T, K, E, idx) != 0) exit(4);
    for (int64_t i = 0; i < TK; ++i)
        if (i % 7 == 3) idx[i] = -1;  /* some slots not selected */
    synth_normal_bf16(synth_stream_key(seed, 91, 1), 0, T * H, x);
    synth_softmax_weights(synth_stream_key(seed, 91, 3), T, K, w);

    const int64_t cap = cgd_dispatch_capacity(T, K, E, A);
    expect(cap == oracle_capacity(T, K, E, A), "capacity", name);

    /* oracle */
    int32_t* o_ntpr = malloc(sizeof(int32_t) * (size_t)R);
    int32_t* o_ntpe = malloc(sizeof(int32_t) * (size_t)E);
    uint8_t* o_itr = malloc((size_t)(T * R));
    int32_t* o_off = malloc(sizeof(int32_t) * (size_t)(E + 1));
    int32_t* o_dst = malloc(sizeof(int32_t) * (size_t)TK);
    int32_t* o_src = malloc(sizeof(int32_t) * (size_t)cap);
    uint16_t* o_recv = calloc((size_t)(cap * H), sizeof(uint16_t));
    if (oracle_layout(idx, T, K, E, R, o_ntpr, o_ntpe, o_itr) != 0) exit(5);
    if (oracle_dispatch(x, T, H, idx, K, E, R, A, o_off, o_dst, o_src, cap, o_recv) != 0) exit(5);

    /* device inputs and outputs */
    void* d_x = dev_copy(x, sizeof(uint16_t) * (size_t)(T * H));
    int64_t* d_idx = dev_copy(idx, sizeof(int64_t) * (size_t)TK);
    float* d_w = dev_copy(w, sizeof(float) * (size_t)TK);
    void* d_recv = dev_alloc(sizeof(uint16_t) * (size_t)(cap * H));
    int32_t* d_ntpr = dev_alloc(sizeof(int32_t) * (size_t)R);
    int32_t* d_ntpe = dev_alloc(sizeof(int32_t) * (size_t)E);
    uint8_t* d_itr = dev_alloc((size_t)(T * R));
    int32_t* d_off = dev_alloc(sizeof(int32_t) * (size_t)(E + 1));
    int32_t* d_counts = dev_alloc(sizeof(int32_t) * (size_t)E);
    int32_t* d_src = dev_alloc(sizeof(int32_t) * (size_t)cap);
    int32_t* d_dst = dev_alloc(sizeof(int32_t) * (size_t)TK);
    const size_t ws_bytes = cgd_dispatch_workspace_bytes(T, K, E, R);
    const size_t lws_bytes = cgd_layout_workspace_bytes(T, K, E, R);
    void* d_ws = dev_alloc(ws_bytes);
    void* d_lws = dev_alloc(lws_bytes);
    HIP_OK(hipMemset(d_ws, 0, ws_bytes));
    HIP_OK(hipMemset(d_lws, 0, lws_bytes));

    /* a receive capacity below the bound is refused before anything is enqueued */
    int s = cgd_dispatch(d_x, T, H, d_idx, K, E, R, A, d_recv, cap - 1, d_off, d_counts, d_src, d_dst, d_ws, ws_bytes,
                         stream);
    expect(s == CGD_ERR_CAPACITY, "capacity check status", name);
    expect(strlen(cgd_last_error()) > 0, "error message", name);

    /* layout alone, then layout and dispatch in one call, on one stream */
    CGD_OK_(cgd_get_dispatch_layout(d_idx, T, K, E, R, d_ntpr, d_ntpe, d_itr, d_lws, lws_bytes, stream));
    HIP_OK(hipStreamSynchronize(stream));
    int32_t* g_ntpr = host_copy(d_ntpr, sizeof(int32_t) * (size_t)R);
    int32_t* g_ntpe = host_copy(d_ntpe, sizeof(int32_t) * (size_t)E);
    uint8_t* g_itr = host_copy(d_itr, (size_t)(T * R));
    expect(!memcmp(g_ntpr, o_ntpr, sizeof(int32_t) * (size_t)R), "layout num_tokens_per_rank", name);
    expect(!memcmp(g_ntpe, o_ntpe, sizeof(int32_t) * (size_t)E), "layout num_tokens_per_expert", name);
    expect(!memcmp(g_itr, o_itr, (size_t)(T * R)), "layout is_token_in_rank", name);
    HIP_OK(hipMemset(d_ntpr, 0xff, sizeof(int32_t) * (size_t)R));
    HIP_OK(hipMemset(d_ntpe, 0xff, sizeof(int32_t) * (size_t)E));
    HIP_OK(hipMemset(d_itr, 0xff, (size_t)(T * R)));

    CGD_OK_(cgd_layout_and_dispatch(d_x, T, H, d_idx, K, E, R, A, d_recv, cap, d_ntpr, d_ntpe, d_itr, d_off,
                                    d_counts, d_src, d_dst, d_ws, ws_bytes, stream));
    HIP_OK(hipStreamSynchronize(stream));
    free(g_ntpr); free(g_ntpe); free(g_itr);
    g_ntpr = host_copy(d_ntpr, sizeof(int32_t) * (size_t)R);
    g_ntpe = host_copy(d_ntpe, sizeof(int32_t) * (size_t)E);
    g_itr = host_copy(d_itr, (size_t)(T * R));
    int32_t* g_off = host_copy(d_off, sizeof(int32_t) * (size_t)(E + 1));
    int32_t* g_counts = host_copy(d_counts, sizeof(int32_t) * (size_t)E);
    int32_t* g_src = host_copy(d_src, sizeof(int32_t) * (size_t)cap);
    int32_t* g_dst = host_copy(d_dst, sizeof(int32_t) * (size_t)TK);
    uint16_t* g_recv = host_copy(d_recv, sizeof(uint16_t) * (size_t)(cap * H));
    expect(!memcmp(g_ntpr, o_ntpr, sizeof(int32_t) * (size_t)R), "num_tokens_per_rank", name);
    expect(!memcmp(g_ntpe, o_ntpe, sizeof(int32_t) * (size_t)E), "num_tokens_per_expert", name);
    expect(!memcmp(g_itr, o_itr, (size_t)(T * R)), "is_token_in_rank", name);
    expect(!memcmp(g_off, o_off, sizeof(int32_t) * (size_t)(E + 1)), "expert_offset", name);
    expect(!memcmp(g_dst, o_dst, sizeof(int32_t) * (size_t)TK), "dst_row", name);
    expect(!memcmp(g_src, o_src, sizeof(int32_t) * (size_t)cap), "recv_src_idx", name);
    int counts_ok = 1, rows_ok = 1;
    for (int e = 0; e < E; ++e) counts_ok &= g_counts[e] == o_off[e + 1] - o_off[e];
    for (int64_t r = 0; r < cap; ++r)
        if (o_src[r] >= 0) rows_ok &= !memcmp(g_recv + r * H, o_recv + r * H, sizeof(uint16_t) * (size_t)H);
    expect(counts_ok, "num_recv_tokens_per_expert", name);
    expect(rows_ok, "received rows", name);

    /* the same call with the FP8 cast on the way (UE8M0 scales): handle as
     * above, every received row the oracle's per-token cast of its token */
    if (H % 128 == 0) {
        const int nsb = H / 128;
        uint8_t* o_q = malloc((size_t)(T * H));
        uint8_t* o_s = malloc((size_t)(T * nsb));
        if (oracle_cast_to_fp8(x, T, H, CGD_SCALE_UE8M0, o_q, o_s) != 0) exit(5);
        void* d_rq = dev_alloc((size_t)(cap * H));
        void* d_rs = dev_alloc((size_t)(cap * nsb));
        CGD_OK_(cgd_layout_and_dispatch_cast_fp8(d_x, T, H, d_idx, K, E, R, A, CGD_SCALE_UE8M0, d_rq, d_rs, cap,
                                                 d_ntpr, d_ntpe, d_itr, d_off, d_counts, d_src, d_dst, d_ws, ws_bytes,
                                                 stream));
        HIP_OK(hipStreamSynchronize(stream));
        int32_t* f_dst = host_copy(d_dst, sizeof(int32_t) * (size_t)TK);
        int32_t* f_src = host_copy(d_src, sizeof(int32_t) * (size_t)cap);
        uint8_t* f_q = host_copy(d_rq, (size_t)(cap * H));
        uint8_t* f_s = host_copy(d_rs, (size_t)(cap * nsb));
        expect(!memcmp(f_dst, o_dst, sizeof(int32_t) * (size_t)TK), "FP8 dst_row", name);
        expect(!memcmp(f_src, o_src, sizeof(int32_t) * (size_t)cap), "FP8 recv_src_idx", name);
        int fp8_ok = 1;
        for (int64_t i = 0; i < TK; ++i) {
            const int32_t r = o_dst[i];
            if (r < 0) continue;
            fp8_ok &= !memcmp(f_q + (int64_t)r * H, o_q + (i / K) * H, (size_t)H);
            fp8_ok &= !memcmp(f_s + (int64_t)r * nsb, o_s + (i / K) * nsb, (size_t)nsb);
        }
        expect(fp8_ok, "received FP8 codes and UE8M0 scales", name);
        printf("[%s] cast on dispatch: FP8 rows as the oracle's cast\n", name);
        free(f_dst); free(f_src); free(f_q); free(f_s); free(o_q); free(o_s);
        HIP_OK(hipFree(d_rq)); HIP_OK(hipFree(d_rs));
    }

    /* combine of independent expert outputs */
    uint16_t* y = malloc(sizeof(uint16_t) * (size_t)(cap * H));
    synth_normal_bf16(synth_stream_key(seed, 91, 4), 0, cap * H, y);
    void* d_y = dev_copy(y, sizeof(uint16_t) * (size_t)(cap * H));
    void* d_out = dev_alloc(sizeof(uint16_t) * (size_t)(T * H));
    CGD_OK_(cgd_combine(d_y, cap, H, d_dst, d_w, T, K, d_out, stream));
    HIP_OK(hipStreamSynchronize(stream));
    uint16_t* g_out = host_copy(d_out, sizeof(uint16_t) * (size_t)(T * H));
    uint16_t* o_out = malloc(sizeof(uint16_t) * (size_t)(T * H));
    if (oracle_combine(y, cap, H, o_dst, w, T, K, o_out) != 0) exit(5);
    int64_t same = 0, bad = 0;
    for (int64_t t = 0; t < T; ++t) {
        for (int h = 0; h < H; ++h) {
            const uint16_t gb = g_out[t * H + h], ob = o_out[t * H + h];
            double mag = 0.0;
            for (int k = 0; k < K; ++k) {
                const int32_t row = o_dst[t * K + k];
                if (row >= 0) mag += fabs((double)w[t * K + k] * bf16_value(y[(int64_t)row * H + h]));
            }
            const double err = fabs(bf16_value(gb) - bf16_value(ob));
            if (!(err <= 1e-2 * mag + ldexp(1.0, -133))) ++bad;
            if (gb == ob || (((gb | ob) & 0x7FFF) == 0)) ++same;
        }
    }
    expect(bad == 0, "combine tolerance", name);
    expect(T == 0 || (double)same / (double)(T * H) > 0.99, "combine bit-identical fraction", name);
    printf("[%s] combine: %lld of %lld values bit-identical\n", name, (long long)same, (long long)(T * H));

    void* dev_bufs[] = {d_x, d_idx, d_w, d_recv, d_ntpr, d_ntpe, d_itr, d_off, d_counts, d_src, d_dst,
                        d_ws, d_lws, d_y, d_out};
    for (size_t i = 0; i < sizeof dev_bufs / sizeof dev_bufs[0]; ++i) HIP_OK(hipFree(dev_bufs[i]));
    void* host_bufs[] = {idx, x, w, o_ntpr, o_ntpe, o_itr, o_off, o_dst, o_src, o_recv, g_ntpr, g_ntpe, g_itr,
                         g_off, g_counts, g_src, g_dst, g_recv, y, g_out, o_out};
    for (size_t i = 0; i < sizeof host_bufs / sizeof host_bufs[0]; ++i) free(host_bufs[i]);
}

/* Rank-granular layout + dispatch in one call (bf16), and with the FP8 cast
 * done by the plan's idle blocks: layout, plan, rows and per-row outputs
 * against the oracle's rank-granular dispatch and per-token cast; an apply
 * from the plan the bf16 call leaves in the workspace gives the same rows. */
static void run_normal_case(const char* name, int64_t T, int K, int E, int R, int H, int A, uint64_t seed,
                            hipStream_t stream) {
    printf("[%s] T=%lld K=%d E=%d R=%d H=%d alignment=%d\n", name, (long long)T, K, E, R, H, A);
    fflush(stdout);
    const int64_t TK = T * K, nsb = H / 128;
    int64_t* idx = malloc(sizeof(int64_t) * (size_t)TK);
    uint16_t* x = malloc(sizeof(uint16_t) * (size_t)(T * H));
    float* w = malloc(sizeof(float) * (size_t)TK);
    if (synth_topk_uniform(synth_stream_key(seed, 92, 2), T, K, E, idx) != 0) exit(4);
    for (int64_t i = 0; i < TK; ++i)
        if (i % 5 == 2) idx[i] = -1;
    synth_normal_bf16(synth_stream_key(seed, 92, 1), 0, T * H, x);
    synth_softmax_weights(synth_stream_key(seed, 92, 3), T, K, w);
    const int64_t cap = cgd_normal_capacity(T, K, R);
    expect(cap == oracle_normal_capacity(T, K, R), "normal capacity", name);

    int32_t* o_ntpr = malloc(sizeof(int32_t) * (size_t)R);
    int32_t* o_ntpe = malloc(sizeof(int32_t) * (size_t)E);
    uint8_t* o_itr = malloc((size_t)(T * R));
    int32_t* o_roff = malloc(sizeof(int32_t) * (size_t)(R + 1));
    int32_t* o_send = malloc(sizeof(int32_t) * (size_t)(T * R));
    int32_t* o_src = malloc(sizeof(int32_t) * (size_t)cap);
    int64_t* o_ridx = malloc(sizeof(int64_t) * (size_t)(cap * K));
    float* o_rw = malloc(sizeof(float) * (size_t)(cap * K));
    int32_t* o_nre = malloc(sizeof(int32_t) * (size_t)E);
    uint16_t* o_recv = calloc((size_t)(cap * H), sizeof(uint16_t));
    uint8_t* o_q = malloc((size_t)(T * H));
    float* o_s = malloc(sizeof(float) * (size_t)(T * nsb));
    if (oracle_layout(idx, T, K, E, R, o_ntpr, o_ntpe, o_itr) != 0) exit(5);
    if (oracle_dispatch_normal(x, T, H, o_itr, o_ntpe, idx, w, K, E, R, A, cap, o_roff, o_send, o_src, o_ridx, o_rw,
                               o_nre, o_recv) != 0)
        exit(5);
    if (oracle_cast_to_fp8(x, T, H, CGD_SCALE_F32, o_q, o_s) != 0) exit(5);

    void* d_x = dev_copy(x, sizeof(uint16_t) * (size_t)(T * H));
    int64_t* d_idx = dev_copy(idx, sizeof(int64_t) * (size_t)TK);
    float* d_w = dev_copy(w, sizeof(float) * (size_t)TK);
    int32_t* d_ntpr = dev_alloc(sizeof(int32_t) * (size_t)R);
    int32_t* d_ntpe = dev_alloc(sizeof(int32_t) * (size_t)E);
    uint8_t* d_itr = dev_alloc((size_t)(T * R));
    int32_t* d_roff = dev_alloc(sizeof(int32_t) * (size_t)(R + 1));
    int32_t* d_nre = dev_alloc(sizeof(int32_t) * (size_t)E);
    int32_t* d_src = dev_alloc(sizeof(int32_t) * (size_t)cap);
    int32_t* d_send = dev_alloc(sizeof(int32_t) * (size_t)(T * R));
    int64_t* d_ridx = dev_alloc(sizeof(int64_t) * (size_t)(cap * K));
    float* d_rw = dev_alloc(sizeof(float) * (size_t)(cap * K));
    void* d_recv = dev_alloc(sizeof(uint16_t) * (size_t)(cap * H));
    void* d_xq = dev_alloc((size_t)(T * H));
    void* d_xs = dev_alloc(sizeof(float) * (size_t)(T * nsb));
    void* d_rq = dev_alloc((size_t)(cap * H));
    void* d_rs = dev_alloc(sizeof(float) * (size_t)(cap * nsb));
    const size_t ws_bytes = cgd_layout_and_normal_workspace_bytes(T, K, E, R);
    void* d_ws = dev_alloc(ws_bytes);
    HIP_OK(hipMemset(d_ws, 0, ws_bytes));

    for (int fp8 = 0; fp8 < 2; ++fp8) {
        if (fp8)
            CGD_OK_(cgd_layout_and_normal_dispatch_cast_fp8(d_x, T, H, d_idx, d_w, K, E, R, A, CGD_SCALE_F32, d_xq,
                                                            d_xs, d_rq, d_rs, cap, d_ntpr, d_ntpe, d_itr, d_roff,
                                                            d_nre, d_src, d_send, d_ridx, d_rw, d_ws, ws_bytes,
                                                            stream));
        else
            CGD_OK_(cgd_layout_and_normal_dispatch(d_x, T, H, d_idx, d_w, K, E, R, A, d_recv, cap, d_ntpr, d_ntpe,
                                                   d_itr, d_roff, d_nre, d_src, d_send, d_ridx, d_rw, d_ws, ws_bytes,
                                                   stream));
        HIP_OK(hipStreamSynchronize(stream));
        int32_t* g_ntpr = host_copy(d_ntpr, sizeof(int32_t) * (size_t)R);
        int32_t* g_ntpe = host_copy(d_ntpe, sizeof(int32_t) * (size_t)E);
        uint8_t* g_itr = host_copy(d_itr, (size_t)(T * R));
        int32_t* g_roff = host_copy(d_roff, sizeof(int32_t) * (size_t)(R + 1));
        int32_t* g_nre = host_copy(d_nre, sizeof(int32_t) * (size_t)E);
        int32_t* g_src = host_copy(d_src, sizeof(int32_t) * (size_t)cap);
        int32_t* g_send = host_copy(d_send, sizeof(int32_t) * (size_t)(T * R));
        int64_t* g_ridx = host_copy(d_ridx, sizeof(int64_t) * (size_t)(cap * K));
        float* g_rw = host_copy(d_rw, sizeof(float) * (size_t)(cap * K));
        expect(!memcmp(g_ntpr, o_ntpr, sizeof(int32_t) * (size_t)R), "normal num_tokens_per_rank", name);
        expect(!memcmp(g_ntpe, o_ntpe, sizeof(int32_t) * (size_t)E), "normal num_tokens_per_expert", name);
        expect(!memcmp(g_itr, o_itr, (size_t)(T * R)), "normal is_token_in_rank", name);
        expect(!memcmp(g_roff, o_roff, sizeof(int32_t) * (size_t)(R + 1)), "rank_offset", name);
        expect(!memcmp(g_nre, o_nre, sizeof(int32_t) * (size_t)E), "normal num_recv_tokens_per_expert", name);
        expect(!memcmp(g_src, o_src, sizeof(int32_t) * (size_t)cap), "normal recv_src_idx", name);
        expect(!memcmp(g_send, o_send, sizeof(int32_t) * (size_t)(T * R)), "send_row", name);
        int meta_ok = 1, rows_ok = 1;
        for (int64_t r = 0; r < cap; ++r) {
            if (o_src[r] < 0) continue;
            meta_ok &= !memcmp(g_ridx + r * K, o_ridx + r * K, sizeof(int64_t) * (size_t)K);
            meta_ok &= !memcmp(g_rw + r * K, o_rw + r * K, sizeof(float) * (size_t)K);
        }
        if (fp8) {
            uint8_t* g_xq = host_copy(d_xq, (size_t)(T * H));
            float* g_xs = host_copy(d_xs, sizeof(float) * (size_t)(T * nsb));
            uint8_t* g_rq = host_copy(d_rq, (size_t)(cap * H));
            float* g_rs = host_copy(d_rs, sizeof(float) * (size_t)(cap * nsb));
            expect(!memcmp(g_xq, o_q, (size_t)(T * H)), "cast codes", name);
            expect(!memcmp(g_xs, o_s, sizeof(float) * (size_t)(T * nsb)), "cast scales", name);
            for (int64_t r = 0; r < cap; ++r) {
                if (o_src[r] < 0) continue;
                rows_ok &= !memcmp(g_rq + r * H, o_q + (int64_t)o_src[r] * H, (size_t)H);
                rows_ok &= !memcmp(g_rs + r * nsb, o_s + (int64_t)o_src[r] * nsb, sizeof(float) * (size_t)nsb);
            }
            free(g_xq); free(g_xs); free(g_rq); free(g_rs);
        } else {
            uint16_t* g_recv = host_copy(d_recv, sizeof(uint16_t) * (size_t)(cap * H));
            for (int64_t r = 0; r < cap; ++r)
                if (o_src[r] >= 0) rows_ok &= !memcmp(g_recv + r * H, o_recv + r * H, sizeof(uint16_t) * (size_t)H);
            free(g_recv);
        }
        expect(meta_ok, "recv_topk_idx / recv_topk_weights", name);
        expect(rows_ok, fp8 ? "received FP8 rows" : "received rows", name);
        if (!fp8) {
            /* the workspace now holds the plan: an apply from it gives the same rows */
            void* d_recv2 = dev_alloc(sizeof(uint16_t) * (size_t)(cap * H));
            int32_t* d_src2 = dev_alloc(sizeof(int32_t) * (size_t)cap);
            int32_t* d_send2 = dev_alloc(sizeof(int32_t) * (size_t)(T * R));
            CGD_OK_(cgd_normal_dispatch_apply(d_x, T, H, NULL, NULL, K, E, R, d_recv2, cap, d_roff, d_src2, d_send2,
                                              NULL, NULL, d_ws, ws_bytes, stream));
            HIP_OK(hipStreamSynchronize(stream));
            int32_t* g_send2 = host_copy(d_send2, sizeof(int32_t) * (size_t)(T * R));
            int32_t* g_src2 = host_copy(d_src2, sizeof(int32_t) * (size_t)cap);
            uint16_t* g_recv2 = host_copy(d_recv2, sizeof(uint16_t) * (size_t)(cap * H));
            expect(!memcmp(g_send2, o_send, sizeof(int32_t) * (size_t)(T * R)), "send_row of the plan left", name);
            expect(!memcmp(g_src2, o_src, sizeof(int32_t) * (size_t)cap), "recv_src_idx of the plan left", name);
            int ok2 = 1;
            for (int64_t r = 0; r < cap; ++r)
                if (o_src[r] >= 0) ok2 &= !memcmp(g_recv2 + r * H, o_recv + r * H, sizeof(uint16_t) * (size_t)H);
            expect(ok2, "rows of the plan left in the workspace", name);
            free(g_send2); free(g_src2); free(g_recv2);
            HIP_OK(hipFree(d_recv2)); HIP_OK(hipFree(d_src2)); HIP_OK(hipFree(d_send2));
        }
        free(g_ntpr); free(g_ntpe); free(g_itr); free(g_roff); free(g_nre); free(g_src); free(g_send);
        free(g_ridx); free(g_rw);
    }
    printf("[%s] rank-granular rows, bf16 and FP8, as the oracle's\n", name);

    void* dev_bufs[] = {d_x, d_idx, d_w, d_ntpr, d_ntpe, d_itr, d_roff, d_nre, d_src, d_send, d_ridx, d_rw,
                        d_recv, d_xq, d_xs, d_rq, d_rs, d_ws};
    for (size_t i = 0; i < sizeof dev_bufs / sizeof dev_bufs[0]; ++i) HIP_OK(hipFree(dev_bufs[i]));
    void* host_bufs[] = {idx, x, w, o_ntpr, o_ntpe, o_itr, o_roff, o_send, o_src, o_ridx, o_rw, o_nre, o_recv,
                         o_q, o_s};
    for (size_t i = 0; i < sizeof host_bufs / sizeof host_bufs[0]; ++i) free(host_bufs[i]);
}

int main(void) {
    printf("libcgd %s\n", cgd_version());
    CGD_OK_(cgd_init());
    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));
    run_case("one launch", 100, 8, 64, 8, 512, 1, 1, stream);
    run_case("several tiles", 1000, 8, 256, 16, 256, 4, 2, stream);
    run_case("top-16", 700, 16, 512, 64, 128, 1, 3, stream);
    run_normal_case("rank-granular, several tiles", 1000, 8, 256, 16, 256, 4, 4, stream);
    run_normal_case("rank-granular, one tile", 100, 6, 64, 8, 128, 1, 5, stream);
    HIP_OK(hipStreamDestroy(stream));
    if (failures) {
        printf("%d checks failed\n", failures);
        return 1;
    }
    printf("ok\n");
    return 0;
}
