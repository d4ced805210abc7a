/*
 * Runs every function of the CPU oracle (oracle/oracle.c) on small inputs,
 * edge cases included, so that a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer sees every loop bound and index.  Prints one
 * checksum line; exits non-zero when a round trip or a cross-check fails.
 * Test infrastructure: only tests/test_sanitizers.py builds and runs it.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void orc_quant_sym_rows(const float*, int64_t, int64_t, float, int8_t*, float*);
void orc_lqq_encode(const int8_t*, int64_t, int64_t, int64_t, uint8_t*, uint8_t*, uint8_t*, int64_t*);
int64_t orc_lqq_decode(const uint8_t*, const uint8_t*, const uint8_t*, int64_t, int64_t, int64_t, int8_t*);
void orc_pack_nibbles(const uint8_t*, int64_t, int64_t, uint8_t*);
void orc_unpack_nibbles(const uint8_t*, int64_t, int64_t, uint8_t*);
void orc_params_to_panels(const uint8_t*, int64_t, int64_t, uint8_t*);
void orc_params_from_panels(const uint8_t*, int64_t, int64_t, uint8_t*);
void orc_gemm_i32(const int8_t*, const int8_t*, int64_t, int64_t, int64_t, int32_t*);
void orc_round_f16(const double*, int64_t, uint16_t*);
void orc_round_bf16(const double*, int64_t, uint16_t*);
void orc_epilogue_f16(const int32_t*, const float*, const float*, int64_t, int64_t, uint16_t*, double*);
void orc_e4m3_decode(const uint8_t*, int64_t, double*);
void orc_e4m3_encode(const float*, int64_t, uint8_t*);
void orc_quant_rows_e4m3(const float*, int64_t, int64_t, uint8_t*, float*);
void orc_int4_sm_codes(const int8_t*, int64_t, uint8_t*);
void orc_int4_sm_values(const uint8_t*, int64_t, int8_t*);
void orc_w4fp8_ref(const uint8_t*, const float*, const int8_t*, const float*, int64_t, int64_t, int64_t, double*, double*);
void orc_w4fp8g_pack(const float*, int64_t, int64_t, int64_t, int8_t*, float*, float*, float*);
void orc_w4fp8g_weights(const int8_t*, const float*, int64_t, int64_t, int64_t, uint8_t*);
void orc_w4fp8g_ref(const uint8_t*, const float*, const uint8_t*, float, int64_t, int64_t, int64_t, double*, double*);
void orc_pack_w8(const int8_t*, int64_t, int64_t, int8_t*);
void orc_unpack_w8(const int8_t*, int64_t, int64_t, int8_t*);

static uint32_t lcg = 12345u;
static float frand(void) {  /* uniform in [-1, 1) */
    lcg = lcg * 1664525u + 1013904223u;
    return (float)((int32_t)lcg) / 2147483648.0f;
}

#define CHECK(c) do { if (!(c)) { fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); return 1; } } while (0)

int main(void) {
    enum { M = 3, N = 64, K = 256, G = 64 };
    float* W = malloc(sizeof(float) * N * K);
    float* X = malloc(sizeof(float) * M * K);
    for (int i = 0; i < N * K; ++i) W[i] = 0.02f * frand();
    for (int i = 0; i < M * K; ++i) X[i] = frand() * (i % 37 == 0 ? 20.0f : 1.0f);
    for (int k = 0; k < K; ++k) W[5 * K + k] = 0.0f;    /* all-zero channel */
    for (int k = 0; k < K; ++k) X[1 * K + k] = 0.0f;    /* all-zero token */
    W[7 * K + 3] = 1e30f;                                /* one huge weight */
    X[2 * K + 9] = -0.0f;

    int8_t* Q = malloc(N * K);
    float* sw = malloc(sizeof(float) * N);
    orc_quant_sym_rows(W, N, K, 127.0f, Q, sw);
    int8_t* X8 = malloc(M * K);
    float* sx = malloc(sizeof(float) * M);
    orc_quant_sym_rows(X, M, K, 127.0f, X8, sx);

    uint8_t* codes = malloc(N * K);
    uint8_t* s8 = malloc(N * K / G);
    uint8_t* a8 = malloc(N * K / G);
    int64_t nsat = -1;
    orc_lqq_encode(Q, N, K, G, codes, s8, a8, &nsat);
    CHECK(nsat >= 0);
    int8_t* Qh = malloc(N * K);
    CHECK(orc_lqq_decode(codes, s8, a8, N, K, G, Qh) == 0);

    uint8_t* wq = malloc(N * K / 2);
    uint8_t* back = malloc(N * K);
    orc_pack_nibbles(codes, N, K, wq);
    orc_unpack_nibbles(wq, N, K, back);
    CHECK(memcmp(back, codes, N * K) == 0);
    uint8_t* pan = malloc(N * K / G);
    uint8_t* pb = malloc(N * K / G);
    orc_params_to_panels(s8, N, K / G, pan);
    orc_params_from_panels(pan, N, K / G, pb);
    CHECK(memcmp(pb, s8, N * K / G) == 0);

    int32_t* acc = malloc(sizeof(int32_t) * M * N);
    orc_gemm_i32(X8, Qh, M, N, K, acc);
    for (int m = 0; m < M; ++m)
        for (int n = 0; n < N; n += 13) {
            int64_t t = 0;
            for (int k = 0; k < K; ++k) t += (int64_t)X8[m * K + k] * Qh[n * K + k];
            CHECK(t == acc[m * N + n]);
        }
    uint16_t* y = malloc(2 * M * N);
    double* yd = malloc(sizeof(double) * M * N);
    orc_epilogue_f16(acc, sx, sw, M, N, y, yd);

    double v[8] = {0.0, -0.0, 1e-9, 65504.0, 65520.0, 1e300, NAN, -3.5};
    uint16_t h[8], b[8];
    orc_round_f16(v, 8, h);
    orc_round_bf16(v, 8, b);
    CHECK(h[4] == 0x7C00);  /* 65520 rounds up to +inf in fp16 */

    uint8_t all[256];
    double dec[256];
    for (int i = 0; i < 256; ++i) all[i] = (uint8_t)i;
    orc_e4m3_decode(all, 256, dec);
    float fx[6] = {0.0f, -0.0f, 448.0f, 1e9f, NAN, 0.001953125f};
    uint8_t e8[6];
    orc_e4m3_encode(fx, 6, e8);
    CHECK(e8[3] == 0x7E && e8[4] == 0x7F && e8[1] == 0x80);
    uint8_t* Xe = malloc(M * K);
    float* sxe = malloc(sizeof(float) * M);
    orc_quant_rows_e4m3(X, M, K, Xe, sxe);

    int8_t* q4 = malloc(N * K);
    float* sw4 = malloc(sizeof(float) * N);
    orc_quant_sym_rows(W, N, K, 7.0f, q4, sw4);
    uint8_t* c4 = malloc(N * K);
    int8_t* q4b = malloc(N * K);
    orc_int4_sm_codes(q4, N * K, c4);
    orc_int4_sm_values(c4, N * K, q4b);
    CHECK(memcmp(q4, q4b, N * K) == 0);
    double* ref = malloc(sizeof(double) * M * N);
    double* pre = malloc(sizeof(double) * M * N);
    orc_w4fp8_ref(Xe, sxe, q4, sw4, M, N, K, ref, pre);

    int8_t* qg = malloc(N * K);
    float* sg = malloc(sizeof(float) * N * K / G);
    float* fg = malloc(sizeof(float) * N * K / G);
    float t = 0.0f;
    orc_w4fp8g_pack(W, N, K, G, qg, sg, fg, &t);
    uint8_t* w8 = malloc(N * K);
    orc_w4fp8g_weights(qg, fg, N, K, G, w8);
    orc_w4fp8g_ref(Xe, sxe, w8, t, M, N, K, ref, pre);

    int8_t* p8 = malloc(N * K);
    int8_t* u8 = malloc(N * K);
    orc_pack_w8(Q, N, K, p8);
    orc_unpack_w8(p8, N, K, u8);
    CHECK(memcmp(u8, Q, N * K) == 0);

    uint64_t sum = 0;
    for (int i = 0; i < M * N; ++i) sum = sum * 31u + y[i] + (uint32_t)acc[i];
    for (int i = 0; i < N * K; ++i) sum = sum * 31u + w8[i] + wq[i / 2];
    printf("oracle driver ok, checksum %016llx\n", (unsigned long long)sum);
    free(W); free(X); free(Q); free(sw); free(X8); free(sx); free(codes); free(s8); free(a8);
    free(Qh); free(wq); free(back); free(pan); free(pb); free(acc); free(y); free(yd); free(Xe);
    free(sxe); free(q4); free(sw4); free(c4); free(q4b); free(ref); free(pre); free(qg); free(sg);
    free(fg); free(w8); free(p8); free(u8);
    return 0;
}
