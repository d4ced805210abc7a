/*
 * CPU oracle for the W4A8 (LiquidQuant) and W4FP8 (INT4 x FP8) GEMM paths.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or constant with the HIP library: everything here is
 * written from the method's definition, in plain loops, one step per
 * function, in the order the method states them.
 *
 * Sources (cited by page title and part of the page):
 *   [LG]  "LiquidGEMM: Hardware-Efficient W4A8 GEMM Kernel for High-
 *         Performance LLM Serving", Pith review of arXiv 2509.01229:
 *         "What carries the argument", the referee summary and major
 *         comment 3 (paper Sec. 4, Eq. 7, Eq. 10, Eq. 12), the circularity
 *         audit (Eq. 11, the [-119, 119] range), minor comment 1 (Sec. 5.3).
 *   [FQ]  "FireQ: Fast INT4-FP8 Kernel and RoPE-aware Quantization for LLM
 *         Inference Acceleration" (arXiv 2505.20839), abstract.
 *
 * Readings where the pages leave a step open are marked READING; they are
 * the plainest ones the rest of the text supports.
 *
 * Parity pins: every function below is pinned by a CPU test against a closed
 * form, an exhaustive enumeration, a library routine on a special case, or a
 * hand-derived example.  None is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_API __attribute__((visibility("default")))

/* ------------------------------------------------------------------------ *
 * 1. Symmetric per-row quantisation to signed integers in [-qmax, qmax].
 *    Used three ways: per-token INT8 activations (qmax 127), per-output-
 *    channel INT8 weights, the first level of LiquidQuant ([LG] referee
 *    summary: a two-level scheme whose first level is INT8), and per-channel
 *    INT4 weights for the FP8 variant (qmax 7, [FQ] abstract: channel-wise
 *    scaling of INT4).
 *    scale = max_k |x[k]| / qmax   (float32, correctly rounded division)
 *    q[k]  = clamp(round_half_even(x[k] / scale), -qmax, qmax)   (float32)
 *    READING: a row whose scale is not positive (all zeros, or a max so
 *    small that max/qmax underflows) gets scale 1 and all-zero codes.
 * ------------------------------------------------------------------------ */
ORC_API void orc_quant_sym_rows(const float* x, int64_t rows, int64_t cols,
                                float qmax, int8_t* q, float* scale) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const float* xr = x + r * cols;
        float amax = 0.0f;
        for (int64_t c = 0; c < cols; ++c) {
            float a = fabsf(xr[c]);
            if (a > amax) amax = a;
        }
        float s = amax / qmax;
        if (!(s > 0.0f)) s = 1.0f;
        scale[r] = s;
        for (int64_t c = 0; c < cols; ++c) {
            float v = rintf(xr[c] / s); /* default mode: nearest, ties to even */
            if (v > qmax) v = qmax;
            if (v < -qmax) v = -qmax;
            q[r * cols + c] = (int8_t)v;
        }
    }
}

/* ------------------------------------------------------------------------ *
 * 2. LiquidQuant second level: INT8 -> UINT4 per group of g along K.
 *    [LG] referee summary: INT8 weights are shifted into the UINT8 domain
 *    and then quantised to UINT4; "What carries the argument": the offset
 *    a = 2^7 + min(Q_i8) is precomputed offline; major comment 3: s_u8 is an
 *    integer scale (Eq. 7) and q is rounded to nearest (minor comment 2,
 *    Eq. 10).
 *      m = min_group Q,  Mx = max_group Q,  R = Mx - m
 *      s = max(1, ceil(R / 15))           READING: ceil keeps R/s <= 15
 *      a = 128 + m                        (UINT8)
 *      u = Q - m  in [0, R]               (the UINT8-domain value)
 *      q = floor((2u + s) / (2s))         READING: nearest, ties upward
 *      q = min(q, floor((127 - m) / s))   READING: saturation so that the
 *          decoded value never exceeds 127.  It is inert when Q lies in the
 *          pages' protective range [-119, 119] (circularity audit, Eq. 11)
 *          and only bites when the first level used the full +-127.
 *    codes[n*K + k] receives q (one code per byte, unpacked); *nsat counts
 *    the codes the saturation lowered.
 * ------------------------------------------------------------------------ */
ORC_API void orc_lqq_encode(const int8_t* Q, int64_t N, int64_t K, int64_t g,
                            uint8_t* codes, uint8_t* s_u8, uint8_t* a_u8,
                            int64_t* nsat) {
    int64_t G = K / g;
    int64_t sat_total = 0;
#pragma omp parallel for schedule(static) reduction(+ : sat_total)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t j = 0; j < G; ++j) {
            const int8_t* qg = Q + n * K + j * g;
            int m = 127, Mx = -128;
            for (int64_t t = 0; t < g; ++t) {
                if (qg[t] < m) m = qg[t];
                if (qg[t] > Mx) Mx = qg[t];
            }
            int R = Mx - m;
            int s = (R + 14) / 15; /* ceil(R / 15) for R >= 0 */
            if (s < 1) s = 1;
            int a = 128 + m;
            int cap = (127 - m) / s; /* 127 - m >= 0 */
            s_u8[n * G + j] = (uint8_t)s;
            a_u8[n * G + j] = (uint8_t)a;
            for (int64_t t = 0; t < g; ++t) {
                int u = qg[t] - m;
                int q = (2 * u + s) / (2 * s);
                if (q > cap) {
                    q = cap;
                    sat_total += 1;
                }
                if (q > 15) q = 15; /* unreachable with the ceil scale */
                codes[n * K + j * g + t] = (uint8_t)q;
            }
        }
    }
    if (nsat) *nsat = sat_total;
}

/* ------------------------------------------------------------------------ *
 * 3. LiquidQuant decode, the identity itself ([LG] "What carries the
 *    argument", Eq. 12):  Q^_i8 = (q_u4 * s_u8 + a) XOR 0x80, computed on a
 *    UINT8 byte and read back as two's complement INT8 (the congruence mod
 *    2^8 of the circularity audit).  Returns the number of elements whose
 *    UINT8 multiply-add would have carried out of the byte (must be 0).
 * ------------------------------------------------------------------------ */
ORC_API int64_t orc_lqq_decode(const uint8_t* codes, const uint8_t* s_u8,
                               const uint8_t* a_u8, int64_t N, int64_t K,
                               int64_t g, int8_t* Qhat) {
    int64_t G = K / g;
    int64_t carries = 0;
#pragma omp parallel for schedule(static) reduction(+ : carries)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) {
            unsigned q = codes[n * K + k];
            unsigned s = s_u8[n * G + k / g];
            unsigned a = a_u8[n * G + k / g];
            unsigned wide = q * s + a;
            if (wide > 255u) carries += 1;
            uint8_t byte = (uint8_t)(wide & 0xFFu);
            byte ^= 0x80u;
            Qhat[n * K + k] = (int8_t)byte;
        }
    }
    return carries;
}

/* ------------------------------------------------------------------------ *
 * 4. Packed nibble layout (the byte order the library documents for wq).
 *    Written from the layout description alone:
 *      the matrix [N][K] of 4-bit codes is cut into tiles of 16 rows x 128
 *      K-columns; tile (nt, kt) occupies bytes [1024*(nt*(K/128)+kt), +1024).
 *      Inside a tile, lane L = 16*G + r (r = row in tile 0..15, G = 0..3)
 *      owns 16 bytes at offset 16*L covering K-columns 32*G .. 32*G+31 of
 *      the tile.  Of those, dword d (0..3) covers columns 32*G+8*d .. +7:
 *      its byte b (0..3) holds column +b in the low nibble and column +4+b
 *      in the high nibble.
 *    codes: one code per byte (low 4 bits used), [N][K].  wq: N*K/2 bytes.
 * ------------------------------------------------------------------------ */
ORC_API void orc_pack_nibbles(const uint8_t* codes, int64_t N, int64_t K,
                              uint8_t* wq) {
    int64_t KT = K / 128;
    memset(wq, 0, (size_t)(N * K / 2));
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) {
            int64_t nt = n / 16, r = n % 16;
            int64_t kt = k / 128, kk = k % 128;
            int64_t G = kk / 32, w = kk % 32;
            int64_t d = w / 8, e = w % 8;
            int64_t b = e % 4, hi = e / 4;
            int64_t lane = 16 * G + r;
            int64_t off = (nt * KT + kt) * 1024 + lane * 16 + d * 4 + b;
            wq[off] |= (uint8_t)((codes[n * K + k] & 0xFu) << (4 * hi));
        }
    }
}

/* Per-group parameter order (panel order): the row-major [N][K/g] array of
 * s (or a) bytes is rewritten so that panel p = n/64 and group j occupy the
 * 64 bytes at 64*(p*(K/g) + j), channel n at byte 4*(n%16) + (n%64)/16. */
ORC_API void orc_params_to_panels(const uint8_t* rowmajor, int64_t N,
                                  int64_t groups, uint8_t* panels) {
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t j = 0; j < groups; ++j) {
            int64_t p = n / 64;
            int64_t off = 64 * (p * groups + j) + 4 * (n % 16) + (n % 64) / 16;
            panels[off] = rowmajor[n * groups + j];
        }
    }
}

/* Inverse of the panel order (tests read device-written parameters). */
ORC_API void orc_params_from_panels(const uint8_t* panels, int64_t N,
                                    int64_t groups, uint8_t* rowmajor) {
    for (int64_t n = 0; n < N; ++n)
        for (int64_t j = 0; j < groups; ++j)
            rowmajor[n * groups + j] =
                panels[64 * ((n / 64) * groups + j) + 4 * (n % 16) + (n % 64) / 16];
}

/* Inverse of the nibble layout, used by tests to read device-packed bytes. */
ORC_API void orc_unpack_nibbles(const uint8_t* wq, int64_t N, int64_t K,
                                uint8_t* codes) {
    int64_t KT = K / 128;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) {
            int64_t nt = n / 16, r = n % 16;
            int64_t kt = k / 128, kk = k % 128;
            int64_t G = kk / 32, w = kk % 32;
            int64_t d = w / 8, e = w % 8;
            int64_t b = e % 4, hi = e / 4;
            int64_t off = (nt * KT + kt) * 1024 + (16 * G + r) * 16 + d * 4 + b;
            codes[n * K + k] = (uint8_t)((wq[off] >> (4 * hi)) & 0xFu);
        }
    }
}

/* ------------------------------------------------------------------------ *
 * 5. INT32 GEMM of the INT8 operands, straight from the definition:
 *    acc[m][n] = sum_k X[m][k] * W[n][k]   (k ascending; integer, exact).
 *    [LG] referee summary: the dequantised INT8 weights feed an INT8 MMA.
 * ------------------------------------------------------------------------ */
ORC_API void orc_gemm_i32(const int8_t* X, const int8_t* W, int64_t M,
                          int64_t N, int64_t K, int32_t* acc) {
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            int64_t s = 0;
            for (int64_t k = 0; k < K; ++k)
                s += (int64_t)X[m * K + k] * (int64_t)W[n * K + k];
            acc[m * N + n] = (int32_t)s;
        }
    }
}

/* ------------------------------------------------------------------------ *
 * 6. Rounding of a double to a binary floating-point format with p
 *    significand bits (implicit bit included) and minimum normal exponent
 *    emin, nearest with ties to even, overflow to +-inf.  Exact steps:
 *    the quantum at |v| is 2^(max(e, emin) - p + 1) where 2^e <= |v| < 2^(e+1);
 *    |v| / quantum is exact in double, rint() rounds it to nearest-even.
 * ------------------------------------------------------------------------ */
static double round_to_format(double v, int p, int emin, double maxfinite) {
    if (v == 0.0 || isnan(v) || isinf(v)) return v;
    double a = fabs(v);
    int ex;
    (void)frexp(a, &ex);       /* a = f * 2^ex with f in [0.5, 1) */
    int e = ex - 1;            /* 2^e <= a < 2^(e+1) */
    if (e < emin) e = emin;    /* subnormal range keeps the fixed quantum */
    double quantum = ldexp(1.0, e - p + 1);
    double r = rint(a / quantum) * quantum;
    if (r > maxfinite) r = INFINITY;
    return v < 0 ? -r : r;
}

/* IEEE binary16 bit pattern of an already-representable double. */
static uint16_t f16_bits(double r) {
    uint16_t sign = signbit(r) ? 0x8000u : 0u;
    double a = fabs(r);
    if (isinf(a)) return sign | 0x7C00u;
    if (a == 0.0) return sign;
    if (a < ldexp(1.0, -14)) /* subnormal: a = mant * 2^-24 */
        return sign | (uint16_t)(a / ldexp(1.0, -24));
    int ex;
    double f = frexp(a, &ex); /* a = f * 2^ex, f in [0.5, 1) */
    int e = ex - 1;
    uint16_t mant = (uint16_t)((f * 2.0 - 1.0) * 1024.0);
    return sign | (uint16_t)((e + 15) << 10) | mant;
}

/* bfloat16 bit pattern of an already-representable double. */
static uint16_t bf16_bits(double r) {
    float f = (float)r; /* exact: every bfloat16 value is a float */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

ORC_API void orc_round_f16(const double* v, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i)
        out[i] = f16_bits(round_to_format(v[i], 11, -14, 65504.0));
}

ORC_API void orc_round_bf16(const double* v, int64_t n, uint16_t* out) {
    double maxbf = ldexp(255.0 / 128.0, 127); /* (2 - 2^-7) * 2^127 */
    for (int64_t i = 0; i < n; ++i)
        out[i] = bf16_bits(round_to_format(v[i], 8, -126, maxbf));
}

/* ------------------------------------------------------------------------ *
 * 7. W4A8 epilogue: y[m][n] = fp16( acc[m][n] * sx[m] * sw[n] ), the
 *    per-token x per-channel rescale, evaluated in double and rounded once.
 *    Also returns the unrounded double values when yd != NULL.
 * ------------------------------------------------------------------------ */
ORC_API void orc_epilogue_f16(const int32_t* acc, const float* sx,
                              const float* sw, int64_t M, int64_t N,
                              uint16_t* y, double* yd) {
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double v = (double)acc[m * N + n] * (double)sx[m] * (double)sw[n];
            if (yd) yd[m * N + n] = v;
            y[m * N + n] = f16_bits(round_to_format(v, 11, -14, 65504.0));
        }
    }
}

/* ------------------------------------------------------------------------ *
 * 8. FP8 e4m3 (OCP "e4m3fn": bias 7, no infinities, S.1111.111 is NaN,
 *    largest finite 448).  [FQ] abstract: activations in FP8.
 *    Decoding is the format definition; encoding takes the nearest finite
 *    value (ties to the even code), found by binary search over the sorted
 *    non-negative finite values, with the sign copied; magnitudes above 448
 *    therefore saturate to 448.  NaN encodes as 0x7F.
 * ------------------------------------------------------------------------ */
static double e4m3_value(unsigned b) {
    unsigned e = (b >> 3) & 0xFu, m = b & 0x7u;
    double mag;
    if (e == 15u && m == 7u) return NAN;
    if (e == 0u) mag = ldexp((double)m, -9);              /* m/8 * 2^(1-7) */
    else mag = ldexp(1.0 + (double)m / 8.0, (int)e - 7);
    return (b & 0x80u) ? -mag : mag;
}

ORC_API void orc_e4m3_decode(const uint8_t* b, int64_t n, double* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = e4m3_value(b[i]);
}

static uint8_t e4m3_encode(float x) {
    if (isnan(x)) return 0x7Fu;
    /* codes 0x00 .. 0x7E are the non-negative finite values, ascending */
    double a = fabs((double)x);
    unsigned lo = 0, hi = 0x7E;
    if (a >= e4m3_value(hi)) {
        lo = hi;
    } else {
        while (hi - lo > 1) { /* invariant: value(lo) <= a < value(hi) */
            unsigned mid = (lo + hi) / 2;
            if (e4m3_value(mid) <= a) lo = mid;
            else hi = mid;
        }
        double dl = a - e4m3_value(lo), dh = e4m3_value(hi) - a;
        if (dh < dl || (dh == dl && (hi & 1u) == 0u)) lo = hi;
    }
    return (uint8_t)(lo | (signbit(x) ? 0x80u : 0u));
}

ORC_API void orc_e4m3_encode(const float* x, int64_t n, uint8_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = e4m3_encode(x[i]);
}

/* Per-token FP8 activations: sx = max|x| / 448 (float32), codes =
 * e4m3(x / sx) with the float32 quotient (same zero-row reading as 1). */
ORC_API void orc_quant_rows_e4m3(const float* x, int64_t rows, int64_t cols,
                                 uint8_t* q, float* scale) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const float* xr = x + r * cols;
        float amax = 0.0f;
        for (int64_t c = 0; c < cols; ++c) {
            float a = fabsf(xr[c]);
            if (a > amax) amax = a;
        }
        float s = amax / 448.0f;
        if (!(s > 0.0f)) s = 1.0f;
        scale[r] = s;
        for (int64_t c = 0; c < cols; ++c) q[r * cols + c] = e4m3_encode(xr[c] / s);
    }
}

/* ------------------------------------------------------------------------ *
 * 9. INT4 weights of the FP8 variant, sign-magnitude nibbles (READING: the
 *    pages fix no INT4 encoding): bit 3 = sign, bits 0..2 = |q|, q in
 *    [-7, 7] from step 1 with qmax 7.  Zero is always the code 0.
 * ------------------------------------------------------------------------ */
ORC_API void orc_int4_sm_codes(const int8_t* q, int64_t n, uint8_t* codes) {
    for (int64_t i = 0; i < n; ++i) {
        int v = q[i];
        codes[i] = (uint8_t)(v < 0 ? (0x8 | (unsigned)(-v)) : (unsigned)v);
    }
}

ORC_API void orc_int4_sm_values(const uint8_t* codes, int64_t n, int8_t* q) {
    for (int64_t i = 0; i < n; ++i) {
        int mag = codes[i] & 0x7, neg = (codes[i] >> 3) & 1;
        q[i] = (int8_t)(neg ? -mag : mag);
    }
}

/* ------------------------------------------------------------------------ *
 * 10. FP8-variant reference in double: ref[m][n] = (sum_k x[m][k] * q[n][k])
 *     * sx[m] * sw[n], x = decoded e4m3, q = INT4 value (exactly an FP8
 *     weight, since |q| <= 7 is representable in e4m3).  Each product has at
 *     most 7 significant bits and the sum spans less than 2^53, so the
 *     double sum is exact; only the two scale multiplications round.
 *     pre[m][n] (if not NULL) receives the unscaled exact sum.
 * ------------------------------------------------------------------------ */
ORC_API void orc_w4fp8_ref(const uint8_t* X8, const float* sx, const int8_t* q,
                           const float* sw, int64_t M, int64_t N, int64_t K,
                           double* ref, double* pre) {
    double* xd = (double*)malloc(sizeof(double) * (size_t)(M * K));
    for (int64_t i = 0; i < M * K; ++i) xd[i] = e4m3_value(X8[i]);
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double s = 0.0;
            for (int64_t k = 0; k < K; ++k) s += xd[m * K + k] * (double)q[n * K + k];
            if (pre) pre[m * N + n] = s;
            ref[m * N + n] = s * (double)sx[m] * (double)sw[n];
        }
    }
    free(xd);
}

/* ------------------------------------------------------------------------ *
 * 11. FP8 variant with per-group scales folded into the FP8 weights and a
 *     per-tensor rescale against underflow (FireQ, arXiv 2505.20839,
 *     abstract: INT4 weights, FP8 activations, "per-tensor scaling to
 *     prevent underflow" of the FP8 weights, finer scaling for the coarse
 *     INT4 grid).  READING (the abstract fixes no formula), all in float32
 *     with correctly rounded division and round-half-even:
 *       per group j of g K-columns of channel n:
 *         s_g[n][j] = max_k |W[n][k]| / 7   (a zero group gets 1)
 *         q[n][k]   = clamp(rne(W[n][k] / s_g[n][j]), -7, 7)
 *       per tensor: t = max |W| / 448       (all-zero W gets 1)
 *       folded factor f[n][j] = s_g[n][j] / t
 *       FP8 weight w8[n][k] = sign(q) * e4m3(float(|q| * f[n][j]))
 *     so W ~= w8 * t, and the largest folded value 7 f is at most 448
 *     (up to one rounding of f): FP8's range holds every group's grid.
 * ------------------------------------------------------------------------ */
ORC_API void orc_w4fp8g_pack(const float* W, int64_t N, int64_t K, int64_t g, int8_t* q,
                             float* sg, float* f, float* t_out) {
    const int64_t G = K / g;
    float wmax = 0.0f;
    for (int64_t i = 0; i < N * K; ++i) {
        float a = fabsf(W[i]);
        if (a > wmax) wmax = a;
    }
    float t = wmax / 448.0f;
    if (!(t > 0.0f)) t = 1.0f;
    *t_out = t;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t j = 0; j < G; ++j) {
            const float* w = W + n * K + j * g;
            float amax = 0.0f;
            for (int64_t k = 0; k < g; ++k) {
                float a = fabsf(w[k]);
                if (a > amax) amax = a;
            }
            float s = amax / 7.0f;
            if (!(s > 0.0f)) s = 1.0f;
            sg[n * G + j] = s;
            f[n * G + j] = s / t;
            for (int64_t k = 0; k < g; ++k) {
                float v = rintf(w[k] / s);
                if (v > 7.0f) v = 7.0f;
                if (v < -7.0f) v = -7.0f;
                q[n * K + j * g + k] = (int8_t)v;
            }
        }
    }
}

/* The folded FP8 weights (e4m3 bytes) of section 11. */
ORC_API void orc_w4fp8g_weights(const int8_t* q, const float* f, int64_t N, int64_t K,
                                int64_t g, uint8_t* w8) {
    const int64_t G = K / g;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) {
            const int v = q[n * K + k];
            const float mag = (float)(v < 0 ? -v : v) * f[n * G + k / g];
            const uint8_t e = e4m3_encode(mag);
            w8[n * K + k] = (uint8_t)(v < 0 ? (e | 0x80u) : e);
        }
    }
}

/* Reference of section 11 in double: ref = (sum_k x * w8) * sx[m] * t.  Both
 * factors are e4m3 values (at most 4 significant bits each), so every
 * product and the whole sum are exact in double; pre = the unscaled sum. */
ORC_API void orc_w4fp8g_ref(const uint8_t* X8, const float* sx, const uint8_t* w8, float t,
                            int64_t M, int64_t N, int64_t K, double* ref, double* pre) {
    double* xd = (double*)malloc(sizeof(double) * (size_t)(M * K));
    double* wd = (double*)malloc(sizeof(double) * (size_t)(N * K));
    for (int64_t i = 0; i < M * K; ++i) xd[i] = e4m3_value(X8[i]);
    for (int64_t i = 0; i < N * K; ++i) wd[i] = e4m3_value(w8[i]);
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double s = 0.0;
            for (int64_t k = 0; k < K; ++k) s += xd[m * K + k] * wd[n * K + k];
            if (pre) pre[m * N + n] = s;
            ref[m * N + n] = s * (double)sx[m] * (double)t;
        }
    }
    free(xd);
    free(wd);
}

/* ------------------------------------------------------------------------ *
 * 12. The W8A8 comparison path.  [LG] ("If this is right") sets W4A8 against
 *     W8A8: lower memory traffic should win in small-batch, memory-bound
 *     runs, and in large-batch, compute-bound runs W4A8 should match or beat
 *     it.  The W8A8 weights are the first LiquidQuant level alone: the
 *     per-channel INT8 codes and scales of section 1 (qmax 127), multiplied
 *     by the INT8 GEMM above with the same epilogue.  This library's 8-bit
 *     tile layout (READING: the pages give none) holds the codes as:
 *       tile (nt, kt) of 16 rows x 128 K at byte 2048 * (nt * (K/128) + kt);
 *       inside it, byte 1024*u + 16*(16*G + r) + j is row 16*nt + r,
 *       column 128*kt + 32*G + 16*u + j   (G 0..3, u 0..1, j 0..15).
 * ------------------------------------------------------------------------ */
ORC_API void orc_pack_w8(const int8_t* Q, int64_t N, int64_t K, int8_t* out) {
    const int64_t KT = K / 128;
    for (int64_t n = 0; n < N; ++n) {
        const int64_t nt = n / 16, r = n % 16;
        for (int64_t k = 0; k < K; ++k) {
            const int64_t kt = k / 128, kk = k % 128;
            const int64_t G = kk / 32, u = (kk % 32) / 16, j = kk % 16;
            const int64_t off = 2048 * (nt * KT + kt) + 1024 * u + 16 * (16 * G + r) + j;
            out[off] = Q[n * K + k];
        }
    }
}

ORC_API void orc_unpack_w8(const int8_t* packed, int64_t N, int64_t K, int8_t* Q) {
    const int64_t KT = K / 128;
    for (int64_t n = 0; n < N; ++n) {
        const int64_t nt = n / 16, r = n % 16;
        for (int64_t k = 0; k < K; ++k) {
            const int64_t kt = k / 128, kk = k % 128;
            const int64_t G = kk / 32, u = (kk % 32) / 16, j = kk % 16;
            Q[n * K + k] = packed[2048 * (nt * KT + kt) + 1024 * u + 16 * (16 * G + r) + j];
        }
    }
}
