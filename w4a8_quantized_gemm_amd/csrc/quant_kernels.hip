// Quantisation kernels for gfx950: offline weight packing (LiquidQuant and
// INT4 sign-magnitude) and per-token activation quantisation (INT8, e4m3).
//
// Sources: LiquidGEMM, Pith review of arXiv 2509.01229 (referee summary:
// per-channel INT8 then per-group UINT4 in the UINT8 domain; "What carries
// the argument": offset a = 2^7 + min; major comment 3: integer scale,
// Sec. 4 Eq. 7; minor comment 2: nearest rounding, Eq. 10).  FireQ, arXiv
// 2505.20839, abstract (INT4 weights with channel-wise scales, FP8
// activations).
//
// Every float step that decides an integer (scale division, quotient,
// rounding) is done in float32 with correctly rounded division and
// round-half-even, so the codes are a deterministic function of the input.
#include "device_common.h"
#include "launch.h"

namespace w4a8 {

// ---------------------------------------------------------------------------
// Row max |x| reduced by one workgroup of 256 threads, then scale =
// max / qmax (a row whose scale is not positive gets scale 1).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float block_absmax_256(const float* row, int K) {
    float m = 0.0f;
    const float4* r4 = reinterpret_cast<const float4*>(row);
    for (int i = threadIdx.x; i < K / 4; i += 256) {
        float4 v = r4[i];
        m = fmaxf(m, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    }
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    __shared__ float part[4];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
    __syncthreads();
    m = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
    __syncthreads();
    return m;
}

__device__ __forceinline__ float scale_of(float amax, float qmax) {
    float s = __fdiv_rn(amax, qmax);
    return (s > 0.0f) ? s : 1.0f;
}

__device__ __forceinline__ int quant_sym(float x, float s, float qmax) {
    float v = __builtin_rintf(__fdiv_rn(x, s));
    v = fminf(fmaxf(v, -qmax), qmax);
    return (int)v;
}

// Per-row scale (weights: per output channel).
__global__ __launch_bounds__(256) void row_scale_kernel(const float* __restrict__ W, int K,
                                                        float qmax, float* __restrict__ sw) {
    const float* row = W + (size_t)blockIdx.x * K;
    float amax = block_absmax_256(row, K);
    if (threadIdx.x == 0) sw[blockIdx.x] = scale_of(amax, qmax);
}

// Byte offset of packed dword d of lane (G, r) in tile (nt, kt).
__device__ __forceinline__ size_t packed_dword_offset(int nt, int kt, int KT, int G, int r, int d) {
    return ((size_t)nt * KT + kt) * kTileBytes + (size_t)(16 * G + r) * 16 + 4 * d;
}

// LiquidQuant second level.  One thread per packed dword (8 consecutive
// columns of one row, read as two float4): it forms the 8 INT8 values once,
// the GW = group / 8 threads of a group (aligned lanes of one wave) combine
// their minima and maxima by XOR shuffles, and each thread then writes its
// dword of UINT4 codes; the group's first thread writes s_u8 / a_u8.  The
// arithmetic is per element and in the same order as a serial loop, so the
// codes do not depend on the thread layout.
template <int GW>
__global__ __launch_bounds__(256) void lqq_group_kernel(const float* __restrict__ W,
                                                        const float* __restrict__ sw, int N, int K,
                                                        float qmax, uint8_t* __restrict__ wq,
                                                        uint8_t* __restrict__ s_u8,
                                                        uint8_t* __restrict__ a_u8) {
    const long long tid = (long long)blockIdx.x * 256 + threadIdx.x;
    const long long per_row = K / 8;
    // N * K / 8 is a multiple of GW and groups are lane-aligned, so a group's
    // threads are all in range or all out of range; out-of-range threads
    // still take part in the shuffles (on row 0) and write nothing
    const bool live = tid < (long long)N * per_row;
    const long long t = live ? tid : 0;
    const int n = (int)(t / per_row);
    const int k = (int)(t % per_row) * 8;
    const float s_ch = sw[n];
    const float4* w4 = reinterpret_cast<const float4*>(W + (size_t)n * K + k);
    const float4 v0 = w4[0], v1 = w4[1];
    const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    int q8[8];
    int mn = 127, mx = -128;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        q8[e] = quant_sym(v[e], s_ch, qmax);
        mn = min(mn, q8[e]);
        mx = max(mx, q8[e]);
    }
#pragma unroll
    for (int off = GW / 2; off > 0; off >>= 1) {
        mn = min(mn, __shfl_xor(mn, off, 64));
        mx = max(mx, __shfl_xor(mx, off, 64));
    }
    if (!live) return;
    const int R = mx - mn;
    int s = (R + 14) / 15;
    s = s < 1 ? 1 : s;
    const int a = 128 + mn;
    const int cap = (127 - mn) / s;
    const int groups = K / (8 * GW);
    const int j = k / (8 * GW);
    if ((threadIdx.x & (GW - 1)) == 0) {
        s_u8[param_offset(n, j, groups)] = (uint8_t)s;
        a_u8[param_offset(n, j, groups)] = (uint8_t)a;
    }
    unsigned word = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int u = q8[e] - mn;
        int q = (2 * u + s) / (2 * s);
        q = min(q, cap);
        q = min(q, 15);
        // column +e -> byte (e & 3), low nibble for e < 4, high for e >= 4
        word |= (unsigned)q << (8 * (e & 3) + 4 * (e >> 2));
    }
    const int KT = K / kTileK, nt = n / kTileN, r = n % kTileN;
    const int kt = k / kTileK, kk = k % kTileK;
    const size_t off = packed_dword_offset(nt, kt, KT, kk / 32, r, (kk % 32) / 8);
    *reinterpret_cast<unsigned*>(wq + off) = word;
}

// INT4 symmetric sign-magnitude nibbles.  One thread per packed dword
// (8 consecutive columns of one row).
__global__ __launch_bounds__(256) void int4_pack_kernel(const float* __restrict__ W,
                                                        const float* __restrict__ sw, int N, int K,
                                                        uint8_t* __restrict__ wq) {
    const long long tid = (long long)blockIdx.x * 256 + threadIdx.x;
    const long long per_row = K / 8;
    if (tid >= (long long)N * per_row) return;
    const int n = (int)(tid / per_row);
    const int k = (int)(tid % per_row) * 8;
    const float s_ch = sw[n];
    const float* w = W + (size_t)n * K + k;
    unsigned word = 0;
    for (int e = 0; e < 8; ++e) {
        int q = quant_sym(w[e], s_ch, 7.0f);
        unsigned c = q < 0 ? (0x8u | (unsigned)(-q)) : (unsigned)q;
        word |= c << (8 * (e & 3) + 4 * (e >> 2));
    }
    const int KT = K / kTileK, nt = n / kTileN, r = n % kTileN;
    const int kt = k / kTileK, kk = k % kTileK;
    size_t off = packed_dword_offset(nt, kt, KT, kk / 32, r, (kk % 32) / 8);
    *reinterpret_cast<unsigned*>(wq + off) = word;
}

// ---------------------------------------------------------------------------
// W8A8 comparison: the per-channel INT8 codes of the first quantisation
// level in the 8-bit tile layout.  One thread per 16-byte piece: piece
// (nt, kt, u, G, r) = row 16nt + r, columns 128kt + 32G + 16u .. +15, stored
// at byte 2048 (nt KT + kt) + 1024 u + 16 (16 G + r).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void w8_pack_kernel(const float* __restrict__ W,
                                                      const float* __restrict__ sw, int N, int K,
                                                      int8_t* __restrict__ wq8) {
    const long long p = (long long)blockIdx.x * 256 + threadIdx.x;
    if (p >= (long long)N * K / 16) return;
    const int KT = K / kTileK;
    const int lane = (int)(p & 63), u = (int)((p >> 6) & 1);
    const long long tile = p >> 7;  // nt * KT + kt
    const int nt = (int)(tile / KT), kt = (int)(tile % KT);
    const int r = lane & 15, G = lane >> 4;
    const int n = nt * kTileN + r;
    const float* w = W + (size_t)n * K + (size_t)kt * kTileK + 32 * G + 16 * u;
    const float s = sw[n];
    unsigned b[4] = {0u, 0u, 0u, 0u};
    for (int j = 0; j < 16; ++j)
        b[j >> 2] |= ((unsigned)quant_sym(w[j], s, 127.0f) & 0xFFu) << (8 * (j & 3));
    *reinterpret_cast<v4i*>(wq8 + (size_t)tile * 2048 + 1024 * u + 16 * lane) =
        v4i{(int)b[0], (int)b[1], (int)b[2], (int)b[3]};
}

// ---------------------------------------------------------------------------
// INT4 with per-group scales folded into FP8 weights and a per-tensor
// rescale (FireQ, arXiv 2505.20839, abstract; the formulas are this
// library's reading): s_g = max|group| / 7, t = max|W| / 448, f = s_g / t,
// q = clamp(rne(W / s_g), -7, 7) in sign-magnitude nibbles.  The GEMM
// turns q into e4m3(|q| f) with q's sign and rescales by t.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void row_absmax_kernel(const float* __restrict__ W, int K,
                                                         float* __restrict__ rmax) {
    const float m = block_absmax_256(W + (size_t)blockIdx.x * K, K);
    if (threadIdx.x == 0) rmax[blockIdx.x] = m;
}

// t = max_n rmax[n] / 448 (an all-zero tensor gets 1); one workgroup.
__global__ __launch_bounds__(256) void tensor_scale_kernel(const float* __restrict__ rmax, int N,
                                                           float* __restrict__ t) {
    float m = 0.0f;
    for (int i = threadIdx.x; i < N; i += 256) m = fmaxf(m, rmax[i]);
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    __shared__ float part[4];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        m = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
        t[0] = scale_of(m, 448.0f);
    }
}

// One thread per (group, row): its scale, folded factor (group-major
// fsc[j][n], so a K-step's factors of consecutive channels are adjacent)
// and packed codes.
__global__ __launch_bounds__(256) void fp8g_group_kernel(const float* __restrict__ W,
                                                         const float* __restrict__ t, int N, int K,
                                                         int group, uint8_t* __restrict__ wq,
                                                         float* __restrict__ fsc) {
    const long long tid = (long long)blockIdx.x * 256 + threadIdx.x;
    const int groups = K / group;
    if (tid >= (long long)N * groups) return;
    const int j = (int)(tid / N), n = (int)(tid % N);
    const float* w = W + (size_t)n * K + (size_t)j * group;
    float amax = 0.0f;
    for (int k = 0; k < group; ++k) amax = fmaxf(amax, fabsf(w[k]));
    const float sg = scale_of(amax, 7.0f);
    fsc[tid] = __fdiv_rn(sg, t[0]);
    const int KT = K / kTileK, nt = n / kTileN, r = n % kTileN;
    for (int k8 = 0; k8 < group; k8 += 8) {
        unsigned word = 0;
        for (int e = 0; e < 8; ++e) {
            const int q = quant_sym(w[k8 + e], sg, 7.0f);
            const unsigned c = q < 0 ? (0x8u | (unsigned)(-q)) : (unsigned)q;
            word |= c << (8 * (e & 3) + 4 * (e >> 2));
        }
        const int k = j * group + k8;
        const int kt = k / kTileK, kk = k % kTileK;
        const size_t off = packed_dword_offset(nt, kt, KT, kk / 32, r, (kk % 32) / 8);
        *reinterpret_cast<unsigned*>(wq + off) = word;
    }
}

// ---------------------------------------------------------------------------
// Per-token activation quantisation: one workgroup per row.  The input is
// float32, fp16 or bf16 (IN = 0, 1, 2); each element is first widened to
// float32, which is exact, so every input type quantises like float32.
// ---------------------------------------------------------------------------
template <int IN>
struct Row8 {  // eight consecutive elements of a row, widened to float32
    float v[8];
};

template <int IN>
struct Raw8 {  // the same eight elements as stored (32 bytes float32, 16 otherwise)
    v4i w[IN == 0 ? 2 : 1];
};

template <int IN>
__device__ __forceinline__ Raw8<IN> load_raw8(const void* row, int i) {  // elements 8i..8i+7
    Raw8<IN> r;
    const v4i* p = reinterpret_cast<const v4i*>(row) + (IN == 0 ? 2 * i : i);
    r.w[0] = p[0];
    if constexpr (IN == 0) r.w[1] = p[1];
    return r;
}

template <int IN>
__device__ __forceinline__ Row8<IN> widen8(const Raw8<IN>& w) {
    Row8<IN> r;
    if constexpr (IN == 0) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            // through a scalar: a bit cast of the vector element itself
            // reads lane 0 of the vector with this compiler
            const int x = w.w[j >> 2][j & 3];
            r.v[j] = __builtin_bit_cast(float, x);
        }
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const unsigned h = ((unsigned)w.w[0][j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
            if constexpr (IN == 1)
                r.v[j] = (float)__builtin_bit_cast(_Float16, (unsigned short)h);
            else
                r.v[j] = __builtin_bit_cast(float, h << 16);
        }
    }
    return r;
}

template <int IN>
__device__ __forceinline__ Row8<IN> load_row8(const void* row, int i) {
    return widen8<IN>(load_raw8<IN>(row, i));
}

// Largest of the TPB threads' values.
template <int TPB = 256>
__device__ __forceinline__ float block_max(float m) {
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    __shared__ float part[TPB / 64];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
    __syncthreads();
    m = part[0];
#pragma unroll
    for (int w = 1; w < TPB / 64; ++w) m = fmaxf(m, part[w]);
    __syncthreads();
    return m;
}

template <int IN>
__device__ __forceinline__ float row_absmax(const void* row, int K) {
    float m = 0.0f;
    for (int i = threadIdx.x; i < K / 8; i += 256) {
        const Row8<IN> r = load_row8<IN>(row, i);
#pragma unroll
        for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(r.v[j]));
    }
    return block_max(m);
}

template <int IN>
__device__ __forceinline__ const void* row_ptr(const void* X, int K) {
    constexpr int EB = IN == 0 ? 4 : 2;
    return reinterpret_cast<const uint8_t*>(X) + (size_t)blockIdx.x * K * EB;
}

template <int IN>
__global__ __launch_bounds__(256) void act_int8_kernel(const void* __restrict__ X, int K,
                                                       int8_t* __restrict__ Xq,
                                                       float* __restrict__ sx) {
    const void* row = row_ptr<IN>(X, K);
    const float s = scale_of(row_absmax<IN>(row, K), 127.0f);
    if (threadIdx.x == 0) sx[blockIdx.x] = s;
    uint2* out = reinterpret_cast<uint2*>(Xq + (size_t)blockIdx.x * K);
    for (int i = threadIdx.x; i < K / 8; i += 256) {
        const Row8<IN> r = load_row8<IN>(row, i);
        unsigned b[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) b[j] = (unsigned)(quant_sym(r.v[j], s, 127.0f) & 0xFF);
        out[i] = uint2{b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24),
                       b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24)};
    }
}

// float32 -> OCP e4m3 ("fn"), nearest-even, saturating to +-448, sign kept.
// Normal inputs: the significand is rounded to 3 fraction bits at the
// input's own binade (2^(e-3) quantum); below 2^-6 the fixed subnormal
// quantum 2^-9 applies.  A carry out of the significand moves to the next
// binade through the plain addition of the exponent and mantissa fields.
__device__ __forceinline__ unsigned f32_to_e4m3(float x) {
    unsigned u = __builtin_bit_cast(unsigned, x);
    unsigned sign = (u >> 24) & 0x80u;
    float a = fabsf(x);
    if (a != a) return 0x7Fu;
    if (a >= 448.0f) return sign | 0x7Eu;
    if (a < 0.015625f) {  // 2^-6
        unsigned m = (unsigned)__builtin_rintf(a * 512.0f);  // exact scaling by 2^9
        return sign | m;  // m == 8 is exactly the smallest normal, code 0x08
    }
    int e = (int)((u >> 23) & 0xFFu) - 127;         // -6 .. 8
    float t = __builtin_ldexpf(a, 3 - e);            // in [8, 16), exact
    unsigned mi = (unsigned)__builtin_rintf(t);      // 8 .. 16
    unsigned code = (unsigned)((e + 7) << 3) + (mi - 8u);
    if (code > 0x7Eu) code = 0x7Eu;
    return sign | code;
}

template <int IN>
__global__ __launch_bounds__(256) void act_e4m3_kernel(const void* __restrict__ X, int K,
                                                       uint8_t* __restrict__ Xq,
                                                       float* __restrict__ sx) {
    const void* row = row_ptr<IN>(X, K);
    const float s = scale_of(row_absmax<IN>(row, K), 448.0f);
    if (threadIdx.x == 0) sx[blockIdx.x] = s;
    uint2* out = reinterpret_cast<uint2*>(Xq + (size_t)blockIdx.x * K);
    for (int i = threadIdx.x; i < K / 8; i += 256) {
        const Row8<IN> r = load_row8<IN>(row, i);
        unsigned b[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) b[j] = f32_to_e4m3(__fdiv_rn(r.v[j], s));
        out[i] = uint2{b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24),
                       b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24)};
    }
}

// The same two quantisers with the row held in registers between the
// absolute maximum and the quantisation (rows of at most 8 TPB CH
// elements): the row is read from memory once instead of twice.  Q: 0 =
// INT8 (qmax 127), 1 = e4m3; arithmetic identical to the kernels above.
// TPB threads per row: 1024 when there are fewer rows than CUs, so that
// each thread converts fewer elements.
template <int IN, int Q, int CH, int TPB>
__global__ __launch_bounds__(TPB) void act_quant_regs_kernel(const void* __restrict__ X, int K,
                                                             uint8_t* __restrict__ Xq,
                                                             float* __restrict__ sx) {
    const void* row = row_ptr<IN>(X, K);
    const int n8 = K / 8;
    Raw8<IN> c[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
        const int i = threadIdx.x + TPB * j;
        c[j] = i < n8 ? load_raw8<IN>(row, i) : Raw8<IN>{};
    }
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
        const Row8<IN> r = widen8<IN>(c[j]);  // zeros past the row end
#pragma unroll
        for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(r.v[e]));
    }
    const float s = scale_of(block_max<TPB>(m), Q == 0 ? 127.0f : 448.0f);
    if (threadIdx.x == 0) sx[blockIdx.x] = s;
    uint2* out = reinterpret_cast<uint2*>(Xq + (size_t)blockIdx.x * K);
#pragma unroll
    for (int j = 0; j < CH; ++j) {
        const int i = threadIdx.x + TPB * j;
        if (i >= n8) continue;
        const Row8<IN> r = widen8<IN>(c[j]);
        if constexpr (Q == 0) {
            unsigned b[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) b[e] = (unsigned)(quant_sym(r.v[e], s, 127.0f) & 0xFF);
            out[i] = uint2{b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24),
                           b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24)};
        } else {
            // |x / s| <= 448 (1 + 2^-23) here, where the hardware conversion
            // (nearest even) gives f32_to_e4m3's codes; a NaN quotient (NaN
            // input) gets f32_to_e4m3's 0x7F whatever its sign
            float t[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) t[e] = __fdiv_rn(r.v[e], s);
            unsigned w[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int l = __builtin_amdgcn_cvt_pk_fp8_f32(t[4 * h], t[4 * h + 1], 0, false);
                w[h] = (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(t[4 * h + 2], t[4 * h + 3], l,
                                                                  true);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (t[4 * h + e] != t[4 * h + e])
                        w[h] = (w[h] & ~(0xFFu << (8 * e))) | (0x7Fu << (8 * e));
            }
            out[i] = uint2{w[0], w[1]};
        }
    }
}

template <int IN, int Q>
static bool launch_act_regs(const void* X, int M, int K, uint8_t* Xq, float* sx,
                            hipStream_t st) {
    const int n8 = K / 8;
#define ACT_REGS(CH, TPB)                                                                   \
    if (n8 <= TPB * CH) {                                                                   \
        hipLaunchKernelGGL((act_quant_regs_kernel<IN, Q, CH, TPB>), dim3(M), dim3(TPB), 0, st, \
                           X, K, Xq, sx);                                                   \
        return true;                                                                        \
    }
    if (M < 256) {
        ACT_REGS(1, 1024)
        ACT_REGS(2, 1024)
        ACT_REGS(4, 1024)
    } else {
        ACT_REGS(2, 256)
        ACT_REGS(4, 256)
        ACT_REGS(8, 256)
        ACT_REGS(16, 256)
    }
#undef ACT_REGS
    return false;  // longer rows: the two-pass kernels
}

// ----------------------------------------------------------- launchers ----
hipError_t launch_pack_lqq(const float* W, int N, int K, int group, int qmax, uint8_t* wq,
                           uint8_t* s_u8, uint8_t* a_u8, float* sw, hipStream_t st) {
    hipLaunchKernelGGL(row_scale_kernel, dim3(N), dim3(256), 0, st, W, K, (float)qmax, sw);
    const long long threads = (long long)N * (K / 8);  // one per packed dword
    const unsigned blocks = (unsigned)((threads + 255) / 256);
    if (group == 64)
        hipLaunchKernelGGL((lqq_group_kernel<8>), dim3(blocks), dim3(256), 0, st, W, sw, N, K,
                           (float)qmax, wq, s_u8, a_u8);
    else
        hipLaunchKernelGGL((lqq_group_kernel<16>), dim3(blocks), dim3(256), 0, st, W, sw, N, K,
                           (float)qmax, wq, s_u8, a_u8);
    return hipGetLastError();
}

hipError_t launch_pack_int4(const float* W, int N, int K, uint8_t* wq, float* sw,
                            hipStream_t st) {
    hipLaunchKernelGGL(row_scale_kernel, dim3(N), dim3(256), 0, st, W, K, 7.0f, sw);
    long long threads = (long long)N * (K / 8);
    unsigned blocks = (unsigned)((threads + 255) / 256);
    hipLaunchKernelGGL(int4_pack_kernel, dim3(blocks), dim3(256), 0, st, W, sw, N, K, wq);
    return hipGetLastError();
}

hipError_t launch_pack_w8(const float* W, int N, int K, int8_t* wq8, float* sw, hipStream_t st) {
    hipLaunchKernelGGL(row_scale_kernel, dim3(N), dim3(256), 0, st, W, K, 127.0f, sw);
    const long long pieces = (long long)N * K / 16;
    const unsigned blocks = (unsigned)((pieces + 255) / 256);
    hipLaunchKernelGGL(w8_pack_kernel, dim3(blocks), dim3(256), 0, st, W, sw, N, K, wq8);
    return hipGetLastError();
}

hipError_t launch_pack_fp8g(const float* W, int N, int K, int group, uint8_t* wq, float* fsc,
                            float* tscale, hipStream_t st) {
    // fsc's first N floats hold the row maxima until the group kernel
    // overwrites them (it reads only tscale).
    hipLaunchKernelGGL(row_absmax_kernel, dim3(N), dim3(256), 0, st, W, K, fsc);
    hipLaunchKernelGGL(tensor_scale_kernel, dim3(1), dim3(256), 0, st, fsc, N, tscale);
    long long threads = (long long)N * (K / group);
    unsigned blocks = (unsigned)((threads + 255) / 256);
    hipLaunchKernelGGL(fp8g_group_kernel, dim3(blocks), dim3(256), 0, st, W, tscale, N, K, group,
                       wq, fsc);
    return hipGetLastError();
}

hipError_t launch_act_int8(const void* X, int in_type, int M, int K, int8_t* Xq, float* sx,
                           hipStream_t st) {
    uint8_t* Xb = reinterpret_cast<uint8_t*>(Xq);
    const bool regs = in_type == 1   ? launch_act_regs<1, 0>(X, M, K, Xb, sx, st)
                      : in_type == 2 ? launch_act_regs<2, 0>(X, M, K, Xb, sx, st)
                                     : launch_act_regs<0, 0>(X, M, K, Xb, sx, st);
    if (regs)
        ;
    else if (in_type == 1)
        hipLaunchKernelGGL(act_int8_kernel<1>, dim3(M), dim3(256), 0, st, X, K, Xq, sx);
    else if (in_type == 2)
        hipLaunchKernelGGL(act_int8_kernel<2>, dim3(M), dim3(256), 0, st, X, K, Xq, sx);
    else
        hipLaunchKernelGGL(act_int8_kernel<0>, dim3(M), dim3(256), 0, st, X, K, Xq, sx);
    return hipGetLastError();
}

hipError_t launch_act_e4m3(const void* X, int in_type, int M, int K, uint8_t* Xq, float* sx,
                           hipStream_t st) {
    const bool regs = in_type == 1   ? launch_act_regs<1, 1>(X, M, K, Xq, sx, st)
                      : in_type == 2 ? launch_act_regs<2, 1>(X, M, K, Xq, sx, st)
                                     : launch_act_regs<0, 1>(X, M, K, Xq, sx, st);
    if (regs)
        ;
    else if (in_type == 1)
        hipLaunchKernelGGL(act_e4m3_kernel<1>, dim3(M), dim3(256), 0, st, X, K, Xq, sx);
    else if (in_type == 2)
        hipLaunchKernelGGL(act_e4m3_kernel<2>, dim3(M), dim3(256), 0, st, X, K, Xq, sx);
    else
        hipLaunchKernelGGL(act_e4m3_kernel<0>, dim3(M), dim3(256), 0, st, X, K, Xq, sx);
    return hipGetLastError();
}

}  // namespace w4a8
