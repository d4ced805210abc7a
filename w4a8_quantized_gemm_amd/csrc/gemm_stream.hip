// Streamed-tile W4A8 and W4FP8 GEMM kernels for gfx950 (any M; the
// weight-bandwidth-bound decode path).
//
// Each wave streams packed weight tiles (16 rows x 128 K = 1 KiB, one
// 16-byte load per lane) straight from HBM into registers, dequantises them
// in registers and feeds the matrix cores:
//   W4A8:  (q*s + a) XOR 0x80 per byte, two 16-bit-lane multiply-adds and
//          one XOR per 8 weights after the nibble split (LiquidGEMM, Pith
//          review of arXiv 2509.01229, "What carries the argument" and
//          minor comment 1: paper Eq. 12 and Sec. 5.3), then two
//          v_mfma_i32_16x16x64_i8 per tile;
//   W4FP8: sign-magnitude INT4 -> e4m3 by a byte-table v_perm_b32, then one
//          v_mfma_scale_f32_16x16x128_f8f6f4 per tile with unit scales
//          (FireQ, arXiv 2505.20839, abstract: INT4 weights x FP8
//          activations).
// The activation rows (16 per workgroup, rows >= M read as zero) come from
// L2.  `ks` waves of a workgroup split the K range of the same output tile;
// their partial sums are reduced in LDS in wave order (exact for int32), and
// the per-token x per-channel scale epilogue is fused into the store.
#include "device_common.h"
#include "launch.h"

namespace w4a8 {

template <int NTW, int OUT>
__global__ __launch_bounds__(1024) void w4a8_stream_kernel(
    const int8_t* __restrict__ X, const float* __restrict__ sx, const uint8_t* __restrict__ wq,
    const uint8_t* __restrict__ s_u8, const uint8_t* __restrict__ a_u8,
    const float* __restrict__ sw, void* __restrict__ Y, int M, int N, int K, int group, int ks) {
    extern __shared__ int red[];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r = lane & 15, G = lane >> 4;
    const int KT = K / kTileK;
    const int groups = K / group;
    const int nt0 = blockIdx.x * NTW;
    const int m0 = blockIdx.y * 16;
    const int kt_begin = (int)((long long)KT * wave / ks);
    const int kt_end = (int)((long long)KT * (wave + 1) / ks);
    const int m = m0 + r;
    const bool mvalid = m < M;
    const int8_t* xrow = X + (size_t)(mvalid ? m : 0) * K + 32 * G;
    const uint8_t* wlane = wq + (size_t)lane * 16;

    v4i acc[NTW];
#pragma unroll
    for (int t = 0; t < NTW; ++t) acc[t] = v4i{0, 0, 0, 0};

    for (int kt = kt_begin; kt < kt_end; ++kt) {
        v4i xa0 = v4i{0, 0, 0, 0}, xa1 = v4i{0, 0, 0, 0};
        if (mvalid) {
            xa0 = load16(xrow + (size_t)kt * kTileK);
            xa1 = load16(xrow + (size_t)kt * kTileK + 16);
        }
        const int j = (kt * kTileK + 32 * G) / group;
#pragma unroll
        for (int t = 0; t < NTW; ++t) {
            const int nt = nt0 + t;
            const v4i w = load16(wlane + ((size_t)nt * KT + kt) * kTileBytes);
            const size_t gi = param_offset(nt * kTileN + r, j, groups);
            const unsigned s = s_u8[gi], a = a_u8[gi];
            const u16x2 s2 = u16x2{(unsigned short)s, (unsigned short)s};
            const unsigned short aa = (unsigned short)(a * 0x101u);
            const u16x2 a4 = u16x2{aa, aa};
            unsigned b[8];
            lqq_dequant8((unsigned)w.x, s2, a4, b[0], b[1]);
            lqq_dequant8((unsigned)w.y, s2, a4, b[2], b[3]);
            lqq_dequant8((unsigned)w.z, s2, a4, b[4], b[5]);
            lqq_dequant8((unsigned)w.w, s2, a4, b[6], b[7]);
            const v4i B0 = v4i{(int)b[0], (int)b[1], (int)b[2], (int)b[3]};
            const v4i B1 = v4i{(int)b[4], (int)b[5], (int)b[6], (int)b[7]};
            acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(xa0, B0, acc[t], 0, 0, 0);
            acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(xa1, B1, acc[t], 0, 0, 0);
        }
    }

    if (ks > 1) {
#pragma unroll
        for (int t = 0; t < NTW; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v) red[((wave * NTW + t) * 4 + v) * 64 + lane] = acc[t][v];
        __syncthreads();
        if (wave != 0) return;
        for (int w = 1; w < ks; ++w)
#pragma unroll
            for (int t = 0; t < NTW; ++t)
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[t][v] += red[((w * NTW + t) * 4 + v) * 64 + lane];
    }

    // Output: lane holds rows m0 + 4G + v, column (nt*16 + r).
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
        const int n = (nt0 + t) * kTileN + r;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int mo = m0 + 4 * G + v;
            if (mo >= M) continue;
            if (OUT == 1) {
                reinterpret_cast<int*>(Y)[(size_t)mo * N + n] = acc[t][v];
            } else {
                const float y = ((float)acc[t][v] * sx[mo]) * sw[n];
                reinterpret_cast<unsigned short*>(Y)[(size_t)mo * N + n] = f32_to_f16_bits(y);
            }
        }
    }
}

template <int NTW, int OUT>
__global__ __launch_bounds__(1024) void w4fp8_stream_kernel(
    const uint8_t* __restrict__ X, const float* __restrict__ sx, const uint8_t* __restrict__ wq,
    const float* __restrict__ sw, void* __restrict__ Y, int M, int N, int K, int ks) {
    extern __shared__ int red[];
    float* redf = reinterpret_cast<float*>(red);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r = lane & 15, G = lane >> 4;
    const int KT = K / kTileK;
    const int nt0 = blockIdx.x * NTW;
    const int m0 = blockIdx.y * 16;
    const int kt_begin = (int)((long long)KT * wave / ks);
    const int kt_end = (int)((long long)KT * (wave + 1) / ks);
    const int m = m0 + r;
    const bool mvalid = m < M;
    const uint8_t* xrow = X + (size_t)(mvalid ? m : 0) * K + 32 * G;
    const uint8_t* wlane = wq + (size_t)lane * 16;

    v4f acc[NTW];
#pragma unroll
    for (int t = 0; t < NTW; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};

    for (int kt = kt_begin; kt < kt_end; ++kt) {
        v4i xa0 = v4i{0, 0, 0, 0}, xa1 = v4i{0, 0, 0, 0};
        if (mvalid) {
            xa0 = load16(xrow + (size_t)kt * kTileK);
            xa1 = load16(xrow + (size_t)kt * kTileK + 16);
        }
        const v8i A = v8i{xa0.x, xa0.y, xa0.z, xa0.w, xa1.x, xa1.y, xa1.z, xa1.w};
#pragma unroll
        for (int t = 0; t < NTW; ++t) {
            const int nt = nt0 + t;
            const v4i w = load16(wlane + ((size_t)nt * KT + kt) * kTileBytes);
            const v8i B = v8i{(int)int4_to_e4m3_lo(w.x), (int)int4_to_e4m3_hi(w.x),
                              (int)int4_to_e4m3_lo(w.y), (int)int4_to_e4m3_hi(w.y),
                              (int)int4_to_e4m3_lo(w.z), (int)int4_to_e4m3_hi(w.z),
                              (int)int4_to_e4m3_lo(w.w), (int)int4_to_e4m3_hi(w.w)};
            // formats 0/0 = e4m3 x e4m3; E8M0 scale 127 = 2^0 on both sides
            acc[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, acc[t], 0, 0, 0, 127,
                                                                      0, 127);
        }
    }

    if (ks > 1) {
#pragma unroll
        for (int t = 0; t < NTW; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v) redf[((wave * NTW + t) * 4 + v) * 64 + lane] = acc[t][v];
        __syncthreads();
        if (wave != 0) return;
        for (int w = 1; w < ks; ++w)
#pragma unroll
            for (int t = 0; t < NTW; ++t)
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[t][v] += redf[((w * NTW + t) * 4 + v) * 64 + lane];
    }

#pragma unroll
    for (int t = 0; t < NTW; ++t) {
        const int n = (nt0 + t) * kTileN + r;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int mo = m0 + 4 * G + v;
            if (mo >= M) continue;
            const float y = (acc[t][v] * sx[mo]) * sw[n];
            if (OUT == 1)
                reinterpret_cast<float*>(Y)[(size_t)mo * N + n] = y;
            else
                reinterpret_cast<unsigned short*>(Y)[(size_t)mo * N + n] = f32_to_bf16_bits(y);
        }
    }
}

// ----------------------------------------------------------- launchers ----
template <int NTW>
static hipError_t w4a8_stream_ntw(const int8_t* X, const float* sx, const uint8_t* wq,
                                  const uint8_t* s_u8, const uint8_t* a_u8, const float* sw,
                                  void* Y, int out_type, int M, int N, int K, int group, int ks,
                                  hipStream_t st) {
    dim3 grid(N / (kTileN * NTW), (M + 15) / 16);
    dim3 block(64 * ks);
    size_t lds = ks > 1 ? (size_t)ks * NTW * 4 * 64 * sizeof(int) : 0;
    if (out_type == 1)
        hipLaunchKernelGGL((w4a8_stream_kernel<NTW, 1>), grid, block, lds, st, X, sx, wq, s_u8,
                           a_u8, sw, Y, M, N, K, group, ks);
    else
        hipLaunchKernelGGL((w4a8_stream_kernel<NTW, 0>), grid, block, lds, st, X, sx, wq, s_u8,
                           a_u8, sw, Y, M, N, K, group, ks);
    return hipGetLastError();
}

hipError_t launch_w4a8_stream(const int8_t* X, const float* sx, const uint8_t* wq,
                              const uint8_t* s_u8, const uint8_t* a_u8, const float* sw,
                              void* Y, int out_type, int M, int N, int K, int group,
                              StreamCfg cfg, hipStream_t st) {
    switch (cfg.nt_per_wave) {
        case 4: return w4a8_stream_ntw<4>(X, sx, wq, s_u8, a_u8, sw, Y, out_type, M, N, K, group, cfg.ks, st);
        case 2: return w4a8_stream_ntw<2>(X, sx, wq, s_u8, a_u8, sw, Y, out_type, M, N, K, group, cfg.ks, st);
        default: return w4a8_stream_ntw<1>(X, sx, wq, s_u8, a_u8, sw, Y, out_type, M, N, K, group, cfg.ks, st);
    }
}

template <int NTW>
static hipError_t w4fp8_stream_ntw(const uint8_t* X, const float* sx, const uint8_t* wq,
                                   const float* sw, void* Y, int out_type, int M, int N, int K,
                                   int ks, hipStream_t st) {
    dim3 grid(N / (kTileN * NTW), (M + 15) / 16);
    dim3 block(64 * ks);
    size_t lds = ks > 1 ? (size_t)ks * NTW * 4 * 64 * sizeof(float) : 0;
    if (out_type == 1)
        hipLaunchKernelGGL((w4fp8_stream_kernel<NTW, 1>), grid, block, lds, st, X, sx, wq, sw, Y,
                           M, N, K, ks);
    else
        hipLaunchKernelGGL((w4fp8_stream_kernel<NTW, 0>), grid, block, lds, st, X, sx, wq, sw, Y,
                           M, N, K, ks);
    return hipGetLastError();
}

hipError_t launch_w4fp8_stream(const uint8_t* X, const float* sx, const uint8_t* wq,
                               const float* sw, void* Y, int out_type, int M, int N, int K,
                               StreamCfg cfg, hipStream_t st) {
    switch (cfg.nt_per_wave) {
        case 4: return w4fp8_stream_ntw<4>(X, sx, wq, sw, Y, out_type, M, N, K, cfg.ks, st);
        case 2: return w4fp8_stream_ntw<2>(X, sx, wq, sw, Y, out_type, M, N, K, cfg.ks, st);
        default: return w4fp8_stream_ntw<1>(X, sx, wq, sw, Y, out_type, M, N, K, cfg.ks, st);
    }
}

}  // namespace w4a8
