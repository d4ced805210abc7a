// Large-M W4A8 GEMM for gfx950 (the matrix-core-bound regime).
//
// Workgroup tile: MT rows of X (M) x 4*64 output channels (N); four waves,
// each owning all MT rows and its own 64 channels, so every weight is
// dequantised exactly once per workgroup tile and goes from registers
// straight into the matrix cores (the consumer dequantises what it
// multiplies, as in the implicit pipeline of LiquidGEMM, Pith review of
// arXiv 2509.01229, "What carries the argument" -- here without a producer
// wave: the loads are asynchronous and prefetched one K-step ahead).
// Dequantisation is the LiquidQuant identity (q*s + a) XOR 0x80, two VALU
// instructions per four weights after the nibble split (same review, paper
// Eq. 12; minor comment 1 / Sec. 5.3 for the instruction count).
//
// Per K-step of 128:
//   X[MT][128] int8 -> LDS (double buffer, row stride 144 B so the 16 rows
//     read by one ds_read_b128 fall in distinct banks);
//   each wave: 4 packed tiles (16 ch x 128 K, 16 B per lane) + their
//     (s_u8, a_u8) -> 32 dequantised operand registers;
//   MT/16 x 4 x 2 v_mfma_i32_16x16x64_i8 into MT/16 x 4 int32 accumulators.
// Epilogue: Y = fp16((float(acc) * sx[m]) * sw[n]) or the raw int32.
#include "device_common.h"
#include "launch.h"

namespace w4a8 {

namespace {

constexpr int kWaves = 4;
constexpr int kColsPerWave = 64;                  // 4 packed tiles
constexpr int kNT = kWaves * kColsPerWave;        // 256 channels per workgroup
constexpr int kLdsRow = 144;                      // 128 data bytes + 16 pad

template <int MT>
struct XStage {
    static constexpr int kChunks = MT * 8;             // 16-byte chunks per K-step
    static constexpr int kPerThread = kChunks / 256;   // 256 threads
};

}  // namespace

template <int MT, int OUT>
__global__ __launch_bounds__(256, 1) void w4a8_mfma_kernel(
    const int8_t* __restrict__ X, const float* __restrict__ sx, const uint8_t* __restrict__ wq,
    const uint8_t* __restrict__ s_u8, const uint8_t* __restrict__ a_u8,
    const float* __restrict__ sw, void* __restrict__ Y, int M, int N, int K, int group,
    int tiles_n, int tiles_m) {
    constexpr int MB = MT / 16;  // 16-row blocks per wave
    constexpr int XP = XStage<MT>::kPerThread;
    __shared__ __attribute__((aligned(16))) uint8_t xs[2][MT * kLdsRow];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int r = lane & 15, G = lane >> 4;

    // Workgroup -> tile.  Consecutive workgroups are dealt round-robin to
    // the 8 XCDs; regroup so each XCD walks a contiguous run of tiles, with
    // the M tiles of one channel panel adjacent (shared weight panel in L2).
    const int nwg = tiles_n * tiles_m;
    const int bid = blockIdx.x;
    int lin = bid;
    if ((nwg & 7) == 0) lin = (bid & 7) * (nwg >> 3) + (bid >> 3);
    const int tm = lin % tiles_m;
    const int tn = lin / tiles_m;
    const int m0 = tm * MT;
    const int n0 = tn * kNT + wave * kColsPerWave;

    const int KT = K / kTileK;
    const int groups = K / group;

    // ---- X staging: thread owns chunks c = tid + 256*p (row c/8, 16-B col c%8)
    v4i xreg[XP];
    auto load_x = [&](int kt) {
#pragma unroll
        for (int p = 0; p < XP; ++p) {
            const int c = tid + 256 * p;
            const int row = c >> 3, col = c & 7;
            const int m = m0 + row;
            xreg[p] = v4i{0, 0, 0, 0};
            if (m < M) xreg[p] = load16(X + (size_t)m * K + (size_t)kt * kTileK + col * 16);
        }
    };
    auto store_x = [&](int buf) {
#pragma unroll
        for (int p = 0; p < XP; ++p) {
            const int c = tid + 256 * p;
            const int row = c >> 3, col = c & 7;
            *reinterpret_cast<v4i*>(&xs[buf][row * kLdsRow + col * 16]) = xreg[p];
        }
    };

    // ---- weights of this wave: 4 tiles (nt0 .. nt0+3) at K-step kt
    const int nt0 = n0 / kTileN;
    const uint8_t* wl = wq + (size_t)lane * 16;
    v4i wreg[4];
    unsigned sreg[4], areg[4];
    auto load_w = [&](int kt) {
        const int j = (kt * kTileK + 32 * G) / group;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            wreg[b] = load16(wl + ((size_t)(nt0 + b) * KT + kt) * kTileBytes);
            const size_t gi = (size_t)((nt0 + b) * kTileN + r) * groups + j;
            sreg[b] = s_u8[gi];
            areg[b] = a_u8[gi];
        }
    };

    v4i acc[MB][4];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[i][b] = v4i{0, 0, 0, 0};

    load_x(0);
    load_w(0);
    store_x(0);
    __syncthreads();

    for (int kt = 0; kt < KT; ++kt) {
        const int buf = kt & 1;
        // dequantise this step's weights into operands B[b][h]
        v4i B[4][2];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const u16x2 s2 = u16x2{(unsigned short)sreg[b], (unsigned short)sreg[b]};
            const unsigned short aa = (unsigned short)(areg[b] * 0x101u);
            const u16x2 a4 = u16x2{aa, aa};
            unsigned d[8];
            lqq_dequant8((unsigned)wreg[b].x, s2, a4, d[0], d[1]);
            lqq_dequant8((unsigned)wreg[b].y, s2, a4, d[2], d[3]);
            lqq_dequant8((unsigned)wreg[b].z, s2, a4, d[4], d[5]);
            lqq_dequant8((unsigned)wreg[b].w, s2, a4, d[6], d[7]);
            B[b][0] = v4i{(int)d[0], (int)d[1], (int)d[2], (int)d[3]};
            B[b][1] = v4i{(int)d[4], (int)d[5], (int)d[6], (int)d[7]};
        }
        // prefetch the next step (global -> registers)
        if (kt + 1 < KT) {
            load_x(kt + 1);
            load_w(kt + 1);
        }
        const uint8_t* xb = &xs[buf][r * kLdsRow + 32 * G];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int i = 0; i < MB; ++i) {
                const v4i A = *reinterpret_cast<const v4i*>(xb + i * 16 * kLdsRow + 16 * h);
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    acc[i][b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, B[b][h], acc[i][b], 0, 0, 0);
            }
        }
        if (kt + 1 < KT) store_x(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: lane holds rows m0 + 16i + 4G + v, channel n0 + 16b + r
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const int n = n0 + 16 * b + r;
        const float swn = (OUT == 1) ? 0.0f : sw[n];
#pragma unroll
        for (int i = 0; i < MB; ++i) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int m = m0 + 16 * i + 4 * G + v;
                if (m >= M) continue;
                if (OUT == 1) {
                    reinterpret_cast<int*>(Y)[(size_t)m * N + n] = acc[i][b][v];
                } else {
                    const float y = ((float)acc[i][b][v] * sx[m]) * swn;
                    reinterpret_cast<unsigned short*>(Y)[(size_t)m * N + n] = f32_to_f16_bits(y);
                }
            }
        }
    }
}

template <int MT>
static hipError_t launch_mt(const int8_t* X, const float* sx, const uint8_t* wq,
                            const uint8_t* s_u8, const uint8_t* a_u8, const float* sw, void* Y,
                            int out_type, int M, int N, int K, int group, hipStream_t st) {
    const int tiles_n = N / kNT;
    const int tiles_m = (M + MT - 1) / MT;
    dim3 grid(tiles_n * tiles_m), block(256);
    if (out_type == 1)
        hipLaunchKernelGGL((w4a8_mfma_kernel<MT, 1>), grid, block, 0, st, X, sx, wq, s_u8, a_u8,
                           sw, Y, M, N, K, group, tiles_n, tiles_m);
    else
        hipLaunchKernelGGL((w4a8_mfma_kernel<MT, 0>), grid, block, 0, st, X, sx, wq, s_u8, a_u8,
                           sw, Y, M, N, K, group, tiles_n, tiles_m);
    return hipGetLastError();
}

hipError_t launch_w4a8_mfma(const int8_t* X, const float* sx, const uint8_t* wq,
                            const uint8_t* s_u8, const uint8_t* a_u8, const float* sw, void* Y,
                            int out_type, int M, int N, int K, int group, int mt,
                            hipStream_t st) {
    if (mt == 128)
        return launch_mt<128>(X, sx, wq, s_u8, a_u8, sw, Y, out_type, M, N, K, group, st);
    return launch_mt<256>(X, sx, wq, s_u8, a_u8, sw, Y, out_type, M, N, K, group, st);
}

}  // namespace w4a8
