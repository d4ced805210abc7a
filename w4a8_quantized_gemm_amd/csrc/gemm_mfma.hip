// Large-M W4A8 GEMM for gfx950 (the matrix-core-bound regime).
//
// Workgroup tile: MT rows of X (M) x 4*64 output channels (N); four waves,
// each owning all MT rows and its own 64 channels, so every weight is
// dequantised exactly once per workgroup tile and goes from registers
// straight into the matrix cores.  The consumer dequantises what it
// multiplies, as in the implicit pipeline of LiquidGEMM (Pith review of
// arXiv 2509.01229, "What carries the argument"); there is no producer wave:
// loads are asynchronous and run ahead of the math.  Dequantisation is the
// LiquidQuant identity (q*s + a) XOR 0x80, two VALU instructions per four
// weights after the nibble split (same review, paper Eq. 12; minor comment 1
// / Sec. 5.3 for the instruction count).
//
// Per K-step of 128 columns:
//   X[MT][128] int8 of the next step: global -> registers at the start of
//     the step, registers -> LDS (double buffer) at its end; 16-byte slots
//     XOR-swizzled per row so the 16 rows read by one ds_read_b128 fall in
//     distinct banks;
//   each wave: 4 packed tiles (16 ch x 128 K, 16 B per lane) of the next
//     step loaded at the start, dequantised at the end of the step;
//   MT/16 x 4 x 2 v_mfma_i32_16x16x64_i8 into MT/16 x 4 int32 accumulators
//     held in accumulation registers, A operands streamed from LDS through a
//     short register ring.
// With 128-row tiles two workgroups share a CU, so one's barrier and
// dequantisation phases overlap the other's matrix-core phase.
// Epilogue: Y = fp16((float(acc) * sx[m]) * sw[n]) or the raw int32.
#include "device_common.h"
#include "launch.h"

namespace w4a8 {

namespace {

constexpr int kWaves = 4;
constexpr int kColsPerWave = 64;              // 4 packed tiles
constexpr int kNT = kWaves * kColsPerWave;    // 256 channels per workgroup

// Row-dependent XOR of the 16-byte slot index: distinct for rows r and r'
// of a 16-row block whenever they share a bank window, for both 32- and
// 64-bank LDS organisations.
__device__ __forceinline__ int xswz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// Raw weights of one K-step for one wave: 4 packed tiles (16 B per lane)
// and the parameter bytes of the lane's row in those tiles (byte b = tile b).
struct WStep {
    v4i w[4];
    unsigned sdw, adw;
};

__device__ __forceinline__ void dequant_half(const WStep& ws, int h, v4i (&B)[4][2]) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const u16x2 s2 = scale_pair(ws.sdw, b);
        const u16x2 a4 = offset_quad(ws.adw, b);
        unsigned d0, d1, d2, d3;
        const unsigned w0 = (unsigned)(h ? ws.w[b].z : ws.w[b].x);
        const unsigned w1 = (unsigned)(h ? ws.w[b].w : ws.w[b].y);
        lqq_dequant8(w0, s2, a4, d0, d1);
        lqq_dequant8(w1, s2, a4, d2, d3);
        B[b][h] = v4i{(int)d0, (int)d1, (int)d2, (int)d3};
    }
}

// Accumulate into an int32 tile that stays in accumulation registers
// (destination = source C).  Written as inline assembly so the register
// allocator cannot split the accumulators between register files.
__device__ __forceinline__ void mfma_i8_acc(v4i& acc, const v4i& a, const v4i& b) {
    asm("v_mfma_i32_16x16x64_i8 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// Wait states between the last accumulation and the first read of the
// accumulators (the compiler does not see the assembly instructions above).
__device__ __forceinline__ void mfma_drain() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

}  // namespace

template <int MT, int OUT>
__global__ __launch_bounds__(256, MT == 128 ? 2 : 1) void w4a8_mfma_kernel(
    const int8_t* __restrict__ X, const float* __restrict__ sx, const uint8_t* __restrict__ wq,
    const uint8_t* __restrict__ s_u8, const uint8_t* __restrict__ a_u8,
    const float* __restrict__ sw, void* __restrict__ Y, int M, int N, int K, int group,
    int tiles_n, int tiles_m) {
    constexpr int MB = MT / 16;          // 16-row blocks per wave
    constexpr int CPT = MT * 8 / 256;    // 16-byte X chunks per thread per K-step
    __shared__ __attribute__((aligned(1024))) uint8_t xs[2][MT * 128];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int r = lane & 15, G = lane >> 4;

    // Workgroup -> tile.  Workgroups are dealt round-robin to the 8 XCDs;
    // regroup so each XCD walks a contiguous run of tiles, with the M tiles
    // of one channel panel adjacent (the weight panel stays in that L2).
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

    // ---- X staging: chunk c = tid + 256p is row c/8, 16-byte column c%8;
    // it is stored in LDS slot (c%8) ^ xswz(row).  Rows past M re-read row
    // M-1: their products land in accumulator rows that are never stored.
    unsigned xoff[CPT];   // byte offsets into X (M*K < 2^32 is checked on the host)
    int xlds[CPT];        // LDS byte offsets within a buffer
#pragma unroll
    for (int p = 0; p < CPT; ++p) {
        const int c = tid + 256 * p;
        const int row = c >> 3, col16 = c & 7;
        const int m = min(m0 + row, M - 1);
        xoff[p] = (unsigned)m * (unsigned)K + (unsigned)(col16 * 16);
        xlds[p] = row * 128 + ((col16 ^ xswz(row & 15)) * 16);
    }
    v4i xr[CPT];
    auto load_x = [&](int kt) {
#pragma unroll
        for (int p = 0; p < CPT; ++p) xr[p] = load16(X + xoff[p] + (unsigned)(kt * kTileK));
    };
    auto store_x = [&](uint8_t* dst) {
#pragma unroll
        for (int p = 0; p < CPT; ++p) *reinterpret_cast<v4i*>(dst + xlds[p]) = xr[p];
    };
    // A operand of row block i, half h: row 16i + r, column 2G + h.
    const int aoff0 = r * 128 + (((2 * G) ^ xswz(r)) * 16);
    const int aoff1 = r * 128 + (((2 * G + 1) ^ xswz(r)) * 16);

    // ---- weights: the wave's 64 channels are one parameter panel.
    const int nt0 = n0 / kTileN;
    const uint8_t* wpanel = wq + (size_t)nt0 * KT * kTileBytes;   // wave-uniform
    const unsigned wlane = (unsigned)lane * 16u;
    const size_t ppanel = (size_t)64 * (size_t)(n0 >> 6) * groups;  // wave-uniform
    const unsigned plane = 4u * (unsigned)r;
    auto load_w = [&](int kt, WStep& ws) {
        const int j = (kt * kTileK + 32 * G) / group;
#pragma unroll
        for (int b = 0; b < 4; ++b)
            ws.w[b] = load16(wpanel + ((size_t)b * KT + kt) * kTileBytes + wlane);
        const size_t po = ppanel + (size_t)64 * j + plane;
        ws.sdw = *reinterpret_cast<const unsigned*>(s_u8 + po);
        ws.adw = *reinterpret_cast<const unsigned*>(a_u8 + po);
    };

    v4i acc[MB][4];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[i][b] = v4i{0, 0, 0, 0};

    WStep wn;
    v4i B[4][2];
    load_x(0);
    load_w(0, wn);
    store_x(&xs[0][0]);
    dequant_half(wn, 0, B);
    dequant_half(wn, 1, B);
    __syncthreads();

    // The loop body is branch-free: the prefetch index is clamped to the
    // last step (the extra loads are never consumed).
    for (int kt = 0; kt < KT; ++kt) {
        const int buf = kt & 1;
        const int kn = min(kt + 1, KT - 1);
        load_x(kn);
        load_w(kn, wn);
        const uint8_t* xb = &xs[buf][0];

        // A operands stream through a ring of kRing registers, each read
        // kRing row blocks before its use (half 0 then half 1).
        constexpr int kRing = 4;
        auto read_a = [&](int j) {
            const int h = j / MB, i = j % MB;
            return *reinterpret_cast<const v4i*>(xb + i * 2048 + (h ? aoff1 : aoff0));
        };
        v4i Ar[kRing];
#pragma unroll
        for (int d = 0; d < kRing; ++d) Ar[d] = read_a(d);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int i = 0; i < MB; ++i) {
                const int j = h * MB + i;
                const v4i a = Ar[j % kRing];
                if (j + kRing < 2 * MB) Ar[j % kRing] = read_a(j + kRing);
#pragma unroll
                for (int b = 0; b < 4; ++b) mfma_i8_acc(acc[i][b], a, B[b][h]);
            }
        }
        store_x(&xs[buf ^ 1][0]);
        dequant_half(wn, 0, B);
        dequant_half(wn, 1, B);
        __syncthreads();
    }

    mfma_drain();

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
