// Streamed-tile W4A8 and W4FP8 GEMM kernels for gfx950 (small M; the
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
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace w4a8 {

// Panels (64 channels, four tiles) that NTW consecutive tiles can touch.
template <int NTW>
__host__ __device__ constexpr int stream_param_span() {
    return (NTW + 3) / 4 + 1;
}

// Swizzled 16-byte piece position of row R's piece c in a 16 x 128-byte X
// tile held in LDS (row stride 128 bytes): conflict-free for the row-wise
// writes and for the MFMA-layout reads below.
__device__ __forceinline__ int xpiece(int R, int c) {
    return R * 128 + 16 * (c ^ ((R & 7) ^ ((R >> 3) & 1)));
}

// W4A8 decode-shaped GEMM (M < 64).  One workgroup per NTW packed tiles
// (16 channels each) and one 16-row block of X (NTW and ks are chosen by
// the host from the shape); its `ks` waves take interleaved K-tiles (wave w:
// w, w + ks, ...), so at any moment a CU reads adjacent tiles of its channel
// rows.  Each wave keeps D K-tiles of weight loads in flight (a register
// ring refilled as each stage is consumed); the weight stream is loaded
// non-temporally.  The per-group parameters of the workgroup's tiles are
// copied to LDS once (whole 64-byte panel rows) when they fit.  X tiles
// (L2-resident) are loaded eight whole 128-byte rows per instruction and
// re-laid out through a per-wave LDS slot into the MFMA operand layout.
// The ks partial tiles are summed by all threads of the workgroup in wave
// order (exact).
// WK selects the weight kind (the rest of the kernel is shared):
//   kWkLQQ  LiquidQuant codes + group parameters, INT8 matrix cores;
//   kWkW8   the W8A8 comparison: INT8 weights in the 8-bit tile layout
//           (2 KiB per tile, a lane's 32 bytes as two 16-byte halves 1 KiB
//           apart), used as B operands without decode;
//   kWkF8   sign-magnitude INT4 codes -> e4m3 by byte table, X is e4m3,
//           one v_mfma_scale_f32_16x16x128_f8f6f4 per tile (unit scales),
//           float32 accumulation; epilogue scale sw[n];
//   kWkF8G  the same with per-group scales folded into the FP8 weights:
//           each tile's table is e4m3(|q| f) for the lane's channel and
//           group (fsc group-major [K/GROUP][N]; with 64-wide groups lane
//           quarter G lies in group 2 kt + G/2), loaded with the weights,
//           and the epilogue scales by tsc[0].
// OUT: 0 = fp16 (INT8 kinds) or bf16 (FP8 kinds), 1 = int32 or float32.
constexpr int kWkLQQ = 0, kWkW8 = 1, kWkF8 = 2, kWkF8G = 3;

template <int NTW, int D, int OUT, int GROUP, bool LDSP, int WK = kWkLQQ, int RB = 1>
__global__ __launch_bounds__(NTW == 1 && RB == 1 ? 1024 : 512) void w4a8_stream_kernel(
    const int8_t* __restrict__ X, const float* __restrict__ sx, const uint8_t* __restrict__ wq,
    const uint8_t* __restrict__ s_u8, const uint8_t* __restrict__ a_u8,
    const float* __restrict__ sw, void* __restrict__ Y, int M, int N, int K, int ks,
    const int* __restrict__ offsets, const float* __restrict__ fsc = nullptr,
    const float* __restrict__ tsc = nullptr) {
    constexpr bool W8 = WK == kWkW8;
    constexpr bool F8 = WK == kWkF8 || WK == kWkF8G;
    using Acc = std::conditional_t<F8, v4f, v4i>;
    extern __shared__ int red[];
    // Grouped problems (offsets != nullptr): expert blockIdx.z owns rows
    // offsets[e] .. offsets[e+1]-1 of X and Y and the e-th slab of the
    // packed weights.  Rows are clamped to [0, M], so bad offsets can only
    // leave rows unwritten, never move an access out of the buffers.
    int row_lo = 0, row_hi = M;
    if (offsets) {
        const int e = blockIdx.z;
        row_lo = min(max(offsets[e], 0), M);
        row_hi = min(max(offsets[e + 1], row_lo), M);
        wq += (size_t)e * N * (W8 ? K : K / 2);
        s_u8 += (size_t)e * N * (K / GROUP);
        a_u8 += (size_t)e * N * (K / GROUP);
        sw += (size_t)e * N;
    }
    const int m0 = row_lo + blockIdx.y * (16 * RB);
    if (m0 >= row_hi) return;  // whole workgroup: no rows of this expert here
    // X through LDS pays where X is a large share of the loads (narrow
    // workgroups: 2 KB of X per K-tile against NTW KB of weights).
    constexpr bool kXlds = true;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15, G = lane >> 4;
    const int KT = K / kTileK;
    const int groups = K / GROUP;
    // Workgroups are dealt round-robin to the eight XCDs (b -> b % 8), each
    // with its own L2: give workgroups b and b + 8 adjacent tile groups, so
    // the parameter panels that neighbouring groups share are read once per
    // XCD (when the group count is a multiple of 8).
    const int nwg = gridDim.x, b = blockIdx.x;
    const int g = (nwg & 7) ? b : (b & 7) * (nwg >> 3) + (b >> 3);
    const int nt0 = g * NTW;
    const int nk = (KT - wave + ks - 1) / ks;  // K-tiles of this wave (>= 1: ks <= KT)
    // i-th K-tile of this wave (i < nk)
    auto kt_of = [&](int i) { return wave + ks * i; };

    const __amdgpu_buffer_rsrc_t x_rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(X), (short)0, M * K, 0x00020000);
    const __amdgpu_buffer_rsrc_t w_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(wq), (short)0, (int)((size_t)N * K / (W8 ? 1 : 2)), 0x00020000);
    const __amdgpu_buffer_rsrc_t f_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(fsc), (short)0,
        WK == kWkF8G ? (int)((size_t)(K / GROUP) * N * sizeof(float)) : 0, 0x00020000);
    const __amdgpu_buffer_rsrc_t s_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(s_u8), (short)0, (int)((size_t)N * K / GROUP), 0x00020000);
    const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(a_u8), (short)0, (int)((size_t)N * K / GROUP), 0x00020000);
    // X loads (a row >= M lies past the buffer end and reads as 0).  With
    // the LDS re-layout, lane l takes 16-byte piece (l & 7) of rows
    // m0 + (l >> 3) and m0 + 8 + (l >> 3); otherwise lane (r, G) loads its
    // MFMA operand directly: row m0 + r, columns 32G .. 32G+31.
    const unsigned xvoff =
        kXlds ? (unsigned)(m0 + (lane >> 3)) * (unsigned)K + 16u * (unsigned)(lane & 7)
              : (unsigned)(m0 + r) * (unsigned)K + 32u * (unsigned)G;
    const unsigned xvoff8 = kXlds ? xvoff + 8u * (unsigned)K : xvoff + 16u;
    const unsigned wvoff = (unsigned)lane * 16u;
    const int gsub = (GROUP == 64) ? (G >> 1) : 0;  // group within the K-tile

    // ---- LDS: [parameters (LDSP)] [one 2 KB X slot per wave]; the
    // reduction at the end reuses it from offset 0.
    const int p0 = nt0 >> 2;
    const int np = ((nt0 + NTW - 1) >> 2) - p0 + 1;
    uint8_t* lds_s = reinterpret_cast<uint8_t*>(red);
    uint8_t* lds_a = lds_s + (size_t)np * groups * 64;
    const int pbytes = LDSP ? 2 * stream_param_span<NTW>() * groups * 64 : 0;
    uint8_t* xslot = reinterpret_cast<uint8_t*>(red) + pbytes + wave * (2048 * RB);
    // MFMA operand layout: lane (r, G) holds row r, columns 32G .. 32G+31.
    const int xw0 = xpiece(lane >> 3, lane & 7), xw1 = xpiece(8 + (lane >> 3), lane & 7);
    const int xr0 = xpiece(r, 2 * G), xr1 = xpiece(r, 2 * G + 1);

    constexpr int WPT = W8 ? 2 : 1;  // 16-byte weight loads per lane and tile
    constexpr int NF = WK == kWkF8G ? NTW : 1;  // folded factors per stage
    struct Stage {
        v4i x0[RB], x1[RB];
        v4i w[NTW * WPT];
        float f[NF];
    };
    auto issue = [&](int kt, Stage& st) {
        const unsigned so = (unsigned)(kt * kTileK);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const unsigned ro = 16u * (unsigned)rb * (unsigned)K;  // row block rb
            st.x0[rb] = __builtin_bit_cast(
                v4i, __builtin_amdgcn_raw_buffer_load_b128(x_rsrc, xvoff + ro, so, 0));
            st.x1[rb] = __builtin_bit_cast(
                v4i, __builtin_amdgcn_raw_buffer_load_b128(x_rsrc, xvoff8 + ro, so, 0));
        }
#pragma unroll
        for (int t = 0; t < NTW; ++t) {
            if constexpr (W8) {
#pragma unroll
                for (int u = 0; u < 2; ++u)
                    st.w[2 * t + u] = __builtin_bit_cast(
                        v4i, __builtin_amdgcn_raw_buffer_load_b128(
                                 w_rsrc, wvoff,
                                 (unsigned)(((size_t)(nt0 + t) * KT + kt) * 2048 + 1024 * u),
                                 kNonTemporal));
            } else {
                st.w[t] = __builtin_bit_cast(
                    v4i, __builtin_amdgcn_raw_buffer_load_b128(
                             w_rsrc, wvoff, (unsigned)(((size_t)(nt0 + t) * KT + kt) * kTileBytes),
                             kNonTemporal));
            }
            if constexpr (WK == kWkF8G) {
                // factor of this lane's channel and group, loaded with the
                // stage so using it waits for nothing younger
                const int gi = GROUP == 64 ? 2 * kt + (G >> 1) : kt;
                st.f[t] = __builtin_bit_cast(
                    float, __builtin_amdgcn_raw_buffer_load_b32(
                               f_rsrc, (unsigned)((size_t)gi * N + (nt0 + t) * kTileN + r) * 4u,
                               0u, 0));
            }
        }
    };
    auto params = [&](int kt, int t, unsigned& s, unsigned& a) {
        const int j = kt * (kTileK / GROUP) + gsub;
        const int nt = nt0 + t;
        if (LDSP) {
            const int o = (((nt >> 2) - p0) * groups + j) * 64 + 4 * r + (nt & 3);
            s = lds_s[o];
            a = lds_a[o];
        } else {
            const unsigned po = (unsigned)param_offset(nt * kTileN + r, j, groups);
            s = __builtin_amdgcn_raw_buffer_load_b8(s_rsrc, po, 0, 0);
            a = __builtin_amdgcn_raw_buffer_load_b8(a_rsrc, po, 0, 0);
        }
    };

    Acc acc[RB][NTW];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int t = 0; t < NTW; ++t) acc[rb][t] = Acc{};

    // Multiply-accumulate of the K-tile held in stage S.
    auto consume = [&](const Stage& S, int kt) {
        v4i x0[RB], x1[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            x0[rb] = S.x0[rb];
            x1[rb] = S.x1[rb];
            if constexpr (kXlds) {
                // X tile -> MFMA layout through this wave's LDS slot (LDS
                // operations of one wave complete in order).
                uint8_t* xs = xslot + rb * 2048;
                *reinterpret_cast<v4i*>(xs + xw0) = S.x0[rb];
                *reinterpret_cast<v4i*>(xs + xw1) = S.x1[rb];
                x0[rb] = *reinterpret_cast<const v4i*>(xs + xr0);
                x1[rb] = *reinterpret_cast<const v4i*>(xs + xr1);
            }
        }
#pragma unroll
        for (int t = 0; t < NTW; ++t) {
            if constexpr (W8) {
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    acc[rb][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(x0[rb], S.w[2 * t],
                                                                       acc[rb][t], 0, 0, 0);
                    acc[rb][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(x1[rb], S.w[2 * t + 1],
                                                                       acc[rb][t], 0, 0, 0);
                }
                continue;
            } else if constexpr (F8) {
                unsigned lo = kE4m3LutLo, hi = kE4m3LutHi;
                if constexpr (WK == kWkF8G) e4m3_fold_table(S.f[t], lo, hi);
                const v4i w = S.w[t];
                const v8i Bf = v8i{(int)int4_to_e4m3_lo(w.x, lo, hi), (int)int4_to_e4m3_hi(w.x, lo, hi),
                                   (int)int4_to_e4m3_lo(w.y, lo, hi), (int)int4_to_e4m3_hi(w.y, lo, hi),
                                   (int)int4_to_e4m3_lo(w.z, lo, hi), (int)int4_to_e4m3_hi(w.z, lo, hi),
                                   (int)int4_to_e4m3_lo(w.w, lo, hi), (int)int4_to_e4m3_hi(w.w, lo, hi)};
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    const v8i A = v8i{x0[rb].x, x0[rb].y, x0[rb].z, x0[rb].w,
                                      x1[rb].x, x1[rb].y, x1[rb].z, x1[rb].w};
                    // formats 0/0 = e4m3 x e4m3; E8M0 scale 127 = 2^0 on both sides
                    acc[rb][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        A, Bf, acc[rb][t], 0, 0, 0, 127, 0, 127);
                }
                continue;
            }
            unsigned s, a;
            params(kt, t, s, a);
            const u16x2 s2 = u16x2{(unsigned short)s, (unsigned short)s};
            const unsigned short aa = (unsigned short)(a * 0x101u);
            const u16x2 a4 = u16x2{aa, aa};
            unsigned b[8];
            lqq_dequant8((unsigned)S.w[t].x, s2, a4, b[0], b[1]);
            lqq_dequant8((unsigned)S.w[t].y, s2, a4, b[2], b[3]);
            lqq_dequant8((unsigned)S.w[t].z, s2, a4, b[4], b[5]);
            lqq_dequant8((unsigned)S.w[t].w, s2, a4, b[6], b[7]);
            const v4i B0 = v4i{(int)b[0], (int)b[1], (int)b[2], (int)b[3]};
            const v4i B1 = v4i{(int)b[4], (int)b[5], (int)b[6], (int)b[7]};
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                acc[rb][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(x0[rb], B0, acc[rb][t], 0, 0, 0);
                acc[rb][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(x1[rb], B1, acc[rb][t], 0, 0, 0);
            }
        }
    };

    // Stage d holds this wave's K-tile i + d.  The steady-state loop has no
    // conditional work, so the load counter waits it needs are exact (one
    // stage at a time) and D stages stay in flight; the last 2D-1 K-tiles
    // at most are drained after it.
    Stage st[D];
#pragma unroll
    for (int d = 0; d < D; ++d)
        if (d < nk) issue(kt_of(d), st[d]);

    // Parameter copy, behind the first weight loads (panels p0 .. p0+np-1
    // are contiguous in the panel-order arrays).
    if (LDSP && WK == kWkLQQ) {
        const int n16 = np * groups * 4;  // 16-byte pieces per array
        const size_t base = (size_t)p0 * groups * 64;
        for (int q = tid; q < n16; q += blockDim.x) {
            const v4i vs = *reinterpret_cast<const v4i*>(s_u8 + base + (size_t)q * 16);
            const v4i va = *reinterpret_cast<const v4i*>(a_u8 + base + (size_t)q * 16);
            *reinterpret_cast<v4i*>(lds_s + q * 16) = vs;
            *reinterpret_cast<v4i*>(lds_a + q * 16) = va;
        }
        __syncthreads();
    }

    int i = 0;
    for (; i + 2 * D <= nk; i += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            consume(st[d], kt_of(i + d));
            issue(kt_of(i + d + D), st[d]);
            // keep each refill right behind its stage's use (the scheduler
            // would otherwise sink every refill to the end of the iteration)
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int d = 0; d < D; ++d) {
        if (i + d < nk) {
            consume(st[d], kt_of(i + d));
            if (i + d + D < nk) issue(kt_of(i + d + D), st[d]);
        }
    }
#pragma unroll
    for (int d = 0; d < D; ++d)
        if (i + D + d < nk) consume(st[d], kt_of(i + D + d));

    // Sum the ks partial tiles: element e = ((rb * NTW + t) * 4 + v) * 64 + l
    // of wave w lives at red[w * RB * NTW * 256 + e] (reusing the parameter
    // LDS).
    // (float32 sums, for the FP8 kinds, are added in the same wave order.)
    using Sum = std::conditional_t<F8, float, int>;
    Sum* reds = reinterpret_cast<Sum*>(red);
    __syncthreads();
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int t = 0; t < NTW; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                reds[(((wave * RB + rb) * NTW + t) * 4 + v) * 64 + lane] = acc[rb][t][v];
    __syncthreads();
    const int nel = RB * NTW * 256;
    const float tval = WK == kWkF8G ? tsc[0] : 0.0f;
    for (int e = tid; e < nel; e += blockDim.x) {
        Sum sum = reds[e];
        for (int w = 1; w < ks; ++w) sum += reds[w * nel + e];
        const int rb = e / (NTW * 256), t = (e >> 8) % NTW, v = (e >> 6) & 3, l = e & 63;
        const int m = m0 + 16 * rb + 4 * (l >> 4) + v;  // accumulator row (X row)
        const int n = (nt0 + t) * kTileN + (l & 15);
        if (m < row_hi) {
            if constexpr (F8) {
                const float y = (sum * sx[m]) * (WK == kWkF8G ? tval : sw[n]);
                if (OUT == 1)
                    reinterpret_cast<float*>(Y)[(size_t)m * N + n] = y;
                else
                    reinterpret_cast<unsigned short*>(Y)[(size_t)m * N + n] = f32_to_bf16_bits(y);
            } else if (OUT == 1) {
                reinterpret_cast<int*>(Y)[(size_t)m * N + n] = sum;
            } else {
                const float y = ((float)sum * sx[m]) * sw[n];
                reinterpret_cast<unsigned short*>(Y)[(size_t)m * N + n] = f32_to_f16_bits(y);
            }
        }
    }
}

// ----------------------------------------------------------- launchers ----
constexpr size_t kMaxLdsBytes = 160 * 1024;  // LDS one workgroup may hold on gfx950

template <int NTW, int D, int RB = 1>
static hipError_t w4a8_stream_ntw(const int8_t* X, const float* sx, const uint8_t* wq,
                                  const uint8_t* s_u8, const uint8_t* a_u8, const float* sw,
                                  void* Y, int out_type, int M, int N, int K, int group, int ks,
                                  const int* offsets, int E, int max_rows, hipStream_t st) {
    dim3 grid(N / (kTileN * NTW), (max_rows + 16 * RB - 1) / (16 * RB), E);
    dim3 block(64 * ks);
    const int groups = K / group;
    const size_t pbytes = (size_t)2 * stream_param_span<NTW>() * groups * 64;
    const size_t xbytes = (size_t)ks * 2048 * RB;  // X slots
    const size_t rbytes = (size_t)ks * RB * NTW * 256 * sizeof(int);
    const bool ldsp = pbytes + xbytes <= 128 * 1024;
    const size_t used = (ldsp ? pbytes : 0) + xbytes;
    const size_t lds = used > rbytes ? used : rbytes;
    if (lds > kMaxLdsBytes) return hipErrorInvalidConfiguration;
#define W4A8_LS(O, G, P)                                                                    \
    hipLaunchKernelGGL((w4a8_stream_kernel<NTW, D, O, G, P, kWkLQQ, RB>), grid, block, lds, \
                       st, X, sx, wq, s_u8, a_u8, sw, Y, M, N, K, ks, offsets)
    if (ldsp) {
        if (out_type == 1) {
            if (group == 64) W4A8_LS(1, 64, true); else W4A8_LS(1, 128, true);
        } else {
            if (group == 64) W4A8_LS(0, 64, true); else W4A8_LS(0, 128, true);
        }
    } else {
        if (out_type == 1) {
            if (group == 64) W4A8_LS(1, 64, false); else W4A8_LS(1, 128, false);
        } else {
            if (group == 64) W4A8_LS(0, 64, false); else W4A8_LS(0, 128, false);
        }
    }
#undef W4A8_LS
    return hipGetLastError();
}

hipError_t launch_w4a8_stream(const int8_t* X, const float* sx, const uint8_t* wq,
                              const uint8_t* s_u8, const uint8_t* a_u8, const float* sw,
                              void* Y, int out_type, int M, int N, int K, int group,
                              StreamCfg cfg, hipStream_t st, const int* offsets, int E,
                              int max_rows) {
    if (!offsets) {
        E = 1;
        max_rows = M;
    }
#define W4A8_NTW(W, D, R)                                                                    \
    return w4a8_stream_ntw<W, D, R>(X, sx, wq, s_u8, a_u8, sw, Y, out_type, M, N, K, group, \
                                    cfg.ks, offsets, E, max_rows, st)
    // several 16-row blocks per workgroup share each decoded weight (ring
    // of two K-tiles: the X operands of every block are held per stage;
    // four blocks of four tiles would not fit the registers)
    switch (cfg.nt_per_wave * 8 + cfg.rb) {
        case 7 * 8 + 1: W4A8_NTW(7, 2, 1);
        case 4 * 8 + 1: W4A8_NTW(4, 2, 1);
        case 4 * 8 + 2: W4A8_NTW(4, 2, 2);
        case 2 * 8 + 1: W4A8_NTW(2, 4, 1);
        case 2 * 8 + 2: W4A8_NTW(2, 2, 2);
        case 2 * 8 + 4: W4A8_NTW(2, 2, 4);
        case 1 * 8 + 1: W4A8_NTW(1, 3, 1);
        case 1 * 8 + 2: W4A8_NTW(1, 2, 2);
        default: return hipErrorInvalidValue;
    }
#undef W4A8_NTW
}

template <int NTW, int D>
static hipError_t w8a8_stream_ntw(const int8_t* X, const float* sx, const int8_t* wq8,
                                  const float* sw, void* Y, int out_type, int M, int N, int K,
                                  int ks, hipStream_t st) {
    dim3 grid(N / (kTileN * NTW), (M + 15) / 16, 1);
    dim3 block(64 * ks);
    const size_t xbytes = (size_t)ks * 2048;
    const size_t rbytes = (size_t)ks * NTW * 256 * sizeof(int);
    const size_t lds = xbytes > rbytes ? xbytes : rbytes;
    const uint8_t* w = reinterpret_cast<const uint8_t*>(wq8);
    if (out_type == 1)
        hipLaunchKernelGGL((w4a8_stream_kernel<NTW, D, 1, 128, false, kWkW8>), grid, block, lds, st,
                           X, sx, w, nullptr, nullptr, sw, Y, M, N, K, ks, nullptr);
    else
        hipLaunchKernelGGL((w4a8_stream_kernel<NTW, D, 0, 128, false, kWkW8>), grid, block, lds, st,
                           X, sx, w, nullptr, nullptr, sw, Y, M, N, K, ks, nullptr);
    return hipGetLastError();
}

hipError_t launch_w8a8_stream(const int8_t* X, const float* sx, const int8_t* wq8,
                              const float* sw, void* Y, int out_type, int M, int N, int K,
                              StreamCfg cfg, hipStream_t st) {
    switch (cfg.nt_per_wave) {
        case 7: return w8a8_stream_ntw<7, 2>(X, sx, wq8, sw, Y, out_type, M, N, K, cfg.ks, st);
        case 4: return w8a8_stream_ntw<4, 3>(X, sx, wq8, sw, Y, out_type, M, N, K, cfg.ks, st);
        case 2: return w8a8_stream_ntw<2, 4>(X, sx, wq8, sw, Y, out_type, M, N, K, cfg.ks, st);
        default: return w8a8_stream_ntw<1, 3>(X, sx, wq8, sw, Y, out_type, M, N, K, cfg.ks, st);
    }
}

template <int NTW, int D, int WK, int GROUP, int RB = 1>
static hipError_t w4fp8_stream_ntw(const uint8_t* X, const float* sx, const uint8_t* wq,
                                   const float* sw, const float* fsc, const float* tsc, void* Y,
                                   int out_type, int M, int N, int K, int ks, hipStream_t st) {
    dim3 grid(N / (kTileN * NTW), (M + 16 * RB - 1) / (16 * RB), 1);
    dim3 block(64 * ks);
    const size_t xbytes = (size_t)ks * 2048 * RB;
    const size_t rbytes = (size_t)ks * RB * NTW * 256 * sizeof(float);
    const size_t lds = xbytes > rbytes ? xbytes : rbytes;
    if (lds > kMaxLdsBytes) return hipErrorInvalidConfiguration;
    const int8_t* Xb = reinterpret_cast<const int8_t*>(X);
    if (out_type == 1)
        hipLaunchKernelGGL((w4a8_stream_kernel<NTW, D, 1, GROUP, false, WK, RB>), grid, block, lds,
                           st, Xb, sx, wq, nullptr, nullptr, sw, Y, M, N, K, ks, nullptr, fsc, tsc);
    else
        hipLaunchKernelGGL((w4a8_stream_kernel<NTW, D, 0, GROUP, false, WK, RB>), grid, block, lds,
                           st, Xb, sx, wq, nullptr, nullptr, sw, Y, M, N, K, ks, nullptr, fsc, tsc);
    return hipGetLastError();
}

template <int WK, int GROUP>
static hipError_t w4fp8_stream_run(const uint8_t* X, const float* sx, const uint8_t* wq,
                                   const float* sw, const float* fsc, const float* tsc, void* Y,
                                   int out_type, int M, int N, int K, StreamCfg cfg,
                                   hipStream_t st) {
#define F8_NTW(W, D, R)                                                                          \
    return w4fp8_stream_ntw<W, D, WK, GROUP, R>(X, sx, wq, sw, fsc, tsc, Y, out_type, M, N, K, \
                                                cfg.ks, st)
    switch (cfg.nt_per_wave * 8 + cfg.rb) {
        case 7 * 8 + 1: F8_NTW(7, 2, 1);
        case 4 * 8 + 1: F8_NTW(4, 2, 1);
        case 4 * 8 + 2: F8_NTW(4, 2, 2);
        case 2 * 8 + 1: F8_NTW(2, 4, 1);
        case 2 * 8 + 2: F8_NTW(2, 2, 2);
        case 2 * 8 + 4: F8_NTW(2, 2, 4);
        case 1 * 8 + 1: F8_NTW(1, 3, 1);
        case 1 * 8 + 2: F8_NTW(1, 2, 2);
        default: return hipErrorInvalidValue;
    }
#undef F8_NTW
}

hipError_t launch_w4fp8_stream(const uint8_t* X, const float* sx, const uint8_t* wq,
                               const float* sw, void* Y, int out_type, int M, int N, int K,
                               StreamCfg cfg, hipStream_t st) {
    return w4fp8_stream_run<kWkF8, 128>(X, sx, wq, sw, nullptr, nullptr, Y, out_type, M, N, K,
                                        cfg, st);
}

hipError_t launch_w4fp8g_stream(const uint8_t* X, const float* sx, const uint8_t* wq,
                                const float* fsc, const float* tsc, void* Y, int out_type, int M,
                                int N, int K, int group, StreamCfg cfg, hipStream_t st) {
    if (group == 64)
        return w4fp8_stream_run<kWkF8G, 64>(X, sx, wq, nullptr, fsc, tsc, Y, out_type, M, N, K,
                                            cfg, st);
    return w4fp8_stream_run<kWkF8G, 128>(X, sx, wq, nullptr, fsc, tsc, Y, out_type, M, N, K, cfg,
                                         st);
}

}  // namespace w4a8
