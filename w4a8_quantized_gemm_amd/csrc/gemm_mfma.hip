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
#include <utility>

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

// Same instruction, volatile: keeps its place relative to the one-instruction
// dequantisation steps interleaved with it below.
__device__ __forceinline__ void mfma_i8_acc_v(v4i& acc, const v4i& a, const v4i& b) {
    asm volatile("v_mfma_i32_16x16x64_i8 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// Dequantisation of the next K-step's four tiles as 120 single-instruction
// steps, so that one can follow each matrix-core instruction of the current
// step and run on the vector ALU while the matrix core is busy.
//   steps 30b + 0, 1:   scale pair / offset quad of tile b (v_perm_b32)
//   steps 30b + 2 + 7d + e, dword d of tile b, e = 0..6:
//     lo = w & 0x0F0F0F0F; t = w >> 4; hi = t & 0x0F0F0F0F;
//     lo = lo*s + a; hi = hi*s + a   (two 16-bit lanes, v_pk_mad_u16);
//     lo ^= 0x80808080; hi ^= 0x80808080
// Results land in B[b][d/2] components 2(d%2), 2(d%2)+1.
struct DequantPipe {
    unsigned s2[4], a4[4];
    unsigned lo, t, hi;
};

template <int OP>
__device__ __forceinline__ void dq_step(DequantPipe& p, const WStep& w, v4i (&B)[4][2]) {
    constexpr int b = OP / 30, q = OP % 30;
    if constexpr (q == 0) {
        constexpr unsigned sel = (unsigned)b | 0x0C00u | ((unsigned)b << 16) | 0x0C000000u;
        asm volatile("v_perm_b32 %0, 0, %1, %2" : "=v"(p.s2[b]) : "v"(w.sdw), "s"(sel));
    } else if constexpr (q == 1) {
        constexpr unsigned sel = (unsigned)b * 0x01010101u;
        asm volatile("v_perm_b32 %0, 0, %1, %2" : "=v"(p.a4[b]) : "v"(w.adw), "s"(sel));
    } else {
        constexpr int d = (q - 2) / 7, e = (q - 2) % 7;
        const unsigned wd = (unsigned)w.w[b][d];
        if constexpr (e == 0) {
            asm volatile("v_and_b32 %0, 0x0f0f0f0f, %1" : "=v"(p.lo) : "v"(wd));
        } else if constexpr (e == 1) {
            asm volatile("v_lshrrev_b32 %0, 4, %1" : "=v"(p.t) : "v"(wd));
        } else if constexpr (e == 2) {
            asm volatile("v_and_b32 %0, 0x0f0f0f0f, %1" : "=v"(p.hi) : "v"(p.t));
        } else if constexpr (e == 3) {
            asm volatile("v_pk_mad_u16 %0, %1, %2, %3"
                         : "=v"(p.lo) : "v"(p.lo), "v"(p.s2[b]), "v"(p.a4[b]));
        } else if constexpr (e == 4) {
            asm volatile("v_pk_mad_u16 %0, %1, %2, %3"
                         : "=v"(p.hi) : "v"(p.hi), "v"(p.s2[b]), "v"(p.a4[b]));
        } else if constexpr (e == 5) {
            unsigned x;
            asm volatile("v_xor_b32 %0, 0x80808080, %1" : "=v"(x) : "v"(p.lo));
            B[b][d >> 1][2 * (d & 1)] = (int)x;
        } else {
            unsigned x;
            asm volatile("v_xor_b32 %0, 0x80808080, %1" : "=v"(x) : "v"(p.hi));
            B[b][d >> 1][2 * (d & 1) + 1] = (int)x;
        }
    }
}

// Compile-time loop: f(std::integral_constant<int, i>) for i = 0 .. N-1.
template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
    (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
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

// 256-row variant (one workgroup per CU), built on v_mfma_i32_32x32x32_i8:
// half as many matrix-core instructions per K-step as the 16x16 form, so
// each one leaves a 32-cycle shadow for the dequantisation, LDS and memory
// instructions of the same wave.
//   wave tile 256 x 64 = 8 row blocks x 2 channel blocks of 32 x 32;
//   B operand of lane (c = lane % 32, h = lane / 32): packed tile row c % 16
//     of tile 2*cb + c/16, slots 2h and 2h+1 (K columns 64h .. 64h+63 of
//     the 128-column step); instruction i (0..3) consumes columns
//     64h + 16i .. +15, and the A operand (X row, same columns) matches;
//   every global load is a buffer load (SGPR step offset, no per-load
//     address arithmetic) issued two K-steps ahead; X rows past M fall
//     outside the buffer and read as zero;
//   the next step's weights are dequantised in single-instruction steps
//     interleaved with this step's matrix-core instructions;
//   the epilogue scales in registers, transposes through LDS and writes
//     whole 128-byte row segments.
namespace {

__device__ __forceinline__ void mfma32_i8_acc(v16i& acc, const v4i& a, const v4i& b) {
    asm volatile("v_mfma_i32_32x32x32_i8 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* p, unsigned bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                             0x00020000);
}
__device__ __forceinline__ v4i buf_load16(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff) {
    return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ unsigned buf_load4(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}

// Raw weights of one K-step for one lane: w[cb][e] = slot 2h+e of the
// lane's row in tile 2cb + c/16; parameter dwords of the lane's panel row.
struct WStep32 {
    v4i w[2][2];
    unsigned sdw, adw;
};

// Scale pair / offset quad of the lane's tiles for one K-step.
struct WParams {
    unsigned s2[2], a4[2];
};

__device__ __forceinline__ void wparams(const WStep32& w, int tb, WParams& p) {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
        const unsigned b = (unsigned)(2 * cb + tb);
        const unsigned sel = b | 0x0C00u | (b << 16) | 0x0C000000u;
        asm volatile("v_perm_b32 %0, 0, %1, %2" : "=v"(p.s2[cb]) : "v"(w.sdw), "v"(sel));
        asm volatile("v_perm_b32 %0, 0, %1, %2" : "=v"(p.a4[cb]) : "v"(w.adw), "v"(b * 0x01010101u));
    }
}

// Operands of instruction i (K columns 64h + 16i .. +15 of the lane) come
// from dwords d = 2(i%2), 2(i%2)+1 of slot e = i/2.  Producing B[*][i] is 28
// single-instruction steps: for cb in {0,1}, for the two dwords:
//   lo = w & 0x0F0F0F0F; t = w >> 4; hi = t & 0x0F0F0F0F;
//   lo = lo*s + a; hi = hi*s + a   (v_pk_mad_u16, two codes per 16-bit lane);
//   B = lo ^ 0x80808080, hi ^ 0x80808080   (LiquidQuant decode)
struct DqTmp {
    unsigned lo, t, hi;
};

template <int I, int OP>
__device__ __forceinline__ void dq_group_step(DqTmp& tmp, const WStep32& w, const WParams& p,
                                              v4i (&B)[2][4]) {
    constexpr int cb = OP / 14, q = OP % 14, dd = q / 7, st = q % 7;
    constexpr int e = I / 2, d = 2 * (I % 2) + dd;
    const unsigned wd = (unsigned)w.w[cb][e][d];
    if constexpr (st == 0) {
        asm volatile("v_and_b32 %0, 0x0f0f0f0f, %1" : "=v"(tmp.lo) : "v"(wd));
    } else if constexpr (st == 1) {
        asm volatile("v_lshrrev_b32 %0, 4, %1" : "=v"(tmp.t) : "v"(wd));
    } else if constexpr (st == 2) {
        asm volatile("v_and_b32 %0, 0x0f0f0f0f, %1" : "=v"(tmp.hi) : "v"(tmp.t));
    } else if constexpr (st == 3) {
        asm volatile("v_pk_mad_u16 %0, %1, %2, %3"
                     : "=v"(tmp.lo) : "v"(tmp.lo), "v"(p.s2[cb]), "v"(p.a4[cb]));
    } else if constexpr (st == 4) {
        asm volatile("v_pk_mad_u16 %0, %1, %2, %3"
                     : "=v"(tmp.hi) : "v"(tmp.hi), "v"(p.s2[cb]), "v"(p.a4[cb]));
    } else if constexpr (st == 5) {
        unsigned x;
        asm volatile("v_xor_b32 %0, 0x80808080, %1" : "=v"(x) : "v"(tmp.lo));
        B[cb][I][2 * dd] = (int)x;
    } else {
        unsigned x;
        asm volatile("v_xor_b32 %0, 0x80808080, %1" : "=v"(x) : "v"(tmp.hi));
        B[cb][I][2 * dd + 1] = (int)x;
    }
}

template <int I>
__device__ __forceinline__ void dq_group_all(const WStep32& w, const WParams& p, v4i (&B)[2][4]) {
    DqTmp tmp;
    static_for<28>([&](auto oc) { dq_group_step<I, decltype(oc)::value>(tmp, w, p, B); });
}

__device__ __forceinline__ void mfma32_drain() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

}  // namespace

template <int OUT, int GROUP>
__global__ __launch_bounds__(256, 1) void w4a8_mfma256_kernel(
    const int8_t* __restrict__ X, const float* __restrict__ sx, const uint8_t* __restrict__ wq,
    const uint8_t* __restrict__ s_u8, const uint8_t* __restrict__ a_u8,
    const float* __restrict__ sw, void* __restrict__ Y, int M, int N, int K, int tiles_n,
    int tiles_m) {
    constexpr int MT = 256;
    constexpr int RB = 8;          // 32-row blocks per wave
    constexpr int CPT = 8;         // 16-byte X chunks per thread per K-step
    __shared__ __attribute__((aligned(1024))) uint8_t xs0[MT * 128];
    __shared__ __attribute__((aligned(1024))) uint8_t xs1[MT * 128];
    __shared__ float sxs[MT];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int c = lane & 31, h = lane >> 5;
    const int tb = c >> 4, r = c & 15;

    const int nwg = tiles_n * tiles_m;
    const int bid = blockIdx.x;
    int lin = bid;
    if ((nwg & 7) == 0) lin = (bid & 7) * (nwg >> 3) + (bid >> 3);
    const int tm = lin % tiles_m;
    const int tn = lin / tiles_m;
    const int m0 = tm * MT;
    const int n0 = tn * kNT + wave * kColsPerWave;
    const int KT = K / kTileK;
    const int groups = K / GROUP;

    // ---- X: chunk p of this thread is row (tid>>3) + 32p, 16-byte column
    // tid & 7, stored in LDS slot col ^ xswz(row & 15) (row & 15 is the same
    // for all p).  Rows >= M lie past the end of the buffer and read as 0.
    const __amdgpu_buffer_rsrc_t xr_rsrc = buf_rsrc(X, (unsigned)M * (unsigned)K);
    const int xrow0 = tid >> 3, xcol = tid & 7;
    const unsigned xvoff = (unsigned)(m0 + xrow0) * (unsigned)K + (unsigned)(xcol * 16);
    const unsigned xrowstep = 32u * (unsigned)K;
    const int xlds0 = xrow0 * 128 + ((xcol ^ xswz(xrow0 & 15)) * 16);
    // A operand (row block rb, instruction i): row 32rb + c, column 4h + i.
    int aoff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) aoff[i] = c * 128 + (((4 * h + i) ^ xswz(r)) * 16);

    // ---- weights of this wave: tiles nt0 .. nt0+3 (one parameter panel)
    const int nt0 = n0 / kTileN;
    const __amdgpu_buffer_rsrc_t w_rsrc = buf_rsrc(wq, (unsigned)((size_t)N * K / 2));
    const __amdgpu_buffer_rsrc_t s_rsrc = buf_rsrc(s_u8, (unsigned)((size_t)N * K / GROUP));
    const __amdgpu_buffer_rsrc_t a_rsrc = buf_rsrc(a_u8, (unsigned)((size_t)N * K / GROUP));
    const unsigned wvoff = (unsigned)(tb * KT) * kTileBytes + (unsigned)(32 * h + r) * 16u;
    const unsigned pvoff = 4u * (unsigned)r + (GROUP == 64 ? 64u * (unsigned)h : 0u);
    const unsigned ppanel = 64u * (unsigned)(n0 >> 6) * (unsigned)groups;
    auto w_load = [&](int kt, int part, WStep32& ws) {  // part 0..5
        if (part < 4) {
            const int cb = part >> 1, e = part & 1;
            ws.w[cb][e] = buf_load16(w_rsrc, wvoff,
                                     (unsigned)(((nt0 + 2 * cb) * KT + kt) * kTileBytes + e * 256));
        } else {
            const unsigned jo = ppanel + 64u * (unsigned)(kt * (kTileK / GROUP));
            if (part == 4) ws.sdw = buf_load4(s_rsrc, pvoff, jo);
            else ws.adw = buf_load4(a_rsrc, pvoff, jo);
        }
    };
    auto x_load = [&](int kt, int p) {
        return buf_load16(xr_rsrc, xvoff + (unsigned)p * xrowstep, (unsigned)(kt * kTileK));
    };

    v16i acc[RB][2];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        acc[rb][0] = v16i{};
        acc[rb][1] = v16i{};
    }

    // ---- prologue: X(0) -> LDS xs0, X(1) staged; W(0) dequantised fully,
    // W(1) raw; A ring primed with step 0's first four operands.
    v4i xe[CPT], xo[CPT];   // X staging for even / odd steps (X(kt) in set kt%2)
    WStep32 we, wo;         // raw weights for even / odd steps
    WParams pp;             // parameters of the raw set being dequantised
    v4i B[2][4];
    v4i ring[8];
    const int k1 = min(1, KT - 1);
#pragma unroll
    for (int p = 0; p < CPT; ++p) xe[p] = x_load(0, p);
#pragma unroll
    for (int p = 0; p < CPT; ++p) xo[p] = x_load(k1, p);
#pragma unroll
    for (int part = 0; part < 6; ++part) w_load(0, part, we);
#pragma unroll
    for (int part = 0; part < 6; ++part) w_load(k1, part, wo);
#pragma unroll
    for (int p = 0; p < CPT; ++p) *reinterpret_cast<v4i*>(xs0 + xlds0 + p * 4096) = xe[p];
    wparams(we, tb, pp);
    dq_group_all<0>(we, pp, B);
    dq_group_all<1>(we, pp, B);
    dq_group_all<2>(we, pp, B);
    dq_group_all<3>(we, pp, B);
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q) ring[q] = *reinterpret_cast<const v4i*>(xs0 + q * 4096 + aoff[0]);

    // ---- one K-step, 64 matrix-core slots.  Slot s: instruction i = s/16,
    // row block rb = (s/2)%8, channel block cb = s%2.  Entering step kt:
    // LDS `cur` = X(kt); ring holds A for slots 0..7; B[*][0..2] = W(kt)
    // operands and B[*][3] is produced in slots 0..15 from `wcur` (raw W(kt),
    // parameters pp); `xnx` = X(kt+1) staged; `wnx` = raw W(kt+1).
    //   slots 0..7    X(kt+2) -> xcur (the set that held X(kt))
    //   slots 16..21  W(kt+2) -> wcur (done with it after slot 15)
    //   slots 16..63  B[*][i-1] for step kt+1 from wnx, i = 1..3
    //   slots 52..59  X(kt+1) -> LDS `nxt`
    //   after slot 59: barrier, then step kt+1's first four A reads, then
    //   slots 60..63 (their operands were read before the barrier).
    auto step = [&](int kt, const uint8_t* cur, uint8_t* nxt, v4i (&xcur)[CPT],
                    v4i (&xnx)[CPT], WStep32& wcur, WStep32& wnx) {
        const int k2 = min(kt + 2, KT - 1);
        DqTmp tmp;
        auto read_a = [&](const uint8_t* buf, int sI) {  // sI = 8i + rb
            return *reinterpret_cast<const v4i*>(buf + (sI & 7) * 4096 + aoff[sI >> 3]);
        };
        static_for<64>([&](auto sc) {
            constexpr int s = decltype(sc)::value;
            constexpr int sI = s / 2, i = sI / 8, rb = sI % 8, cb = s % 2;
            if constexpr (s == 60) {
                __syncthreads();
#pragma unroll
                for (int q = 0; q < 4; ++q) ring[q] = read_a(nxt, q);
            }
            mfma32_i8_acc(acc[rb][cb], ring[sI % 8], B[cb][i]);
            if constexpr (cb == 1 && sI + 4 < 32) ring[(sI + 4) % 8] = read_a(cur, sI + 4);
            if constexpr (s < 8) xcur[s] = x_load(k2, s);
            if constexpr (s >= 16 && s < 22) w_load(k2, s - 16, wcur);
            if constexpr (s >= 52 && s < 60)
                *reinterpret_cast<v4i*>(nxt + xlds0 + (s - 52) * 4096) = xnx[s - 52];
            // dequantisation: 28 steps per 16 slots, 2 per slot (the
            // parameter extraction for wnx takes slot 16's pair)
            if constexpr (s < 16) {
                constexpr int o0 = 2 * s;
                if constexpr (o0 < 28) dq_group_step<3, o0>(tmp, wcur, pp, B);
                if constexpr (o0 + 1 < 28) dq_group_step<3, o0 + 1>(tmp, wcur, pp, B);
            } else if constexpr (s == 16) {
                wparams(wnx, tb, pp);
            } else {
                constexpr int g = s / 16;            // producing B[*][g-1]
                constexpr int o0 = 2 * (s % 16) - (g == 1 ? 2 : 0);
                if constexpr (o0 >= 0 && o0 < 28) dq_group_step<g - 1, o0>(tmp, wnx, pp, B);
                if constexpr (o0 + 1 >= 0 && o0 + 1 < 28)
                    dq_group_step<g - 1, o0 + 1>(tmp, wnx, pp, B);
            }
        });
    };

    int kt = 0;
    for (; kt + 1 < KT; kt += 2) {
        step(kt, xs0, xs1, xe, xo, we, wo);
        step(kt + 1, xs1, xs0, xo, xe, wo, we);
    }
    if (kt < KT) step(kt, xs0, xs1, xe, xo, we, wo);

    mfma32_drain();
    __syncthreads();  // all waves done with the X buffers

    // ---- epilogue.  Accumulator (rb, cb) register v of lane (c, h): row
    // 32rb + 8(v/4) + 4h + (v%4), channel n0 + 32cb + c.  Scaled values go
    // to a per-wave LDS block [32 rows][64 channels]; each row is then
    // written as whole 16-byte pieces.
    if (OUT == 0) sxs[tid] = (m0 + tid < M) ? sx[m0 + tid] : 0.0f;
    const float sw0 = (OUT == 0) ? sw[n0 + c] : 0.0f;
    const float sw1 = (OUT == 0) ? sw[n0 + 32 + c] : 0.0f;
    __syncthreads();
    constexpr int EB = (OUT == 1) ? 4 : 2;   // output element bytes
    constexpr int ROWB = 64 * EB;             // bytes per staged row
    uint8_t* stage = xs0 + wave * (32 * ROWB);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = 8 * (v >> 2) + 4 * h + (v & 3);
                const int col = 32 * cb + c;
                if (OUT == 1) {
                    *reinterpret_cast<int*>(stage + row * ROWB + col * 4) = acc[rb][cb][v];
                } else {
                    const float y = ((float)acc[rb][cb][v] * sxs[32 * rb + row]) * (cb ? sw1 : sw0);
                    *reinterpret_cast<unsigned short*>(stage + row * ROWB + col * 2) =
                        f32_to_f16_bits(y);
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes done
        __builtin_amdgcn_wave_barrier();
        constexpr int PIECES = 32 * ROWB / 16;  // 16-byte pieces per block
        constexpr int PPR = ROWB / 16;          // pieces per row
#pragma unroll
        for (int u = 0; u < PIECES / 64; ++u) {
            const int q = lane + 64 * u;
            const int row = q / PPR, piece = q % PPR;
            const int m = m0 + 32 * rb + row;
            const v4i val = *reinterpret_cast<const v4i*>(stage + row * ROWB + piece * 16);
            if (m < M)
                *reinterpret_cast<v4i*>(reinterpret_cast<uint8_t*>(Y) +
                                        ((size_t)m * N + n0) * EB + piece * 16) = val;
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_wave_barrier();
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
    const int tiles_n = N / kNT;
    const int tiles_m = (M + 255) / 256;
    dim3 grid(tiles_n * tiles_m), block(256);
#define W4A8_L256(O, G)                                                                         \
    hipLaunchKernelGGL((w4a8_mfma256_kernel<O, G>), grid, block, 0, st, X, sx, wq, s_u8, a_u8, \
                       sw, Y, M, N, K, tiles_n, tiles_m)
    if (out_type == 1) {
        if (group == 64) W4A8_L256(1, 64); else W4A8_L256(1, 128);
    } else {
        if (group == 64) W4A8_L256(0, 64); else W4A8_L256(0, 128);
    }
#undef W4A8_L256
    return hipGetLastError();
}

}  // namespace w4a8
