// Large-M W4A8 GEMM for gfx950 (the matrix-core-bound regime).
//
// Workgroup tile: MT (128 or 256) rows of X x 256 output channels; four
// waves, each owning all MT rows and its own 64 channels, so every weight is
// dequantised exactly once per workgroup tile and goes from registers
// straight into the matrix cores.  The consumer dequantises what it
// multiplies, as in the implicit pipeline of LiquidGEMM (Pith review of
// arXiv 2509.01229, "What carries the argument"); there is no producer wave:
// loads are asynchronous and run ahead of the math.  Dequantisation is the
// LiquidQuant identity (q*s + a) XOR 0x80, two VALU instructions per four
// weights after the nibble split (same review, paper Eq. 12; minor comment 1
// / Sec. 5.3 for the instruction count).
//
// Per K-step of 128 columns: X[MT][128] int8 goes global -> LDS directly
// (three rotating tiles, 16-byte slots XOR-swizzled per row); each wave loads
// its 4 packed tiles of a later step and dequantises them in single
// instructions interleaved with the current step's matrix-core
// instructions (v_mfma_i32_32x32x32_i8, accumulators in AGPRs).
// Epilogue: Y = fp16((float(acc) * sx[m]) * sw[n]) or the raw int32.
#include "launch.h"
#include "mfma_common.h"

namespace w4a8 {

// Built on v_mfma_i32_32x32x32_i8: each instruction leaves a 32-cycle
// shadow for the dequantisation, LDS and memory instructions of the same
// wave.
//   wave tile MT x 64 = MT/32 row blocks x 2 channel blocks of 32 x 32;
//   B operand of lane (c = lane % 32, h = lane / 32): packed tile row c % 16
//     of tile 2*cb + c/16, slots 2h and 2h+1 (K columns 64h .. 64h+63 of
//     the 128-column step); instruction i (0..3) consumes columns
//     64h + 16i .. +15, and the A operand (X row, same columns) matches;
//   every global load is a buffer load (SGPR step offset, no per-load
//     address arithmetic); weights are loaded two K-steps ahead into
//     registers, X tiles two K-steps ahead into LDS; X rows past M fall
//     outside the buffer and read as zero;
//   the next step's weights are dequantised in single-instruction steps
//     interleaved with this step's matrix-core instructions;
//   the epilogue scales in registers, transposes through LDS and writes
//     whole 128-byte row segments.
namespace {

__device__ __forceinline__ void mfma32_i8_acc(v16i& acc, const v4i& a, const v4i& b) {
    asm volatile("v_mfma_i32_32x32x32_i8 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// Raw weights of one K-step for one lane: w[cb][e] = slot 2h+e of the
// lane's row in tile 2cb + c/16; parameter dwords of the lane's panel row.
struct WStep32 {
    v4i w[2][2];
    unsigned sdw, adw;
};

// Decoders of one K-step's raw weights into the B operands, as policies
// with single-instruction steps so the kernel can spread them over the
// matrix-core slots:
//   kParamOps  steps that turn the parameter dwords into per-lane operands;
//   kOps       steps that produce B[*][i] of one instruction group i (both
//              channel blocks, two packed dwords each);
// plus the same work in one call (params(), group<i>()).
//
// LiquidQuant decode (the default): per packed dword (8 codes),
//   lo = w & 0x0F0F0F0F; t = w >> 4; hi = t & 0x0F0F0F0F;
//   lo = lo*s + a; hi = hi*s + a   (v_pk_mad_u16, two codes per 16-bit lane);
//   B = lo ^ 0x80808080, hi ^ 0x80808080
// 7 instructions per 8 weights (LiquidGEMM, Pith review of arXiv 2509.01229,
// paper Eq. 12 and minor comment 1 / Sec. 5.3).
// Empty assembly reading every register of a raw set: the compiler must
// have all of its loads complete at this point.
__device__ __forceinline__ void touch_raw(const WStep32& w) {
    asm volatile("" ::"v"(w.w[0][0]), "v"(w.w[0][1]), "v"(w.w[1][0]), "v"(w.w[1][1]), "v"(w.sdw),
                 "v"(w.adw));
}

struct DecLQQ {
    using Raw = WStep32;
    static constexpr bool kW8 = false;
    static constexpr int kLoads = 6;  // raw loads per K-step: 4 weight slots, s, a
    struct Params {
        unsigned s2[2], a4[2];  // scale pair, offset quad per channel block
    };
    struct Tmp {  // the two dwords decoded together (index dd)
        unsigned lo[2], t[2], hi[2];
    };
    static constexpr int kParamOps = 4;
    static constexpr int kOps = 28;

    template <int K_>
    __device__ __forceinline__ static void param_step(const WStep32& w, int tb, Params& p) {
        constexpr int cb = K_ / 2;
        const unsigned b = (unsigned)(2 * cb + tb);
        if constexpr (K_ % 2 == 0) {
            const unsigned sel = b | 0x0C00u | (b << 16) | 0x0C000000u;
            asm volatile("v_perm_b32 %0, 0, %1, %2" : "=v"(p.s2[cb]) : "v"(w.sdw), "v"(sel));
        } else {
            asm volatile("v_perm_b32 %0, 0, %1, %2"
                         : "=v"(p.a4[cb]) : "v"(w.adw), "v"(b * 0x01010101u));
        }
    }

    // Instruction group I takes dwords d = 2(I%2), 2(I%2)+1 of slot e = I/2;
    // their steps alternate (dd = q % 2), so no step reads the result of the
    // one just before it.
    template <int I, int OP>
    __device__ __forceinline__ static void step(Tmp& tmp, const WStep32& w, const Params& p,
                                                v4i (&B)[2][4]) {
        constexpr int cb = OP / 14, q = OP % 14, dd = q % 2, st = q / 2;
        constexpr int e = I / 2, d = 2 * (I % 2) + dd;
        const unsigned wd = (unsigned)w.w[cb][e][d];
        if constexpr (st == 0) {
            asm volatile("v_and_b32 %0, 0x0f0f0f0f, %1" : "=v"(tmp.lo[dd]) : "v"(wd));
        } else if constexpr (st == 1) {
            asm volatile("v_lshrrev_b32 %0, 4, %1" : "=v"(tmp.t[dd]) : "v"(wd));
        } else if constexpr (st == 2) {
            asm volatile("v_and_b32 %0, 0x0f0f0f0f, %1" : "=v"(tmp.hi[dd]) : "v"(tmp.t[dd]));
        } else if constexpr (st == 3) {
            asm volatile("v_pk_mad_u16 %0, %1, %2, %3"
                         : "=v"(tmp.lo[dd]) : "v"(tmp.lo[dd]), "v"(p.s2[cb]), "v"(p.a4[cb]));
        } else if constexpr (st == 4) {
            asm volatile("v_pk_mad_u16 %0, %1, %2, %3"
                         : "=v"(tmp.hi[dd]) : "v"(tmp.hi[dd]), "v"(p.s2[cb]), "v"(p.a4[cb]));
        } else if constexpr (st == 5) {
            unsigned x;
            asm volatile("v_xor_b32 %0, 0x80808080, %1" : "=v"(x) : "v"(tmp.lo[dd]));
            B[cb][I][2 * dd] = (int)x;
        } else {
            unsigned x;
            asm volatile("v_xor_b32 %0, 0x80808080, %1" : "=v"(x) : "v"(tmp.hi[dd]));
            B[cb][I][2 * dd + 1] = (int)x;
        }
    }
};

// Conventional sign-safe decode, for the ablation: the same stored codes
// and parameters decoded as the plain affine value s*q + min (min = a - 128)
// in signed 16-bit lanes, one code per lane, because a negative result in
// a byte lane would borrow from its neighbour -- the overflow handling the
// LiquidQuant shift into UINT8 removes (same review, "What carries the
// argument").  Per packed dword: the nibble split, then for each half two
// byte spreads, two v_pk_mad_i16 and one byte gather: 13 instructions per 8
// weights.  Equal to the LiquidQuant decode value for value (the identity
// (q*s + a) XOR 0x80 = q*s + a - 128 on INT8 results).
struct DecAffine16 {
    using Raw = WStep32;
    static constexpr bool kW8 = false;
    static constexpr int kLoads = 6;
    struct Params {
        unsigned s2[2], m2[2];  // scale, min in both 16-bit lanes
    };
    struct Tmp {  // the two dwords decoded together (index dd)
        unsigned lo[2], t[2], hi[2], e0[2], e1[2];
    };
    static constexpr int kParamOps = 6;
    static constexpr int kOps = 52;

    template <int K_>
    __device__ __forceinline__ static void param_step(const WStep32& w, int tb, Params& p) {
        constexpr int cb = K_ / 3, st = K_ % 3;
        const unsigned b = (unsigned)(2 * cb + tb);
        const unsigned sel = b | 0x0C00u | (b << 16) | 0x0C000000u;
        if constexpr (st == 0) {
            asm volatile("v_perm_b32 %0, 0, %1, %2" : "=v"(p.s2[cb]) : "v"(w.sdw), "v"(sel));
        } else if constexpr (st == 1) {
            asm volatile("v_perm_b32 %0, 0, %1, %2" : "=v"(p.m2[cb]) : "v"(w.adw), "v"(sel));
        } else {
            asm volatile("v_pk_sub_u16 %0, %1, %2" : "=v"(p.m2[cb]) : "v"(p.m2[cb]), "s"(0x00800080u));
        }
    }

    template <int I, int OP>
    __device__ __forceinline__ static void step(Tmp& tmp, const WStep32& w, const Params& p,
                                                v4i (&B)[2][4]) {
        constexpr int cb = OP / 26, q = OP % 26, dd = q % 2, st = q / 2;  // dwords alternate
        constexpr int e = I / 2, d = 2 * (I % 2) + dd;
        const unsigned wd = (unsigned)w.w[cb][e][d];
        constexpr unsigned kEven = 0x0C020C00u, kOdd = 0x0C030C01u, kGather = 0x06020400u;
        if constexpr (st == 0) {
            asm volatile("v_and_b32 %0, 0x0f0f0f0f, %1" : "=v"(tmp.lo[dd]) : "v"(wd));
        } else if constexpr (st == 1) {
            asm volatile("v_lshrrev_b32 %0, 4, %1" : "=v"(tmp.t[dd]) : "v"(wd));
        } else if constexpr (st == 2) {
            asm volatile("v_and_b32 %0, 0x0f0f0f0f, %1" : "=v"(tmp.hi[dd]) : "v"(tmp.t[dd]));
        } else if constexpr (st == 3 || st == 8) {
            const unsigned src = st == 3 ? tmp.lo[dd] : tmp.hi[dd];
            asm volatile("v_perm_b32 %0, 0, %1, %2" : "=v"(tmp.e0[dd]) : "v"(src), "s"(kEven));
        } else if constexpr (st == 4 || st == 9) {
            const unsigned src = st == 4 ? tmp.lo[dd] : tmp.hi[dd];
            asm volatile("v_perm_b32 %0, 0, %1, %2" : "=v"(tmp.e1[dd]) : "v"(src), "s"(kOdd));
        } else if constexpr (st == 5 || st == 10) {
            asm volatile("v_pk_mad_i16 %0, %1, %2, %3"
                         : "=v"(tmp.e0[dd]) : "v"(tmp.e0[dd]), "v"(p.s2[cb]), "v"(p.m2[cb]));
        } else if constexpr (st == 6 || st == 11) {
            asm volatile("v_pk_mad_i16 %0, %1, %2, %3"
                         : "=v"(tmp.e1[dd]) : "v"(tmp.e1[dd]), "v"(p.s2[cb]), "v"(p.m2[cb]));
        } else {
            unsigned x;
            asm volatile("v_perm_b32 %0, %1, %2, %3" : "=v"(x) : "v"(tmp.e1[dd]), "v"(tmp.e0[dd]), "s"(kGather));
            B[cb][I][2 * dd + (st == 12 ? 1 : 0)] = (int)x;
        }
    }
};

// No decode, for the W8A8 comparison: the INT8 weights of the first
// quantisation level alone, in the 8-bit tile layout.  A lane's raw K-step
// (w[cb][i] = its 16 bytes for instruction i, read straight from the 8-bit
// tile layout) is already the B operand set; "decoding" copies it into B.
struct WStep8 {
    v4i w[2][4];
};
__device__ __forceinline__ void touch_raw(const WStep8& w) {
    asm volatile("" ::"v"(w.w[0][0]), "v"(w.w[0][1]), "v"(w.w[0][2]), "v"(w.w[0][3]),
                 "v"(w.w[1][0]), "v"(w.w[1][1]), "v"(w.w[1][2]), "v"(w.w[1][3]));
}

struct DecW8 {
    using Raw = WStep8;
    static constexpr bool kW8 = true;
    static constexpr int kLoads = 8;
    struct Params {};
    struct Tmp {};
    static constexpr int kParamOps = 0;
    static constexpr int kOps = 8;

    template <int K_>
    __device__ __forceinline__ static void param_step(const Raw&, int, Params&) {}

    // one dword per step (explicit moves: a copy the register allocator
    // could fold would leave loop-carried copies of registers still being
    // loaded)
    template <int I, int OP>
    __device__ __forceinline__ static void step(Tmp&, const Raw& w, const Params&,
                                                v4i (&B)[2][4]) {
        constexpr int cb = OP / 4, d = OP % 4;
        int x;
        asm volatile("v_mov_b32 %0, %1" : "=v"(x) : "v"(w.w[cb][I][d]));
        B[cb][I][d] = x;
    }
};

template <class DEC>
__device__ __forceinline__ void dec_params(const typename DEC::Raw& w, int tb,
                                           typename DEC::Params& p) {
    static_for<DEC::kParamOps>([&](auto k) { DEC::template param_step<decltype(k)::value>(w, tb, p); });
}

template <class DEC, int I>
__device__ __forceinline__ void dec_group(const typename DEC::Raw& w, const typename DEC::Params& p,
                                          v4i (&B)[2][4]) {
    typename DEC::Tmp tmp;
    static_for<DEC::kOps>([&](auto oc) { DEC::template step<I, decltype(oc)::value>(tmp, w, p, B); });
}

template <class DEC>
__device__ __forceinline__ void dec_all(const typename DEC::Raw& w, int tb, typename DEC::Params& p,
                                        v4i (&B)[2][4]) {
    dec_params<DEC>(w, tb, p);
    dec_group<DEC, 0>(w, p, B);
    dec_group<DEC, 1>(w, p, B);
    dec_group<DEC, 2>(w, p, B);
    dec_group<DEC, 3>(w, p, B);
}

}  // namespace

// DEC: weight decoder policy (DecLQQ; DecAffine16 for the ablation; DecW8
// for the W8A8 comparison, whose `wq` is the 8-bit tile layout).
// COARSE: decode each K-step's weights in one block after that step's
// matrix-core instructions instead of interleaving them (ablation of the
// fine-grained overlap).
template <int MT, int OUT, int GROUP, bool PARTIAL, class DEC, bool COARSE>
__global__ __launch_bounds__(256, 1) void w4a8_mfma_kernel(
    const int8_t* __restrict__ X, const float* __restrict__ sx, const uint8_t* __restrict__ wq,
    const uint8_t* __restrict__ s_u8, const uint8_t* __restrict__ a_u8,
    const float* __restrict__ sw, void* __restrict__ Y, int* __restrict__ part, int M, int N,
    int K, int tiles_n, int tiles_m, int splits, const int* __restrict__ offsets) {
    constexpr int RB = MT / 32;        // 32-row blocks per wave
    constexpr int CPT = MT / 32;       // 16-byte X chunks per thread per K-step
    constexpr int SLOTS = 8 * RB;      // matrix-core instructions per wave per K-step
    constexpr int GS = SLOTS / 4;      // slots per instruction group i
    constexpr int DQ = (DEC::kParamOps + DEC::kOps + GS - 1) / GS;  // decode steps per slot
    constexpr unsigned XB = MT * 128;  // bytes of one X tile (MT rows x 128 K)
    __shared__ __attribute__((aligned(1024))) uint8_t xs[3 * XB];  // X(kt), X(kt+1), X(kt+2)
    __shared__ float sxs[MT];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int c = lane & 31, h = lane >> 5;
    const int tb = c >> 4, r = c & 15;

    const TileCoord tc = tile_coord(blockIdx.x, tiles_m, tiles_n, splits);
    const int ks = tc.ks;
    // Grouped problems (offsets != nullptr): expert blockIdx.y owns rows
    // offsets[e] .. offsets[e+1]-1 (clamped to [0, M]) and the e-th weight
    // slab; its M tiles start at offsets[e].
    int row_lo = 0, row_hi = M;
    if (offsets) {
        const int e = blockIdx.y;
        row_lo = min(max(offsets[e], 0), M);
        row_hi = min(max(offsets[e + 1], row_lo), M);
        wq += (size_t)e * N * (DEC::kW8 ? K : K / 2);
        s_u8 += (size_t)e * N * (K / GROUP);
        a_u8 += (size_t)e * N * (K / GROUP);
        sw += (size_t)e * N;
    }
    const int m0 = row_lo + tc.tm * MT;
    if (m0 >= row_hi) return;  // whole workgroup: no rows of this expert here
    const int n0 = tc.tn * kNT + wave * kColsPerWave;
    const int KTall = K / kTileK;
    const int kt0 = (int)((long long)KTall * ks / splits);
    const int KT = (int)((long long)KTall * (ks + 1) / splits) - kt0;  // >= 1
    // The main loop runs K-steps in pairs with a single exit; an odd count
    // gets one more step whose X tile reads as zero (contributing exactly 0).
    const int KTe = KT + (KT & 1);
    const int groups = K / GROUP;

    // ---- X goes from global memory straight into one of three LDS tiles
    // (no register round trip).  Tile row R keeps its 16-byte column chunk
    // k in slot k ^ xswz(R & 15).  Wave w's load p (p < CPT) fills rows
    // 32p + 8w .. +7 (1 KiB): lane l writes slot l % 8 of row
    // 32p + 8w + l / 8, so it fetches that row's chunk (l % 8) ^ xswz(row & 15)
    // (row & 15 does not depend on p).  Rows >= M lie past the end of the
    // buffer and read as 0.
    const __amdgpu_buffer_rsrc_t xr_rsrc = buf_rsrc(X, (unsigned)M * (unsigned)K);
    const int xr = 8 * wave + (lane >> 3);
    const int xc = (lane & 7) ^ xswz(xr & 15);
    const unsigned xvoff =
        (unsigned)(m0 + xr) * (unsigned)K + (unsigned)(xc * 16) + (unsigned)(kt0 * kTileK);
    const unsigned xrowstep = 32u * (unsigned)K;
    const unsigned xsbase = lds_addr(xs);
    // A operand (row block rb, instruction i): row 32rb + c, column 4h + i.
    int aoff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) aoff[i] = c * 128 + (((4 * h + i) ^ xswz(r)) * 16);

    // ---- weights of this wave: tiles nt0 .. nt0+3 (one parameter panel)
    const int nt0 = n0 / kTileN;
    const __amdgpu_buffer_rsrc_t w_rsrc =
        buf_rsrc(wq, (unsigned)((size_t)N * K / (DEC::kW8 ? 1 : 2)));
    const __amdgpu_buffer_rsrc_t s_rsrc = buf_rsrc(s_u8, (unsigned)((size_t)N * K / GROUP));
    const __amdgpu_buffer_rsrc_t a_rsrc = buf_rsrc(a_u8, (unsigned)((size_t)N * K / GROUP));
    const unsigned wvoff = (unsigned)(tb * KTall) * kTileBytes + (unsigned)(32 * h + r) * 16u;
    const unsigned pvoff = 4u * (unsigned)r + (GROUP == 64 ? 64u * (unsigned)h : 0u);
    const unsigned ppanel = 64u * (unsigned)(n0 >> 6) * (unsigned)groups;
    // 8-bit layout: tile (nt, kt) of 2 KiB; the bytes for instruction i of
    // lane (c, h) (K columns 64h + 16i .. +15 of row r) sit at
    // 1024 (i & 1) + 256 (2h + i / 2) + 16 r inside it.
    const unsigned w8voff = (unsigned)(tb * KTall) * 2048u + 512u * (unsigned)h + 16u * (unsigned)r;
    auto w_load = [&](int kt, int part_i, typename DEC::Raw& ws) {  // part_i < DEC::kLoads
        const int ktg = kt0 + kt;
        if constexpr (DEC::kW8) {
            const int cb = part_i >> 2, i = part_i & 3;
            ws.w[cb][i] = buf_load16(w_rsrc, w8voff,
                                     (unsigned)(((nt0 + 2 * cb) * KTall + ktg) * 2048 +
                                                1024 * (i & 1) + 256 * (i >> 1)));
        } else if (part_i < 4) {
            const int cb = part_i >> 1, e = part_i & 1;
            ws.w[cb][e] = buf_load16(
                w_rsrc, wvoff, (unsigned)(((nt0 + 2 * cb) * KTall + ktg) * kTileBytes + e * 256));
        } else {
            const unsigned jo = ppanel + 64u * (unsigned)(ktg * (kTileK / GROUP));
            if (part_i == 4) ws.sdw = buf_load4(s_rsrc, pvoff, jo);
            else ws.adw = buf_load4(a_rsrc, pvoff, jo);
        }
    };
    auto x_load = [&](int kt, int p, unsigned buf) {  // into LDS tile at byte `buf`
        const bool live = kt < KT;  // kt >= KT: offset past the buffer, reads 0
        const unsigned vo = live ? xvoff + (unsigned)p * xrowstep : 0xFFFFFFF0u;
        const unsigned so = live ? (unsigned)(kt * kTileK) : 0u;
        buf_load16_lds(xr_rsrc, vo, so, xsbase + buf + (unsigned)(4 * p + wave) * 1024u);
    };

    v16i acc[RB][2];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        acc[rb][0] = v16i{};
        acc[rb][1] = v16i{};
    }

    // ---- prologue: X(0), X(1) -> LDS tiles 0, 1; W(0) dequantised fully,
    // W(1) raw; A ring primed with step 0's first four operands.
    typename DEC::Raw we, wo;  // raw weights for even / odd steps
    typename DEC::Params pp;  // parameters of the raw set being decoded
    v4i B[2][4];
    v4i ring[8];
    // X of the padding step reads as zero; its weights (and factors) are
    // those of the last real step, so no load leaves this split's K range.
    const int k1 = min(1, KTe - 1), kw1 = min(1, KT - 1);
    unsigned bc = 0, bn = XB, bd = 2 * XB;  // LDS tiles of X(kt), X(kt+1), X(kt+2)
#pragma unroll
    for (int p = 0; p < CPT; ++p) x_load(0, p, bc);
#pragma unroll
    for (int p = 0; p < CPT; ++p) x_load(k1, p, bn);
#pragma unroll
    for (int pi = 0; pi < DEC::kLoads; ++pi) w_load(0, pi, we);
#pragma unroll
    for (int pi = 0; pi < DEC::kLoads; ++pi) w_load(kw1, pi, wo);
    dec_all<DEC>(we, tb, pp, B);
    // X(0) and X(1) were issued before W(0) and W(1): once at most the W(1)
    // loads are outstanding, every wave's part of the two X tiles is in LDS.
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(DEC::kLoads, 0));
    __syncthreads();
    auto read_a = [&](unsigned buf, int sI) {  // sI = RB*i + rb
        return *reinterpret_cast<const v4i*>(xs + buf + (sI % RB) * 4096 + aoff[sI / RB]);
    };
#pragma unroll
    for (int q = 0; q < 4; ++q) ring[q] = read_a(bc, q);

    // ---- one K-step, SLOTS matrix-core slots.  Slot s: instruction group
    // i = s / GS, row block rb = (s/2) % RB, channel block cb = s % 2.
    // Entering step kt: LDS tile `cur` = X(kt), `nxt` = X(kt+1) (loads in
    // flight), `dst` free (its X(kt-1) was last read before the previous
    // barrier); ring holds A for the first slots; B[*][0..2] = W(kt)
    // operands and B[*][3] is produced during group 0 from `wcur` (raw W(kt),
    // parameters pp); `wnx` = raw W(kt+1).
    //   group 0 slots      B[*][3] of step kt
    //   group 1 slots      W(kt+2) -> wcur; parameters of wnx, B[*][0] of kt+1
    //   groups 2, 3        B[*][1], B[*][2] of step kt+1
    //   CPT slots from XS  X(kt+2) -> LDS `dst`, after this step's first use
    //                      of wnx: the compiler does not see these loads, so
    //                      its wait before that use covers only loads a
    //                      step old
    //   before the last 4  wait for this wave's X(kt+1) loads (CPT + kLoads
    //                      loads were issued after them), barrier, then step
    //                      kt+1's first four A reads; the last four slots
    //                      use operands read earlier.
    auto step = [&](int kt, unsigned cur, unsigned nxt, unsigned dst, typename DEC::Raw& wcur,
                    typename DEC::Raw& wnx) {
        const int k2 = min(kt + 2, KTe - 1), kw2 = min(kt + 2, KT - 1);
        constexpr int XS = GS + DEC::kLoads;  // first X load slot
        static_assert(XS + CPT <= SLOTS - 4, "X loads must precede the barrier");
        typename DEC::Tmp tmp;
        static_for<SLOTS>([&](auto sc) {
            constexpr int s = decltype(sc)::value;
            constexpr int sI = s / 2, i = sI / RB, rb = sI % RB, cb = s % 2;
            constexpr int g = s / GS, sg = s % GS;
            if constexpr (s == SLOTS - 4) {
                __builtin_amdgcn_sched_barrier(0);
                __builtin_amdgcn_s_waitcnt(waitcnt_imm(CPT + DEC::kLoads, 0));
                __syncthreads();
#pragma unroll
                for (int q = 0; q < 4; ++q) ring[q] = read_a(nxt, q);
            }
            mfma32_i8_acc(acc[rb][cb], B[cb][i], ring[sI % 8]);
            if constexpr (cb == 1 && sI + 4 < 4 * RB) ring[(sI + 4) % 8] = read_a(cur, sI + 4);
            if constexpr (s >= GS && s < GS + DEC::kLoads) w_load(kw2, s - GS, wcur);
            // All of wnx complete here, before the X loads: the compiler's
            // wait for a part first used later would also cover X loads
            // issued in between, which it does not see.
            if constexpr (s == GS) touch_raw(wnx);
            if constexpr (s >= XS && s < XS + CPT) x_load(k2, s - XS, dst);
            if constexpr (!COARSE) {
                constexpr int PO = DEC::kParamOps, NO = DEC::kOps;
                static_for<DQ>([&](auto dc) {
                    constexpr int o = DQ * sg + decltype(dc)::value;
                    if constexpr (g == 0) {
                        if constexpr (o < NO) DEC::template step<3, o>(tmp, wcur, pp, B);
                    } else if constexpr (g == 1) {
                        if constexpr (o < PO) DEC::template param_step<o>(wnx, tb, pp);
                        else if constexpr (o - PO < NO)
                            DEC::template step<0, o - PO>(tmp, wnx, pp, B);
                    } else {
                        if constexpr (o < NO) DEC::template step<g - 1, o>(tmp, wnx, pp, B);
                    }
                });
            }
        });
        // Coarse variant: the whole next step decoded here, the matrix cores idle.
        if constexpr (COARSE) dec_all<DEC>(wnx, tb, pp, B);
    };

    for (int kt = 0; kt < KTe; kt += 2) {
        step(kt, bc, bn, bd, we, wo);
        step(kt + 1, bn, bd, bc, wo, we);
        const unsigned t0 = bc;  // next pair: X(kt+2) in bd, X(kt+3) in bc
        bc = bd;
        bd = bn;
        bn = t0;
        if (kt + 2 >= KTe) mfma_loop_exit_wait();  // the iteration that leaves the loop
    }
    mfma32_drain(acc);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));  // the last steps' X loads
    __syncthreads();  // all waves done with the X tiles

    // ---- epilogue.  The weights are the instruction's first operand and X
    // its second, so it accumulates (W X^T) blocks: accumulator (rb, cb)
    // register 4i + e of lane (c, h) holds row 32rb + c, channel
    // n0 + 32cb + 8i + 4h + e -- runs of four consecutive channels.  Each run
    // goes to a per-wave LDS block [32 rows][64 channels] as one 8-byte
    // (fp16) or 16-byte (int32) piece, rows padded by 16 bytes; each row is
    // then written as whole 16-byte pieces (final output, or this split's
    // int32 partial).
    constexpr bool SCALED = (OUT == 0) && !PARTIAL;
    if (SCALED) sxs[tid % MT] = (m0 + tid % MT < row_hi) ? sx[m0 + tid % MT] : 0.0f;
    float swv[2][4][4];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                swv[cb][i][e] = SCALED ? sw[n0 + 32 * cb + 8 * i + 4 * h + e] : 0.0f;
    __syncthreads();
    constexpr int EB = SCALED ? 2 : 4;  // output element bytes
    constexpr int ROWB = 64 * EB;       // bytes per row of the block
    constexpr int RSTR = ROWB + 16;     // padded row stride in LDS
    static_assert(kWaves * 32 * RSTR <= 3 * XB, "epilogue staging fits in the X tiles");
    uint8_t* stage = xs + wave * (32 * RSTR);
    uint8_t* out = PARTIAL ? reinterpret_cast<uint8_t*>(part + (size_t)ks * M * N)
                           : reinterpret_cast<uint8_t*>(Y);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        uint8_t* srow = stage + c * RSTR;
        const float sm = SCALED ? sxs[32 * rb + c] : 0.0f;
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int col = 32 * cb + 8 * i + 4 * h;
                if constexpr (SCALED) {
                    unsigned short hv[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        hv[e] = f32_to_f16_bits(((float)acc[rb][cb][4 * i + e] * sm) *
                                                swv[cb][i][e]);
                    uint2 pk;
                    pk.x = hv[0] | ((unsigned)hv[1] << 16);
                    pk.y = hv[2] | ((unsigned)hv[3] << 16);
                    *reinterpret_cast<uint2*>(srow + col * 2) = pk;
                } else {
                    *reinterpret_cast<v4i*>(srow + col * 4) =
                        v4i{acc[rb][cb][4 * i], acc[rb][cb][4 * i + 1], acc[rb][cb][4 * i + 2],
                            acc[rb][cb][4 * i + 3]};
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes done
        __builtin_amdgcn_wave_barrier();
        constexpr int PPR = ROWB / 16;  // 16-byte pieces per row
#pragma unroll
        for (int u = 0; u < 32 * PPR / 64; ++u) {
            const int q = lane + 64 * u;
            const int row = q / PPR, piece = q % PPR;
            const int m = m0 + 32 * rb + row;
            const v4i val = *reinterpret_cast<const v4i*>(stage + row * RSTR + piece * 16);
            if (m < row_hi)
                store16_result<PARTIAL>(out + ((size_t)m * N + n0) * EB + piece * 16, val);
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_wave_barrier();
    }
}

// Sum of the split-K partial tiles in split order (exact int32), then the
// per-token x per-channel scale to fp16, or the raw int32 sums.  Workgroup
// (x, y) covers 1024 channels of row y; each thread four consecutive
// channels.  The split count is a template argument, so a thread's S partial
// loads are all in flight before the first add.
template <int OUT, int S>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(
    const int* __restrict__ part, int M, int N, const float* __restrict__ sx,
    const float* __restrict__ sw, void* __restrict__ Y) {
    const int n = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (n >= N) return;
    const int m = blockIdx.y;
    const size_t MN = (size_t)M * N;
    const size_t e = (size_t)m * N + n;
    v4i v[S];
#pragma unroll
    for (int s = 0; s < S; ++s) v[s] = *reinterpret_cast<const v4i*>(part + s * MN + e);
    v4i acc = v[0];
#pragma unroll
    for (int s = 1; s < S; ++s) acc += v[s];
    if (OUT == 1) {
        *reinterpret_cast<v4i*>(reinterpret_cast<int*>(Y) + e) = acc;
    } else {
        const float sm = sx[m];
        unsigned short hv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) hv[j] = f32_to_f16_bits(((float)acc[j] * sm) * sw[n + j]);
        uint2 pk;
        pk.x = hv[0] | ((unsigned)hv[1] << 16);
        pk.y = hv[2] | ((unsigned)hv[3] << 16);
        *reinterpret_cast<uint2*>(reinterpret_cast<unsigned short*>(Y) + e) = pk;
    }
}

// splits in 2 .. 16 (the plans' range), one instantiation each.
template <int OUT, int S = 2>
static hipError_t splitk_reduce_run(const int* part, int splits, int M, int N, const float* sx,
                                    const float* sw, void* Y, hipStream_t st) {
    if constexpr (S > 16) {
        return hipErrorInvalidValue;
    } else {
        if (splits != S)
            return splitk_reduce_run<OUT, S + 1>(part, splits, M, N, sx, sw, Y, st);
        const dim3 grid((unsigned)((N / 4 + 255) / 256), (unsigned)M);
        hipLaunchKernelGGL((splitk_reduce_kernel<OUT, S>), grid, dim3(256), 0, st, part, M, N,
                           sx, sw, Y);
        return hipGetLastError();
    }
}

hipError_t launch_splitk_reduce(const int* part, int splits, int M, int N, const float* sx,
                                const float* sw, void* Y, int out_type, hipStream_t st) {
    if (M == 0) return hipSuccess;
    if (out_type == 1) return splitk_reduce_run<1>(part, splits, M, N, sx, sw, Y, st);
    return splitk_reduce_run<0>(part, splits, M, N, sx, sw, Y, st);
}

// Workgroup tile height and K split for the matrix-core kernel.
MfmaPlan plan_w4a8_mfma(int M, int N, int K, bool k_parts) {
    MfmaPlan p;
    const int KT = K / kTileK;
    const long long t256 = (long long)(N / kNT) * ((M + 255) / 256);
    // 256-row tiles decode each weight for twice the rows (a few per cent
    // faster per tile) when the grid stays full and they pad M by at most
    // 3 % more rows than 128-row tiles would
    const long long pad256 = (long long)((M + 255) / 256) * 256;
    const long long pad128 = (long long)((M + 127) / 128) * 128;
    p.mt = (M > 128 && t256 >= 256 && pad256 * 100 <= pad128 * 103) ? 256 : 128;
    const long long tiles = (long long)(N / kNT) * ((M + p.mt - 1) / p.mt);
    // Few tiles: split K so the grid fills one wave of the 256 CUs (the
    // largest split count with tiles * splits <= 256; each split keeps at
    // least 8 K-steps).  Overshooting to a second, partial wave costs more
    // than the idle CUs of an exact fit, and every split adds M*N int32
    // partials to write and read back.
    p.splits = 1;
    if (tiles < 256) {
        int s = (int)(256 / tiles);
        if (s > 16) s = 16;
        while (s > 1 && KT < 8 * s) --s;
        p.splits = s;
    }
    p.workspace = p.splits > 1 ? (size_t)p.splits * M * N * sizeof(int) : 0;
    // Integer kernels: workgroups with at most 64 K-steps run 128-row tiles
    // on the 16 x 16 kernel, two per CU, so one workgroup's prologue and
    // epilogue overlap the other's main loop, where 256-row tiles would make
    // fewer than four waves (measured: 2048 x 11008 x 4096 20 % faster,
    // 1024 x 28672 x 8192 6 %, 4096 x 8192 x 8192 2.5 %, the split-K mid-M
    // plans 1-6 %).  With more waves (4096 x 28672 x 8192: equal time, 1.4x
    // the HBM traffic, each weight read for twice as many row tiles) and for
    // longer K, 256-row tiles stay; 128-row plans with long K keep the
    // 32 x 32 kernel.  A 256 -> 128 switch keeps splits = 1.
    const bool short_k = KT / p.splits <= 64;
    const bool few_waves = p.mt == 128 || t256 < 4 * 256;
    p.mt16 = (short_k && few_waves) ? 128 : (p.mt == 256 ? 256 : 0);
    // Integer 16 x 16 kernel with an even split count: workgroups of 128
    // channels whose two wave pairs take the two K halves (exact int32 sums
    // through LDS) cover the same grid with half the splits -- the same
    // K-steps per wave and half the partials, but every workgroup reads X
    // for half as many channels, so X is read once more per 256 channels.
    // Taken when that removes the partials and the second launch (two
    // splits), or when the X bytes it adds are at most the partial bytes it
    // saves (written once and read once).  Measured, alternating launches on
    // one GPU: 128 x 28672 x 8192 48.0 -> 42.6 us, 64 x 28672 x 8192 42.1 ->
    // 38.2, 128 x 4096 x 4096 (four splits) 17.6 -> 16.1; not taken at
    // 128 x 8192 x 28672 (eight splits: 48.1 -> 50.1) or 256 x 8192 x 8192
    // (four: 30.7 -> 31.1).
    p.kin = 1;
    if (k_parts && p.mt16 == 128 && p.mt == 128 && p.splits % 2 == 0) {
        const long long x_extra = (long long)(N / kNT) * (((M + 127) / 128) * 128LL) * K;
        const long long saved = (long long)p.splits * M * N * (long long)sizeof(int);
        if (p.splits == 2 || x_extra <= saved) {
            p.kin = 2;
            p.splits /= 2;
            p.workspace = p.splits > 1 ? (size_t)p.splits * M * N * sizeof(int) : 0;
        }
    }
    return p;
}

template <int MT, int OUT, bool PARTIAL, class DEC = DecLQQ, bool COARSE = false>
static void launch_tile(const int8_t* X, const float* sx, const uint8_t* wq, const uint8_t* s_u8,
                        const uint8_t* a_u8, const float* sw, void* Y, int* part, int M, int N,
                        int K, int group, int splits, hipStream_t st,
                        const int* offsets = nullptr, int E = 1, int max_rows = 0) {
    const int tiles_n = N / kNT;
    const int tiles_m = ((offsets ? max_rows : M) + MT - 1) / MT;
    dim3 grid(tiles_n * tiles_m * splits, offsets ? E : 1), block(256);
    if (group == 64)
        hipLaunchKernelGGL((w4a8_mfma_kernel<MT, OUT, 64, PARTIAL, DEC, COARSE>), grid, block, 0,
                           st, X, sx, wq, s_u8, a_u8, sw, Y, part, M, N, K, tiles_n, tiles_m,
                           splits, offsets);
    else
        hipLaunchKernelGGL((w4a8_mfma_kernel<MT, OUT, 128, PARTIAL, DEC, COARSE>), grid, block, 0,
                           st, X, sx, wq, s_u8, a_u8, sw, Y, part, M, N, K, tiles_n, tiles_m,
                           splits, offsets);
}

// Grouped 128-row tiles: from this many rows in the largest expert on, the
// 16 x 16 kernel at two workgroups per CU (Mixtral experts at 8192 tokens,
// about 2100 rows each: 5-6 % faster; at 512 tokens, about 140 rows: 3-4 %
// slower, so fewer rows keep the 32 x 32 kernel).
constexpr int kGrouped16Rows = 1024;

hipError_t launch_w4a8_mfma_grouped(const int8_t* X, const float* sx, const uint8_t* wq,
                                    const uint8_t* s_u8, const uint8_t* a_u8, const float* sw,
                                    void* Y, int out_type, int M, int N, int K, int group,
                                    const int* offsets, int E, int max_rows, int mt,
                                    hipStream_t st) {
    if (mt == 256) {
        if (out_type == 1) launch_tile<256, 1, false>(X, sx, wq, s_u8, a_u8, sw, Y, nullptr, M, N, K, group, 1, st, offsets, E, max_rows);
        else launch_tile<256, 0, false>(X, sx, wq, s_u8, a_u8, sw, Y, nullptr, M, N, K, group, 1, st, offsets, E, max_rows);
    } else if (max_rows >= kGrouped16Rows) {
        const MfmaPlan p{128, 1, 0, 128};
        return launch_w4a8_mfma16(X, sx, wq, s_u8, a_u8, sw, Y, out_type, M, N, K, group, p,
                                  nullptr, st, offsets, E, max_rows);
    } else {
        if (out_type == 1) launch_tile<128, 1, false>(X, sx, wq, s_u8, a_u8, sw, Y, nullptr, M, N, K, group, 1, st, offsets, E, max_rows);
        else launch_tile<128, 0, false>(X, sx, wq, s_u8, a_u8, sw, Y, nullptr, M, N, K, group, 1, st, offsets, E, max_rows);
    }
    return hipGetLastError();
}

template <class DEC>
static hipError_t run_mfma(const int8_t* X, const float* sx, const uint8_t* wq,
                           const uint8_t* s_u8, const uint8_t* a_u8, const float* sw, void* Y,
                           int out_type, int M, int N, int K, int group, const MfmaPlan& plan,
                           void* workspace, hipStream_t st) {
    int* part = reinterpret_cast<int*>(workspace);
    if (plan.splits == 1) {
        if (plan.mt == 256) {
            if (out_type == 1) launch_tile<256, 1, false, DEC>(X, sx, wq, s_u8, a_u8, sw, Y, part, M, N, K, group, 1, st);
            else launch_tile<256, 0, false, DEC>(X, sx, wq, s_u8, a_u8, sw, Y, part, M, N, K, group, 1, st);
        } else {
            if (out_type == 1) launch_tile<128, 1, false, DEC>(X, sx, wq, s_u8, a_u8, sw, Y, part, M, N, K, group, 1, st);
            else launch_tile<128, 0, false, DEC>(X, sx, wq, s_u8, a_u8, sw, Y, part, M, N, K, group, 1, st);
        }
        return hipGetLastError();
    }
    if (plan.mt == 256)
        launch_tile<256, 1, true, DEC>(X, sx, wq, s_u8, a_u8, sw, Y, part, M, N, K, group, plan.splits, st);
    else
        launch_tile<128, 1, true, DEC>(X, sx, wq, s_u8, a_u8, sw, Y, part, M, N, K, group, plan.splits, st);
    return launch_splitk_reduce(part, plan.splits, M, N, sx, sw, Y, out_type, st);
}

// Kernel choice by plan.mt16: the 16 x 16 x 64 kernel (256-row tiles, 3-6 %
// faster than this one there; or 128-row tiles two per CU for short K), else
// this kernel with 128-row tiles (faster than the 16 x 16 one at that height
// with one workgroup per CU).  Results are the same bit for bit.
hipError_t launch_w4a8_mfma(const int8_t* X, const float* sx, const uint8_t* wq,
                            const uint8_t* s_u8, const uint8_t* a_u8, const float* sw, void* Y,
                            int out_type, int M, int N, int K, int group, const MfmaPlan& plan,
                            void* workspace, hipStream_t st) {
    if (plan.mt16 != 0) {
        MfmaPlan p = plan;
        p.mt = plan.mt16;
        return launch_w4a8_mfma16(X, sx, wq, s_u8, a_u8, sw, Y, out_type, M, N, K, group, p,
                                  workspace, st);
    }
    return run_mfma<DecLQQ>(X, sx, wq, s_u8, a_u8, sw, Y, out_type, M, N, K, group, plan,
                            workspace, st);
}

hipError_t launch_w8a8_mfma(const int8_t* X, const float* sx, const int8_t* wq8, const float* sw,
                            void* Y, int out_type, int M, int N, int K, const MfmaPlan& plan,
                            void* workspace, hipStream_t st) {
    if (plan.mt16 != 0) {  // same kernel choice as the W4A8 GEMM
        MfmaPlan p = plan;
        p.mt = plan.mt16;
        return launch_w8a8_mfma16(X, sx, wq8, sw, Y, out_type, M, N, K, p, workspace, st);
    }
    return run_mfma<DecW8>(X, sx, reinterpret_cast<const uint8_t*>(wq8), nullptr, nullptr, sw, Y,
                           out_type, M, N, K, 128, plan, workspace, st);
}

template <class DEC, bool COARSE>
static void launch_ablation(const int8_t* X, const float* sx, const uint8_t* wq,
                            const uint8_t* s_u8, const uint8_t* a_u8, const float* sw, void* Y,
                            int out_type, int M, int N, int K, int group, int mt, hipStream_t st) {
    if (mt == 256) {
        if (out_type == 1) launch_tile<256, 1, false, DEC, COARSE>(X, sx, wq, s_u8, a_u8, sw, Y, nullptr, M, N, K, group, 1, st);
        else launch_tile<256, 0, false, DEC, COARSE>(X, sx, wq, s_u8, a_u8, sw, Y, nullptr, M, N, K, group, 1, st);
    } else {
        if (out_type == 1) launch_tile<128, 1, false, DEC, COARSE>(X, sx, wq, s_u8, a_u8, sw, Y, nullptr, M, N, K, group, 1, st);
        else launch_tile<128, 0, false, DEC, COARSE>(X, sx, wq, s_u8, a_u8, sw, Y, nullptr, M, N, K, group, 1, st);
    }
}

hipError_t launch_w4a8_mfma_ablation(int variant, const int8_t* X, const float* sx,
                                     const uint8_t* wq, const uint8_t* s_u8, const uint8_t* a_u8,
                                     const float* sw, void* Y, int out_type, int M, int N, int K,
                                     int group, const MfmaPlan& plan, hipStream_t st) {
    // all three decoders on this (32 x 32 x 32) skeleton
    if (variant == 0)
        launch_ablation<DecLQQ, false>(X, sx, wq, s_u8, a_u8, sw, Y, out_type, M, N, K, group,
                                       plan.mt, st);
    else if (variant == 1)
        launch_ablation<DecAffine16, false>(X, sx, wq, s_u8, a_u8, sw, Y, out_type, M, N, K,
                                            group, plan.mt, st);
    else
        launch_ablation<DecLQQ, true>(X, sx, wq, s_u8, a_u8, sw, Y, out_type, M, N, K, group,
                                      plan.mt, st);
    return hipGetLastError();
}

}  // namespace w4a8
