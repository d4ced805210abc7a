// Large-M W4A8 GEMM for gfx950 on v_mfma_i32_16x16x64_i8 (the matrix-core-
// bound regime).  Same method and data flow as the 32 x 32 tile kernel
// (LiquidGEMM, Pith review of arXiv 2509.01229: "What carries the argument"
// and minor comment 1 -- the consumer dequantises what it multiplies, with
// the identity (q*s + a) XOR 0x80 in two VALU instructions per four
// weights), with the 16 x 16 x 64 instruction.  Per operation that shape
// moves less register-file data (a 16 x 16 accumulator is four registers
// against sixteen), and the kernel is power-bound: on random register data
// the 16 x 16 x 64 loop sustains more of the peak than the 32 x 32 x 32 one.
//
// Workgroup tile MT (128 or 256) rows x 256 channels, four waves, each
// owning all MT rows and its 64 channels = packed tiles nt0 .. nt0+3, so a
// weight is dequantised once per workgroup tile.  Lane (r = lane % 16,
// G = lane / 16) of a 16 x 16 block:
//   weight operand B[cb][u] (channel block cb = tile nt0 + cb, half u of the
//     K-step): the lane's 16 packed bytes of the tile hold codes
//     32G .. 32G+31 of row r; decoded, codes 32G + 16u .. +15;
//   X operand (row block rb, half u): X row 16 rb + r, columns
//     32G + 16u .. +15 -- the same K columns, so the two agree whatever the
//     instruction's internal K order;
//   the instruction takes the weights as its first operand and X as its
//   second, so it accumulates (W X^T) blocks: accumulator register v of the
//   lane holds row 16 rb + r, channel 16 cb + 4G + v -- four consecutive
//   channels of one row, which the epilogue writes as one piece.
// One K-step (128 columns) is 8 MT/16 instructions in two groups of half
// the slots (u = 0, 1), each walking row blocks with the four channel
// blocks innermost.  Group 0 decodes B[*][1] of this step from the raw
// weights `wcur`; group 1 loads the step after next into `wcur` and decodes
// the next step's parameters and B[*][0] from `wnx`.  X goes global -> LDS
// directly (three rotating tiles), as in the 32 x 32 kernel.
//
// K parts (KIN = 2, 128-row tiles): the workgroup covers 128 channels, and
// waves 0-1 and 2-3 take the two halves of its K range, each pair with its
// own X tiles; at the end each wave hands its partner the sums of the rows
// the partner writes (exact int32 adds through LDS).  For the shapes that
// would otherwise split K across workgroups, the same grid then needs half
// as many splits, and no partials or second launch when it was two
// (128 x 28672 x 8192: 48.0 -> 42.6 us).
#include <type_traits>

#include "launch.h"
#include "mfma_common.h"

namespace w4a8 {

namespace {

__device__ __forceinline__ void mfma16_i8_acc(v4i& acc, const v4i& a, const v4i& b) {
    asm volatile("v_mfma_i32_16x16x64_i8 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// Raw weights of one K-step for one lane: w[cb] = the lane's 16 bytes of
// tile nt0 + cb; sdw / adw = the lane's panel-row parameter dwords (byte cb
// = scale / offset of tile nt0 + cb, channel r).
struct WRaw16 {
    v4i w[4];
    unsigned sdw, adw;
};

__device__ __forceinline__ void touch_raw16(const WRaw16& w) {
    asm volatile("" ::"v"(w.w[0]), "v"(w.w[1]), "v"(w.w[2]), "v"(w.w[3]), "v"(w.sdw),
                 "v"(w.adw));
}

// W8A8 comparison: raw INT8 weights in the 8-bit tile layout, w[cb][u] =
// the lane's 16 bytes of half u of tile nt0 + cb (already the B operand).
struct WRaw8x16 {
    v4i w[4][2];
};

__device__ __forceinline__ void touch_raw16(const WRaw8x16& w) {
    asm volatile("" ::"v"(w.w[0][0]), "v"(w.w[0][1]), "v"(w.w[1][0]), "v"(w.w[1][1]),
                 "v"(w.w[2][0]), "v"(w.w[2][1]), "v"(w.w[3][0]), "v"(w.w[3][1]));
}

// W8 "decode": one explicit move per dword (OP 0..15: channel block OP / 4,
// dword OP % 4) of B[*][U].
template <int U, int OP>
__device__ __forceinline__ void mov16_step(const WRaw8x16& w, v4i (&B)[4][2]) {
    constexpr int cb = OP / 4, d = OP % 4;
    int x;
    asm volatile("v_mov_b32 %0, %1" : "=v"(x) : "v"(w.w[cb][U][d]));
    B[cb][U][d] = x;
}

struct Par16 {
    unsigned s2[4], a4[4];  // per channel block: scale pair, offset quad
};

// Temporaries of the two packed dwords decoded together (index dd).
struct Tmp16 {
    unsigned lo[2], t[2], hi[2];
};

// Parameter step K_ (0..7): scale pair (even) or offset quad (odd) of
// channel block K_/2.
template <int K_>
__device__ __forceinline__ void par16_step(const WRaw16& w, Par16& p) {
    constexpr int cb = K_ / 2;
    constexpr unsigned b = (unsigned)cb;
    if constexpr (K_ % 2 == 0) {
        constexpr unsigned sel = b | 0x0C00u | (b << 16) | 0x0C000000u;
        asm volatile("v_perm_b32 %0, 0, %1, %2" : "=v"(p.s2[cb]) : "v"(w.sdw), "v"(sel));
    } else {
        asm volatile("v_perm_b32 %0, 0, %1, %2" : "=v"(p.a4[cb]) : "v"(w.adw), "v"(b * 0x01010101u));
    }
}

// Decode step OP (0..55) producing B[*][U]: channel block cb = OP / 14,
// packed dword d = 2U + dd with dd = (OP % 14) % 2, instruction
// st = (OP % 14) / 2:
//   lo = w & 0x0F0F0F0F; t = w >> 4; hi = t & 0x0F0F0F0F;
//   lo = lo*s + a; hi = hi*s + a (two codes per 16-bit lane);
//   B[cb][U] dwords 2dd, 2dd+1 = lo ^ 0x80808080, hi ^ 0x80808080
// The two dwords' steps alternate, so no step reads the result of the one
// just before it (the compiler puts a wait state between two dependent
// assembly statements, not knowing what they are).
template <int U, int OP>
__device__ __forceinline__ void dec16_step(Tmp16& t, const WRaw16& w, const Par16& p,
                                           v4i (&B)[4][2]) {
    constexpr int cb = OP / 14, q = OP % 14, dd = q % 2, st = q / 2;
    constexpr int d = 2 * U + dd;
    const unsigned wd = (unsigned)w.w[cb][d];
    if constexpr (st == 0) {
        asm volatile("v_and_b32 %0, 0x0f0f0f0f, %1" : "=v"(t.lo[dd]) : "v"(wd));
    } else if constexpr (st == 1) {
        asm volatile("v_lshrrev_b32 %0, 4, %1" : "=v"(t.t[dd]) : "v"(wd));
    } else if constexpr (st == 2) {
        asm volatile("v_and_b32 %0, 0x0f0f0f0f, %1" : "=v"(t.hi[dd]) : "v"(t.t[dd]));
    } else if constexpr (st == 3) {
        asm volatile("v_pk_mad_u16 %0, %1, %2, %3"
                     : "=v"(t.lo[dd]) : "v"(t.lo[dd]), "v"(p.s2[cb]), "v"(p.a4[cb]));
    } else if constexpr (st == 4) {
        asm volatile("v_pk_mad_u16 %0, %1, %2, %3"
                     : "=v"(t.hi[dd]) : "v"(t.hi[dd]), "v"(p.s2[cb]), "v"(p.a4[cb]));
    } else if constexpr (st == 5) {
        unsigned x;
        asm volatile("v_xor_b32 %0, 0x80808080, %1" : "=v"(x) : "v"(t.lo[dd]));
        B[cb][U][2 * dd] = (int)x;
    } else {
        unsigned x;
        asm volatile("v_xor_b32 %0, 0x80808080, %1" : "=v"(x) : "v"(t.hi[dd]));
        B[cb][U][2 * dd + 1] = (int)x;
    }
}

template <int RB>
__device__ __forceinline__ void mfma16_drain(v4i (&acc)[RB][4]) {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) asm volatile("" : "+a"(acc[rb][cb]));
    __builtin_amdgcn_sched_barrier(0);
}

}  // namespace

// W8: the W8A8 comparison on this skeleton (no decode, no parameters).
// 128-row tiles fit two workgroups per CU (128 accumulator registers per
// lane, at most 128 others), 256-row tiles one; with K parts (KIN = 2) the
// X tiles take 96 KiB of LDS, one workgroup per CU.
template <int MT, int OUT, int GROUP, bool PARTIAL, bool W8, int KIN>
__global__ __launch_bounds__(256, (MT == 128 && KIN == 1) ? 2 : 1) void w4a8_mfma16_kernel(
    const int8_t* __restrict__ X, const float* __restrict__ sx, const uint8_t* __restrict__ wq,
    const uint8_t* __restrict__ s_u8, const uint8_t* __restrict__ a_u8,
    const float* __restrict__ sw, void* __restrict__ Y, int* __restrict__ part, int M, int N,
    int K, int tiles_n, int tiles_m, int splits, const int* __restrict__ offsets) {
    static_assert(KIN == 1 || (KIN == 2 && MT == 128), "K parts: 128-row tiles only");
    constexpr int RB = MT / 16;        // 16-row blocks per wave
    constexpr int NWX = kWaves / KIN;  // waves per K part (sharing its X tiles)
    constexpr int CPT = MT / (8 * NWX);  // X loads (1 KiB per wave) per K-step
    constexpr int SLOTS = 8 * RB;      // matrix-core instructions per wave per K-step
    constexpr int GS = SLOTS / 2;      // slots per group u
    constexpr int kLoads = W8 ? 8 : 6;  // raw loads per K-step: 4 tiles, s, a (W8: 8 halves)
    constexpr int NOPS = W8 ? 16 : 56;  // decode steps per group
    constexpr int NPAR = W8 ? 0 : 8;    // parameter steps
    constexpr int DQ0 = (NOPS + GS - 1) / GS;         // group-0 decode steps per slot
    constexpr int DQ1 = (NPAR + NOPS + GS - 1) / GS;  // group-1 parameter + decode steps per slot
    using Raw = std::conditional_t<W8, WRaw8x16, WRaw16>;
    constexpr unsigned XB = MT * 128;     // bytes of one X tile
    constexpr unsigned XSTEP = KIN * XB;  // one K-step's X tiles, one per K part
    __shared__ __attribute__((aligned(1024))) uint8_t xs[3 * XSTEP];
    __shared__ float sxs[MT];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15, G = lane >> 4;
    const int kp = wave / NWX;  // K part of this wave
    const int wc = wave % NWX;  // its 64-channel panel within the workgroup

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
        wq += (size_t)e * N * (W8 ? K : K / 2);
        s_u8 += (size_t)e * N * (K / GROUP);
        a_u8 += (size_t)e * N * (K / GROUP);
        sw += (size_t)e * N;
    }
    const int m0 = row_lo + tc.tm * MT;
    if (m0 >= row_hi) return;  // whole workgroup: no rows of this expert here
    const int n0 = tc.tn * (kNT / KIN) + wc * kColsPerWave;
    const int KTall = K / kTileK;
    // K is cut into splits * KIN parts; this wave takes part ks * KIN + kp
    const int parts = splits * KIN;
    const int pidx = ks * KIN + kp;
    const int kt0 = (int)((long long)KTall * pidx / parts);
    const int KT = (int)((long long)KTall * (pidx + 1) / parts) - kt0;  // >= 1
    // Every wave of the workgroup runs the same number of K-steps (one
    // barrier per step): the longest part's, in pairs with a single loop
    // exit.  Steps past a wave's own part read an X tile of zeros (their
    // weights are the part's last real step's, so no load leaves the part's
    // K range).
    int KTmax = KT;
    if constexpr (KIN == 2) {
        const int q0 = ks * KIN;
        const int a0 = (int)((long long)KTall * q0 / parts);
        const int a1 = (int)((long long)KTall * (q0 + 1) / parts);
        const int a2 = (int)((long long)KTall * (q0 + 2) / parts);
        KTmax = max(a1 - a0, a2 - a1);
    }
    const int KTe = KTmax + (KTmax & 1);
    const int groups = K / GROUP;

    // ---- X straight into LDS (same tile format and load mapping as the
    // 32 x 32 kernel): the X tile of K part kp is filled by its NWX waves;
    // load p of panel wave wc fills rows 8 (NWX p + wc) .. +7, lane l writing
    // slot l % 8 of row 8 (NWX p + wc) + l / 8 from that row's chunk
    // (l % 8) ^ xswz(row & 15).
    const __amdgpu_buffer_rsrc_t xr_rsrc = buf_rsrc(X, (unsigned)M * (unsigned)K);
    const int xr = 8 * wc + (lane >> 3);
    const int xc = (lane & 7) ^ xswz(xr & 15);
    const unsigned xvoff =
        (unsigned)(m0 + xr) * (unsigned)K + (unsigned)(xc * 16) + (unsigned)(kt0 * kTileK);
    const unsigned xrowstep = 8u * NWX * (unsigned)K;
    const unsigned xsbase = lds_addr(xs) + (unsigned)kp * XB;
    auto x_load = [&](int kt, int p, unsigned buf) {
        const bool live = kt < KT;  // kt >= KT: offset past the buffer, reads 0
        const unsigned vo = live ? xvoff + (unsigned)p * xrowstep : 0xFFFFFFF0u;
        const unsigned so = live ? (unsigned)(kt * kTileK) : 0u;
        buf_load16_lds(xr_rsrc, vo, so, xsbase + buf + (unsigned)(NWX * p + wc) * 1024u);
    };
    // A operand (row block rb, half u): row 16 rb + r, chunk 2G + u.
    int aoff[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) aoff[u] = r * 128 + (((2 * G + u) ^ xswz(r)) * 16);

    // ---- weights of this wave: tiles nt0 .. nt0+3 (one parameter panel)
    const int nt0 = n0 / kTileN;
    const __amdgpu_buffer_rsrc_t w_rsrc = buf_rsrc(wq, (unsigned)((size_t)N * K / (W8 ? 1 : 2)));
    const __amdgpu_buffer_rsrc_t s_rsrc = buf_rsrc(s_u8, (unsigned)((size_t)N * K / GROUP));
    const __amdgpu_buffer_rsrc_t a_rsrc = buf_rsrc(a_u8, (unsigned)((size_t)N * K / GROUP));
    const unsigned wvoff = (unsigned)lane * 16u;
    // the lane's 32 K columns lie in the K-step's group G / 2 when GROUP = 64
    const unsigned pvoff = 4u * (unsigned)r + (GROUP == 64 ? 64u * (unsigned)(G >> 1) : 0u);
    const unsigned ppanel = 64u * (unsigned)(n0 >> 6) * (unsigned)groups;
    auto w_load = [&](int kt, int part_i, Raw& ws) {  // part_i < kLoads
        const int ktg = kt0 + kt;
        if constexpr (W8) {  // 8-bit layout: 2 KiB tiles, halves 1 KiB apart
            const int cb = part_i >> 1, u = part_i & 1;
            ws.w[cb][u] = buf_load16(
                w_rsrc, wvoff, (unsigned)(((nt0 + cb) * KTall + ktg) * 2048 + 1024 * u));
        } else if (part_i < 4) {
            ws.w[part_i] = buf_load16(
                w_rsrc, wvoff, (unsigned)(((nt0 + part_i) * KTall + ktg) * kTileBytes));
        } else {
            const unsigned jo = ppanel + 64u * (unsigned)(ktg * (kTileK / GROUP));
            if (part_i == 4) ws.sdw = buf_load4(s_rsrc, pvoff, jo);
            else ws.adw = buf_load4(a_rsrc, pvoff, jo);
        }
    };

    v4i acc[RB][4];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = v4i{0, 0, 0, 0};

    // ---- prologue: X(0), X(1) -> LDS tiles 0, 1; parameters and B[*][0]
    // of W(0); W(1) raw; A ring primed with step 0's first two operands.
    Raw we, wo;     // raw weights for even / odd steps
    Par16 pp;       // parameters of the raw set being decoded
    v4i B[4][2];
    v4i ring[4];
    const int k1 = min(1, KTe - 1), kw1 = min(1, KT - 1);
    unsigned bc = 0, bn = XSTEP, bd = 2 * XSTEP;  // LDS tiles of X(kt), X(kt+1), X(kt+2)
#pragma unroll
    for (int p = 0; p < CPT; ++p) x_load(0, p, bc);
#pragma unroll
    for (int p = 0; p < CPT; ++p) x_load(k1, p, bn);
#pragma unroll
    for (int pi = 0; pi < kLoads; ++pi) w_load(0, pi, we);
#pragma unroll
    for (int pi = 0; pi < kLoads; ++pi) w_load(kw1, pi, wo);
    if constexpr (W8) {
        static_for<16>([&](auto k) { mov16_step<0, decltype(k)::value>(we, B); });
    } else {
        Tmp16 t;
        static_for<8>([&](auto k) { par16_step<decltype(k)::value>(we, pp); });
        static_for<56>([&](auto k) { dec16_step<0, decltype(k)::value>(t, we, pp, B); });
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(kLoads, 0));  // X(0), X(1), W(0) complete
    __syncthreads();
    const uint8_t* xsk = xs + kp * XB;  // this K part's X tiles
    auto read_a = [&](unsigned buf, int sI) {  // sI = RB*u + rb
        return *reinterpret_cast<const v4i*>(xsk + buf + (sI % RB) * 2048 + aoff[sI / RB]);
    };
    ring[0] = read_a(bc, 0);
    ring[1] = read_a(bc, 1);

    // ---- one K-step.  Slot s: group u = s / GS, row block rb = (s % GS) / 4,
    // channel block cb = s % 4; operand index sI = RB*u + rb (ring sI % 4,
    // read two row blocks ahead at the row block's first slot).
    //   group 0 slots      B[*][1] of step kt from wcur (parameters pp)
    //   group 1 slot GS    W(kt+2) -> wcur begins; all of wnx waited for
    //   group 1 slots      parameters of wnx, B[*][0] of step kt+1
    //   slots XS ..        X(kt+2) -> LDS tile `dst` (after the wait on wnx:
    //                      the compiler does not see these loads)
    //   before the last 4  wait for this wave's X(kt+1) loads (CPT + kLoads
    //                      loads were issued after them), barrier, then the
    //                      next step's first two A reads.
    constexpr int XS = GS + kLoads;
    static_assert(XS + CPT <= SLOTS - 4, "X loads must precede the barrier");
    auto step = [&](int kt, unsigned cur, unsigned nxt, unsigned dst, Raw& wcur, Raw& wnx) {
        const int k2 = min(kt + 2, KTe - 1), kw2 = min(kt + 2, KT - 1);
        Tmp16 tmp;
        static_for<SLOTS>([&](auto sc) {
            constexpr int s = decltype(sc)::value;
            constexpr int u = s / GS, q = s % GS, rb = q / 4, cb = q % 4;
            constexpr int sI = RB * u + rb;
            if constexpr (s == SLOTS - 4) {
                __builtin_amdgcn_sched_barrier(0);
                __builtin_amdgcn_s_waitcnt(waitcnt_imm(CPT + kLoads, 0));
                __syncthreads();
                ring[0] = read_a(nxt, 0);
                ring[1] = read_a(nxt, 1);
            }
            mfma16_i8_acc(acc[rb][cb], B[cb][u], ring[sI % 4]);
            if constexpr (cb == 0 && sI + 2 < 2 * RB) ring[(sI + 2) % 4] = read_a(cur, sI + 2);
            if constexpr (s >= GS && s < GS + kLoads) w_load(kw2, s - GS, wcur);
            if constexpr (s == GS) touch_raw16(wnx);
            if constexpr (s >= XS && s < XS + CPT) x_load(k2, s - XS, dst);
            if constexpr (u == 0) {
                static_for<DQ0>([&](auto dc) {
                    constexpr int o = DQ0 * q + decltype(dc)::value;
                    if constexpr (o < NOPS) {
                        if constexpr (W8) mov16_step<1, o>(wcur, B);
                        else dec16_step<1, o>(tmp, wcur, pp, B);
                    }
                });
            } else {
                static_for<DQ1>([&](auto dc) {
                    constexpr int o = DQ1 * q + decltype(dc)::value;
                    if constexpr (W8) {
                        if constexpr (o < NOPS) mov16_step<0, o>(wnx, B);
                    } else {
                        if constexpr (o < NPAR) par16_step<o>(wnx, pp);
                        else if constexpr (o - NPAR < NOPS) dec16_step<0, o - NPAR>(tmp, wnx, pp, B);
                    }
                });
            }
        });
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
    mfma16_drain(acc);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));  // the last steps' X loads
    __syncthreads();  // all waves done with the X tiles

    // ---- epilogue.  Accumulator (rb, cb) register v of lane (r, G): row
    // 16 rb + r, channel n0 + 16 cb + 4G + v.  Two row blocks at a time go to
    // a per-wave LDS block [32 rows][64 channels] -- each lane writes its four
    // consecutive channels as one 8-byte (fp16) or 16-byte (int32) piece, rows
    // padded by 16 bytes so a write touches distinct banks -- and each row is
    // then written to memory as whole 16-byte pieces of one 128-byte segment
    // (final output, or this split's int32 partial).
    constexpr bool SCALED = (OUT == 0) && !PARTIAL;
    if (SCALED) sxs[tid % MT] = (m0 + tid % MT < row_hi) ? sx[m0 + tid % MT] : 0.0f;
    float swv[4][4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int v = 0; v < 4; ++v) swv[cb][v] = SCALED ? sw[n0 + 16 * cb + 4 * G + v] : 0.0f;
    // K parts: the two waves of a channel panel hold sums over the two K
    // halves.  Part kp writes row blocks [kp HB, kp HB + HB): each wave first
    // stores its sums of the other half's row blocks to LDS (block (receiving
    // part, panel, row block, channel block) of 64 lanes x 16 bytes), then,
    // after the barrier, adds its partner's sums of its own into `fin`.  Row
    // blocks are chosen by a select on kp (uniform), so every accumulator
    // index stays a constant and both parts share one code path.
    constexpr int HB = RB / 2;
    constexpr int FB = KIN == 2 ? HB : 1;
    v4i fin[FB][4];
    if constexpr (KIN == 2) {
        static_assert(KIN * NWX * HB * 4 * 1024 <= 3 * XSTEP, "K-part exchange fits in LDS");
        v4i* xch = reinterpret_cast<v4i*>(xs);
        auto xidx = [&](int d, int i, int cb) {
            return ((d * NWX + wc) * HB * 4 + i * 4 + cb) * 64 + lane;
        };
        const bool hi = kp != 0;
#pragma unroll
        for (int i = 0; i < HB; ++i)
#pragma unroll
            for (int cb = 0; cb < 4; ++cb)
                xch[xidx(1 - kp, i, cb)] = hi ? acc[i][cb] : acc[HB + i][cb];
        __syncthreads();
#pragma unroll
        for (int i = 0; i < HB; ++i)
#pragma unroll
            for (int cb = 0; cb < 4; ++cb)
                fin[i][cb] = (hi ? acc[HB + i][cb] : acc[i][cb]) + xch[xidx(kp, i, cb)];
    }
    __syncthreads();  // sxs written; the exchange blocks read before staging reuses them
    constexpr int EB = SCALED ? 2 : 4;  // output element bytes
    constexpr int ROWB = 64 * EB;       // bytes per row of the block
    constexpr int RSTR = ROWB + 16;     // padded row stride in LDS
    static_assert(kWaves * 32 * RSTR <= 3 * XSTEP, "epilogue staging fits in the X tiles");
    uint8_t* stage = xs + wave * (32 * RSTR);
    uint8_t* out = PARTIAL ? reinterpret_cast<uint8_t*>(part + (size_t)ks * M * N)
                           : reinterpret_cast<uint8_t*>(Y);
    // Row-block pairs 0 .. NP-1 from row r0 of the tile on; value(rb, cb) is
    // the sum of local row block rb, channel block cb.
    auto epi = [&](auto npc, int r0, auto value) {
        constexpr int NP = decltype(npc)::value;
#pragma unroll
        for (int rp = 0; rp < NP; ++rp) {
#pragma unroll
            for (int rr = 0; rr < 2; ++rr) {
                const int rb = 2 * rp + rr;
                uint8_t* srow = stage + (16 * rr + r) * RSTR;
                const float sm = SCALED ? sxs[r0 + 16 * rb + r] : 0.0f;
#pragma unroll
                for (int cb = 0; cb < 4; ++cb) {
                    const int col = 16 * cb + 4 * G;
                    const v4i a = value(rb, cb);
                    if constexpr (SCALED) {
                        unsigned short h[4];
#pragma unroll
                        for (int v = 0; v < 4; ++v)
                            h[v] = f32_to_f16_bits(((float)a[v] * sm) * swv[cb][v]);
                        uint2 pk;
                        pk.x = h[0] | ((unsigned)h[1] << 16);
                        pk.y = h[2] | ((unsigned)h[3] << 16);
                        *reinterpret_cast<uint2*>(srow + col * 2) = pk;
                    } else {
                        *reinterpret_cast<v4i*>(srow + col * 4) = a;
                    }
                }
            }
            __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes done
            __builtin_amdgcn_wave_barrier();
            constexpr int PPR = ROWB / 16;  // 16-byte pieces per row
#pragma unroll
            for (int w = 0; w < 32 * PPR / 64; ++w) {
                const int q = lane + 64 * w;
                const int row = q / PPR, piece = q % PPR;
                const int m = m0 + r0 + 32 * rp + row;
                const v4i val = *reinterpret_cast<const v4i*>(stage + row * RSTR + piece * 16);
                if (m < row_hi)
                    store16_result<PARTIAL>(out + ((size_t)m * N + n0) * EB + piece * 16, val);
            }
            __builtin_amdgcn_s_waitcnt(0xc07f);
            __builtin_amdgcn_wave_barrier();
        }
    };
    if constexpr (KIN == 1)
        epi(std::integral_constant<int, RB / 2>{}, 0,
            [&](int rb, int cb) { return acc[rb][cb]; });
    else
        epi(std::integral_constant<int, HB / 2>{}, 16 * HB * kp,
            [&](int rb, int cb) { return fin[rb][cb]; });
}

template <int MT, int OUT, bool PARTIAL, bool W8, int KIN = 1>
static void launch_tile16(const int8_t* X, const float* sx, const uint8_t* wq,
                          const uint8_t* s_u8, const uint8_t* a_u8, const float* sw, void* Y,
                          int* part, int M, int N, int K, int group, int splits, hipStream_t st,
                          const int* offsets, int E, int max_rows) {
    const int tiles_n = N / (kNT / KIN);
    const int tiles_m = ((offsets ? max_rows : M) + MT - 1) / MT;
    dim3 grid(tiles_n * tiles_m * splits, offsets ? E : 1), block(256);
    if (group == 64 && !W8)
        hipLaunchKernelGGL((w4a8_mfma16_kernel<MT, OUT, 64, PARTIAL, W8, KIN>), grid, block, 0,
                           st, X, sx, wq, s_u8, a_u8, sw, Y, part, M, N, K, tiles_n, tiles_m,
                           splits, offsets);
    else
        hipLaunchKernelGGL((w4a8_mfma16_kernel<MT, OUT, 128, PARTIAL, W8, KIN>), grid, block, 0,
                           st, X, sx, wq, s_u8, a_u8, sw, Y, part, M, N, K, tiles_n, tiles_m,
                           splits, offsets);
}

template <bool W8>
static hipError_t run_mfma16(const int8_t* X, const float* sx, const uint8_t* wq,
                             const uint8_t* s_u8, const uint8_t* a_u8, const float* sw, void* Y,
                             int out_type, int M, int N, int K, int group, const MfmaPlan& plan,
                             void* workspace, hipStream_t st, const int* offsets, int E,
                             int max_rows) {
    int* part = reinterpret_cast<int*>(workspace);
    if (plan.kin == 2) {  // 128-row tiles, no grouped problems
        if (plan.splits == 1) {
            if (out_type == 1)
                launch_tile16<128, 1, false, W8, 2>(X, sx, wq, s_u8, a_u8, sw, Y, part, M, N, K,
                                                    group, 1, st, nullptr, 1, 0);
            else
                launch_tile16<128, 0, false, W8, 2>(X, sx, wq, s_u8, a_u8, sw, Y, part, M, N, K,
                                                    group, 1, st, nullptr, 1, 0);
            return hipGetLastError();
        }
        launch_tile16<128, 1, true, W8, 2>(X, sx, wq, s_u8, a_u8, sw, Y, part, M, N, K, group,
                                           plan.splits, st, nullptr, 1, 0);
        return launch_splitk_reduce(part, plan.splits, M, N, sx, sw, Y, out_type, st);
    }
    if (plan.splits == 1) {
#define T16(MT_, O_) \
    launch_tile16<MT_, O_, false, W8>(X, sx, wq, s_u8, a_u8, sw, Y, part, M, N, K, group, 1, st, \
                                      offsets, E, max_rows)
        if (plan.mt == 256) {
            if (out_type == 1) T16(256, 1);
            else T16(256, 0);
        } else {
            if (out_type == 1) T16(128, 1);
            else T16(128, 0);
        }
#undef T16
        return hipGetLastError();
    }
    if (plan.mt == 256)
        launch_tile16<256, 1, true, W8>(X, sx, wq, s_u8, a_u8, sw, Y, part, M, N, K, group,
                                        plan.splits, st, nullptr, 1, 0);
    else
        launch_tile16<128, 1, true, W8>(X, sx, wq, s_u8, a_u8, sw, Y, part, M, N, K, group,
                                        plan.splits, st, nullptr, 1, 0);
    return launch_splitk_reduce(part, plan.splits, M, N, sx, sw, Y, out_type, st);
}

hipError_t launch_w4a8_mfma16(const int8_t* X, const float* sx, const uint8_t* wq,
                              const uint8_t* s_u8, const uint8_t* a_u8, const float* sw, void* Y,
                              int out_type, int M, int N, int K, int group, const MfmaPlan& plan,
                              void* workspace, hipStream_t st, const int* offsets, int E,
                              int max_rows) {
    return run_mfma16<false>(X, sx, wq, s_u8, a_u8, sw, Y, out_type, M, N, K, group, plan,
                             workspace, st, offsets, E, max_rows);
}

hipError_t launch_w8a8_mfma16(const int8_t* X, const float* sx, const int8_t* wq8,
                              const float* sw, void* Y, int out_type, int M, int N, int K,
                              const MfmaPlan& plan, void* workspace, hipStream_t st) {
    return run_mfma16<true>(X, sx, reinterpret_cast<const uint8_t*>(wq8), nullptr, nullptr, sw,
                            Y, out_type, M, N, K, 128, plan, workspace, st, nullptr, 1, 0);
}

}  // namespace w4a8
