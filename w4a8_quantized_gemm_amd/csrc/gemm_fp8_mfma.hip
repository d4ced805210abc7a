// Large-M W4FP8 GEMM for gfx950: INT4 weights (sign-magnitude nibbles, per
// output channel scale) converted to FP8 e4m3 in registers, multiplied with
// e4m3 activations on the matrix cores with float32 accumulation (the
// INT4-FP8 scheme of FireQ, arXiv 2505.20839, abstract); epilogue
// Y = bf16((acc * sx[m]) * sw[n]) or float32.
//
// Same skeleton as the W4A8 tile kernel: workgroup tile MT (128 or 256)
// rows x 256 channels, four waves of MT x 64, X global -> LDS directly
// (three rotating tiles, swizzled 16-byte slots), weights loaded two K-steps
// ahead and converted in single instructions interleaved with the matrix-
// core instructions.  Per 128-column K-step and 32 x 32 block there are two
// v_mfma_f32_32x32x64_f8f6f4 (e4m3 x e4m3): instruction j of lane
// (c = lane % 32, h = lane / 32) takes K columns 64h + 32j .. +31, which is
// packed slot 2h + j of the lane's weight row (32 consecutive codes, low
// nibble of byte i = code 8d+i, high nibble = code 8d+4+i for dword d) and
// 16-byte X chunks 4h + 2j, 4h + 2j + 1 of the lane's row.
//
// |q| <= 7 is exact in e4m3; conversion of one packed dword (8 codes) is 8
// VALU instructions: magnitude mask, byte permute through the 8-entry e4m3
// table, sign moved to bit 7 -- for the low nibbles (sign at bit 3) and the
// high nibbles (sign already at bit 7).
//
// GROUP = 64 or 128 selects the folded per-group format (per-group scale
// folded into the FP8 weights, per-tensor rescale; FireQ abstract): the
// table then holds e4m3(|q| f) for the lane's channel and group, rebuilt
// every K-step from the folded factor f (six multiplies and four packed
// conversions per 32-channel block), and the epilogue scales by the tensor
// scale t instead of sw[n].  One K-step of a lane lies in one group for
// both group sizes (lane half h selects the 64-column group).
#include "launch.h"
#include "mfma_common.h"

namespace w4a8 {

namespace {

__device__ __forceinline__ void mfma32_f8_acc(v16f& acc, const v8i& a, const v8i& b) {
    asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// Raw weights of one K-step for one lane: w[cb][j] = slot 2h+j of the lane's
// row in tile 2cb + c/16.
struct F8Step {
    v4i w[2][2];
};

// e4m3 magnitudes of 0..7 as two byte tables for v_perm_b32 (bytes 0..3 in
// `lo`, 4..7 in `hi`), one table per 32-channel block cb; kept in registers
// (one VOP3 reads one scalar only).
struct F8Lut {
    unsigned lo[2], hi[2];
};

struct F8Tmp {  // the two dwords converted together (index h)
    unsigned m[2], e[2], s[2];
};

// Producing operand B[cb][j] of a K-step is 32 single-instruction steps:
// for cb in {0,1}, for the slot's four dwords d:
//   m = w & 0x07070707; e = perm(table, m); s = w & 0x08080808;
//   B[2d] = (s << 4) | e                               (low nibbles)
//   t = w >> 4; m = t & 0x07070707; e = perm(table, m);
//   B[2d+1] = (w & 0x80808080) | e                      (high nibbles)
// Dwords go in pairs (d = 2 (q / 16) + h) whose steps alternate, so no
// step reads the result of the one just before it (the compiler puts a wait
// state between two dependent assembly statements, not knowing what they
// are).
template <int J, int OP>
__device__ __forceinline__ void f8_step(F8Tmp& t, const F8Step& w, const F8Lut& lut,
                                        unsigned sgn, v8i (&B)[2][2]) {
    constexpr int cb = OP / 32, q = OP % 32, h = q % 2, d = 2 * (q / 16) + h, st = (q % 16) / 2;
    const unsigned wd = (unsigned)w.w[cb][J][d];
    if constexpr (st == 0) {
        asm volatile("v_and_b32 %0, 0x07070707, %1" : "=v"(t.m[h]) : "v"(wd));
    } else if constexpr (st == 1) {
        asm volatile("v_perm_b32 %0, %1, %2, %3"
                     : "=v"(t.e[h])
                     : "v"(lut.hi[cb]), "v"(lut.lo[cb]), "v"(t.m[h]));
    } else if constexpr (st == 2) {
        asm volatile("v_and_b32 %0, 0x08080808, %1" : "=v"(t.s[h]) : "v"(wd));
    } else if constexpr (st == 3) {
        unsigned x;
        asm volatile("v_lshl_or_b32 %0, %1, 4, %2" : "=v"(x) : "v"(t.s[h]), "v"(t.e[h]));
        B[cb][J][2 * d] = (int)x;
    } else if constexpr (st == 4) {
        asm volatile("v_lshrrev_b32 %0, 4, %1" : "=v"(t.m[h]) : "v"(wd));
    } else if constexpr (st == 5) {
        asm volatile("v_and_b32 %0, 0x07070707, %1" : "=v"(t.m[h]) : "v"(t.m[h]));
    } else if constexpr (st == 6) {
        asm volatile("v_perm_b32 %0, %1, %2, %3"
                     : "=v"(t.e[h])
                     : "v"(lut.hi[cb]), "v"(lut.lo[cb]), "v"(t.m[h]));
    } else {
        unsigned x;
        asm volatile("v_and_or_b32 %0, %1, %2, %3" : "=v"(x) : "v"(wd), "v"(sgn), "v"(t.e[h]));
        B[cb][J][2 * d + 1] = (int)x;
    }
}

template <int J>
__device__ __forceinline__ void f8_all(const F8Step& w, const F8Lut& lut, unsigned sgn,
                                       v8i (&B)[2][2]) {
    F8Tmp t;
    static_for<64>([&](auto oc) { f8_step<J, decltype(oc)::value>(t, w, lut, sgn, B); });
}

}  // namespace

// 128-row tiles fit two workgroups per CU (128 accumulator and at most 128
// other registers per lane), 256-row tiles one.
template <int MT, int OUT, bool PARTIAL, int GROUP>
__global__ __launch_bounds__(256, MT == 128 ? 2 : 1) void w4fp8_mfma_kernel(
    const uint8_t* __restrict__ X, const float* __restrict__ sx, const uint8_t* __restrict__ wq,
    const float* __restrict__ sw, const float* __restrict__ fsc, const float* __restrict__ tsc,
    void* __restrict__ Y, float* __restrict__ part, int M, int N, int K, int tiles_n,
    int tiles_m, int splits) {
    constexpr bool FOLD = GROUP != 0;
    constexpr int RB = MT / 32;        // 32-row blocks per wave
    constexpr int CPT = MT / 32;       // 16-byte X chunks per thread per K-step
    constexpr int SLOTS = 4 * RB;      // matrix-core instructions per wave per K-step
    constexpr int GS = SLOTS / 2;      // slots per instruction group j
    constexpr int DQ = (64 + GS - 1) / GS;  // conversion steps per slot
    constexpr unsigned XB = MT * 128;  // bytes of one X tile (MT rows x 128 K)
    __shared__ __attribute__((aligned(1024))) uint8_t xs[3 * XB];  // X(kt), X(kt+1), X(kt+2)
    __shared__ float sxs[MT];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int c = lane & 31, h = lane >> 5;
    const int tb = c >> 4, r = c & 15;

    const TileCoord tcd = tile_coord(blockIdx.x, tiles_m, tiles_n, splits);
    const int ks = tcd.ks;
    const int m0 = tcd.tm * MT;
    const int n0 = tcd.tn * kNT + wave * kColsPerWave;
    const int KTall = K / kTileK;
    const int kt0 = (int)((long long)KTall * ks / splits);
    const int KT = (int)((long long)KTall * (ks + 1) / splits) - kt0;  // >= 1
    // The main loop runs K-steps in pairs with a single exit; an odd count
    // gets one more step whose X tile reads as zero (contributing exactly 0).
    const int KTe = KT + (KT & 1);

    // ---- X goes from global memory straight into one of three LDS tiles.
    // Tile row R keeps its 16-byte column chunk k in slot k ^ xswz(R & 15).
    // Wave w's load p (p < CPT) fills rows 32p + 8w .. +7: lane l writes
    // slot l % 8 of row 32p + 8w + l / 8, so it fetches that row's chunk
    // (l % 8) ^ xswz(row & 15).  Rows >= M lie past the end of the buffer
    // and read as 0.
    const __amdgpu_buffer_rsrc_t xr_rsrc = buf_rsrc(X, (unsigned)M * (unsigned)K);
    const int xr = 8 * wave + (lane >> 3);
    const int xc = (lane & 7) ^ xswz(xr & 15);
    const unsigned xvoff =
        (unsigned)(m0 + xr) * (unsigned)K + (unsigned)(xc * 16) + (unsigned)(kt0 * kTileK);
    const unsigned xrowstep = 32u * (unsigned)K;
    const unsigned xsbase = lds_addr(xs);
    // A operand of instruction group j: row 32rb + c, chunks 4h+2j, 4h+2j+1.
    int aoff[2][2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int u = 0; u < 2; ++u) aoff[j][u] = c * 128 + (((4 * h + 2 * j + u) ^ xswz(r)) * 16);

    // ---- weights of this wave: tiles n0/16 .. n0/16+3
    const int nt0 = n0 / kTileN;
    const __amdgpu_buffer_rsrc_t w_rsrc = buf_rsrc(wq, (unsigned)((size_t)N * K / 2));
    const unsigned wvoff = (unsigned)(tb * KTall) * kTileBytes + (unsigned)(32 * h + r) * 16u;
    auto w_load = [&](int kt, int part_i, F8Step& ws) {  // part_i 0..3
        const int ktg = kt0 + kt;
        const int cb = part_i >> 1, j = part_i & 1;
        ws.w[cb][j] = buf_load16(
            w_rsrc, wvoff, (unsigned)(((nt0 + 2 * cb) * KTall + ktg) * kTileBytes + j * 256));
    };
    auto x_load = [&](int kt, int p, unsigned buf) {  // into LDS tile at byte `buf`
        const bool live = kt < KT;  // kt >= KT: offset past the buffer, reads 0
        const unsigned vo = live ? xvoff + (unsigned)p * xrowstep : 0xFFFFFFF0u;
        const unsigned so = live ? (unsigned)(kt * kTileK) : 0u;
        buf_load16_lds(xr_rsrc, vo, so, xsbase + buf + (unsigned)(4 * p + wave) * 1024u);
    };
    // Folded factors, group-major fsc[g][N]: K-step ktg of channel n lies in
    // group ktg * (128 / GROUP) + (GROUP == 64 ? h : 0).
    constexpr int GPS = FOLD ? 128 / GROUP : 1;  // groups per K-step
    const __amdgpu_buffer_rsrc_t f_rsrc =
        buf_rsrc(fsc, FOLD ? (unsigned)((size_t)KTall * GPS * N * 4) : 0u);
    const unsigned fvoff = (unsigned)(n0 + c) * 4u + (GROUP == 64 ? (unsigned)h * N * 4u : 0u);
    auto f_load = [&](int kt, float (&fv)[2]) {
        const unsigned so = (unsigned)((kt0 + kt) * GPS) * (unsigned)N * 4u;
        fv[0] = __builtin_bit_cast(float, buf_load4(f_rsrc, fvoff, so));
        fv[1] = __builtin_bit_cast(float, buf_load4(f_rsrc, fvoff + 128u, so));
    };
    const unsigned sgn = 0x80808080u;
    F8Lut le, lo;  // tables of even / odd K-steps
    float fe[2] = {0.f, 0.f}, fo[2] = {0.f, 0.f};
    if constexpr (!FOLD) {
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
            le.lo[cb] = lo.lo[cb] = 0x44403800u;  // e4m3 of 3, 2, 1, 0
            le.hi[cb] = lo.hi[cb] = 0x4E4C4A48u;  // e4m3 of 7, 6, 5, 4
        }
    }

    v16f acc[RB][2];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        acc[rb][0] = v16f{};
        acc[rb][1] = v16f{};
    }

    // ---- prologue: X(0), X(1) -> LDS tiles 0, 1; B[*][0] of step 0
    // converted, W(0) kept raw for B[*][1], W(1) raw; A ring primed.
    F8Step we, wo;         // raw weights for even / odd steps
    v8i B[2][2];
    v8i ring[4];
    // X of the padding step reads as zero; its weights (and factors) are
    // those of the last real step, so no load leaves this split's K range.
    const int k1 = min(1, KTe - 1), kw1 = min(1, KT - 1);
    unsigned bc = 0, bn = XB, bd = 2 * XB;  // LDS tiles of X(kt), X(kt+1), X(kt+2)
#pragma unroll
    for (int p = 0; p < CPT; ++p) x_load(0, p, bc);
#pragma unroll
    for (int p = 0; p < CPT; ++p) x_load(k1, p, bn);
    if constexpr (FOLD) {
        f_load(0, fe);
        f_load(kw1, fo);
    }
#pragma unroll
    for (int pi = 0; pi < 4; ++pi) w_load(0, pi, we);
#pragma unroll
    for (int pi = 0; pi < 4; ++pi) w_load(kw1, pi, wo);
    if constexpr (FOLD) {
        e4m3_fold_table(fe[0], le.lo[0], le.hi[0]);
        e4m3_fold_table(fe[1], le.lo[1], le.hi[1]);
    }
    f8_all<0>(we, le, sgn, B);
    // X(0) and X(1) were issued first: once at most the W(1) loads are
    // outstanding, every wave's part of the two X tiles is in LDS.
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(4, 0));
    __syncthreads();
    auto read_a = [&](unsigned buf, int sI) {  // sI = RB*j + rb
        const int j = sI / RB, rb = sI % RB;
        const v4i lo = *reinterpret_cast<const v4i*>(xs + buf + rb * 4096 + aoff[j][0]);
        const v4i hi = *reinterpret_cast<const v4i*>(xs + buf + rb * 4096 + aoff[j][1]);
        return v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    };
    ring[0] = read_a(bc, 0);
    ring[1] = read_a(bc, 1);

    // ---- one K-step, SLOTS matrix-core slots.  Slot s: group j = s / GS,
    // row block rb = (s/2) % RB, channel block cb = s % 2.  Entering step
    // kt: LDS tile `cur` = X(kt), `nxt` = X(kt+1) (loads possibly in
    // flight), `dst` free (X(kt-1), last read before the previous barrier);
    // ring holds A for the first two operand slots; B[*][0] = W(kt)
    // operands; `wcur` = raw W(kt), `wnx` = raw W(kt+1).
    //   group 0 slots      B[*][1] of step kt from wcur
    //   group 1 slots      W(kt+2) -> wcur; B[*][0] of step kt+1 from wnx
    //   CPT slots from XS  X(kt+2) -> LDS `dst`, after this step's first use
    //                      of wnx (the compiler does not see these loads, so
    //                      its wait before that use covers only older ones);
    //                      with 128-row tiles some follow the barrier
    //   before the last 4  wait for this wave's X(kt+1) loads, barrier, then
    //                      step kt+1's first two A reads.
    // Folded format: `lcur` = table of step kt (group 0), `lnx` = table of
    // step kt+1 (group 1), built from `fnx` in the last two group-0 slots;
    // f(kt+2) -> `fcur` at slot 0.
    constexpr int XS = GS + 4;  // first X load slot
    static_assert(XS + CPT <= SLOTS, "X loads fit in the step");
    // Loads issued after a step's last X load, up to the next step's
    // barrier: that step's factor, weight and pre-barrier X loads.
    constexpr int XPRE = (SLOTS - 4 - XS) < 0 ? 0 : ((SLOTS - 4 - XS) > CPT ? CPT : (SLOTS - 4 - XS));
    constexpr int XWAIT = (FOLD ? 2 : 0) + 4 + XPRE;
    auto step = [&](int kt, unsigned cur, unsigned nxt, unsigned dst, F8Step& wcur, F8Step& wnx,
                    F8Lut& lcur, F8Lut& lnx, float (&fcur)[2], float (&fnx)[2]) {
        const int k2 = min(kt + 2, KTe - 1), kw2 = min(kt + 2, KT - 1);
        F8Tmp tmp;
        static_for<SLOTS>([&](auto sc) {
            constexpr int s = decltype(sc)::value;
            constexpr int sI = s / 2, j = sI / RB, rb = sI % RB, cb = s % 2;
            constexpr int g = s / GS, sg = s % GS;
            if constexpr (s == SLOTS - 4) {
                __builtin_amdgcn_sched_barrier(0);
                __builtin_amdgcn_s_waitcnt(waitcnt_imm(XWAIT, 0));
                __syncthreads();
                ring[0] = read_a(nxt, 0);
                ring[1] = read_a(nxt, 1);
            }
            mfma32_f8_acc(acc[rb][cb], ring[sI % 4], B[cb][j]);
            if constexpr (FOLD && s == 0) f_load(kw2, fcur);
            if constexpr (FOLD && (s == GS - 2 || s == GS - 1))
                e4m3_fold_table(fnx[s - (GS - 2)], lnx.lo[s - (GS - 2)], lnx.hi[s - (GS - 2)]);
            if constexpr (cb == 1 && sI + 2 < 2 * RB) ring[(sI + 2) % 4] = read_a(cur, sI + 2);
            if constexpr (s >= GS && s < GS + 4) w_load(kw2, s - GS, wcur);
            // All of wnx must be complete here, before the X loads: the
            // compiler's wait for a part first used later (here or in the
            // next step's group 0) would also wait for X loads issued since.
            if constexpr (s == GS) {
                asm volatile("" ::"v"(wnx.w[0][0]), "v"(wnx.w[1][0]), "v"(wnx.w[0][1]),
                             "v"(wnx.w[1][1]));
                // likewise this step's factors, which the next step's tables use
                if constexpr (FOLD) asm volatile("" ::"v"(fcur[0]), "v"(fcur[1]));
            }
            if constexpr (s >= XS && s < XS + CPT) x_load(k2, s - XS, dst);
            static_for<DQ>([&](auto dc) {
                constexpr int o = DQ * sg + decltype(dc)::value;
                if constexpr (o < 64) {
                    if constexpr (g == 0) f8_step<1, o>(tmp, wcur, lcur, sgn, B);
                    else f8_step<0, o>(tmp, wnx, lnx, sgn, B);
                }
            });
        });
    };

    for (int kt = 0; kt < KTe; kt += 2) {
        step(kt, bc, bn, bd, we, wo, le, lo, fe, fo);
        step(kt + 1, bn, bd, bc, wo, we, lo, le, fo, fe);
        const unsigned t0 = bc;  // next pair: X(kt+2) in bd, X(kt+3) in bc
        bc = bd;
        bd = bn;
        bn = t0;
        if (kt + 2 >= KTe) mfma_loop_exit_wait();  // the iteration that leaves the loop
    }
    mfma32_drain(acc);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));  // the last steps' X loads
    __syncthreads();  // all waves done with the X tiles

    // ---- epilogue.  Accumulator (rb, cb) register v of lane (c, h): row
    // 32rb + 8(v/4) + 4h + (v%4), channel n0 + 32cb + c.  Values go to a
    // per-wave LDS block [32 rows][64 channels]; each row is then written as
    // whole 16-byte pieces (final output, or this split's float32 partial).
    constexpr bool SCALED = !PARTIAL;
    constexpr bool BF16 = (OUT == 0) && !PARTIAL;
    if (SCALED) sxs[tid % MT] = (m0 + tid % MT < M) ? sx[m0 + tid % MT] : 0.0f;
    const float tval = (SCALED && FOLD) ? tsc[0] : 0.0f;
    const float sw0 = SCALED ? (FOLD ? tval : sw[n0 + c]) : 0.0f;
    const float sw1 = SCALED ? (FOLD ? tval : sw[n0 + 32 + c]) : 0.0f;
    __syncthreads();
    constexpr int EB = BF16 ? 2 : 4;          // output element bytes
    constexpr int ROWB = 64 * EB;             // bytes per staged row
    static_assert(kWaves * 32 * ROWB <= 3 * XB, "epilogue staging fits in the X tiles");
    uint8_t* stage = xs + wave * (32 * ROWB);
    uint8_t* out = PARTIAL ? reinterpret_cast<uint8_t*>(part + (size_t)ks * M * N)
                           : reinterpret_cast<uint8_t*>(Y);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = 8 * (v >> 2) + 4 * h + (v & 3);
                const int col = 32 * cb + c;
                float y = acc[rb][cb][v];
                if (SCALED) y = (y * sxs[32 * rb + row]) * (cb ? sw1 : sw0);
                if (BF16)
                    *reinterpret_cast<unsigned short*>(stage + row * ROWB + col * 2) =
                        f32_to_bf16_bits(y);
                else
                    *reinterpret_cast<float*>(stage + row * ROWB + col * 4) = y;
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
                store16_result<PARTIAL>(out + ((size_t)m * N + n0) * EB + piece * 16, val);
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_wave_barrier();
    }
}

// Sum of the split-K float32 partial tiles in split order, then the
// per-token x per-channel scale (or, with `tsc`, the per-tensor scale) to
// bf16 or float32.  Workgroup (x, y) covers 1024 channels of row y; each
// thread four consecutive channels, its S partial loads all in flight
// before the first add (the adds keep split order).
template <int OUT, int S>
__global__ __launch_bounds__(256) void splitk_reduce_f32_kernel(
    const float* __restrict__ part, int M, int N, const float* __restrict__ sx,
    const float* __restrict__ sw, const float* __restrict__ tsc, void* __restrict__ Y) {
    const int n = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (n >= N) return;
    const int m = blockIdx.y;
    const size_t MN = (size_t)M * N;
    const size_t e = (size_t)m * N + n;
    v4f v[S];
#pragma unroll
    for (int s = 0; s < S; ++s) v[s] = *reinterpret_cast<const v4f*>(part + s * MN + e);
    v4f acc = v[0];
#pragma unroll
    for (int s = 1; s < S; ++s) acc += v[s];
    const float sm = sx[m];
    float y[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) y[j] = (acc[j] * sm) * (tsc ? tsc[0] : sw[n + j]);
    if (OUT == 1) {
        *reinterpret_cast<v4f*>(reinterpret_cast<float*>(Y) + e) = v4f{y[0], y[1], y[2], y[3]};
    } else {
        uint2 pk;
        pk.x = f32_to_bf16_bits(y[0]) | ((unsigned)f32_to_bf16_bits(y[1]) << 16);
        pk.y = f32_to_bf16_bits(y[2]) | ((unsigned)f32_to_bf16_bits(y[3]) << 16);
        *reinterpret_cast<uint2*>(reinterpret_cast<unsigned short*>(Y) + e) = pk;
    }
}

// splits in 2 .. 16 (the plans' range), one instantiation each.
template <int OUT, int S = 2>
static hipError_t splitk_reduce_f32_run(const float* part, int splits, int M, int N,
                                        const float* sx, const float* sw, const float* tsc,
                                        void* Y, hipStream_t st) {
    if constexpr (S > 16) {
        return hipErrorInvalidValue;
    } else {
        if (splits != S)
            return splitk_reduce_f32_run<OUT, S + 1>(part, splits, M, N, sx, sw, tsc, Y, st);
        const dim3 grid((unsigned)((N / 4 + 255) / 256), (unsigned)M);
        hipLaunchKernelGGL((splitk_reduce_f32_kernel<OUT, S>), grid, dim3(256), 0, st, part, M,
                           N, sx, sw, tsc, Y);
        return hipGetLastError();
    }
}

template <int MT, int OUT, bool PARTIAL, int GROUP>
static void launch_fp8_tile(const uint8_t* X, const float* sx, const uint8_t* wq, const float* sw,
                            const float* fsc, const float* tsc, void* Y, float* part, int M,
                            int N, int K, int splits, hipStream_t st) {
    const int tiles_n = N / kNT;
    const int tiles_m = (M + MT - 1) / MT;
    dim3 grid(tiles_n * tiles_m * splits), block(256);
    hipLaunchKernelGGL((w4fp8_mfma_kernel<MT, OUT, PARTIAL, GROUP>), grid, block, 0, st, X, sx,
                       wq, sw, fsc, tsc, Y, part, M, N, K, tiles_n, tiles_m, splits);
}

template <int GROUP>
static hipError_t w4fp8_mfma_group(const uint8_t* X, const float* sx, const uint8_t* wq,
                                   const float* sw, const float* fsc, const float* tsc, void* Y,
                                   int out_type, int M, int N, int K, const MfmaPlan& plan,
                                   void* workspace, hipStream_t st) {
    float* part = reinterpret_cast<float*>(workspace);
    // Same tile-height rule as the integer GEMM: short-K grids under four
    // waves of 256-row tiles run 128-row tiles, two workgroups per CU
    // (2048 x 8192 x 8192: 8 % faster per-channel, 11 % folded; 2048 x 11008
    // x 4096: 13-14 %; no shape slower; same results bit for bit).
    const int mt = plan.mt16 == 128 ? 128 : plan.mt;
#define FP8_TILE(MT_, O_, P_, S_) \
    launch_fp8_tile<MT_, O_, P_, GROUP>(X, sx, wq, sw, fsc, tsc, Y, part, M, N, K, S_, st)
    if (plan.splits == 1) {
        if (mt == 256) {
            if (out_type == 1) FP8_TILE(256, 1, false, 1);
            else FP8_TILE(256, 0, false, 1);
        } else {
            if (out_type == 1) FP8_TILE(128, 1, false, 1);
            else FP8_TILE(128, 0, false, 1);
        }
        return hipGetLastError();
    }
    if (mt == 256) FP8_TILE(256, 1, true, plan.splits);
    else FP8_TILE(128, 1, true, plan.splits);
#undef FP8_TILE
    if (M == 0) return hipGetLastError();
    if (out_type == 1)
        return splitk_reduce_f32_run<1>(part, plan.splits, M, N, sx, sw, tsc, Y, st);
    return splitk_reduce_f32_run<0>(part, plan.splits, M, N, sx, sw, tsc, Y, st);
}

hipError_t launch_w4fp8_mfma(const uint8_t* X, const float* sx, const uint8_t* wq,
                             const float* sw, void* Y, int out_type, int M, int N, int K,
                             const MfmaPlan& plan, void* workspace, hipStream_t st) {
    return w4fp8_mfma_group<0>(X, sx, wq, sw, nullptr, nullptr, Y, out_type, M, N, K, plan,
                               workspace, st);
}

hipError_t launch_w4fp8g_mfma(const uint8_t* X, const float* sx, const uint8_t* wq,
                              const float* fsc, const float* tsc, void* Y, int out_type, int M,
                              int N, int K, int group, const MfmaPlan& plan, void* workspace,
                              hipStream_t st) {
    if (group == 64)
        return w4fp8_mfma_group<64>(X, sx, wq, nullptr, fsc, tsc, Y, out_type, M, N, K, plan,
                                    workspace, st);
    return w4fp8_mfma_group<128>(X, sx, wq, nullptr, fsc, tsc, Y, out_type, M, N, K, plan,
                                 workspace, st);
}

}  // namespace w4a8
