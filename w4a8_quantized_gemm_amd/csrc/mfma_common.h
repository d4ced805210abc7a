// Building blocks shared by the matrix-core tile kernels (W4A8 int8 and
// W4FP8 e4m3): compile-time loops, buffer loads, the X tile swizzle, the
// workgroup -> output tile order and the accumulator drain.
#pragma once
#include <stdint.h>

#include <utility>

#include "device_common.h"

namespace w4a8 {

constexpr int kWaves = 4;
constexpr int kColsPerWave = 64;              // 4 packed tiles
constexpr int kNT = kWaves * kColsPerWave;    // 256 channels per workgroup

// Row-dependent XOR of the 16-byte slot index of an X row held in LDS (row
// stride 128 bytes): distinct for rows r and r' of a 16-row block whenever
// they share a bank window, for both 32- and 64-bank LDS organisations.
__device__ __forceinline__ int xswz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// Compile-time loop: f(std::integral_constant<int, i>) for i = 0 .. N-1.
template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
    (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
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

// 32-bit LDS address of a pointer into a __shared__ object.
__device__ __forceinline__ unsigned lds_addr(const void* p) {
    return (unsigned)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Global -> LDS load of 16 bytes per lane, no register round trip: lane l's
// bytes land at LDS address `lds` + 16 l (`lds` wave-uniform); a lane whose
// offset lies outside the buffer writes zeros.  Written as assembly so the
// compiler does not track it: its own load-counter waits stay exact for the
// register loads, and the kernel waits for these loads itself (a
// s_waitcnt on the load counter before the barrier that publishes the
// tile).  M0 carries the LDS address; the compiler keeps nothing in M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void buf_load16_lds(__amdgpu_buffer_rsrc_t r, unsigned voff,
                                               unsigned soff, unsigned lds) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(lds), "v"(voff), "s"(r), "s"(soff)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt immediate: load counter <= vm and LDS/scalar counter <= lgkm
// (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4 left at 7).
constexpr int waitcnt_imm(int vm, int lgkm) {
    return (vm & 15) | (7 << 4) | ((lgkm & 15) << 8) | ((vm >> 4) << 14);
}

// Wait states between the last accumulation written in inline assembly and
// any read of the accumulators.  The compiler sees neither the matrix-core
// instructions nor their latency, so after the wait every accumulator is
// passed through an empty assembly statement that it must treat as the
// accumulator's new definition: copies the register allocator makes (into
// VGPRs for the epilogue, or between the allocations of two control-flow
// paths) can then only come after the wait.  Call at the end of every path
// that leaves the main loop.
template <typename ACC, int RB>
__device__ __forceinline__ void mfma32_drain(ACC (&acc)[RB][2]) {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        asm volatile("" : "+a"(acc[rb][0]));
        asm volatile("" : "+a"(acc[rb][1]));
    }
    __builtin_amdgcn_sched_barrier(0);
}

// Wait states at the bottom of the main loop's last iteration, after its
// last matrix-core instruction (called under a uniform branch on the loop
// counter).  The register allocator may split an accumulator's live range at
// the loop exit and copy it out of its AGPR there, before the drain that
// follows the loop: neither the scheduling barriers nor the drain's
// redefinitions constrain where it puts such copies.  With these wait states
// inside the loop, every path out of it is far enough from the last write.
// An XDL write of a register and a vector read of it need passes + 3 wait
// states on CDNA3, one more on gfx950: at most 20 for the 16-pass
// instructions used here.  Waiting in every iteration instead cost 0.2-1.0 %
// on the 70B shapes.  A CPU test checks the distance on every path in this
// build's assembly.
__device__ __forceinline__ void mfma_loop_exit_wait() {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3");
}

// Workgroup -> (output tile, K split).  Workgroups are dealt round-robin to
// the 8 XCDs (each with its own L2); regroup so each XCD walks a contiguous
// run of tiles, and order the tiles in 4 (M) x 8 (channel panel) blocks so
// that the 32 workgroups one XCD runs together share 4 X panels and 8
// weight panels (X is re-fetched tiles_n / 8 times rather than once per
// pair of channel panels).
struct TileCoord {
    int tm, tn, ks;
};
__device__ __forceinline__ TileCoord tile_coord(int bid, int tiles_m, int tiles_n, int splits) {
    const int ntiles = tiles_n * tiles_m;
    const int nwg = ntiles * splits;
    int lin = bid;
    if ((nwg & 7) == 0) lin = (bid & 7) * (nwg >> 3) + (bid >> 3);
    TileCoord t;
    t.ks = lin / ntiles;
    const int tile = lin % ntiles;
    if ((tiles_m & 3) == 0 && (tiles_n & 7) == 0) {
        const int blk = tile >> 5, in = tile & 31;
        const int bm = tiles_m >> 2;
        t.tm = (blk % bm) * 4 + (in & 3);
        t.tn = (blk / bm) * 8 + (in >> 2);
    } else {
        t.tm = tile % tiles_m;
        t.tn = tile / tiles_m;
    }
    return t;
}

}  // namespace w4a8
