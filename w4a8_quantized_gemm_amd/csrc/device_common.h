// Device helpers shared by the gfx950 kernels of libw4a8.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a8 {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr int kTileN = 16;     // rows of one packed tile
constexpr int kTileK = 128;    // K columns of one packed tile
constexpr int kTileBytes = 1024;
// Cache-policy operand of buffer loads: non-temporal, for data read once
// (the packed weight stream), so it does not displace L2-resident operands.
constexpr int kNonTemporal = 2;

// 16-byte global load through the vector memory path.
__device__ __forceinline__ v4i load16(const void* p) {
    return *reinterpret_cast<const v4i*>(p);
}

// 16-byte store of a tile kernel's result.
//   Final output: non-temporal.  Nothing reads it back, so it does not
//   displace the panels other workgroups are reading from L2
//   (4096 x 28672 x 8192: 704 -> 696 us).
//   Split-K partials (KEEP): device scope (sc1).  The reduction launch reads
//   them on every XCD, and each XCD has its own L2, so they have to reach
//   memory anyway.  A device-scope store writes them through during the
//   kernel, instead of leaving tens of MB dirty in L2 for the end-of-kernel
//   writeback that the next launch waits on (128 x 8192 x 28672, eight
//   splits: 45.5 -> 43.2 us; 256 x 8192 x 8192: 30.7 -> 29.5; plans without
//   partials unchanged).  The store comes from inline assembly because no
//   builtin gives a plain 16-byte vector store a scope; it has no outputs,
//   and a load-counter wait the compiler places after it only waits longer.
template <bool KEEP>
__device__ __forceinline__ void store16_result(void* p, v4i v) {
    if constexpr (KEEP)
        asm volatile("global_store_dwordx4 %0, %1, off sc1" : : "v"(p), "v"(v) : "memory");
    else
        __builtin_nontemporal_store(v, reinterpret_cast<v4i*>(p));
}

// LiquidQuant dequantisation of four codes held one per byte of `c`
// (LiquidGEMM, Pith review of arXiv 2509.01229, "What carries the
// argument" / paper Eq. 12): byte = (q*s + a) XOR 0x80.  The multiply-add
// runs as two 16-bit lanes, each holding two code bytes; the byte lanes
// cannot carry because every q*s + a <= 255.  `s2` = s in both 16-bit
// halves, `a4` = a in all four bytes.
__device__ __forceinline__ unsigned lqq_dequant4(unsigned c, u16x2 s2, u16x2 a4) {
    u16x2 v = __builtin_bit_cast(u16x2, c);
    v = v * s2 + a4;
    return __builtin_bit_cast(unsigned, v) ^ 0x80808080u;
}

// Byte offset of the group parameters (s_u8 / a_u8, panel order) of output
// channel n, group j: panels of 64 channels, 64 bytes per (panel, group),
// channel n at 4*(n%16) + (n%64)/16.
__device__ __forceinline__ size_t param_offset(int n, int j, int groups) {
    return (size_t)64 * ((size_t)(n >> 6) * groups + j) + 4 * (n & 15) + ((n & 63) >> 4);
}

// From the 4 parameter bytes of one panel row (tile b in byte b): the scale
// of tile b in both 16-bit halves, and its offset in all four bytes.
// v_perm_b32 selector 0x0C yields a zero byte.
__device__ __forceinline__ u16x2 scale_pair(unsigned sdw, int b) {
    const unsigned sel = (unsigned)b | 0x0C00u | ((unsigned)b << 16) | 0x0C000000u;
    return __builtin_bit_cast(u16x2, __builtin_amdgcn_perm(0u, sdw, sel));
}
__device__ __forceinline__ u16x2 offset_quad(unsigned adw, int b) {
    return __builtin_bit_cast(u16x2, __builtin_amdgcn_perm(0u, adw, (unsigned)b * 0x01010101u));
}

// Dequantise the 8 codes of one packed dword into 8 INT8 bytes in K order:
// .x = columns +0..+3 (low nibbles), .y = columns +4..+7 (high nibbles).
__device__ __forceinline__ void lqq_dequant8(unsigned w, u16x2 s2, u16x2 a4,
                                             unsigned& lo, unsigned& hi) {
    lo = lqq_dequant4(w & 0x0F0F0F0Fu, s2, a4);
    hi = lqq_dequant4((w >> 4) & 0x0F0F0F0Fu, s2, a4);
}

// Sign-magnitude INT4 (bit 3 sign, bits 0..2 magnitude) to OCP e4m3 for
// the four codes in the low nibbles of the bytes of `c` (high nibbles of
// `c` must be the sign bits' neighbours of nothing: callers mask first).
// Magnitudes 0..7 map exactly: 0, 1.0, 2.0, 3.0, 4.0, 5.0, 6.0, 7.0 ->
// 0x00 0x38 0x40 0x44 0x48 0x4A 0x4C 0x4E.  The byte lookup is one
// v_perm_b32 over the 8-byte table {lut_hi, lut_lo}.
constexpr unsigned kE4m3LutLo = 0x44403800u;  // bytes for 3,2,1,0
constexpr unsigned kE4m3LutHi = 0x4E4C4A48u;  // bytes for 7,6,5,4

__device__ __forceinline__ unsigned int4_to_e4m3_lo(unsigned w, unsigned lut_lo = kE4m3LutLo,
                                                    unsigned lut_hi = kE4m3LutHi) {
    // low nibbles: magnitude bits 0..2, sign bit 3 -> e4m3 sign bit 7
    unsigned mag = w & 0x07070707u;
    unsigned e = __builtin_amdgcn_perm(lut_hi, lut_lo, mag);
    return e | ((w << 4) & 0x80808080u);
}

__device__ __forceinline__ unsigned int4_to_e4m3_hi(unsigned w, unsigned lut_lo = kE4m3LutLo,
                                                    unsigned lut_hi = kE4m3LutHi) {
    // high nibbles: magnitude bits 4..6, sign bit 7 is already in place
    unsigned mag = (w >> 4) & 0x07070707u;
    unsigned e = __builtin_amdgcn_perm(lut_hi, lut_lo, mag);
    return e | (w & 0x80808080u);
}

// Table words of e4m3(|q| f) for |q| = 0..7 (entry 0 is +0) in the layout
// above, by the hardware conversion (nearest even; for the products used,
// which stay below 464, it agrees with OCP e4m3).
__device__ __forceinline__ void e4m3_fold_table(float f, unsigned& lo, unsigned& hi) {
    const float f2 = 2.0f * f, f3 = 3.0f * f, f4 = 4.0f * f;
    const float f5 = 5.0f * f, f6 = 6.0f * f, f7 = 7.0f * f;
    const int l = __builtin_amdgcn_cvt_pk_fp8_f32(0.0f, f, 0, false);
    lo = (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(f2, f3, l, true);
    const int u = __builtin_amdgcn_cvt_pk_fp8_f32(f4, f5, 0, false);
    hi = (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(f6, f7, u, true);
}

// float -> IEEE binary16 bits, nearest-even (hardware conversion).  The
// empty statement makes `v` a rounded float first: without it the compiler
// may fuse the multiply that produced `v` with the conversion (one rounding
// instead of two) in some kernels and not in others, and the epilogues of
// the different kernels would not agree bit for bit.
__device__ __forceinline__ unsigned short f32_to_f16_bits(float v) {
    asm("" : "+v"(v));
    _Float16 h = (_Float16)v;
    return __builtin_bit_cast(unsigned short, h);
}

// float -> bfloat16 bits, nearest-even on the float32 bit pattern.
__device__ __forceinline__ unsigned short f32_to_bf16_bits(float v) {
    unsigned u = __builtin_bit_cast(unsigned, v);
    if ((u & 0x7F800000u) == 0x7F800000u) {  // inf / nan
        return (unsigned short)((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u));
    }
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (unsigned short)(u >> 16);
}

}  // namespace w4a8
