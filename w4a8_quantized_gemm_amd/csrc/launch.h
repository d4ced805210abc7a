// Internal host-side launchers of libw4a8 (not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a8 {

hipError_t launch_pack_lqq(const float* W, int N, int K, int group, int qmax, uint8_t* wq,
                           uint8_t* s_u8, uint8_t* a_u8, float* sw, hipStream_t st);
hipError_t launch_pack_int4(const float* W, int N, int K, uint8_t* wq, float* sw,
                            hipStream_t st);
// INT4 codes with per-group scales folded into FP8 (fsc [K/group][N] float32
// folded factors, tscale[0] the per-tensor scale).
hipError_t launch_pack_fp8g(const float* W, int N, int K, int group, uint8_t* wq, float* fsc,
                            float* tscale, hipStream_t st);
// Per-token activation quantisation; in_type 0 = float32, 1 = fp16, 2 = bf16.
hipError_t launch_act_int8(const void* X, int in_type, int M, int K, int8_t* Xq, float* sx,
                           hipStream_t st);
hipError_t launch_act_e4m3(const void* X, int in_type, int M, int K, uint8_t* Xq, float* sx,
                           hipStream_t st);

// Streamed-tile GEMMs: one workgroup per (16*nt_per_wave rows of N, 16 rows
// of M); `ks` waves split K and reduce in LDS.
struct StreamCfg {
    int nt_per_wave;  // 16-row weight tiles per workgroup (1, 2, 4 or 7)
    int ks;           // waves per workgroup splitting K (1..16)
    int rb = 1;       // 16-row blocks of M per workgroup (1, 2 or 4; not W8A8)
};

// offsets != nullptr: grouped problem of E experts (rows offsets[e] ..
// offsets[e+1]-1, e-th weight slab), at most max_rows rows per expert.
hipError_t launch_w4a8_stream(const int8_t* X, const float* sx, const uint8_t* wq,
                              const uint8_t* s_u8, const uint8_t* a_u8, const float* sw,
                              void* Y, int out_type, int M, int N, int K, int group,
                              StreamCfg cfg, hipStream_t st, const int* offsets = nullptr,
                              int E = 1, int max_rows = 0);

// Grouped problem on the matrix-core tile kernel (no K split): expert
// blockIdx.y, M tiles up to ceil(max_rows / mt).
hipError_t launch_w4a8_mfma_grouped(const int8_t* X, const float* sx, const uint8_t* wq,
                                    const uint8_t* s_u8, const uint8_t* a_u8, const float* sw,
                                    void* Y, int out_type, int M, int N, int K, int group,
                                    const int* offsets, int E, int max_rows, int mt,
                                    hipStream_t st);

// Matrix-core tile kernel (N % 256 == 0): workgroup tiles of mt = 128 or
// 256 rows x 256 channels; with splits > 1 each workgroup covers 1/splits of
// K and writes int32 partial tiles to the workspace, then a reduction
// kernel sums them in split order and applies the epilogue.
struct MfmaPlan {
    int mt;
    int splits;
    size_t workspace;  // bytes of 4-byte partials (0 when splits == 1)
    // Integer kernels: tile height for the 16 x 16 x 64 kernel (128: two
    // workgroups per CU), or 0 for the 32 x 32 x 32 kernel at mt.  The FP8
    // tile kernel runs 128-row tiles (two per CU) when mt16 == 128, else mt.
    int mt16;
    // K parts per workgroup of the integer 16 x 16 kernel: 2 = workgroups of
    // 128 channels whose wave pairs take the two halves of the split's K
    // range (only with mt16 == 128; splits then counts workgroups per tile).
    int kin = 1;
};
// k_parts: the caller runs the integer 16 x 16 kernel, which can take K
// parts; the workspace of such a plan is at most that of the plan without.
MfmaPlan plan_w4a8_mfma(int M, int N, int K, bool k_parts = false);
hipError_t launch_w4a8_mfma(const int8_t* X, const float* sx, const uint8_t* wq,
                            const uint8_t* s_u8, const uint8_t* a_u8, const float* sw, void* Y,
                            int out_type, int M, int N, int K, int group, const MfmaPlan& plan,
                            void* workspace, hipStream_t st);

// Ablation variants of the W4A8 tile kernel (plan.splits must be 1):
// variant 1 = conventional signed affine decode in 16-bit lanes, variant 2 =
// LiquidQuant decode done per K-step in one block (no fine-grained overlap).
hipError_t launch_w4a8_mfma_ablation(int variant, const int8_t* X, const float* sx,
                                     const uint8_t* wq, const uint8_t* s_u8, const uint8_t* a_u8,
                                     const float* sw, void* Y, int out_type, int M, int N, int K,
                                     int group, const MfmaPlan& plan, hipStream_t st);

// W4FP8 matrix-core tile kernel: same tiles and plan as the W4A8 one, with
// float32 partials in the workspace when plan.splits > 1.
hipError_t launch_w4fp8_mfma(const uint8_t* X, const float* sx, const uint8_t* wq,
                             const float* sw, void* Y, int out_type, int M, int N, int K,
                             const MfmaPlan& plan, void* workspace, hipStream_t st);

hipError_t launch_w4fp8_stream(const uint8_t* X, const float* sx, const uint8_t* wq,
                               const float* sw, void* Y, int out_type, int M, int N, int K,
                               StreamCfg cfg, hipStream_t st);

// Sum of `splits` int32 partial tiles in split order, then the fp16
// epilogue (out_type 0) or the raw int32 sums (out_type 1).
hipError_t launch_splitk_reduce(const int* part, int splits, int M, int N, const float* sx,
                                const float* sw, void* Y, int out_type, hipStream_t st);

// The W4A8 tile kernel on v_mfma_i32_16x16x64_i8 (offsets != nullptr: the
// grouped problem with E experts and max_rows rows at most per expert).
hipError_t launch_w4a8_mfma16(const int8_t* X, const float* sx, const uint8_t* wq,
                              const uint8_t* s_u8, const uint8_t* a_u8, const float* sw, void* Y,
                              int out_type, int M, int N, int K, int group, const MfmaPlan& plan,
                              void* workspace, hipStream_t st, const int* offsets = nullptr,
                              int E = 1, int max_rows = 0);

// The W8A8 comparison on the 16 x 16 x 64 tile kernel.
hipError_t launch_w8a8_mfma16(const int8_t* X, const float* sx, const int8_t* wq8,
                              const float* sw, void* Y, int out_type, int M, int N, int K,
                              const MfmaPlan& plan, void* workspace, hipStream_t st);

// W8A8 comparison: per-channel INT8 weights in the 8-bit tile layout.
hipError_t launch_pack_w8(const float* W, int N, int K, int8_t* wq8, float* sw, hipStream_t st);

hipError_t launch_w8a8_mfma(const int8_t* X, const float* sx, const int8_t* wq8, const float* sw,
                            void* Y, int out_type, int M, int N, int K, const MfmaPlan& plan,
                            void* workspace, hipStream_t st);

hipError_t launch_w8a8_stream(const int8_t* X, const float* sx, const int8_t* wq8,
                              const float* sw, void* Y, int out_type, int M, int N, int K,
                              StreamCfg cfg, hipStream_t st);

// Folded per-group FP8 weights (fsc [K/group][N] factors, tsc[0] tensor scale).
hipError_t launch_w4fp8g_mfma(const uint8_t* X, const float* sx, const uint8_t* wq,
                              const float* fsc, const float* tsc, void* Y, int out_type, int M,
                              int N, int K, int group, const MfmaPlan& plan, void* workspace,
                              hipStream_t st);

hipError_t launch_w4fp8g_stream(const uint8_t* X, const float* sx, const uint8_t* wq,
                                const float* fsc, const float* tsc, void* Y, int out_type, int M,
                                int N, int K, int group, StreamCfg cfg, hipStream_t st);

// Device address of this library's static scratch array on the current
// device (looked up once per device); W4A8_NOALLOC_SCRATCH_BYTES long.
hipError_t noalloc_scratch(void** ptr);

}  // namespace w4a8
