// C ABI of libw4a8 (declared in include/w4a8.h): argument validation on the
// host, then kernel dispatch on the caller's stream.  Validation makes no
// HIP call, so every error path below can be exercised without a GPU.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <cstring>

#include "launch.h"
#include "mfma_common.h"
#include "w4a8.h"

#define W4A8_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local int g_last_hip_error = 0;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

w4a8_status_t hip_status(hipError_t e) {
    if (e == hipSuccess) return W4A8_OK;
    g_last_hip_error = (int)e;
    return W4A8_ERR_HIP;
}

// Per-device cache: 0 unknown, 1 gfx950, 2 other.
std::atomic<int> g_arch_ok[64];

w4a8_status_t check_device() {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e);
    if (dev < 0 || dev >= 64) return W4A8_ERR_UNSUPPORTED;
    int c = g_arch_ok[dev].load(std::memory_order_relaxed);
    if (c == 0) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess) return hip_status(e);
        c = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
        g_arch_ok[dev].store(c, std::memory_order_relaxed);
    }
    return c == 1 ? W4A8_OK : W4A8_ERR_UNSUPPORTED;
}

bool valid_nk(int N, int K) { return N >= 0 && K > 0 && K % 128 == 0 && N % 64 == 0; }
bool valid_group(int g) { return g == 64 || g == 128; }

// GEMM operand sizes the kernels address with 32-bit buffer ranges: the
// activations M*K bytes < 2^31, the weights N*K < 2^32 codes.
bool valid_extent(int M, int N, int K) {
    return (long long)M * K < (1LL << 31) && (long long)N * K < (1LL << 32);
}

int k_tiles(int K) { return K / 128; }

// Streamed kernel: NTW 16-channel tiles per workgroup, ks waves splitting K,
// RB 16-row blocks of M per workgroup.
// Width: the widest of 4, 2, 1 tiles that divides the tile count and still
// leaves at least 160 workgroups.  Measured at M = 16 against one workgroup
// per CU: 4 tiles are 8-11 % faster on 28672 x 8192, 14336 x 4096,
// 11008 x 4096 and 10240 x 8192 although they leave CUs idle on the last
// three, while 4 tiles at 128 workgroups (N = 8192) are 25-30 % slower than
// 2 at 256.
// Row blocks (W4A8 and FP8, `row_blocks`): a workgroup takes four blocks at
// 33-63 rows when that still allows 2 tiles or more (four blocks of four
// tiles do not fit the registers), else two blocks from 17 rows on when
// some width allows them, so each decoded weight feeds several blocks
// instead of being fetched and decoded again per 16 rows (measured against
// one block per workgroup: 28672 x 8192 at M = 32 / 48 32 % / 22 % faster,
// 8192 x 28672 at M = 48 39 %, 11008 x 4096 at M = 32 / 48 23 % / 18 %,
// 2048 x 4096 at M = 40 4 %).  One tile per workgroup fetches every row
// block's activations per 16 channels: where one row block per workgroup at
// 4 tiles leaves 160 workgroups, that is taken instead.
// With one row block per workgroup (the W8A8 comparison) seven tiles are
// taken from three 16-row blocks on when they leave at least 256 workgroups
// per block (28672 x 8192 at M = 48: 8 % faster than 4; 14336 x 4096: 15 %
// slower).
// K-splitting waves: eight per workgroup, halved while the grid would hold
// more than 2048 waves, and never more than K has K-tiles.  An explicit
// split keeps one tile and one row block per workgroup (up to 16 waves).
w4a8::StreamCfg choose_stream(int M, int N, int K, int splitk, bool row_blocks = false) {
    w4a8::StreamCfg c;
    const int tiles = N / 16;
    const long long rblocks = (M + 15) / 16;
    // widest width leaving at least 160 workgroups with rb row blocks each
    // (0: none does)
    auto width_for = [&](int rb) {
        const long long mgroups = (rblocks + rb - 1) / rb;  // workgroups along M
        const int widths[4] = {7, 4, 2, 1};
        for (int i = 0; i < 4; ++i) {
            const int w = widths[i];
            if (w == 7 && (rb > 1 || rblocks < 3 || tiles / 7 < 256)) continue;
            if (w == 4 && rb == 4) continue;
            if (tiles % w == 0 && (tiles / w) * mgroups >= 160) return w;
        }
        return 0;
    };
    c.rb = 1;
    if (row_blocks && splitk == 0) {
        if (rblocks >= 3 && width_for(4) >= 2)
            c.rb = 4;
        else if (rblocks >= 2 && width_for(2) >= 1)
            c.rb = 2;
    }
    c.nt_per_wave = width_for(c.rb) > 0 ? width_for(c.rb) : 1;
    if (c.rb > 1 && c.nt_per_wave == 1 && width_for(1) == 4) {
        c.rb = 1;
        c.nt_per_wave = 4;
    }
    const int ks_max = 8;
    if (splitk > 0) {
        c.nt_per_wave = 1;
        c.ks = splitk;
    } else {
        c.ks = ks_max;
        const long long wgs = (long long)(tiles / c.nt_per_wave) * ((rblocks + c.rb - 1) / c.rb);
        while (c.ks > 1 && wgs * c.ks > 8 * 256) c.ks /= 2;
        while (c.ks > 1 && k_tiles(K) < c.ks) c.ks /= 2;
    }
    return c;
}

// Kernel choice (a pure function of the shape, so tests can reach both):
// the matrix-core tile kernel takes M >= 64 when N is a multiple of its
// 256-channel workgroup tile; smaller M streams weight tiles per 16 rows.
bool use_mfma_tiles(int M, int N, int K) {
    return M >= 64 && N % 256 == 0 && (long long)M * K < (1LL << 32);
}

bool valid_splitk(int splitk, int K) {
    if (splitk == 0) return true;
    if (splitk != 1 && splitk != 2 && splitk != 4 && splitk != 8 && splitk != 16) return false;
    return splitk <= k_tiles(K);
}

}  // namespace

W4A8_EXPORT const char* w4a8_status_str(w4a8_status_t s) {
    // A C caller may pass any int (an unknown or future code): read the
    // argument's bits as an int, since a value outside the enumerators'
    // range may not be read through the enum type in C++.
    int code;
    std::memcpy(&code, &s, sizeof code);
    static_assert(sizeof(w4a8_status_t) == sizeof(int), "status codes travel as int");
    switch (code) {
        case W4A8_OK: return "ok";
        case W4A8_ERR_NULL_PTR: return "a required pointer is NULL";
        case W4A8_ERR_SHAPE: return "invalid shape, group, qmax or split factor";
        case W4A8_ERR_ALIGNMENT: return "a device pointer is misaligned (16 bytes for arrays, 4 for scale vectors)";
        case W4A8_ERR_WORKSPACE: return "workspace is smaller than w4a8_workspace_size()";
        case W4A8_ERR_UNSUPPORTED: return "unsupported device, mode or output type";
        case W4A8_ERR_HIP: return "HIP runtime error (see w4a8_last_hip_error)";
    }
    return "unknown status";
}

W4A8_EXPORT int w4a8_last_hip_error(void) { return g_last_hip_error; }

W4A8_EXPORT int w4a8_layout_version(void) { return W4A8_LAYOUT_VERSION; }

W4A8_EXPORT w4a8_status_t w4a8_gemm_plan(int M, int N, int K, int splitk, int* kernel,
                                         int* tile_rows, int* tile_channels, int* splits,
                                         int* k_parts) {
    if (!kernel || !tile_rows || !tile_channels || !splits || !k_parts) return W4A8_ERR_NULL_PTR;
    if (M < 0 || !valid_nk(N, K) || !valid_splitk(splitk, K)) return W4A8_ERR_SHAPE;
    // (an empty problem, M or N = 0, launches nothing; it reports the
    // streamed kernel's plan and never reaches the tile plan's arithmetic)
    if (splitk == 0 && M > 0 && N > 0 && use_mfma_tiles(M, N, K)) {  // as launch_w4a8_mfma
        const w4a8::MfmaPlan p = w4a8::plan_w4a8_mfma(M, N, K, true);
        *kernel = p.mt16 != 0 ? 1 : 2;
        *tile_rows = p.mt16 != 0 ? p.mt16 : p.mt;
        *tile_channels = w4a8::kNT / p.kin;
        *splits = p.splits;
        *k_parts = p.kin;
    } else {
        const w4a8::StreamCfg c = choose_stream(M, N, K, splitk, true);
        *kernel = 0;
        *tile_rows = 16 * c.rb;
        *tile_channels = 16 * c.nt_per_wave;
        *splits = 1;
        *k_parts = c.ks;
    }
    return W4A8_OK;
}

W4A8_EXPORT size_t w4a8_workspace_size(int M, int N, int K, int splitk) {
    if (M <= 0 || !valid_nk(N, K) || N == 0 || splitk != 0) return 0;
    if (!use_mfma_tiles(M, N, K)) return 0;
    return w4a8::plan_w4a8_mfma(M, N, K).workspace;
}

W4A8_EXPORT w4a8_status_t w4a8_pack(const float* W, int N, int K, int group, int qmax_i8,
                                    int mode, uint8_t* wq, uint8_t* s_u8, uint8_t* a_u8,
                                    float* sw, hipStream_t stream) {
    if (mode != W4A8_PACK_LQQ && mode != W4A8_PACK_INT4_SYM) return W4A8_ERR_UNSUPPORTED;
    if (!valid_nk(N, K)) return W4A8_ERR_SHAPE;
    if (mode == W4A8_PACK_LQQ && (!valid_group(group) || qmax_i8 < 1 || qmax_i8 > 127))
        return W4A8_ERR_SHAPE;
    if (N == 0) return W4A8_OK;  // nothing to read or write
    if (!W || !wq || !sw) return W4A8_ERR_NULL_PTR;
    if (mode == W4A8_PACK_LQQ && (!s_u8 || !a_u8)) return W4A8_ERR_NULL_PTR;
    if (!aligned16(W) || !aligned16(wq) || !aligned4(sw)) return W4A8_ERR_ALIGNMENT;
    if (mode == W4A8_PACK_LQQ && (!aligned16(s_u8) || !aligned16(a_u8))) return W4A8_ERR_ALIGNMENT;
    w4a8_status_t d = check_device();
    if (d != W4A8_OK) return d;
    if (mode == W4A8_PACK_LQQ)
        return hip_status(w4a8::launch_pack_lqq(W, N, K, group, qmax_i8, wq, s_u8, a_u8, sw, stream));
    return hip_status(w4a8::launch_pack_int4(W, N, K, wq, sw, stream));
}

W4A8_EXPORT w4a8_status_t w4a8_quant_act_ex(const void* X, int in_type, int M, int K,
                                            int8_t* Xq, float* sx, hipStream_t stream) {
    if (in_type != W4A8_IN_F32 && in_type != W4A8_IN_F16 && in_type != W4A8_IN_BF16)
        return W4A8_ERR_UNSUPPORTED;
    if (M < 0 || K <= 0 || K % 16 != 0) return W4A8_ERR_SHAPE;
    if (M == 0) return W4A8_OK;  // nothing to read or write
    if (!X || !Xq || !sx) return W4A8_ERR_NULL_PTR;
    if (!aligned16(X) || !aligned16(Xq) || !aligned4(sx)) return W4A8_ERR_ALIGNMENT;
    w4a8_status_t d = check_device();
    if (d != W4A8_OK) return d;
    return hip_status(w4a8::launch_act_int8(X, in_type, M, K, Xq, sx, stream));
}

W4A8_EXPORT w4a8_status_t w4fp8_quant_act_ex(const void* X, int in_type, int M, int K,
                                             uint8_t* Xq, float* sx, hipStream_t stream) {
    if (in_type != W4A8_IN_F32 && in_type != W4A8_IN_F16 && in_type != W4A8_IN_BF16)
        return W4A8_ERR_UNSUPPORTED;
    if (M < 0 || K <= 0 || K % 16 != 0) return W4A8_ERR_SHAPE;
    if (M == 0) return W4A8_OK;  // nothing to read or write
    if (!X || !Xq || !sx) return W4A8_ERR_NULL_PTR;
    if (!aligned16(X) || !aligned16(Xq) || !aligned4(sx)) return W4A8_ERR_ALIGNMENT;
    w4a8_status_t d = check_device();
    if (d != W4A8_OK) return d;
    return hip_status(w4a8::launch_act_e4m3(X, in_type, M, K, Xq, sx, stream));
}

W4A8_EXPORT w4a8_status_t w4a8_quant_act(const float* X, int M, int K, int8_t* Xq, float* sx,
                                         hipStream_t stream) {
    return w4a8_quant_act_ex(X, W4A8_IN_F32, M, K, Xq, sx, stream);
}

W4A8_EXPORT w4a8_status_t w4fp8_quant_act(const float* X, int M, int K, uint8_t* Xq, float* sx,
                                          hipStream_t stream) {
    return w4fp8_quant_act_ex(X, W4A8_IN_F32, M, K, Xq, sx, stream);
}

namespace w4a8 {

// w4a8_gemm's validation and dispatch.  use_scratch: the workspace is this
// library's static device scratch (w4a8_gemm_noalloc), workspace_bytes its
// capacity; its address is looked up only once the arguments are valid.
w4a8_status_t gemm_entry(const int8_t* X, const float* sx, const uint8_t* wq,
                         const uint8_t* s_u8, const uint8_t* a_u8, const float* sw, void* Y,
                         int out_type, int M, int N, int K, int group, int splitk,
                         void* workspace, size_t workspace_bytes, bool use_scratch,
                         hipStream_t stream) {
    if (out_type != W4A8_OUT_F16 && out_type != W4A8_OUT_I32) return W4A8_ERR_UNSUPPORTED;
    if (M < 0 || !valid_nk(N, K) || !valid_group(group) || !valid_splitk(splitk, K))
        return W4A8_ERR_SHAPE;
    if (!valid_extent(M, N, K)) return W4A8_ERR_SHAPE;
    if (M == 0 || N == 0) return W4A8_OK;  // nothing to read or write
    if (!X || !wq || !s_u8 || !a_u8 || !Y) return W4A8_ERR_NULL_PTR;
    if (out_type == W4A8_OUT_F16 && (!sx || !sw)) return W4A8_ERR_NULL_PTR;
    if (!aligned16(X) || !aligned16(wq) || !aligned16(Y)) return W4A8_ERR_ALIGNMENT;
    if (!aligned16(s_u8) || !aligned16(a_u8)) return W4A8_ERR_ALIGNMENT;
    if ((sx && !aligned4(sx)) || (sw && !aligned4(sw))) return W4A8_ERR_ALIGNMENT;
    const size_t need = w4a8_workspace_size(M, N, K, splitk);
    if (workspace_bytes < need) return W4A8_ERR_WORKSPACE;
    if (!use_scratch && need > 0 && !workspace) return W4A8_ERR_NULL_PTR;
    if (!use_scratch && need > 0 && !aligned16(workspace)) return W4A8_ERR_ALIGNMENT;
    w4a8_status_t d = check_device();
    if (d != W4A8_OK) return d;
    if (use_scratch) {
        workspace = nullptr;
        if (need > 0) {
            const hipError_t e = noalloc_scratch(&workspace);
            if (e != hipSuccess) return hip_status(e);
        }
    }
    if (splitk == 0 && use_mfma_tiles(M, N, K))
        return hip_status(w4a8::launch_w4a8_mfma(X, sx, wq, s_u8, a_u8, sw, Y, out_type, M, N, K,
                                                 group, w4a8::plan_w4a8_mfma(M, N, K, true), workspace,
                                                 stream));
    return hip_status(w4a8::launch_w4a8_stream(X, sx, wq, s_u8, a_u8, sw, Y, out_type, M, N, K,
                                               group, choose_stream(M, N, K, splitk, true),
                                               stream));
}

}  // namespace w4a8

W4A8_EXPORT w4a8_status_t w4a8_gemm(const int8_t* X, const float* sx, const uint8_t* wq,
                                    const uint8_t* s_u8, const uint8_t* a_u8, const float* sw,
                                    void* Y, int out_type, int M, int N, int K, int group,
                                    int splitk, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream) {
    return w4a8::gemm_entry(X, sx, wq, s_u8, a_u8, sw, Y, out_type, M, N, K, group, splitk,
                            workspace, workspace_bytes, false, stream);
}

W4A8_EXPORT w4a8_status_t w4a8_gemm_grouped(const int8_t* X, const float* sx,
                                            const int32_t* offsets, int E, const uint8_t* wq,
                                            const uint8_t* s_u8, const uint8_t* a_u8,
                                            const float* sw, void* Y, int out_type, int M, int N,
                                            int K, int group, int max_rows, hipStream_t stream) {
    if (out_type != W4A8_OUT_F16 && out_type != W4A8_OUT_I32) return W4A8_ERR_UNSUPPORTED;
    if (M < 0 || E < 1 || E > 65535 || max_rows < 0 || !valid_nk(N, K) || !valid_group(group))
        return W4A8_ERR_SHAPE;
    if (!valid_extent(M, N, K)) return W4A8_ERR_SHAPE;
    if (M == 0 || N == 0 || max_rows == 0) return W4A8_OK;  // nothing to read or write
    if (!X || !offsets || !wq || !s_u8 || !a_u8 || !Y) return W4A8_ERR_NULL_PTR;
    if (out_type == W4A8_OUT_F16 && (!sx || !sw)) return W4A8_ERR_NULL_PTR;
    if (!aligned16(X) || !aligned16(wq) || !aligned16(Y)) return W4A8_ERR_ALIGNMENT;
    if (!aligned16(s_u8) || !aligned16(a_u8)) return W4A8_ERR_ALIGNMENT;
    if (!aligned4(offsets) || (sx && !aligned4(sx)) || (sw && !aligned4(sw)))
        return W4A8_ERR_ALIGNMENT;
    w4a8_status_t d = check_device();
    if (d != W4A8_OK) return d;
    const int rows = max_rows < M ? max_rows : M;
    if (rows >= 64 && N % 256 == 0) {
        // matrix-core tiles of 128 rows: every expert's last tile is partly
        // empty, and routed row counts fall anywhere, so the shorter tile
        // wastes less (measured faster than 256-row tiles on Mixtral expert
        // shapes at 512 .. 8192 tokens)
        return hip_status(w4a8::launch_w4a8_mfma_grouped(X, sx, wq, s_u8, a_u8, sw, Y, out_type,
                                                         M, N, K, group, offsets, E, rows, 128,
                                                         stream));
    }
    // streamed tiles: the width rule of the dense problem applied to all
    // experts' tiles together; four K-splitting waves (most experts hold
    // fewer rows than max_rows, so the padded grid overstates the active
    // workgroups; four measured best at 16 and 64 tokens on Mixtral shapes);
    // two 16-row blocks per workgroup above 16 rows per expert (Mixtral
    // expert shapes at 64 / 96 tokens: 16-17 % / 25-28 % faster; four
    // blocks were slower)
    w4a8::StreamCfg c = choose_stream(16, N * E, K, 0);
    while (c.nt_per_wave > 1 && (N / 16) % c.nt_per_wave != 0) {
        c.nt_per_wave = c.nt_per_wave == 7 ? 4 : c.nt_per_wave == 4 ? 2 : 1;
    }
    c.ks = 4;
    while (c.ks > 1 && k_tiles(K) < c.ks) c.ks /= 2;
    if (rows > 16 && c.nt_per_wave != 7) c.rb = 2;
    return hip_status(w4a8::launch_w4a8_stream(X, sx, wq, s_u8, a_u8, sw, Y, out_type, M, N, K,
                                               group, c, stream, offsets, E, rows));
}

W4A8_EXPORT w4a8_status_t w4a8_gemm_ablation(int variant, const int8_t* X, const float* sx,
                                             const uint8_t* wq, const uint8_t* s_u8,
                                             const uint8_t* a_u8, const float* sw, void* Y,
                                             int out_type, int M, int N, int K, int group,
                                             hipStream_t stream) {
    if (variant != W4A8_ABL_LQQ && variant != W4A8_ABL_AFFINE16 &&
        variant != W4A8_ABL_LQQ_COARSE)
        return W4A8_ERR_UNSUPPORTED;
    if (out_type != W4A8_OUT_F16 && out_type != W4A8_OUT_I32) return W4A8_ERR_UNSUPPORTED;
    if (M < 0 || !valid_nk(N, K) || !valid_group(group)) return W4A8_ERR_SHAPE;
    if (!valid_extent(M, N, K)) return W4A8_ERR_SHAPE;
    if (M == 0 || N == 0) return W4A8_OK;  // nothing to read or write
    if (!use_mfma_tiles(M, N, K) || w4a8::plan_w4a8_mfma(M, N, K).splits != 1)
        return W4A8_ERR_UNSUPPORTED;  // the variants exist for the unsplit tile kernel only
    if (!X || !wq || !s_u8 || !a_u8 || !Y) return W4A8_ERR_NULL_PTR;
    if (out_type == W4A8_OUT_F16 && (!sx || !sw)) return W4A8_ERR_NULL_PTR;
    if (!aligned16(X) || !aligned16(wq) || !aligned16(Y)) return W4A8_ERR_ALIGNMENT;
    if (!aligned16(s_u8) || !aligned16(a_u8)) return W4A8_ERR_ALIGNMENT;
    if ((sx && !aligned4(sx)) || (sw && !aligned4(sw))) return W4A8_ERR_ALIGNMENT;
    w4a8_status_t d = check_device();
    if (d != W4A8_OK) return d;
    const w4a8::MfmaPlan plan = w4a8::plan_w4a8_mfma(M, N, K);
    return hip_status(w4a8::launch_w4a8_mfma_ablation(variant, X, sx, wq, s_u8, a_u8, sw, Y,
                                                      out_type, M, N, K, group, plan, stream));
}

W4A8_EXPORT w4a8_status_t w4fp8_gemm(const uint8_t* X_e4m3, const float* sx, const uint8_t* wq,
                                     const float* sw, void* Y, int out_type, int M, int N, int K,
                                     int splitk, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream) {
    if (out_type != W4FP8_OUT_BF16 && out_type != W4FP8_OUT_F32) return W4A8_ERR_UNSUPPORTED;
    if (M < 0 || !valid_nk(N, K) || !valid_splitk(splitk, K)) return W4A8_ERR_SHAPE;
    if (!valid_extent(M, N, K)) return W4A8_ERR_SHAPE;
    if (M == 0 || N == 0) return W4A8_OK;  // nothing to read or write
    if (!X_e4m3 || !sx || !wq || !sw || !Y) return W4A8_ERR_NULL_PTR;
    if (!aligned16(X_e4m3) || !aligned16(wq) || !aligned16(Y)) return W4A8_ERR_ALIGNMENT;
    if (!aligned4(sx) || !aligned4(sw)) return W4A8_ERR_ALIGNMENT;
    const size_t need = w4a8_workspace_size(M, N, K, splitk);
    if (workspace_bytes < need) return W4A8_ERR_WORKSPACE;
    if (need > 0 && !workspace) return W4A8_ERR_NULL_PTR;
    if (need > 0 && !aligned16(workspace)) return W4A8_ERR_ALIGNMENT;
    w4a8_status_t d = check_device();
    if (d != W4A8_OK) return d;
    if (splitk == 0 && use_mfma_tiles(M, N, K))
        return hip_status(w4a8::launch_w4fp8_mfma(X_e4m3, sx, wq, sw, Y, out_type, M, N, K,
                                                  w4a8::plan_w4a8_mfma(M, N, K), workspace,
                                                  stream));
    return hip_status(w4a8::launch_w4fp8_stream(X_e4m3, sx, wq, sw, Y, out_type, M, N, K,
                                                choose_stream(M, N, K, splitk, true), stream));
}

W4A8_EXPORT w4a8_status_t w4fp8g_pack(const float* W, int N, int K, int group, uint8_t* wq,
                                      float* fsc, float* tscale, hipStream_t stream) {
    if (!valid_nk(N, K) || !valid_group(group)) return W4A8_ERR_SHAPE;
    if ((long long)N * (K / group) >= (1LL << 29)) return W4A8_ERR_SHAPE;
    if (N == 0) return W4A8_OK;  // nothing to read or write
    if (!W || !wq || !fsc || !tscale) return W4A8_ERR_NULL_PTR;
    if (!aligned16(W) || !aligned16(wq) || !aligned4(fsc) || !aligned4(tscale))
        return W4A8_ERR_ALIGNMENT;
    w4a8_status_t d = check_device();
    if (d != W4A8_OK) return d;
    return hip_status(w4a8::launch_pack_fp8g(W, N, K, group, wq, fsc, tscale, stream));
}

W4A8_EXPORT w4a8_status_t w4fp8g_gemm(const uint8_t* X_e4m3, const float* sx, const uint8_t* wq,
                                      const float* fsc, const float* tscale, void* Y,
                                      int out_type, int M, int N, int K, int group, int splitk,
                                      void* workspace, size_t workspace_bytes,
                                      hipStream_t stream) {
    if (out_type != W4FP8_OUT_BF16 && out_type != W4FP8_OUT_F32) return W4A8_ERR_UNSUPPORTED;
    if (M < 0 || !valid_nk(N, K) || !valid_group(group) || !valid_splitk(splitk, K))
        return W4A8_ERR_SHAPE;
    if ((long long)N * (K / group) >= (1LL << 29)) return W4A8_ERR_SHAPE;
    if (!valid_extent(M, N, K)) return W4A8_ERR_SHAPE;
    if (M == 0 || N == 0) return W4A8_OK;  // nothing to read or write
    if (!X_e4m3 || !sx || !wq || !fsc || !tscale || !Y) return W4A8_ERR_NULL_PTR;
    if (!aligned16(X_e4m3) || !aligned16(wq) || !aligned16(Y)) return W4A8_ERR_ALIGNMENT;
    if (!aligned4(sx) || !aligned4(fsc) || !aligned4(tscale)) return W4A8_ERR_ALIGNMENT;
    const size_t need = w4a8_workspace_size(M, N, K, splitk);
    if (workspace_bytes < need) return W4A8_ERR_WORKSPACE;
    if (need > 0 && !workspace) return W4A8_ERR_NULL_PTR;
    if (need > 0 && !aligned16(workspace)) return W4A8_ERR_ALIGNMENT;
    w4a8_status_t d = check_device();
    if (d != W4A8_OK) return d;
    if (splitk == 0 && use_mfma_tiles(M, N, K))
        return hip_status(w4a8::launch_w4fp8g_mfma(X_e4m3, sx, wq, fsc, tscale, Y, out_type, M, N,
                                                   K, group, w4a8::plan_w4a8_mfma(M, N, K),
                                                   workspace, stream));
    return hip_status(w4a8::launch_w4fp8g_stream(X_e4m3, sx, wq, fsc, tscale, Y, out_type, M, N,
                                                 K, group, choose_stream(M, N, K, splitk, true),
                                                 stream));
}

W4A8_EXPORT w4a8_status_t w8a8_pack(const float* W, int N, int K, int8_t* wq8, float* sw,
                                    hipStream_t stream) {
    if (!valid_nk(N, K)) return W4A8_ERR_SHAPE;
    if ((long long)N * K >= (1LL << 31)) return W4A8_ERR_SHAPE;
    if (N == 0) return W4A8_OK;  // nothing to read or write
    if (!W || !wq8 || !sw) return W4A8_ERR_NULL_PTR;
    if (!aligned16(W) || !aligned16(wq8) || !aligned4(sw)) return W4A8_ERR_ALIGNMENT;
    w4a8_status_t d = check_device();
    if (d != W4A8_OK) return d;
    return hip_status(w4a8::launch_pack_w8(W, N, K, wq8, sw, stream));
}

W4A8_EXPORT w4a8_status_t w8a8_gemm(const int8_t* X, const float* sx, const int8_t* wq8,
                                    const float* sw, void* Y, int out_type, int M, int N, int K,
                                    int splitk, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream) {
    if (out_type != W4A8_OUT_F16 && out_type != W4A8_OUT_I32) return W4A8_ERR_UNSUPPORTED;
    if (M < 0 || !valid_nk(N, K) || !valid_splitk(splitk, K)) return W4A8_ERR_SHAPE;
    if ((long long)N * K >= (1LL << 31)) return W4A8_ERR_SHAPE;
    if (!valid_extent(M, N, K)) return W4A8_ERR_SHAPE;
    if (M == 0 || N == 0) return W4A8_OK;  // nothing to read or write
    if (!X || !wq8 || !Y) return W4A8_ERR_NULL_PTR;
    if (out_type == W4A8_OUT_F16 && (!sx || !sw)) return W4A8_ERR_NULL_PTR;
    if (!aligned16(X) || !aligned16(wq8) || !aligned16(Y)) return W4A8_ERR_ALIGNMENT;
    if ((sx && !aligned4(sx)) || (sw && !aligned4(sw))) return W4A8_ERR_ALIGNMENT;
    const size_t need = w4a8_workspace_size(M, N, K, splitk);
    if (workspace_bytes < need) return W4A8_ERR_WORKSPACE;
    if (need > 0 && !workspace) return W4A8_ERR_NULL_PTR;
    if (need > 0 && !aligned16(workspace)) return W4A8_ERR_ALIGNMENT;
    w4a8_status_t d = check_device();
    if (d != W4A8_OK) return d;
    if (splitk == 0 && use_mfma_tiles(M, N, K))
        return hip_status(w4a8::launch_w8a8_mfma(X, sx, wq8, sw, Y, out_type, M, N, K,
                                                 w4a8::plan_w4a8_mfma(M, N, K, true), workspace,
                                                 stream));
    return hip_status(w4a8::launch_w8a8_stream(X, sx, wq8, sw, Y, out_type, M, N, K,
                                               choose_stream(M, N, K, splitk), stream));
}
