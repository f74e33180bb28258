// C ABI of the BitLinear library: host-side argument checks, then kernel
// launches on the caller's stream.  Declarations and the full contract of
// each call are in include/bitnet.h.
#include "../../include/bitnet.h"
#include "common.h"

#include <mutex>

namespace {

constexpr int kVersion = 10000;  // 1.0.0

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }
int hip_status(hipError_t e) { return e == hipSuccess ? BITNET_OK : BITNET_E_HIP; }
bool float_dtype(int d) { return d == BITNET_F32 || d == BITNET_BF16; }

// int8 GEMM / GEMV path limits: |acc| <= 128*K must fit int32.
constexpr int64_t kMaxK = (int64_t)1 << 24;
constexpr int64_t kMaxFwdN = (int64_t)1 << 23;  // tile loads and stores use 32-bit offsets
constexpr int64_t kMaxDim = ((int64_t)1 << 31) - 1;  // kernels index rows with int
constexpr int64_t kGemvBlocksMaxM = 64;  // forward: up to this many tokens as GEMV blocks of 16
constexpr int kMaxGatePolls = 1024;  // bitnet_set_gate_polls' upper bound

}  // namespace

extern "C" {

int bitnet_version(void) { return kVersion; }

int bitnet_set_gate_polls(int reads) {
    if (reads < 0 || reads > kMaxGatePolls) return BITNET_E_ARG;
    return bitnet::set_gate_polls(reads);
}

const char* bitnet_status_str(int status) {
    switch (status) {
        case BITNET_OK: return "ok";
        case BITNET_E_ARG: return "null required pointer or bad flag";
        case BITNET_E_SHAPE: return "size out of range (M, N, K >= 1; K % 4 or K % 16 as required)";
        case BITNET_E_DTYPE: return "unsupported dtype";
        case BITNET_E_ALIGN: return "pointer not 16-byte aligned";
        case BITNET_E_WORKSPACE: return "workspace missing or too small";
        case BITNET_E_HIP: return "HIP launch or runtime error";
        case BITNET_E_SCRATCH: return "size beyond the fixed scratch of a no-allocation call";
        default: return "unknown status";
    }
}

size_t bitnet_workspace_bytes(int op, int64_t M, int64_t N, int64_t K) {
    if (M < 0 || N < 0 || K < 0) return 0;
    switch (op) {
        case BITNET_OP_WEIGHT_QUANT: return bitnet::weight_quant_ws_bytes(N);
        case BITNET_OP_LINEAR_BWD_STE: return bitnet::bwd_ws_bytes(M, N, K);
        case BITNET_OP_CODE_COUNTS: return bitnet::code_counts_ws_bytes();
        case BITNET_OP_WEIGHT_QUANT_ROWS: return bitnet::weight_quant_rows_ws_bytes(N);
        case BITNET_OP_WEIGHT_QUANT_COUNTED: return bitnet::weight_quant_counted_ws_bytes(N, K);
        default: return 0;
    }
}

int bitnet_weight_quant(const void* W, int w_dtype, int64_t N, int64_t K, uint8_t* W_packed,
                        float* gamma, void* workspace, size_t workspace_bytes, void* stream) {
    if (!W || !W_packed || !gamma) return BITNET_E_ARG;
    if (!float_dtype(w_dtype)) return BITNET_E_DTYPE;
    if (N < 1 || K < 1 || K % 4 != 0 || N > kMaxDim || K > kMaxDim) return BITNET_E_SHAPE;
    if (!aligned16(W) || !aligned16(W_packed) || !aligned4(gamma)) return BITNET_E_ALIGN;
    if (!workspace || workspace_bytes < bitnet::weight_quant_ws_bytes(N)) return BITNET_E_WORKSPACE;
    if (!aligned16(workspace)) return BITNET_E_ALIGN;
    return hip_status(bitnet::launch_weight_quant(W, w_dtype == BITNET_BF16, N, K, W_packed, gamma,
                                                  workspace, as_stream(stream)));
}

int bitnet_weight_quant_counted(const void* W, int w_dtype, int64_t N, int64_t K, uint8_t* W_packed,
                                float* gamma, uint64_t* counts, void* workspace, size_t workspace_bytes,
                                void* stream) {
    if (!W || !W_packed || !gamma || !counts) return BITNET_E_ARG;
    if (!float_dtype(w_dtype)) return BITNET_E_DTYPE;
    if (N < 1 || K < 1 || K % 4 != 0 || N > kMaxDim || K > kMaxDim) return BITNET_E_SHAPE;
    if (!aligned16(W) || !aligned16(W_packed) || !aligned4(gamma)) return BITNET_E_ALIGN;
    if ((reinterpret_cast<uintptr_t>(counts) & 7u) != 0) return BITNET_E_ALIGN;
    if (!workspace || workspace_bytes < bitnet::weight_quant_counted_ws_bytes(N, K)) return BITNET_E_WORKSPACE;
    if (!aligned16(workspace)) return BITNET_E_ALIGN;
    return hip_status(bitnet::launch_weight_quant_counted(W, w_dtype == BITNET_BF16, N, K, W_packed, gamma, counts,
                                                          workspace, as_stream(stream)));
}

int bitnet_act_quant(const void* X, int x_dtype, int64_t M, int64_t K, float eps, int8_t* Xq,
                     float* scale_x, void* stream) {
    if (!X || !Xq || !scale_x) return BITNET_E_ARG;
    if (!float_dtype(x_dtype)) return BITNET_E_DTYPE;
    if (M < 1 || K < 1 || M > kMaxDim || K > kMaxDim) return BITNET_E_SHAPE;
    if (!(eps >= 0.0f)) return BITNET_E_ARG;
    if (!aligned16(X) || !aligned16(Xq) || !aligned4(scale_x)) return BITNET_E_ALIGN;
    return hip_status(bitnet::launch_act_quant(X, x_dtype == BITNET_BF16, M, K, eps, Xq, scale_x,
                                               as_stream(stream)));
}

int bitnet_quant_operands(const void* X, int x_dtype, int64_t M, int64_t K, float eps, int8_t* Xq,
                          float* scale_x, const void* W, int w_dtype, int64_t N, uint8_t* W_packed,
                          float* gamma, void* workspace, size_t workspace_bytes, void* stream) {
    if (!X || !Xq || !scale_x || !W || !W_packed || !gamma) return BITNET_E_ARG;
    if (!float_dtype(x_dtype) || !float_dtype(w_dtype)) return BITNET_E_DTYPE;
    if (M < 1 || N < 1 || K < 1 || K % 4 != 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim)
        return BITNET_E_SHAPE;
    if (!(eps >= 0.0f)) return BITNET_E_ARG;
    if (!aligned16(X) || !aligned16(Xq) || !aligned4(scale_x) || !aligned16(W) || !aligned16(W_packed) ||
        !aligned4(gamma))
        return BITNET_E_ALIGN;
    if (!workspace || workspace_bytes < bitnet::weight_quant_ws_bytes(N)) return BITNET_E_WORKSPACE;
    if (!aligned16(workspace)) return BITNET_E_ALIGN;
    return hip_status(bitnet::launch_quant_operands(X, x_dtype == BITNET_BF16, M, K, eps, Xq, scale_x, W,
                                                    w_dtype == BITNET_BF16, N, W_packed, gamma, workspace,
                                                    as_stream(stream)));
}

}  // extern "C"

namespace {

int linear_fwd(const int8_t* Xq, const float* scale_x, const uint8_t* W_packed, const float* gamma,
               int64_t M, int64_t N, int64_t K, float* Y, int32_t* acc, void* stream, bool channel) {
    if (!Xq || !scale_x || !W_packed || !gamma || !Y) return BITNET_E_ARG;
    if (M < 1 || N < 1 || K < 1 || K % 16 != 0 || K >= kMaxK || M > kMaxDim || N >= kMaxFwdN)
        return BITNET_E_SHAPE;
    if (!aligned16(Xq) || !aligned16(W_packed) || !aligned16(Y) || !aligned4(scale_x) ||
        !aligned4(gamma) || (acc && !aligned16(acc)))
        return BITNET_E_ALIGN;
    if (bitnet::gemv_supported(M, K))
        return hip_status(bitnet::launch_gemv_t2(Xq, scale_x, W_packed, gamma, M, N, K, Y, acc,
                                                 as_stream(stream), channel));
    // A few token blocks past the GEMV's 16: the GEMM would run one 128- or
    // 256-row tile per CU through the whole K loop, so each block of 16
    // tokens goes through the GEMV instead (the weights stream once per
    // block; same output bits).  Measured at 11008 x 4096: the GEMM 32-34 us
    // from 17 to 256 tokens, the GEMV 5.4 us per block.
    if (M <= kGemvBlocksMaxM && bitnet::gemv_supported(16, K)) {
        for (int64_t m0 = 0; m0 < M; m0 += 16) {
            const int64_t mb = std::min<int64_t>(16, M - m0);
            const hipError_t e = bitnet::launch_gemv_t2(Xq + m0 * K, scale_x + m0, W_packed, gamma, mb, N, K,
                                                        Y + m0 * N, acc ? acc + m0 * N : nullptr,
                                                        as_stream(stream), channel);
            if (e != hipSuccess) return hip_status(e);
        }
        return BITNET_OK;
    }
    return hip_status(bitnet::launch_gemm_i8t2(Xq, scale_x, W_packed, gamma, M, N, K, Y, acc,
                                               as_stream(stream), channel));
}

}  // namespace

extern "C" {

int bitnet_linear_fwd(const int8_t* Xq, const float* scale_x, const uint8_t* W_packed,
                      const float* gamma, int64_t M, int64_t N, int64_t K, float* Y, int32_t* acc,
                      void* stream) {
    return linear_fwd(Xq, scale_x, W_packed, gamma, M, N, K, Y, acc, stream, false);
}

int bitnet_linear_fwd_channel(const int8_t* Xq, const float* scale_x, const uint8_t* W_packed,
                              const float* s, int64_t M, int64_t N, int64_t K, float* Y, int32_t* acc,
                              void* stream) {
    return linear_fwd(Xq, scale_x, W_packed, s, M, N, K, Y, acc, stream, true);
}

int bitnet_linear_fwd_decode(const void* X, int x_dtype, const uint8_t* W_packed, int w_layout,
                             const float* gamma, int64_t M, int64_t N, int64_t K, float eps, float* Y,
                             int8_t* Xq, float* scale_x, void* stream) {
    if (!X || !W_packed || !gamma || !Y) return BITNET_E_ARG;
    if (!float_dtype(x_dtype)) return BITNET_E_DTYPE;
    if (!(eps >= 0.0f) || (w_layout != BITNET_LAYOUT_ROWS && w_layout != BITNET_LAYOUT_DECODE))
        return BITNET_E_ARG;
    if (M < 1 || N < 1 || K < 1 || K % 16 != 0 || N >= kMaxFwdN ||
        !bitnet::gemv_decode_fits(x_dtype == BITNET_BF16, M, K) ||
        (w_layout == BITNET_LAYOUT_DECODE && !bitnet::decode_layout_supported(K)))
        return BITNET_E_SHAPE;
    if (!aligned16(X) || !aligned16(W_packed) || !aligned16(Y) || !aligned4(gamma) ||
        (Xq && !aligned16(Xq)) || (scale_x && !aligned4(scale_x)))
        return BITNET_E_ALIGN;
    return hip_status(bitnet::launch_gemv_decode(X, x_dtype == BITNET_BF16, W_packed, gamma, M, N, K, eps,
                                                 Y, Xq, scale_x, as_stream(stream),
                                                 w_layout == BITNET_LAYOUT_DECODE));
}

int64_t bitnet_decode_layout_bytes(int64_t N, int64_t K) {
    if (N < 1 || N >= kMaxFwdN || !bitnet::decode_layout_supported(K)) return -1;
    return bitnet::decode_layout_bytes(N, K);
}

int bitnet_pack_decode(const uint8_t* W_packed, int64_t N, int64_t K, uint8_t* W_decode, void* stream) {
    if (!W_packed || !W_decode) return BITNET_E_ARG;
    if (N < 1 || N >= kMaxFwdN || !bitnet::decode_layout_supported(K)) return BITNET_E_SHAPE;
    if (!aligned16(W_packed) || !aligned16(W_decode)) return BITNET_E_ALIGN;
    return hip_status(bitnet::launch_pack_decode(W_packed, N, K, W_decode, as_stream(stream)));
}

int bitnet_weight_quant_rows(const void* W, int w_dtype, int64_t N, int64_t K, uint8_t* W_packed,
                             float* gamma, void* workspace, size_t workspace_bytes, void* stream) {
    if (!W || !W_packed || !gamma) return BITNET_E_ARG;
    if (!float_dtype(w_dtype)) return BITNET_E_DTYPE;
    if (N < 1 || K < 1 || K % 4 != 0 || N > kMaxDim || K > kMaxDim) return BITNET_E_SHAPE;
    if (!aligned16(W) || !aligned16(W_packed) || !aligned4(gamma)) return BITNET_E_ALIGN;
    if (!workspace || workspace_bytes < bitnet::weight_quant_rows_ws_bytes(N)) return BITNET_E_WORKSPACE;
    if (!aligned16(workspace)) return BITNET_E_ALIGN;
    return hip_status(bitnet::launch_weight_quant_rows(W, w_dtype == BITNET_BF16, N, K, W_packed, gamma,
                                                       workspace, as_stream(stream)));
}

}  // extern "C"

namespace {

int linear_bwd(const void* grad_y, int gy_dtype, const int8_t* Xq, const float* scale_x,
               const uint8_t* W_packed, const float* gamma, int64_t M, int64_t N, int64_t K, void* grad_x,
               int gx_dtype, float* grad_W, void* workspace, size_t workspace_bytes, void* stream, bool channel) {
    if (!grad_y || !Xq || !scale_x || !W_packed || !gamma) return BITNET_E_ARG;
    if (!grad_x && !grad_W) return BITNET_E_ARG;
    if (gy_dtype != BITNET_BF16 || !float_dtype(gx_dtype)) return BITNET_E_DTYPE;
    if (M < 1 || N < 1 || K < 1 || K % 16 != 0 || M > kMaxDim || N >= kMaxFwdN || K >= kMaxK)
        return BITNET_E_SHAPE;
    if (!aligned16(grad_y) || !aligned16(Xq) || !aligned16(W_packed) || !aligned4(scale_x) ||
        !aligned4(gamma) || (grad_x && !aligned16(grad_x)) || (grad_W && !aligned16(grad_W)))
        return BITNET_E_ALIGN;
    const size_t need = grad_W ? bitnet::bwd_ws_bytes(M, N, K) : 0;
    if (need > 0 && (!workspace || workspace_bytes < need)) return BITNET_E_WORKSPACE;
    if (need > 0 && !aligned16(workspace)) return BITNET_E_ALIGN;
    return hip_status(bitnet::launch_bwd_ste(static_cast<const uint16_t*>(grad_y), Xq, scale_x,
                                             W_packed, gamma, M, N, K, grad_x,
                                             gx_dtype == BITNET_BF16, grad_W, workspace,
                                             as_stream(stream), bitnet::SteGate{}, channel));
}

}  // namespace

extern "C" {

int bitnet_linear_bwd_ste(const void* grad_y, int gy_dtype, const int8_t* Xq, const float* scale_x,
                          const uint8_t* W_packed, const float* gamma, int64_t M, int64_t N,
                          int64_t K, void* grad_x, int gx_dtype, float* grad_W, void* workspace,
                          size_t workspace_bytes, void* stream) {
    return linear_bwd(grad_y, gy_dtype, Xq, scale_x, W_packed, gamma, M, N, K, grad_x, gx_dtype, grad_W,
                      workspace, workspace_bytes, stream, false);
}

int bitnet_linear_bwd_ste_channel(const void* grad_y, int gy_dtype, const int8_t* Xq, const float* scale_x,
                                  const uint8_t* W_packed, const float* s, int64_t M, int64_t N, int64_t K,
                                  void* grad_x, int gx_dtype, float* grad_W, void* workspace,
                                  size_t workspace_bytes, void* stream) {
    return linear_bwd(grad_y, gy_dtype, Xq, scale_x, W_packed, s, M, N, K, grad_x, gx_dtype, grad_W,
                      workspace, workspace_bytes, stream, true);
}

int bitnet_linear_bwd_ste_gated(const void* grad_y, int gy_dtype, const int8_t* Xq, const float* scale_x,
                                const uint8_t* W_packed, const float* gamma, const void* W, int w_dtype,
                                float w_lo, float w_hi, int64_t M, int64_t N, int64_t K, void* grad_x,
                                int gx_dtype, float* grad_W, void* workspace, size_t workspace_bytes,
                                void* stream) {
    if (!W) return BITNET_E_ARG;
    if (!float_dtype(w_dtype)) return BITNET_E_DTYPE;
    if (w_lo != w_lo || w_hi != w_hi) return BITNET_E_ARG;  // NaN bounds
    if (!aligned16(W)) return BITNET_E_ALIGN;
    if (!grad_y || !Xq || !scale_x || !W_packed || !gamma) return BITNET_E_ARG;
    if (!grad_x && !grad_W) return BITNET_E_ARG;
    if (gy_dtype != BITNET_BF16 || !float_dtype(gx_dtype)) return BITNET_E_DTYPE;
    if (M < 1 || N < 1 || K < 1 || K % 16 != 0 || M > kMaxDim || N >= kMaxFwdN || K >= kMaxK)
        return BITNET_E_SHAPE;
    if (!aligned16(grad_y) || !aligned16(Xq) || !aligned16(W_packed) || !aligned4(scale_x) ||
        !aligned4(gamma) || (grad_x && !aligned16(grad_x)) || (grad_W && !aligned16(grad_W)))
        return BITNET_E_ALIGN;
    const size_t need = grad_W ? bitnet::bwd_ws_bytes(M, N, K) : 0;
    if (need > 0 && (!workspace || workspace_bytes < need)) return BITNET_E_WORKSPACE;
    if (need > 0 && !aligned16(workspace)) return BITNET_E_ALIGN;
    bitnet::SteGate gate;
    gate.w = W;
    gate.bf16 = w_dtype == BITNET_BF16;
    gate.lo = w_lo;
    gate.hi = w_hi;
    return hip_status(bitnet::launch_bwd_ste(static_cast<const uint16_t*>(grad_y), Xq, scale_x,
                                             W_packed, gamma, M, N, K, grad_x,
                                             gx_dtype == BITNET_BF16, grad_W, workspace,
                                             as_stream(stream), gate));
}

int bitnet_weight_clamp(void* W, int w_dtype, int64_t N, int64_t K, float lo, float hi, void* stream) {
    if (!W) return BITNET_E_ARG;
    if (!float_dtype(w_dtype)) return BITNET_E_DTYPE;
    if (N < 1 || K < 1 || N > kMaxDim || K > kMaxDim) return BITNET_E_SHAPE;
    if (!(lo <= hi)) return BITNET_E_ARG;  // also rejects NaN bounds
    if (!aligned16(W)) return BITNET_E_ALIGN;
    return hip_status(bitnet::launch_weight_clamp(W, w_dtype == BITNET_BF16, N * K, lo, hi, as_stream(stream)));
}

int bitnet_code_counts(const uint8_t* W_packed, int64_t N, int64_t K, uint64_t* counts, void* workspace,
                       size_t workspace_bytes, void* stream) {
    if (!W_packed || !counts) return BITNET_E_ARG;
    if (N < 1 || K < 1 || K % 4 != 0 || N > kMaxDim || K > kMaxDim) return BITNET_E_SHAPE;
    if (!aligned16(W_packed) || (reinterpret_cast<uintptr_t>(counts) & 7u) != 0) return BITNET_E_ALIGN;
    if (!workspace || workspace_bytes < bitnet::code_counts_ws_bytes()) return BITNET_E_WORKSPACE;
    if (!aligned16(workspace)) return BITNET_E_ALIGN;
    return hip_status(bitnet::launch_code_counts(W_packed, N * (K / 4), counts, workspace, as_stream(stream)));
}

int bitnet_rmsnorm_bwd(const void* X, int x_dtype, const void* grad_n, int g_dtype, int64_t M,
                       int64_t K, float eps, void* grad_X, int out_dtype, void* stream) {
    if (!X || !grad_n || !grad_X) return BITNET_E_ARG;
    if (!float_dtype(x_dtype) || !float_dtype(g_dtype) || !float_dtype(out_dtype)) return BITNET_E_DTYPE;
    if (M < 1 || K < 1 || K % 8 != 0 || M > kMaxDim || K > kMaxDim) return BITNET_E_SHAPE;
    if (!(eps >= 0.0f)) return BITNET_E_ARG;
    if (!aligned16(X) || !aligned16(grad_n) || !aligned16(grad_X)) return BITNET_E_ALIGN;
    return hip_status(bitnet::launch_rmsnorm_bwd(X, x_dtype == BITNET_BF16, grad_n, g_dtype == BITNET_BF16,
                                                 M, K, eps, grad_X, out_dtype == BITNET_BF16,
                                                 as_stream(stream)));
}

int bitnet_channel_scale_grad(const float* grad_W, const uint8_t* W_packed, int64_t N, int64_t K, float* grad_s,
                              void* stream) {
    if (!grad_W || !W_packed || !grad_s) return BITNET_E_ARG;
    if (N < 1 || K < 1 || K % 16 != 0 || K >= kMaxK || N > kMaxDim) return BITNET_E_SHAPE;
    if (!aligned16(grad_W) || !aligned16(W_packed) || !aligned4(grad_s)) return BITNET_E_ALIGN;
    return hip_status(bitnet::launch_channel_scale_grad(grad_W, W_packed, N, K, grad_s, as_stream(stream)));
}

int bitnet_pack_ternary(const int8_t* codes, int64_t N, int64_t K, uint8_t* W_packed,
                        void* stream) {
    if (!codes || !W_packed) return BITNET_E_ARG;
    if (N < 1 || K < 1 || K % 4 != 0 || N > kMaxDim || K > kMaxDim) return BITNET_E_SHAPE;
    if (!aligned16(codes) || !aligned16(W_packed)) return BITNET_E_ALIGN;
    return hip_status(bitnet::launch_pack_ternary(codes, N, K, W_packed, as_stream(stream)));
}

}  // extern "C"

// ------------------------------------------------ no-allocation weight quant
// bitnet_weight_quant_noalloc keeps the weight quantizer's scratch (the N row
// sums and the code threshold) in this file-scope device array instead of a
// caller workspace.  Each device the library runs on holds its own copy until
// the process ends.  In host code `scratch` names a host-side stand-in, so
// its device address is looked up once per device (hipGetSymbolAddress with
// that device current) and only that address reaches the kernels.
namespace {

constexpr size_t kNoAllocScratchBytes = bitnet::weight_quant_ws_size(BITNET_NOALLOC_MAX_N);

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch` (looked up on the first call on
// that device); BITNET_E_HIP when the lookup fails.
int scratch_ptr(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return BITNET_E_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return BITNET_E_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return BITNET_OK;
}

}  // namespace

extern "C" int bitnet_weight_quant_noalloc(const void* W, int w_dtype, int64_t N, int64_t K, uint8_t* W_packed,
                                           float* gamma, void* stream) {
    if (!W || !W_packed || !gamma) return BITNET_E_ARG;
    if (!float_dtype(w_dtype)) return BITNET_E_DTYPE;
    if (N < 1 || K < 1 || K % 4 != 0 || N > kMaxDim || K > kMaxDim) return BITNET_E_SHAPE;
    if (N > BITNET_NOALLOC_MAX_N) return BITNET_E_SCRATCH;
    if (!aligned16(W) || !aligned16(W_packed) || !aligned4(gamma)) return BITNET_E_ALIGN;
    if (bitnet::weight_quant_ws_bytes(N) > kNoAllocScratchBytes) return BITNET_E_SCRATCH;
    void* ws = nullptr;
    const int st = scratch_ptr(&ws);
    if (st != BITNET_OK) return st;
    // the kernels overwrite every scratch word they read (row sums, then the
    // threshold): nothing needs clearing
    return hip_status(bitnet::launch_weight_quant(W, w_dtype == BITNET_BF16, N, K, W_packed, gamma, ws,
                                                  as_stream(stream)));
}
