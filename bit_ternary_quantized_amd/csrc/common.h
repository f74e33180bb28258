// Internal helpers shared by the gfx950 kernels of the BitLinear library.
// Not part of the public ABI (include/bitnet.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace bitnet {

constexpr int kWave = 64;  // CDNA wavefront width
// s_waitcnt operand (gfx9 encoding) that waits for lgkmcnt 0 only: vmcnt at
// its maximum 63 (bits 3:0 and 15:14), expcnt at its maximum 7 (bits 6:4)
constexpr int kWaitLgkm0 = 0xC07F;
// s_waitcnt operand that waits for vmcnt 0 only (expcnt 7, lgkmcnt 15)
constexpr int kWaitVm0 = 0x0F70;

// ------------------------------------------------------------ element loads
// bf16 -> fp32 is exact: the 16 bits are the high half of the binary32.
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
    return __uint_as_float(b16 << 16);
}

// 16 bytes of a row as floats: 4 fp32 or 8 bf16 elements.
template <typename T> struct Vec16;
template <> struct Vec16<float> {
    static constexpr int E = 4;
    __device__ __forceinline__ static void load(const float* p, float (&v)[4]) {
        const float4 q = *reinterpret_cast<const float4*>(p);
        v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
    }
};
template <> struct Vec16<uint16_t> {  // bf16 stored as raw bits
    static constexpr int E = 8;
    __device__ __forceinline__ static void load(const uint16_t* p, float (&v)[8]) {
        const uint4 q = *reinterpret_cast<const uint4*>(p);
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(w[i] << 16);
            v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
};

// the 16 raw bytes of a Vec16 load, widened to floats
template <typename T>
__device__ __forceinline__ void widen16(const uint4& r, float (&v)[Vec16<T>::E]) {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
    if constexpr (Vec16<T>::E == 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(w[i]);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(w[i] << 16);
            v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
}

__device__ __forceinline__ float load_elem(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float load_elem(const uint16_t* p, int64_t i) {
    return bf16_bits_to_f32(p[i]);
}

// ------------------------------------------------------------ buffer loads
// Raw buffer loads through a resource descriptor (gfx9 layout).  The
// hardware checks every offset against the descriptor's size: an offset at
// or past it reads zeros and touches no memory.  Tile loads use this for
// their tails (offset kBufOOB) instead of a branch or a clamped address, and
// the loads can neither be predicated away nor moved under a branch by the
// compiler.  Valid offsets stay below 2^31 (the callers bound their sizes).
constexpr uint32_t kBufOOB = 0x80000000u;
constexpr int kBufMaxBytes = 0x7fffffff;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_buf(const void* base) {
    // word 3 = 0x00020000: 32-bit data format, no swizzle, no added thread id
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, kBufMaxBytes,
                                             0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ uint2 buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
__device__ __forceinline__ uint32_t buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

// ---------------------------------------------------- canonical tree sums
// The library's summation order: pad to a power of two with +0 and add as a
// perfect binary tree in index order.  Aligned power-of-two blocks may be
// summed independently and then combined as a tree; both helpers below keep
// that structure exactly.

// In-lane tree over E (power of two) consecutive values.
template <int E>
__device__ __forceinline__ float lane_tree(const float (&v)[E]) {
    float t[E];
#pragma unroll
    for (int i = 0; i < E; ++i) t[i] = v[i];
#pragma unroll
    for (int w = 1; w < E; w *= 2) {
#pragma unroll
        for (int i = 0; i < E; i += 2 * w) t[i] = t[i] + t[i + w];
    }
    return t[0];
}

// The tree over the 64 lanes in lane order; every lane ends with the total.
// Level m adds each lane's subtree sum to its sibling's (lane l ^ m), so the
// two lanes of a pair add the same two values (commutative: identical bits).
// Levels 1 and 2 read the sibling with a DPP quad permutation.  Levels 4 and
// 8: every lane of an aligned group of m already holds that group's sum, so
// any lane of the sibling group will do, and the row half-mirror (lane i of
// 8 reads 7 - i) and row mirror (i of 16 reads 15 - i) reach one.  The last
// two levels add the four 16-lane sums read from lanes 0, 16, 32, 48.
// Every lane must be active.
template <int CTRL>
__device__ __forceinline__ float dpp_read(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}
constexpr int kDppXor1 = 0xb1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4e;        // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

__device__ __forceinline__ float lane_read(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

__device__ __forceinline__ float wave_tree_sum(float v) {
    v = v + dpp_read<kDppXor1>(v);
    v = v + dpp_read<kDppXor2>(v);
    v = v + dpp_read<kDppHalfMirror>(v);
    v = v + dpp_read<kDppMirror>(v);
    return (lane_read(v, 0) + lane_read(v, 16)) + (lane_read(v, 32) + lane_read(v, 48));
}

// The int8 codes of four quantizer products y = fl(fl(x * inv) * scale),
// packed into one dword (element 0 in the low byte): clamp to [-128, 127],
// then round half to even by adding 1.5 * 2^23 (in [2^23, 2^24) the unit in
// the last place is 1, so the addition itself rounds to the nearest integer,
// ties to even, and leaves that integer in the low mantissa bits as two's
// complement); two byte permutes and an or gather the four low bytes.  For
// every non-NaN y this equals clamp(rint(y), -128, 127): clamping to integer
// bounds commutes with rounding to an integer.
__device__ __forceinline__ uint32_t q8x4(float y0, float y1, float y2, float y3) {
    constexpr float kRound = 12582912.0f;  // 1.5 * 2^23
    const uint32_t a = __float_as_uint(fminf(fmaxf(y0, -128.0f), 127.0f) + kRound);
    const uint32_t b = __float_as_uint(fminf(fmaxf(y1, -128.0f), 127.0f) + kRound);
    const uint32_t c = __float_as_uint(fminf(fmaxf(y2, -128.0f), 127.0f) + kRound);
    const uint32_t d = __float_as_uint(fminf(fmaxf(y3, -128.0f), 127.0f) + kRound);
    // v_perm_b32(S0, S1, sel): selector byte 0-3 picks a byte of S1, 4-7 of S0, 0x0c gives 0
    return __builtin_amdgcn_perm(b, a, 0x0c0c0400u) | __builtin_amdgcn_perm(d, c, 0x04000c0cu);
}

__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp_read<kDppXor1>(v));
    v = fmaxf(v, dpp_read<kDppXor2>(v));
    v = fmaxf(v, dpp_read<kDppHalfMirror>(v));
    v = fmaxf(v, dpp_read<kDppMirror>(v));
    return fmaxf(fmaxf(lane_read(v, 0), lane_read(v, 16)), fmaxf(lane_read(v, 32), lane_read(v, 48)));
}

// Pairwise combination of a stream of equal-size, consecutive, aligned
// blocks (a binary counter): after pushing leaves 0..n-1, total() is the
// tree over them zero-padded to a power of two.  The leaf count must be
// uniform across the wave so that every branch is uniform.
struct PairwiseStack {
    static constexpr int kLevels = 26;
    float part[kLevels];
    uint32_t n = 0;
    __device__ __forceinline__ void push(float s) {
        bool done = false;
#pragma unroll
        for (int l = 0; l < kLevels; ++l) {
            if (!done) {
                if ((n >> l) & 1u) {
                    s = part[l] + s;
                } else {
                    part[l] = s;
                    done = true;
                }
            }
        }
        ++n;
    }
    __device__ __forceinline__ float total() const {
        float acc = 0.0f;
        bool have = false;
#pragma unroll
        for (int l = 0; l < kLevels; ++l) {
            if ((n >> l) & 1u) {
                acc = have ? part[l] + acc : part[l];
                have = true;
            }
        }
        return acc;
    }
};

// ------------------------------------------------------------ 2-bit codes
// Packed layout: code of column k in bits 2(k%4)..2(k%4)+1 of byte k/4;
// 00 = 0, 01 = +1, 10 = -1.
//
// unpack16: one packed dword (16 codes, columns c0..c0+15) -> 16 int8 in
// four dwords.  Dword j holds the codes of columns c0+j, c0+4+j, c0+8+j,
// c0+12+j in bytes 0..3 (a 4x4 byte transpose of the natural order); the
// other matrix-core operand is brought into the same order with
// transpose4x4_bytes() so that every dot product pairs equal columns.
//
// Nine VALU operations per 16 codes.  v_perm_b32 picks byte sel (0..7) of
// {S0, S1} (S1 = bytes 0..3), and for sel 8 the sign of byte 1 replicated,
// for sel 12 the byte 0x00.  Codes 0 and 2 of each byte are masked in place
// (sel 0..3) and looked up in kLut; codes 1 and 3 are masked without a shift
// (sel 0, 4, 8, 12 for the codes 00, 01, 10, 11) and looked up in the pair
// {S0 = 0x01, S1 = 0x8000}: sel 0 -> 0x00, 4 -> 0x01, 8 -> 0xff (sign of
// 0x80), 12 -> 0x00.  The unused code 11 unpacks to 0 in every position.
__device__ __forceinline__ void unpack16(uint32_t w, uint32_t (&out)[4]) {
    // byte LUT indexed by the 2-bit code: 0 -> 0x00, 1 -> 0x01, 2 -> 0xff
    constexpr uint32_t kLut = 0x00ff0100u;
    out[0] = __builtin_amdgcn_perm(0u, kLut, w & 0x03030303u);
    out[1] = __builtin_amdgcn_perm(0x00000001u, 0x00008000u, w & 0x0C0C0C0Cu);
    const uint32_t w4 = w >> 4;
    out[2] = __builtin_amdgcn_perm(0u, kLut, w4 & 0x03030303u);
    out[3] = __builtin_amdgcn_perm(0x00000001u, 0x00008000u, w4 & 0x0C0C0C0Cu);
}

// a[j] byte b -> out[b] byte j.
__device__ __forceinline__ void transpose4x4_bytes(const uint32_t (&a)[4], uint32_t (&o)[4]) {
    // perm(S0, S1, sel): selector byte 0..3 picks S1 bytes, 4..7 picks S0.
    const uint32_t t0 = __builtin_amdgcn_perm(a[1], a[0], 0x06020400u);  // a0.0 a1.0 a0.2 a1.2
    const uint32_t t1 = __builtin_amdgcn_perm(a[1], a[0], 0x07030501u);  // a0.1 a1.1 a0.3 a1.3
    const uint32_t t2 = __builtin_amdgcn_perm(a[3], a[2], 0x06020400u);  // a2.0 a3.0 a2.2 a3.2
    const uint32_t t3 = __builtin_amdgcn_perm(a[3], a[2], 0x07030501u);  // a2.1 a3.1 a2.3 a3.3
    o[0] = __builtin_amdgcn_perm(t2, t0, 0x05040100u);
    o[1] = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
    o[2] = __builtin_amdgcn_perm(t2, t0, 0x07060302u);
    o[3] = __builtin_amdgcn_perm(t3, t1, 0x07060302u);
}

// ------------------------------------------------------------- launchers
// Host-side launchers, one per kernel family; arguments are validated by the
// ABI layer before these run.  Each returns hipSuccess or the launch error.
hipError_t launch_act_quant(const void* X, bool x_bf16, int64_t M, int64_t K, float eps,
                            int8_t* Xq, float* scale_x, hipStream_t s);
hipError_t launch_weight_quant(const void* W, bool w_bf16, int64_t N, int64_t K,
                               uint8_t* W_packed, float* gamma, void* ws, hipStream_t s);
// weight_quant's workspace: the N row sums, the code threshold and the
// ceil(N/4) four-row tree nodes, each 256-byte aligned
constexpr size_t weight_quant_ws_size(int64_t N) {
    return (size_t)(((N * 4 + 255) / 256) * 256 + 256 + (((N + 3) / 4 * 4 + 255) / 256) * 256);
}
size_t weight_quant_ws_bytes(int64_t N);
// reads of the published weight-quant threshold before a pack workgroup
// evaluates it itself; returns the previous value
int set_gate_polls(int n);
// weight_quant and the code counts (zeros, +1, -1, 11) of the codes it packs
hipError_t launch_weight_quant_counted(const void* W, bool w_bf16, int64_t N, int64_t K, uint8_t* W_packed,
                                       float* gamma, uint64_t* counts, void* ws, hipStream_t s);
size_t weight_quant_counted_ws_bytes(int64_t N, int64_t K);
// act_quant of X and weight_quant of W (same K) with one launch fewer;
// outputs bit-identical to the two; ws as weight_quant's
hipError_t launch_quant_operands(const void* X, bool x_bf16, int64_t M, int64_t K, float eps, int8_t* Xq,
                                 float* scale_x, const void* W, bool w_bf16, int64_t N, uint8_t* W_packed,
                                 float* gamma, void* ws, hipStream_t s);
hipError_t launch_weight_quant_rows(const void* W, bool w_bf16, int64_t N, int64_t K, uint8_t* W_packed,
                                    float* gamma, void* ws, hipStream_t s);
size_t weight_quant_rows_ws_bytes(int64_t N);
hipError_t launch_pack_ternary(const int8_t* codes, int64_t N, int64_t K, uint8_t* W_packed,
                               hipStream_t s);
// channel: gamma holds one scale per output channel [N] (else one scalar)
hipError_t launch_gemm_i8t2(const int8_t* Xq, const float* scale_x, const uint8_t* Wp,
                            const float* gamma, int64_t M, int64_t N, int64_t K, float* Y,
                            int32_t* acc, hipStream_t s, bool channel = false);
hipError_t launch_gemv_t2(const int8_t* Xq, const float* scale_x, const uint8_t* Wp,
                          const float* gamma, int64_t M, int64_t N, int64_t K, float* Y,
                          int32_t* acc, hipStream_t s, bool channel = false);
constexpr int64_t kGemvMaxM = 16;
bool gemv_supported(int64_t M, int64_t K);  // M <= 16 and the activations fit LDS
// Fused decode: act_quant of X (fp32 or bf16) and the packed GEMV in one
// launch; xq_out / sx_out (optional) receive q and scale_x.
hipError_t launch_gemv_decode(const void* X, bool x_bf16, const uint8_t* Wp, const float* gamma,
                              int64_t M, int64_t N, int64_t K, float eps, float* Y, int8_t* xq_out,
                              float* sx_out, hipStream_t s, bool decode_layout);
// the decode layout of a packed W (gemv.hip): supported K, bytes, the repack
bool decode_layout_supported(int64_t K);
int64_t decode_layout_bytes(int64_t N, int64_t K);
hipError_t launch_pack_decode(const uint8_t* Wp, int64_t N, int64_t K, uint8_t* Wd, hipStream_t s);
// M <= 16, K <= 4096 and M * ceil(K / (64 * elements per 16 bytes)) <= 128
// (every bf16 shape; fp32: M * ceil(K / 256) <= 128, e.g. 8 rows of 4096)
bool gemv_decode_fits(bool x_bf16, int64_t M, int64_t K);
// Range gate of the master-weight gradient: grad_W[n][k] is kept where
// lo <= W[n][k] <= hi and set to 0 elsewhere; w == nullptr: no gate.
struct SteGate {
    const void* w = nullptr;
    int bf16 = 0;  // W is bf16 (else fp32)
    float lo = 0.0f, hi = 0.0f;
};
// channel: gamma holds one scale per output channel [N] (grad_x only uses it)
hipError_t launch_bwd_ste(const uint16_t* gy, const int8_t* Xq, const float* scale_x,
                          const uint8_t* Wp, const float* gamma, int64_t M, int64_t N, int64_t K,
                          void* grad_x, bool gx_bf16, float* grad_W, void* ws, hipStream_t s,
                          const SteGate& gate = SteGate{}, bool channel = false);
hipError_t launch_weight_clamp(void* W, bool w_bf16, int64_t count, float lo, float hi, hipStream_t s);
hipError_t launch_code_counts(const uint8_t* W_packed, int64_t nbytes, uint64_t* counts, void* ws,
                              hipStream_t s);
size_t code_counts_ws_bytes();
size_t bwd_ws_bytes(int64_t M, int64_t N, int64_t K);
// grad_s[n] = sum_k code[n][k] * G[n][k] (canonical tree; K % 16 == 0)
hipError_t launch_channel_scale_grad(const float* G, const uint8_t* Wp, int64_t N, int64_t K, float* gs,
                                     hipStream_t s);
hipError_t launch_rmsnorm_bwd(const void* X, bool x_bf16, const void* G, bool g_bf16, int64_t M,
                              int64_t K, float eps, void* Out, bool out_bf16, hipStream_t s);

}  // namespace bitnet
