// Calibration kernels: the measured ceilings the BitLinear kernels are
// compared with on the part they run on (include/bitnet_calib.h).
//
//  - stream_read_kernel: the plainest one-launch read of a byte range (16-byte
//    loads, grid-stride, several loads in flight per thread).  Its time for
//    the byte count of a bandwidth-bound call (the decode GEMV's packed
//    weights, the quantizers' operands) is the single-launch ceiling of that
//    call: launch, ramp and drain included, no arithmetic.
//  - mfma_loop_kernel: back-to-back v_mfma_i32_32x32x32_i8 (int8) or
//    v_mfma_f32_32x32x16_bf16 (bf16) on pseudo-random register operands,
//    four independent accumulators per wave, consecutive MFMAs on different
//    operands (the multipliers toggle as in a GEMM on random data).  Its rate
//    is the matrix cores' ceiling at the clock they hold under that load,
//    which each workgroup reports from the shader cycle counter against the
//    100 MHz real-time counter.
#include "../../include/bitnet_calib.h"
#include "common.h"

namespace bitnet {
namespace calib {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 4;  // 16-byte loads in flight per thread and step
constexpr uint32_t kNever = 0x9e3779b9u;  // a sum the sink is written for (never, in practice)

__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const uint4* __restrict__ src, int64_t n16,
                                                                   uint32_t* __restrict__ sink) {
    const int64_t stride = (int64_t)gridDim.x * kReadThreads;
    int64_t i = (int64_t)blockIdx.x * kReadThreads + threadIdx.x;
    uint32_t x = 0;
    for (; i + (kReadUnroll - 1) * stride < n16; i += kReadUnroll * stride) {
        uint4 v[kReadUnroll];
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) v[u] = src[i + u * stride];
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += stride) {
        const uint4 v = src[i];
        x ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (x == kNever) sink[0] = x;  // keeps the loads; a plain vector store
}

__device__ __forceinline__ uint32_t mix(uint32_t h) {
    h ^= h >> 16;
    h *= 0x7feb352du;
    h ^= h >> 15;
    h *= 0x846ca68bu;
    h ^= h >> 16;
    return h;
}

// bf16 bits of a value in [1, 2) with random mantissa (no denormals, no Inf)
__device__ __forceinline__ uint32_t bf16_pair(uint32_t h) {
    return ((h & 0x007f007fu) | 0x3f803f80u) ^ ((h & 0x80008000u));
}

// one ternary code from 8 random bits: 0 with probability 90/256 (about
// 0.35), else +1 or -1 with equal probability
__device__ __forceinline__ uint32_t ternary_of(uint32_t v8) { return v8 < 90u ? 0u : ((v8 & 1u) ? 1u : 0xffu); }

// four ternary codes as int8 bytes
__device__ __forceinline__ uint32_t ternary_bytes(uint32_t h) {
    return ternary_of(h & 0xffu) | (ternary_of((h >> 8) & 0xffu) << 8) | (ternary_of((h >> 16) & 0xffu) << 16) |
           (ternary_of(h >> 24) << 24);
}

// two ternary codes as bf16 bits (0, +1.0 = 0x3f80, -1.0 = 0xbf80)
__device__ __forceinline__ uint32_t ternary_bf16_pair(uint32_t h) {
    const uint32_t lo = ternary_of(h & 0xffu), hi = ternary_of((h >> 8) & 0xffu);
    const uint32_t blo = lo == 0u ? 0u : (lo == 1u ? 0x3f80u : 0xbf80u);
    const uint32_t bhi = hi == 0u ? 0u : (hi == 1u ? 0x3f80u : 0xbf80u);
    return blo | (bhi << 16);
}

// KIND: 0 = int8 32x32x32 on random bytes, 1 = bf16 32x32x16 on random
// values, 2 = int8 with ternary codes as the second operand, 3 = bf16 with
// ternary codes as the second operand
template <int KIND>
__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, uint32_t* __restrict__ sink,
                                                        uint64_t* __restrict__ clocks) {
    const uint32_t seed = mix(blockIdx.x * 256u + threadIdx.x + 1u);
    uint64_t c0 = 0, r0 = 0;
    if (threadIdx.x == 0) {
        c0 = __builtin_readcyclecounter();
        r0 = __builtin_amdgcn_s_memrealtime();
    }
    uint32_t fold = 0;
    if constexpr (KIND == 0 || KIND == 2) {
        v4i a[4], b[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                a[j][e] = (int)mix(seed + 97u * (j * 4 + e));
                const uint32_t hb = mix(seed ^ (0x51ed27u * (j * 4 + e + 1)));
                b[j][e] = (int)(KIND == 2 ? ternary_bytes(hb) : hb);
            }
        v16i acc[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = v16i{};
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[j], b[(j + 1) & 3], acc[j], 0, 0, 0);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[(j + 2) & 3], b[j], acc[j], 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) fold ^= (uint32_t)acc[j][e];
    } else {
        v8bf a[4], b[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t pa = bf16_pair(mix(seed + 97u * (j * 4 + e)));
                const uint32_t hb = mix(seed ^ (0x51ed27u * (j * 4 + e + 1)));
                const uint32_t pb = KIND == 3 ? ternary_bf16_pair(hb) : bf16_pair(hb);
                a[j][2 * e] = __builtin_bit_cast(__bf16, (uint16_t)(pa & 0xffffu));
                a[j][2 * e + 1] = __builtin_bit_cast(__bf16, (uint16_t)(pa >> 16));
                b[j][2 * e] = __builtin_bit_cast(__bf16, (uint16_t)(pb & 0xffffu));
                b[j][2 * e + 1] = __builtin_bit_cast(__bf16, (uint16_t)(pb >> 16));
            }
        v16f acc[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = v16f{};
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j], b[(j + 1) & 3], acc[j], 0, 0, 0);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(j + 2) & 3], b[j], acc[j], 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) fold ^= __float_as_uint(acc[j][e]);
    }
    if (threadIdx.x == 0) {
        const uint64_t c1 = __builtin_readcyclecounter();
        const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
        uint64_t* out = clocks + 2 * (int64_t)blockIdx.x;
        out[0] = c1 - c0;  // shader clock cycles of wave 0
        out[1] = r1 - r0;  // 100 MHz real-time ticks over the same span
    }
    if (fold == kNever) sink[0] = fold;
}

}  // namespace calib
}  // namespace bitnet

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

using bitnet::calib::kReadThreads;
using bitnet::calib::mfma_loop_kernel;
using bitnet::calib::stream_read_kernel;

extern "C" {

int bitnet_calib_stream_read(const void* src, int64_t bytes, int workgroups, uint32_t* sink, void* stream) {
    if (!src || !sink) return BITNET_E_ARG;
    if (bytes < 16 || bytes % 16 != 0 || workgroups < 1 || workgroups > (1 << 20)) return BITNET_E_SHAPE;
    if (!aligned16(src) || (reinterpret_cast<uintptr_t>(sink) & 3u) != 0) return BITNET_E_ALIGN;
    hipLaunchKernelGGL(stream_read_kernel, dim3(workgroups), dim3(kReadThreads), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint4*>(src), bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? BITNET_OK : BITNET_E_HIP;
}

int bitnet_calib_mfma(int kind, int workgroups, int iters, uint32_t* sink, uint64_t* clocks, void* stream) {
    if (!sink || !clocks) return BITNET_E_ARG;
    if (kind < BITNET_CALIB_MFMA_I8 || kind > BITNET_CALIB_MFMA_BF16_TERNARY) return BITNET_E_ARG;
    if (workgroups < 1 || workgroups > (1 << 20) || iters < 1) return BITNET_E_SHAPE;
    if ((reinterpret_cast<uintptr_t>(sink) & 3u) != 0 || (reinterpret_cast<uintptr_t>(clocks) & 7u) != 0)
        return BITNET_E_ALIGN;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    switch (kind) {
        case BITNET_CALIB_MFMA_I8:
            hipLaunchKernelGGL(mfma_loop_kernel<0>, dim3(workgroups), dim3(256), 0, s, iters, sink, clocks);
            break;
        case BITNET_CALIB_MFMA_BF16:
            hipLaunchKernelGGL(mfma_loop_kernel<1>, dim3(workgroups), dim3(256), 0, s, iters, sink, clocks);
            break;
        case BITNET_CALIB_MFMA_I8_TERNARY:
            hipLaunchKernelGGL(mfma_loop_kernel<2>, dim3(workgroups), dim3(256), 0, s, iters, sink, clocks);
            break;
        default:
            hipLaunchKernelGGL(mfma_loop_kernel<3>, dim3(workgroups), dim3(256), 0, s, iters, sink, clocks);
            break;
    }
    return hipGetLastError() == hipSuccess ? BITNET_OK : BITNET_E_HIP;
}

double bitnet_calib_mfma_ops(int kind, int workgroups, int iters) {
    // 4 waves a workgroup, 8 MFMAs a wave and iteration; 2*32*32*32 int8 ops
    // or 2*32*32*16 bf16 flops each
    const bool i8 = kind == BITNET_CALIB_MFMA_I8 || kind == BITNET_CALIB_MFMA_I8_TERNARY;
    const double per = i8 ? 65536.0 : 32768.0;
    if (workgroups < 1 || iters < 1 || kind < BITNET_CALIB_MFMA_I8 || kind > BITNET_CALIB_MFMA_BF16_TERNARY)
        return 0.0;
    return (double)workgroups * 4.0 * 8.0 * (double)iters * per;
}

}  // extern "C"
