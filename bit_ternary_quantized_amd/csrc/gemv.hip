// Packed-weight GEMV for decode (M <= 16 tokens) on gfx950.
//
//   acc[m][n] = sum_k Xq[m][k] * code[n][k]     exact int32
//   Y[m][n]   = acc[m][n] * (gamma / scale_x[m])
//
// Decode is bound by streaming the 2-bit weights from HBM once (the memory
// wall of "1.58-bit量化技术突破AI算力与内存墙限制", section 1); the
// add / subtract / skip of its 3.1 is computed as an exact int8 dot product.
// Unpacking codes costs VALU work per weight regardless of M, so the
// products run on v_mfma_i32_16x16x64_i8 with the tokens padded to 16: the
// matrix-core time is then independent of M as well.
//
// One 256-thread workgroup owns 16 weight rows; its 4 waves split K into
// quarters.  Inside a wave, lane group g = lane/16 owns a contiguous quarter
// of the wave's K range, and MFMA step s takes the s-th 16-column chunk of
// every group's range, so each lane streams one contiguous run of packed
// bytes of its weight row (the sum over k is order-free, and activations are
// gathered with the same mapping).  Partial int32 tiles meet in LDS.
#include "common.h"

namespace bitnet {

namespace {
typedef int v4i __attribute__((ext_vector_type(4)));
constexpr int kRows = 16;    // weight rows per workgroup (MFMA N)
constexpr int kWaves = 4;    // K split
constexpr int kMaxSteps = 64;  // MFMA steps per wave handled by the template
}  // namespace

// STEPS: MFMA k-steps (64 columns each) per wave; lane group range = 16*STEPS.
template <int STEPS>
__global__ __launch_bounds__(kWaves * 64) void gemv_t2_kernel(
    const int8_t* __restrict__ Xq, const float* __restrict__ scale_x,
    const uint8_t* __restrict__ Wp, const float* __restrict__ gamma_p, int M, int N, int K,
    float* __restrict__ Y, int32_t* __restrict__ acc_out) {
    __shared__ int red[kWaves][kRows * 16];
    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int n0 = blockIdx.x * kRows;
    const int col = lane & 15;  // weight row inside the tile / token for A
    const int g = lane >> 4;    // lane group
    constexpr int GR = 16 * STEPS;                     // columns per lane group
    const int kbase = wave * (4 * GR) + g * GR;        // first column of this lane
    const int KB = K / 4;
    const bool vec = (KB % 16) == 0;  // packed rows 16-byte aligned

    // weights: row n0+col, columns [kbase, kbase + GR): GR/4 packed bytes
    uint32_t wq[STEPS];
    {
        const int n = n0 + col;
        const uint8_t* src = Wp + (int64_t)n * KB + kbase / 4;
#pragma unroll
        for (int s = 0; s < STEPS; s += 4) {
            // 16 bytes = 4 steps when fully inside the row
            if (vec && n < N && kbase + 16 * (s + 4) <= K) {
                const uint4 v = *reinterpret_cast<const uint4*>(src + 4 * s);
                wq[s] = v.x; wq[s + 1] = v.y; wq[s + 2] = v.z; wq[s + 3] = v.w;
            } else {
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    wq[s + u] = (n < N && kbase + 16 * (s + u) < K)
                                    ? *reinterpret_cast<const uint32_t*>(src + 4 * (s + u))
                                    : 0u;
            }
        }
    }

    v4i acc = {0, 0, 0, 0};
    const int tok = col;
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
        const int k = kbase + 16 * s;
        uint32_t a4[4] = {0u, 0u, 0u, 0u};
        if (tok < M && k < K) {
            const uint4 v = *reinterpret_cast<const uint4*>(Xq + (int64_t)tok * K + k);
            a4[0] = v.x; a4[1] = v.y; a4[2] = v.z; a4[3] = v.w;
        }
        uint32_t at[4], b[4];
        transpose4x4_bytes(a4, at);
        unpack16(wq[s], b);
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(
            v4i{(int)at[0], (int)at[1], (int)at[2], (int)at[3]},
            v4i{(int)b[0], (int)b[1], (int)b[2], (int)b[3]}, acc, 0, 0, 0);
    }
    // 16x16 output layout: lane holds column lane%16 (weight row) and rows
    // (tokens) 4*(lane/16) + r.
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][(4 * g + r) * 16 + col] = acc[r];
    __syncthreads();
    {
        const int tk = t >> 4, nn = t & 15;  // 256 threads = 16 tokens x 16 rows
        const int sum = red[0][t] + red[1][t] + red[2][t] + red[3][t];
        if (tk < M && n0 + nn < N) {
            const float rs = *gamma_p / scale_x[tk];
            Y[(int64_t)tk * N + n0 + nn] = (float)sum * rs;
            if (acc_out) acc_out[(int64_t)tk * N + n0 + nn] = sum;
        }
    }
}

hipError_t launch_gemv_t2(const int8_t* Xq, const float* scale_x, const uint8_t* Wp,
                          const float* gamma, int64_t M, int64_t N, int64_t K, float* Y,
                          int32_t* acc, hipStream_t s) {
    // steps per wave: K / (4 waves * 4 groups * 16 columns), rounded up to 4
    int64_t steps = (K + 255) / 256;
    steps = (steps + 3) / 4 * 4;
    const dim3 grid((unsigned)((N + kRows - 1) / kRows)), block(kWaves * 64);
#define BITNET_GEMV_CASE(S)                                                                    \
    if (steps <= S) {                                                                          \
        gemv_t2_kernel<S><<<grid, block, 0, s>>>(Xq, scale_x, Wp, gamma, (int)M, (int)N,       \
                                                 (int)K, Y, acc);                              \
        return hipGetLastError();                                                              \
    }
    BITNET_GEMV_CASE(4)
    BITNET_GEMV_CASE(8)
    BITNET_GEMV_CASE(16)
    BITNET_GEMV_CASE(32)
    BITNET_GEMV_CASE(64)
#undef BITNET_GEMV_CASE
    (void)kMaxSteps;
    return hipErrorInvalidValue;  // K beyond 16384: the ABI routes it to the GEMM
}

}  // namespace bitnet
