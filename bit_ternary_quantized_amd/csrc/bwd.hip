// Straight-through-estimator backward of the BitLinear layer on gfx950
// bf16 matrix cores.
//
// "BitNet 1.5技术解析：2比特量化在神经网络中的应用与挑战" (2.1, 2.2) writes both
// quantizers with the detach trick and "1.58-bit量化技术突破AI算力与内存墙限制"
// (3.2) returns the incoming gradient unchanged, so the layer's gradients are
// those of a plain linear map at the dequantized operands:
//   grad_x[m][k] = gamma * sum_n gy[m][n] * code[n][k]
//   grad_W[n][k] =         sum_m gy[m][n] * (Xq[m][k] / scale_x[m])
// "BitNet 三元权重量化训练工程" (gradient-clipping section) pairs a bf16
// forward with fp32 gradients: operands are bf16 (codes and gy exactly, the
// dequantized activations rounded once), accumulation is fp32.
//
// Both products contract over the slow index of one operand, so three
// layout passes first write contraction-contiguous bf16 operands into the
// workspace (codes^T [K][N], gy^T [N][M], X_deq^T [K][M]); one bf16 NT GEMM
// kernel (C = alpha * A * B^T, A [M'][K'], B [N'][K'], both K'-contiguous)
// then computes either gradient.
#include "common.h"

namespace bitnet {

namespace {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // NaN stays NaN
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

constexpr int TT = 64;  // transpose tile edge

}  // namespace

// ------------------------------------------------------------ layout passes
// codes (packed [N][K/4]) -> Ct [K][N] bf16 (+1 = 0x3f80, -1 = 0xbf80, 0 = 0).
__global__ __launch_bounds__(256) void codes_to_bf16_t_kernel(const uint8_t* __restrict__ Wp,
                                                              int N, int K,
                                                              uint16_t* __restrict__ Ct) {
    __shared__ uint16_t tile[TT][TT + 2];  // [k][n]
    const int n0 = blockIdx.x * TT, k0 = blockIdx.y * TT;
    const int t = threadIdx.x;
    {
        const int nl = t >> 2, d = t & 3;  // row, packed dword (16 codes)
        const int n = n0 + nl, k = k0 + 16 * d;
        uint32_t w = 0u;
        if (n < N && k < K) w = *reinterpret_cast<const uint32_t*>(Wp + (int64_t)n * (K / 4) + k / 4);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const uint32_t c = (w >> (2 * j)) & 3u;
            tile[16 * d + j][nl] = c == 1u ? 0x3f80u : (c == 2u ? 0xbf80u : 0u);
        }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < (TT * TT) / (256 * 2); ++u) {  // two bf16 per store
        const int idx = t + u * 256;
        const int kl = idx / (TT / 2), np = idx % (TT / 2);
        const int k = k0 + kl, n = n0 + 2 * np;
        if (k < K) {
            if (n + 1 < N && (N % 2) == 0) {  // 4-byte aligned pair
                const uint32_t v = (uint32_t)tile[kl][2 * np] | ((uint32_t)tile[kl][2 * np + 1] << 16);
                *reinterpret_cast<uint32_t*>(Ct + (int64_t)k * N + n) = v;
            } else {
                if (n < N) Ct[(int64_t)k * N + n] = tile[kl][2 * np];
                if (n + 1 < N) Ct[(int64_t)k * N + n + 1] = tile[kl][2 * np + 1];
            }
        }
    }
}

// gy [M][N] bf16 -> gyT [N][M] bf16
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const uint16_t* __restrict__ src,
                                                             int R, int C,
                                                             uint16_t* __restrict__ dst) {
    __shared__ uint16_t tile[TT][TT + 2];
    const int r0 = blockIdx.y * TT, c0 = blockIdx.x * TT;
    const int t = threadIdx.x;
#pragma unroll
    for (int u = 0; u < (TT * TT) / 256; ++u) {
        const int idx = t + u * 256;
        const int rl = idx / TT, cl = idx % TT;
        const int r = r0 + rl, c = c0 + cl;
        tile[rl][cl] = (r < R && c < C) ? src[(int64_t)r * C + c] : (uint16_t)0;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < (TT * TT) / 256; ++u) {
        const int idx = t + u * 256;
        const int cl = idx / TT, rl = idx % TT;
        const int r = r0 + rl, c = c0 + cl;
        if (r < R && c < C) dst[(int64_t)c * R + r] = tile[rl][cl];
    }
}

// Xq [M][K] int8, scale_x [M] -> XdT [K][M] bf16 = bf16(Xq / scale_x)
__global__ __launch_bounds__(256) void xdeq_t_kernel(const int8_t* __restrict__ Xq,
                                                     const float* __restrict__ scale_x, int M,
                                                     int K, uint16_t* __restrict__ XdT) {
    __shared__ uint16_t tile[TT][TT + 2];  // [m][k]
    const int m0 = blockIdx.y * TT, k0 = blockIdx.x * TT;
    const int t = threadIdx.x;
#pragma unroll
    for (int u = 0; u < (TT * TT) / 256; ++u) {
        const int idx = t + u * 256;
        const int ml = idx / TT, kl = idx % TT;
        const int m = m0 + ml, k = k0 + kl;
        uint16_t v = 0;
        if (m < M && k < K) v = f32_to_bf16_rne((float)Xq[(int64_t)m * K + k] / scale_x[m]);
        tile[ml][kl] = v;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < (TT * TT) / 256; ++u) {
        const int idx = t + u * 256;
        const int kl = idx / TT, ml = idx % TT;
        const int m = m0 + ml, k = k0 + kl;
        if (m < M && k < K) XdT[(int64_t)k * M + m] = tile[ml][kl];
    }
}

// ------------------------------------------------------------ bf16 NT GEMM
// C[m][n] = alpha * sum_k A[m][k] * B[n][k]; 256 x 256 tile per 512-thread
// workgroup, 8 waves as 2 x 4, each 128 x 64 = 4 x 2 blocks of
// v_mfma_f32_32x32x16_bf16; K advances 32 per step.  Lane group g reads
// 16-byte chunks 2g and 2g+1 of a step for both operands (any common
// assignment of k to MFMA slots gives the same sum).
namespace {
constexpr int GBM = 256, GBN = 256, GBK = 32;
constexpr int GT = 512;
constexpr int G_STRIDE = 80;  // 64 data bytes + 16 pad
constexpr int G_TILE = GBM * G_STRIDE;

__device__ __forceinline__ void tile_of2(int wg, int tiles_m, int tiles_n, int& tm, int& tn) {
    const int G = tiles_m * tiles_n;
    const int q = G / 8, r = G % 8;
    const int x = wg % 8, local = wg / 8;
    const int id = (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + local;
    tm = id / tiles_n;
    tn = id % tiles_n;
}
}  // namespace

template <bool OUT_BF16>
__global__ __launch_bounds__(GT) void gemm_bf16_nt_kernel(const uint16_t* __restrict__ A,
                                                          const uint16_t* __restrict__ B, int M,
                                                          int N, int K,
                                                          const float* __restrict__ alpha_p,
                                                          void* __restrict__ Cout) {
    __shared__ __align__(16) uint8_t smem[2][2 * G_TILE];
    int tm, tn;
    tile_of2(blockIdx.x, (M + GBM - 1) / GBM, (N + GBN - 1) / GBN, tm, tn);
    const int m0 = tm * GBM, n0 = tn * GBN;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wm = wave >> 2, wn = wave & 3;
    const int nk = (K + GBK - 1) / GBK;
    const bool vec = (K % 8) == 0;

    auto load = [&](const uint16_t* P, int rows, int r0, int k0, int row, int ch) -> uint4 {
        const int r = r0 + row, k = k0 + ch * 8;
        if (r < rows && k < K) {
            const uint16_t* p = P + (int64_t)r * K + k;
            if (vec && k + 8 <= K) return *reinterpret_cast<const uint4*>(p);
            uint16_t e[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) e[i] = (k + i < K) ? p[i] : (uint16_t)0;
            uint32_t w[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) w[i] = (uint32_t)e[2 * i] | ((uint32_t)e[2 * i + 1] << 16);
            return make_uint4(w[0], w[1], w[2], w[3]);
        }
        return make_uint4(0, 0, 0, 0);
    };
    uint4 pa[2], pb[2];
    auto load_global = [&](int it) {
        const int k0 = it * GBK;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int c = t + u * GT;  // 256 rows x 4 chunks of 8 bf16
            pa[u] = load(A, M, m0, k0, c >> 2, c & 3);
            pb[u] = load(B, N, n0, k0, c >> 2, c & 3);
        }
    };
    auto store_lds = [&](int buf) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int c = t + u * GT;
            const int off = (c >> 2) * G_STRIDE + (c & 3) * 16;
            *reinterpret_cast<uint4*>(&smem[buf][off]) = pa[u];
            *reinterpret_cast<uint4*>(&smem[buf][G_TILE + off]) = pb[u];
        }
    };

    v16f acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    load_global(0);
    store_lds(0);
    __syncthreads();
    const int g = lane >> 5, l32 = lane & 31;
    for (int it = 0; it < nk; ++it) {
        const int buf = it & 1;
        if (it + 1 < nk) load_global(it + 1);
        const uint8_t* As = smem[buf];
        const uint8_t* Bs = smem[buf] + G_TILE;
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
            v8bf a[4], b[2];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                a[i] = *reinterpret_cast<const v8bf*>(As + (wm * 128 + i * 32 + l32) * G_STRIDE +
                                                      32 * g + 16 * kh);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                b[j] = *reinterpret_cast<const v8bf*>(Bs + (wn * 64 + j * 32 + l32) * G_STRIDE +
                                                      32 * g + 16 * kh);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        if (it + 1 < nk) store_lds(buf ^ 1);
        __syncthreads();
    }

    const float alpha = alpha_p ? *alpha_p : 1.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int col = n0 + wn * 64 + j * 32 + l32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm * 128 + i * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
                if (row < M && col < N) {
                    const float v = acc[i][j][r] * alpha;
                    if constexpr (OUT_BF16)
                        static_cast<uint16_t*>(Cout)[(int64_t)row * N + col] = f32_to_bf16_rne(v);
                    else
                        static_cast<float*>(Cout)[(int64_t)row * N + col] = v;
                }
            }
        }
    }
}

// ------------------------------------------------------------ launcher
namespace {
size_t align256(size_t b) { return (b + 255) / 256 * 256; }
}  // namespace

size_t bwd_ws_bytes(int64_t M, int64_t N, int64_t K) {
    return align256((size_t)K * N * 2) + align256((size_t)N * M * 2) + align256((size_t)K * M * 2);
}

hipError_t launch_bwd_ste(const uint16_t* gy, const int8_t* Xq, const float* scale_x,
                          const uint8_t* Wp, const float* gamma, int64_t M, int64_t N, int64_t K,
                          void* grad_x, bool gx_bf16, float* grad_W, void* ws, hipStream_t s) {
    uint8_t* base = static_cast<uint8_t*>(ws);
    uint16_t* Ct = reinterpret_cast<uint16_t*>(base);
    uint16_t* gyT = reinterpret_cast<uint16_t*>(base + align256((size_t)K * N * 2));
    uint16_t* XdT = reinterpret_cast<uint16_t*>(base + align256((size_t)K * N * 2) +
                                                align256((size_t)N * M * 2));
    const int m = (int)M, n = (int)N, k = (int)K;
    if (grad_x) {
        codes_to_bf16_t_kernel<<<dim3((n + TT - 1) / TT, (k + TT - 1) / TT), 256, 0, s>>>(Wp, n, k, Ct);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const unsigned tiles = (unsigned)(((M + GBM - 1) / GBM) * ((K + GBN - 1) / GBN));
        if (gx_bf16)
            gemm_bf16_nt_kernel<true><<<tiles, GT, 0, s>>>(gy, Ct, m, k, n, gamma, grad_x);
        else
            gemm_bf16_nt_kernel<false><<<tiles, GT, 0, s>>>(gy, Ct, m, k, n, gamma, grad_x);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (grad_W) {
        transpose_bf16_kernel<<<dim3((n + TT - 1) / TT, (m + TT - 1) / TT), 256, 0, s>>>(gy, m, n, gyT);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        xdeq_t_kernel<<<dim3((k + TT - 1) / TT, (m + TT - 1) / TT), 256, 0, s>>>(Xq, scale_x, m, k, XdT);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        const unsigned tiles = (unsigned)(((N + GBM - 1) / GBM) * ((K + GBN - 1) / GBN));
        gemm_bf16_nt_kernel<false><<<tiles, GT, 0, s>>>(gyT, XdT, n, k, m, nullptr, grad_W);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace bitnet
