// Ternary x int8 GEMM on gfx950 int8 matrix cores (prefill / training shapes).
//
//   acc[m][n] = sum_k Xq[m][k] * code[n][k]     exact int32
//   Y[m][n]   = acc[m][n] * (gamma / scale_x[m])
//
// The linear layer of "BitNet 1.5技术解析：2比特量化在神经网络中的应用与挑战"
// (3.1) on the integer operands, with the wide accumulator asked for in its
// 5.2; the +1 / -1 / 0 codes are the add / subtract / skip of
// "1.58-bit量化技术突破AI算力与内存墙限制" (3.1), evaluated here as an exact
// int8 dot product on v_mfma_i32_32x32x32_i8.
//
// Tiling: a 256 x 256 output tile per 512-thread workgroup, 8 waves as 2 (M)
// x 4 (N), each wave 128 x 64 = 4 x 2 MFMA blocks of 32 x 32.  K advances 64
// per step.  The activation tile (256 x 64 B) is staged in LDS with each
// 16-byte chunk byte-transposed 4 x 4; the weight tile stays 2-bit packed in
// LDS (256 x 16 B, a quarter of the int8 bytes) and each wave unpacks its
// operand in registers right before the MFMA (unpack16 yields the same
// transposed column order, so every product pairs equal columns; the sum over
// k is exact and order-free).  Two LDS buffers; the next step's global loads
// are in flight while the current step computes.
#include "common.h"

namespace bitnet {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kThreads = 512;
constexpr int A_STRIDE = 80;  // 64 data bytes + 16 pad: conflict-free b128 reads
constexpr int B_STRIDE = 24;  // 16 packed bytes + 8 pad: conflict-free b64 reads
constexpr int A_BYTES = BM * A_STRIDE;
constexpr int B_BYTES = BN * B_STRIDE;
constexpr int BUF_BYTES = A_BYTES + B_BYTES;

// Workgroup id -> tile, XCD-aware: consecutive ids go round-robin over the
// 8 XCDs, so ids are regrouped to give each XCD a contiguous run of tiles
// (row-major over tiles), which then share A rows in that XCD's L2.
__device__ __forceinline__ void tile_of(int wg, int tiles_m, int tiles_n, int& tm, int& tn) {
    const int G = tiles_m * tiles_n;
    const int q = G / 8, r = G % 8;
    const int x = wg % 8, local = wg / 8;
    const int id = (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + local;
    tm = id / tiles_n;
    tn = id % tiles_n;
}

struct Prefetch {
    uint4 a[2];      // two 16-byte activation chunks
    uint32_t b[2];   // two packed weight dwords
};

}  // namespace

__global__ __launch_bounds__(kThreads) void gemm_i8t2_kernel(
    const int8_t* __restrict__ Xq, const float* __restrict__ scale_x,
    const uint8_t* __restrict__ Wp, const float* __restrict__ gamma_p, int M, int N, int K,
    float* __restrict__ Y, int32_t* __restrict__ acc_out) {
    __shared__ __align__(16) uint8_t smem[2 * BUF_BYTES];
    __shared__ float row_scale[BM];

    int tm, tn;
    tile_of(blockIdx.x, (M + BM - 1) / BM, (N + BN - 1) / BN, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int wm = wave >> 2, wn = wave & 3;  // 2 x 4 waves
    const int KB = K / 4;                     // packed bytes per weight row
    const int nk = (K + BK - 1) / BK;

    {
        const float g = *gamma_p;
        if (t < BM) row_scale[t] = (m0 + t < M) ? g / scale_x[m0 + t] : 0.0f;
    }

    auto load_global = [&](int it, Prefetch& p) {
        const int k0 = it * BK;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int c = t + u * kThreads;  // 0..1023: 256 rows x 4 chunks
            const int row = c >> 2, ch = c & 3;
            const int k = k0 + ch * 16;
            if (m0 + row < M && k < K)
                p.a[u] = *reinterpret_cast<const uint4*>(Xq + (int64_t)(m0 + row) * K + k);
            else
                p.a[u] = make_uint4(0, 0, 0, 0);
            if (n0 + row < N && k < K)
                p.b[u] = *reinterpret_cast<const uint32_t*>(Wp + (int64_t)(n0 + row) * KB + k / 4);
            else
                p.b[u] = 0u;
        }
    };
    auto store_lds = [&](int buf, const Prefetch& p) {
        uint8_t* As = smem + buf * BUF_BYTES;
        uint8_t* Bs = As + A_BYTES;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int c = t + u * kThreads;
            const int row = c >> 2, ch = c & 3;
            const uint32_t in[4] = {p.a[u].x, p.a[u].y, p.a[u].z, p.a[u].w};
            uint32_t o[4];
            transpose4x4_bytes(in, o);
            *reinterpret_cast<uint4*>(As + row * A_STRIDE + ch * 16) = make_uint4(o[0], o[1], o[2], o[3]);
            *reinterpret_cast<uint32_t*>(Bs + row * B_STRIDE + ch * 4) = p.b[u];
        }
    };

    v16i acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

    Prefetch pf;
    load_global(0, pf);
    store_lds(0, pf);
    __syncthreads();

    const int g = lane >> 5;    // lane group: k chunks 2g, 2g+1 of the step
    const int l32 = lane & 31;  // row (A) / column (B) inside a 32-block
    for (int it = 0; it < nk; ++it) {
        const int buf = it & 1;
        if (it + 1 < nk) load_global(it + 1, pf);
        const uint8_t* As = smem + buf * BUF_BYTES;
        const uint8_t* Bs = As + A_BYTES;
        uint2 bp[2];
#pragma unroll
        for (int j = 0; j < 2; ++j)
            bp[j] = *reinterpret_cast<const uint2*>(Bs + (wn * 64 + j * 32 + l32) * B_STRIDE + 8 * g);
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
            v4i a[4], b[2];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint4 v = *reinterpret_cast<const uint4*>(
                    As + (wm * 128 + i * 32 + l32) * A_STRIDE + 32 * g + 16 * kh);
                a[i] = v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                uint32_t u[4];
                unpack16(kh ? bp[j].y : bp[j].x, u);
                b[j] = v4i{(int)u[0], (int)u[1], (int)u[2], (int)u[3]};
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        if (it + 1 < nk) store_lds(buf ^ 1, pf);
        __syncthreads();
    }

    // Epilogue.  32x32 block layout: lane holds column l32 and rows
    // 8*(r/4) + 4*g + r%4 for r = 0..15.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int col = n0 + wn * 64 + j * 32 + l32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int rloc = wm * 128 + i * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
                const int row = m0 + rloc;
                if (row < M && col < N) {
                    const int v = acc[i][j][r];
                    Y[(int64_t)row * N + col] = (float)v * row_scale[rloc];
                    if (acc_out) acc_out[(int64_t)row * N + col] = v;
                }
            }
        }
    }
}

hipError_t launch_gemm_i8t2(const int8_t* Xq, const float* scale_x, const uint8_t* Wp,
                            const float* gamma, int64_t M, int64_t N, int64_t K, float* Y,
                            int32_t* acc, hipStream_t s) {
    const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    gemm_i8t2_kernel<<<(unsigned)tiles, kThreads, 0, s>>>(Xq, scale_x, Wp, gamma, (int)M, (int)N,
                                                          (int)K, Y, acc);
    return hipGetLastError();
}

}  // namespace bitnet
