// Backward of the unit-gain RMSNorm in front of the activation quantizer.
//
// "BitNet 1.5技术解析：2比特量化在神经网络中的应用与挑战" (3.1) normalises the
// BitLinear input with an RMSNorm before the absmax quantizer; the pages give
// no backward for it, so this is the exact derivative of that forward (mean
// of squares over the row, eps inside the root, unit gain).  Per row, with
// r = 1/sqrt(sum_k x_k^2 / K + eps) and n = x * r:
//   dL/dx_j = r * (g_j - n_j * c),   c = (sum_k g_k * n_k) / K = r * (sum_k g_k x_k) / K
// g = dL/dn is the STE backward's grad_x.  One pass accumulates sum x^2 and
// sum g*x per row, a second writes dL/dx.  fp32 arithmetic throughout; the
// result decides no integer (a gradient checked against a float64 reference).
//
// HBM-bound: x, g read once (a second time from cache for long rows), dx
// written once.  One wave per row; lane l holds 8 consecutive elements of
// every 512-element block, so each load is a coalesced 16-byte (bf16) or
// 2 x 16-byte (fp32) piece.  Rows of at most 16 blocks (8 with fp32 x and g)
// stay in registers between the passes, as the raw loaded bytes; longer
// rows are read twice.
#include "common.h"

namespace bitnet {

namespace {

constexpr int kNbWaves = 4;
constexpr int kNbChunk = 8;                 // elements per lane and block
constexpr int kNbBlock = kWave * kNbChunk;  // 512

// 16-byte pieces holding 8 elements of T
template <typename T>
constexpr int kPieces = (int)sizeof(T) / 2;
// raw bytes of 8 elements at byte offset `off` (kBufOOB: zeros)
template <typename T>
__device__ __forceinline__ void load_raw(__amdgpu_buffer_rsrc_t r, uint32_t off, uint4 (&p)[kPieces<T>]) {
#pragma unroll
    for (int i = 0; i < kPieces<T>; ++i) p[i] = buf_load16(r, off == kBufOOB ? kBufOOB : off + 16 * i);
}
__device__ __forceinline__ void widen(const uint4 (&p)[2], float (&v)[8]) {  // fp32
    const uint32_t w[8] = {p[0].x, p[0].y, p[0].z, p[0].w, p[1].x, p[1].y, p[1].z, p[1].w};
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = __uint_as_float(w[i]);
}
__device__ __forceinline__ void widen(const uint4 (&p)[1], float (&v)[8]) {  // bf16
    const uint32_t w[4] = {p[0].x, p[0].y, p[0].z, p[0].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}
// rows of NB blocks fit the register cache (at most 192 registers of raw bytes)
template <typename TX, typename TG>
constexpr bool cache_fits(int nb) { return nb * (kPieces<TX> + kPieces<TG>) * 4 <= 192; }

__device__ __forceinline__ void store8(float* p, const float (&v)[8]) {
    reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
    reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
}
__device__ __forceinline__ void store8(uint16_t* p, const float (&v)[8]) {  // bf16, round to nearest even
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const __bf16 lo = (__bf16)v[2 * i], hi = (__bf16)v[2 * i + 1];
        w[i] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
    *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
}

}  // namespace

// TX, TG: float or uint16_t (bf16 bits); TO: float or uint16_t (bf16).
// NB > 0: the row (at most NB blocks) stays in registers; NB == 0: any K.
template <typename TX, typename TG, typename TO, int NB>
__global__ __launch_bounds__(kNbWaves * kWave) void rmsnorm_bwd_kernel(
    const TX* __restrict__ X, const TG* __restrict__ G, int64_t M, int64_t K, float eps,
    TO* __restrict__ Out) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t row =
        (int64_t)blockIdx.x * kNbWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (row >= M) return;  // uniform per wave
    const __amdgpu_buffer_rsrc_t rx = make_buf(X + row * K), rg = make_buf(G + row * K);
    const int64_t nblk = (K + kNbBlock - 1) / kNbBlock;
    // lane's chunk of block b: first element, and whether it lies in the row
    // (K % 8 == 0, so a chunk is all in or all out)
    auto first = [&](int64_t b) { return b * kNbBlock + (int64_t)lane * kNbChunk; };
    auto offset = [&](int64_t b, int elem_bytes) -> uint32_t {
        return first(b) < K ? (uint32_t)(first(b) * elem_bytes) : kBufOOB;
    };
    using RawX = uint4[kPieces<TX>];
    using RawG = uint4[kPieces<TG>];
    auto load_pair_raw = [&](int64_t b, RawX& x, RawG& g) {
        load_raw<TX>(rx, offset(b, (int)sizeof(TX)), x);
        load_raw<TG>(rg, offset(b, (int)sizeof(TG)), g);
    };
    auto load_pair = [&](int64_t b, float (&x)[8], float (&g)[8]) {
        RawX xr;
        RawG gr;
        load_pair_raw(b, xr, gr);
        widen(xr, x);
        widen(gr, g);
    };
    float sq = 0.0f, gx = 0.0f;
    auto accumulate = [&](const float (&x)[8], const float (&g)[8]) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            sq += x[i] * x[i];
            gx += g[i] * x[i];
        }
    };
    float r = 0.0f, c = 0.0f;
    auto finish_sums = [&] {
        const float ss = wave_tree_sum(sq), sgx = wave_tree_sum(gx);
        const float ms = ss / (float)K;
        const float d = sqrtf(ms + eps);
        r = 1.0f / d;
        c = (r * sgx) / (float)K;
    };
    auto write = [&](int64_t b, const float (&x)[8], const float (&g)[8]) {
        if (first(b) >= K) return;
        float o[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = r * (g[i] - (x[i] * r) * c);
        store8(Out + row * K + first(b), o);
    };

    if constexpr (NB > 0) {
        static_assert(cache_fits<TX, TG>(NB), "row cache exceeds the register budget");
        RawX xr[NB];
        RawG gr[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) load_pair_raw(b, xr[b], gr[b]);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            float x[8], g[8];
            widen(xr[b], x);
            widen(gr[b], g);
            accumulate(x, g);
        }
        finish_sums();
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            // an empty register constraint: the floats widened for the sums
            // are not kept live until here
#pragma unroll
            for (int i = 0; i < kPieces<TX>; ++i) asm volatile("" : "+v"(xr[b][i].x), "+v"(xr[b][i].y), "+v"(xr[b][i].z), "+v"(xr[b][i].w));
#pragma unroll
            for (int i = 0; i < kPieces<TG>; ++i) asm volatile("" : "+v"(gr[b][i].x), "+v"(gr[b][i].y), "+v"(gr[b][i].z), "+v"(gr[b][i].w));
            float x[8], g[8];
            widen(xr[b], x);
            widen(gr[b], g);
            write(b, x, g);
        }
    } else {
        constexpr int kInFlight = 2;  // blocks loaded per round
        for (int64_t b0 = 0; b0 < nblk; b0 += kInFlight) {
            float xs[kInFlight][8], gs[kInFlight][8];
#pragma unroll
            for (int u = 0; u < kInFlight; ++u) load_pair(b0 + u < nblk ? b0 + u : nblk, xs[u], gs[u]);
#pragma unroll
            for (int u = 0; u < kInFlight; ++u) accumulate(xs[u], gs[u]);
        }
        finish_sums();
        for (int64_t b0 = 0; b0 < nblk; b0 += kInFlight) {
            float xs[kInFlight][8], gs[kInFlight][8];
#pragma unroll
            for (int u = 0; u < kInFlight; ++u) load_pair(b0 + u < nblk ? b0 + u : nblk, xs[u], gs[u]);
#pragma unroll
            for (int u = 0; u < kInFlight; ++u)
                if (b0 + u < nblk) write(b0 + u, xs[u], gs[u]);
        }
    }
}

namespace {

template <typename TX, typename TG, typename TO>
hipError_t rmsnorm_bwd_dispatch(const TX* X, const TG* G, int64_t M, int64_t K, float eps, TO* Out,
                                hipStream_t s) {
    const int64_t nblk = (K + kNbBlock - 1) / kNbBlock;
    const dim3 grid((unsigned)((M + kNbWaves - 1) / kNbWaves)), block(kNbWaves * kWave);
    if (nblk <= 1)
        rmsnorm_bwd_kernel<TX, TG, TO, 1><<<grid, block, 0, s>>>(X, G, M, K, eps, Out);
    else if (nblk <= 2)
        rmsnorm_bwd_kernel<TX, TG, TO, 2><<<grid, block, 0, s>>>(X, G, M, K, eps, Out);
    else if (nblk <= 4)
        rmsnorm_bwd_kernel<TX, TG, TO, 4><<<grid, block, 0, s>>>(X, G, M, K, eps, Out);
    else if (nblk <= 8)
        rmsnorm_bwd_kernel<TX, TG, TO, 8><<<grid, block, 0, s>>>(X, G, M, K, eps, Out);
    else if (nblk <= 16 && cache_fits<TX, TG>(16))
        rmsnorm_bwd_kernel<TX, TG, TO, cache_fits<TX, TG>(16) ? 16 : 0><<<grid, block, 0, s>>>(X, G, M, K, eps, Out);
    else
        rmsnorm_bwd_kernel<TX, TG, TO, 0><<<grid, block, 0, s>>>(X, G, M, K, eps, Out);
    return hipGetLastError();
}

template <typename TX, typename TG>
hipError_t rmsnorm_bwd_out(const TX* X, const TG* G, int64_t M, int64_t K, float eps, void* Out,
                           bool out_bf16, hipStream_t s) {
    if (out_bf16) return rmsnorm_bwd_dispatch(X, G, M, K, eps, static_cast<uint16_t*>(Out), s);
    return rmsnorm_bwd_dispatch(X, G, M, K, eps, static_cast<float*>(Out), s);
}

template <typename TX>
hipError_t rmsnorm_bwd_g(const TX* X, const void* G, bool g_bf16, int64_t M, int64_t K, float eps,
                         void* Out, bool out_bf16, hipStream_t s) {
    if (g_bf16) return rmsnorm_bwd_out(X, static_cast<const uint16_t*>(G), M, K, eps, Out, out_bf16, s);
    return rmsnorm_bwd_out(X, static_cast<const float*>(G), M, K, eps, Out, out_bf16, s);
}

}  // namespace

hipError_t launch_rmsnorm_bwd(const void* X, bool x_bf16, const void* G, bool g_bf16, int64_t M,
                              int64_t K, float eps, void* Out, bool out_bf16, hipStream_t s) {
    if (M <= 0 || K <= 0 || K % kNbChunk != 0) return hipErrorInvalidValue;
    if (x_bf16) return rmsnorm_bwd_g(static_cast<const uint16_t*>(X), G, g_bf16, M, K, eps, Out, out_bf16, s);
    return rmsnorm_bwd_g(static_cast<const float*>(X), G, g_bf16, M, K, eps, Out, out_bf16, s);
}

}  // namespace bitnet
