// Gradient of a learned per-output-channel weight scale.
//
// "BitNet量化感知训练中的梯度传播优化" (blog.hotdry.top), section on the
// BitLinear implementation, 1 (weight scaling): output = (sign(W) . s) x with
// s in R^{d_out x 1}, one scale per output row learned by gradient descent.
// With y[m][n] = s[n] * sum_k X_deq[m][k] * code[n][k], the chain rule gives
//   grad_s[n] = sum_m grad_y[m][n] * sum_k X_deq[m][k] * code[n][k]
//             = sum_k code[n][k] * G[n][k],   G = grad_y^T X_deq,
// and G is exactly the STE backward's grad_W (the gradient with respect to
// the dequantized weights), so the scale gradient is one pass over grad_W
// and the packed codes: a row-wise dot product with codes in {-1, 0, +1}.
//
// channel_scale_grad_kernel: one wave per output row.  Lane l holds
// elements 4l .. 4l+3 of every 256-element block of the row (a 16-byte
// grad_W load, coalesced 1 KB per wave instruction) and the byte of packed
// codes that covers them (a dword load shared by four lanes).  Each product
// code * G is one binary32 multiplication (exact); the row is summed in the
// library's canonical order: the in-lane tree over 4, the 64-lane tree, then
// the pairwise tree over the blocks, and a zero total is returned as +0.
// Bound: HBM, N*K*4 + N*K/4 bytes read, 4*N written.
#include "common.h"

namespace bitnet {

namespace {

constexpr int kRowsPerGroup = 4;  // waves (rows) per 256-thread workgroup
constexpr int kInFlight = 4;      // 256-element blocks requested ahead per wave

__device__ __forceinline__ float code_value(uint32_t bits2) {
    // 00 -> 0, 01 -> +1, 10 -> -1 (11 is never written; read as 0)
    return bits2 == 1u ? 1.0f : (bits2 == 2u ? -1.0f : 0.0f);
}

}  // namespace

__global__ __launch_bounds__(kRowsPerGroup * kWave) void channel_scale_grad_kernel(
    const float* __restrict__ G, const uint8_t* __restrict__ Wp, int64_t N, int K, float* __restrict__ gs) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t n = (int64_t)blockIdx.x * kRowsPerGroup + (threadIdx.x >> 6);
    if (n >= N) return;  // uniform in the wave
    const int KB = K / 4;  // packed bytes per row (a multiple of 4: K % 16 == 0)
    const __amdgpu_buffer_rsrc_t rg = make_buf(G + n * (int64_t)K);
    const __amdgpu_buffer_rsrc_t rc = make_buf(Wp + n * (int64_t)KB);
    const int nblk = (K + 255) / 256;
    PairwiseStack stack;
    for (int b0 = 0; b0 < nblk; b0 += kInFlight) {
        uint4 gv[kInFlight];
        uint32_t cw[kInFlight];
#pragma unroll
        for (int u = 0; u < kInFlight; ++u) {
            // element 4*lane of block b0 + u, and the dword of packed codes
            // holding its byte; K % 16 == 0, so both are wholly in or out of
            // the row (out: the buffer reads zeros)
            const int k = (b0 + u) * 256 + 4 * lane;
            const bool in = b0 + u < nblk && k < K;
            gv[u] = buf_load16(rg, in ? (uint32_t)k * 4u : kBufOOB);
            cw[u] = buf_load4(rc, in ? (uint32_t)((k >> 2) & ~3) : kBufOOB);
        }
#pragma unroll
        for (int u = 0; u < kInFlight; ++u) {
            if (b0 + u >= nblk) break;  // uniform
            const uint32_t byte = (cw[u] >> (8 * (lane & 3))) & 0xffu;
            const float g[4] = {__uint_as_float(gv[u].x), __uint_as_float(gv[u].y), __uint_as_float(gv[u].z),
                                __uint_as_float(gv[u].w)};
            float p[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) p[i] = code_value((byte >> (2 * i)) & 3u) * g[i];
            stack.push(wave_tree_sum(lane_tree<4>(p)));
        }
    }
    if (lane == 0) gs[n] = stack.total() + 0.0f;
}

hipError_t launch_channel_scale_grad(const float* G, const uint8_t* Wp, int64_t N, int64_t K, float* gs,
                                     hipStream_t s) {
    const int64_t groups = (N + kRowsPerGroup - 1) / kRowsPerGroup;
    channel_scale_grad_kernel<<<(unsigned)groups, kRowsPerGroup * kWave, 0, s>>>(G, Wp, N, (int)K, gs);
    return hipGetLastError();
}

}  // namespace bitnet
