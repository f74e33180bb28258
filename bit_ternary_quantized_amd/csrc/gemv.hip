// Packed-weight GEMV for decode (M <= 16 tokens) on gfx950.
//
//   acc[m][n] = sum_k Xq[m][k] * code[n][k]     exact int32
//   Y[m][n]   = acc[m][n] * (gamma / scale_x[m])
//
// Decode is bound by streaming the 2-bit weights from HBM once (the memory
// wall of "1.58-bit量化技术突破AI算力与内存墙限制", section 1); the
// add / subtract / skip of its 3.1 is computed as an exact int8 dot product.
// Unpacking codes costs VALU work per weight whatever M is, so the products
// run on v_mfma_i32_16x16x64_i8 with the tokens padded to 16 and the
// matrix-core time is independent of M as well.
//
// Data flow.  One 1024-thread workgroup per CU (16 waves).  Weight rows come
// in groups of 16 (one MFMA N block); workgroup w owns groups w, w+G, ...
// Every packed weight byte the workgroup needs is requested first, with no
// branch in front of the loads, so the whole matrix is in flight at once.
// The activations (16 x K int8, tokens >= M zero) are staged once in LDS,
// each 16-byte chunk byte-transposed 4 x 4 to match the column order
// unpack16 produces.  The 16 waves split K: wave v owns columns
// [v*Kw, (v+1)*Kw), its lane group g = lane/16 the contiguous quarter
// [v*Kw + g*Kw/4, ...), and MFMA step s the s-th 16-column chunk of every
// quarter (the sum over k is exact and order-free).  The 16 partial int32
// tiles meet in LDS.
#include "common.h"

namespace bitnet {

namespace {
typedef int v4i __attribute__((ext_vector_type(4)));
constexpr int kWaves = 16;
constexpr int kThreads = kWaves * 64;
constexpr int kMaxKLds = 8192;            // activation tile K bound (LDS)
constexpr int kAStride = kMaxKLds + 16;   // bytes per token row in LDS (+pad)
constexpr int kMaxGroups = 8;             // row groups prefetched per pass
}  // namespace

// S: MFMA steps (64 columns) per wave, Kw = 64*S; FULL: K == 16*Kw, so every
// lane's column range lies inside the row and loads are 16-byte vectors.
template <int S, bool FULL>
__global__ __launch_bounds__(kThreads) void gemv_t2_kernel(
    const int8_t* __restrict__ Xq, const float* __restrict__ scale_x,
    const uint8_t* __restrict__ Wp, const float* __restrict__ gamma_p, int M, int N, int K,
    float* __restrict__ Y, int32_t* __restrict__ acc_out) {
    __shared__ __align__(16) uint8_t As[16 * kAStride];
    __shared__ int red[kWaves][256];
    constexpr int Kw = 64 * S;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int col = lane & 15, g = lane >> 4;
    const int kb = wave * Kw + g * (Kw / 4);  // first column of this lane
    const int KB = K / 4;
    const int ngroups = (N + 15) / 16;

    for (int base = blockIdx.x; base < ngroups; base += gridDim.x * kMaxGroups) {
        // ---- weights for up to kMaxGroups row groups, all loads first
        uint32_t wq[kMaxGroups][S];
#pragma unroll
        for (int r = 0; r < kMaxGroups; ++r) {
            const int grp = base + r * gridDim.x;
            const int n = grp * 16 + col;
            const bool nv = grp < ngroups && n < N;
            const int nc = nv ? n : 0;  // clamped address, value dropped below
            const uint8_t* src = Wp + (int64_t)nc * KB + kb / 4;
            if constexpr (FULL && S % 4 == 0) {
#pragma unroll
                for (int s = 0; s < S; s += 4) {
                    const uint4 v = *reinterpret_cast<const uint4*>(src + 4 * s);
                    wq[r][s] = nv ? v.x : 0u;
                    wq[r][s + 1] = nv ? v.y : 0u;
                    wq[r][s + 2] = nv ? v.z : 0u;
                    wq[r][s + 3] = nv ? v.w : 0u;
                }
            } else {
#pragma unroll
                for (int s = 0; s < S; ++s) {
                    const bool kv = kb + 16 * s < K;
                    const uint32_t v = *reinterpret_cast<const uint32_t*>(
                        Wp + (int64_t)nc * KB + (kv ? (kb + 16 * s) / 4 : 0));
                    wq[r][s] = (nv && kv) ? v : 0u;
                }
            }
        }

        // ---- activations -> LDS (first pass only; they do not change)
        if (base == (int)blockIdx.x) {
            const int kch = K / 16;  // 16-byte chunks per token row
            for (int c = t; c < 16 * kch; c += kThreads) {
                const int tok = c / kch, kc = c - tok * kch;
                const bool tv = tok < M;
                const uint4 v = *reinterpret_cast<const uint4*>(Xq + (int64_t)(tv ? tok : 0) * K + 16 * kc);
                const uint32_t a[4] = {tv ? v.x : 0u, tv ? v.y : 0u, tv ? v.z : 0u, tv ? v.w : 0u};
                uint32_t o[4];
                transpose4x4_bytes(a, o);
                *reinterpret_cast<uint4*>(As + tok * kAStride + 16 * kc) = make_uint4(o[0], o[1], o[2], o[3]);
            }
            __syncthreads();
        }

        // ---- products, one row group at a time
#pragma unroll
        for (int r = 0; r < kMaxGroups; ++r) {
            const int grp = base + r * gridDim.x;
            if (grp >= ngroups) break;  // uniform over the workgroup
            v4i acc = {0, 0, 0, 0};
#pragma unroll
            for (int s = 0; s < S; ++s) {
                const int k = kb + 16 * s;
                uint4 av = make_uint4(0, 0, 0, 0);
                if (FULL || k < K) av = *reinterpret_cast<const uint4*>(As + col * kAStride + k);
                uint32_t b[4];
                unpack16(wq[r][s], b);
                acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                    v4i{(int)av.x, (int)av.y, (int)av.z, (int)av.w},
                    v4i{(int)b[0], (int)b[1], (int)b[2], (int)b[3]}, acc, 0, 0, 0);
            }
            // 16x16 layout: lane holds weight row lane%16, tokens 4*(lane/16)+i
#pragma unroll
            for (int i = 0; i < 4; ++i) red[wave][(4 * g + i) * 16 + col] = acc[i];
            __syncthreads();
            if (t < 256) {
                const int tk = t >> 4, nn = grp * 16 + (t & 15);
                int sum = 0;
#pragma unroll
                for (int v = 0; v < kWaves; ++v) sum += red[v][t];
                if (tk < M && nn < N) {
                    const float rs = *gamma_p / scale_x[tk];
                    Y[(int64_t)tk * N + nn] = (float)sum * rs;
                    if (acc_out) acc_out[(int64_t)tk * N + nn] = sum;
                }
            }
            __syncthreads();
        }
    }
}

bool gemv_supported(int64_t M, int64_t K) { return M <= kGemvMaxM && K <= kMaxKLds; }

hipError_t launch_gemv_t2(const int8_t* Xq, const float* scale_x, const uint8_t* Wp,
                          const float* gamma, int64_t M, int64_t N, int64_t K, float* Y,
                          int32_t* acc, hipStream_t s) {
    if (!gemv_supported(M, K)) return hipErrorInvalidValue;
    const int64_t ngroups = (N + 15) / 16;
    const unsigned grid = (unsigned)std::min<int64_t>(ngroups, 256);
    const int64_t steps = (K + 16 * 64 - 1) / (16 * 64);  // MFMA steps per wave
    const bool full = K % (16 * 64) == 0;
#define BITNET_GEMV_CASE(S_)                                                                   \
    if (steps <= S_) {                                                                         \
        if (full && steps == S_)                                                               \
            gemv_t2_kernel<S_, true><<<grid, kThreads, 0, s>>>(Xq, scale_x, Wp, gamma, (int)M, \
                                                              (int)N, (int)K, Y, acc);         \
        else                                                                                   \
            gemv_t2_kernel<S_, false><<<grid, kThreads, 0, s>>>(Xq, scale_x, Wp, gamma, (int)M,\
                                                               (int)N, (int)K, Y, acc);        \
        return hipGetLastError();                                                              \
    }
    BITNET_GEMV_CASE(1)
    BITNET_GEMV_CASE(2)
    BITNET_GEMV_CASE(4)
    BITNET_GEMV_CASE(8)
#undef BITNET_GEMV_CASE
    return hipErrorInvalidValue;
}

}  // namespace bitnet
