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
// in groups of 16 (one MFMA N block); workgroup w owns groups w, w + grid,
// ...  The 16 waves split K: wave v owns columns [v*Kw, (v+1)*Kw), its lane
// group g = lane/16 the contiguous quarter [v*Kw + g*Kw/4, ...), and MFMA
// step s the s-th 16-column chunk of every quarter (the sum over k is exact
// and order-free).  A lane's activation operand is then the same columns for
// every row group, held in registers (byte-transposed 4 x 4 to match the
// column order unpack16 produces; tokens >= M are zero).  Its loads are
// issued first, so the later wait for them does not wait for the weight
// stream (loads retire in issue order).  Then every packed
// weight byte of the pass is requested with no branch in front of the loads;
// all row groups are computed before one reduction of the 16 partial int32
// tiles in LDS.
#include "common.h"

namespace bitnet {

namespace {
typedef int v4i __attribute__((ext_vector_type(4)));
constexpr int kWaves = 16;
constexpr int kThreads = kWaves * 64;
constexpr int kMaxGroups = 4;  // row groups per pass when S <= 4
}  // namespace

// S: MFMA steps (64 columns) per wave, Kw = 64*S; FULL: K == 16*Kw, so every
// lane's column range lies inside the row and loads are 16-byte vectors.
// STAGE: the activations come in with coalesced 16-byte loads through an LDS
// tile (M > 8: 16 token rows would otherwise be fetched as scattered pieces
// by every lane); without it each lane loads its own chunks (few tokens).
constexpr int kStageMaxK = 4096;  // LDS activation tile bound
constexpr int kStageStride = kStageMaxK + 16;

// CH: gamma_p holds one scale per output channel (see the GEMM).
template <int S, bool FULL, bool STAGE, bool CH>
__global__ __launch_bounds__(kThreads) void gemv_t2_kernel(
    const int8_t* __restrict__ Xq, const float* __restrict__ scale_x,
    const uint8_t* __restrict__ Wp, const float* __restrict__ gamma_p, int M, int N, int K,
    float* __restrict__ Y, int32_t* __restrict__ acc_out) {
    // row groups per pass: weight (G*S) and activation (4*S) registers stay
    // within the budget of 4 waves per SIMD
    constexpr int G = S >= 16 ? 1 : (S >= 8 ? 2 : kMaxGroups);
    __shared__ int red[G][kWaves][256];
    __shared__ __align__(16) uint8_t As[STAGE ? 16 * kStageStride : 16];
    constexpr int Kw = 64 * S;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int col = lane & 15, g = lane >> 4;
    const int kb = wave * Kw + g * (Kw / 4);  // first column of this lane
    const int KB = K / 4;
    const int ngroups = (N + 15) / 16;

    // ---- activation operand: token col, columns kb + 16 s
    uint4 av[S];
    constexpr int kAPer = STAGE ? (16 * kStageMaxK / 16) / kThreads : 1;
    uint4 ac[kAPer];  // coalesced chunks for the LDS tile (STAGE)
    const int kch = K / 16;
    if constexpr (STAGE) {
#pragma unroll
        for (int i = 0; i < kAPer; ++i) {
            const int c = t + i * kThreads;
            const int tok = c / kch;
            ac[i] = make_uint4(0, 0, 0, 0);
            if (c < 16 * kch && tok < M)
                ac[i] = *reinterpret_cast<const uint4*>(Xq + (int64_t)tok * K + 16 * (c - tok * kch));
        }
    } else {
        const bool tv = col < M;
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const int k = kb + 16 * s;
            av[s] = make_uint4(0, 0, 0, 0);
            if (tv && (FULL || k < K)) av[s] = *reinterpret_cast<const uint4*>(Xq + (int64_t)col * K + k);
        }
    }
    bool transposed = false;

    for (int base = blockIdx.x; base < ngroups; base += gridDim.x * G) {
        // ---- weights for up to G row groups, all loads in flight
        uint32_t wq[G][S];
#pragma unroll
        for (int r = 0; r < G; ++r) {
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
        if (!transposed) {
            if constexpr (STAGE) {
#pragma unroll
                for (int i = 0; i < kAPer; ++i) {
                    const int c = t + i * kThreads;
                    if (c < 16 * kch) {
                        const int tok = c / kch, kc = c - tok * kch;
                        const uint32_t a[4] = {ac[i].x, ac[i].y, ac[i].z, ac[i].w};
                        uint32_t o[4];
                        transpose4x4_bytes(a, o);
                        *reinterpret_cast<uint4*>(As + tok * kStageStride + 16 * kc) =
                            make_uint4(o[0], o[1], o[2], o[3]);
                    }
                }
                __syncthreads();
#pragma unroll
                for (int s = 0; s < S; ++s) {
                    const int k = kb + 16 * s;
                    av[s] = (FULL || k < K) ? *reinterpret_cast<const uint4*>(As + col * kStageStride + k)
                                            : make_uint4(0, 0, 0, 0);
                }
            } else {
#pragma unroll
                for (int s = 0; s < S; ++s) {
                    const uint32_t a[4] = {av[s].x, av[s].y, av[s].z, av[s].w};
                    uint32_t o[4];
                    transpose4x4_bytes(a, o);
                    av[s] = make_uint4(o[0], o[1], o[2], o[3]);
                }
            }
            transposed = true;
        }

        // ---- products of every row group, then one reduction
        int nr = 0;
#pragma unroll
        for (int r = 0; r < G; ++r) {
            const int grp = base + r * gridDim.x;
            if (grp >= ngroups) break;  // uniform over the workgroup
            v4i acc = {0, 0, 0, 0};
#pragma unroll
            for (int s = 0; s < S; ++s) {
                uint32_t b[4];
                unpack16(wq[r][s], b);
                acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                    v4i{(int)av[s].x, (int)av[s].y, (int)av[s].z, (int)av[s].w},
                    v4i{(int)b[0], (int)b[1], (int)b[2], (int)b[3]}, acc, 0, 0, 0);
            }
            // 16x16 layout: lane holds weight row lane%16, tokens 4*(lane/16)+i
#pragma unroll
            for (int i = 0; i < 4; ++i) red[r][wave][(4 * g + i) * 16 + col] = acc[i];
            nr = r + 1;
        }
        __syncthreads();
        for (int o = t; o < nr * 256; o += kThreads) {
            const int r = o >> 8, e = o & 255;
            const int grp = base + r * gridDim.x;
            const int tk = e >> 4, nn = grp * 16 + (e & 15);
            int sum = 0;
#pragma unroll
            for (int v = 0; v < kWaves; ++v) sum += red[r][v][e];
            if (tk < M && nn < N) {
                if constexpr (CH) {
                    const float rs = 1.0f / scale_x[tk];
                    Y[(int64_t)tk * N + nn] = ((float)sum * rs) * gamma_p[nn];
                } else {
                    const float rs = *gamma_p / scale_x[tk];
                    Y[(int64_t)tk * N + nn] = (float)sum * rs;
                }
                if (acc_out) acc_out[(int64_t)tk * N + nn] = sum;
            }
        }
        __syncthreads();
    }
}

bool gemv_supported(int64_t M, int64_t K) { return M <= kGemvMaxM && K <= 16 * 64 * 16; }

hipError_t launch_gemv_t2(const int8_t* Xq, const float* scale_x, const uint8_t* Wp,
                          const float* gamma, int64_t M, int64_t N, int64_t K, float* Y,
                          int32_t* acc, hipStream_t s, bool channel) {
    if (!gemv_supported(M, K)) return hipErrorInvalidValue;
    const int64_t ngroups = (N + 15) / 16;
    const unsigned grid = (unsigned)std::min<int64_t>(ngroups, 256);
    const int64_t steps = (K + 16 * 64 - 1) / (16 * 64);  // MFMA steps per wave
    const bool full = K % (16 * 64) == 0;
    const bool stage = M > 8 && K <= kStageMaxK;  // measured: direct loads win up to 8 tokens
#define BITNET_GEMV_LAUNCH(S_, F_, G_)                                                          \
    do {                                                                                       \
        if (channel)                                                                           \
            gemv_t2_kernel<S_, F_, G_, true><<<grid, kThreads, 0, s>>>(Xq, scale_x, Wp, gamma, (int)M, \
                                                                     (int)N, (int)K, Y, acc);  \
        else                                                                                   \
            gemv_t2_kernel<S_, F_, G_, false><<<grid, kThreads, 0, s>>>(Xq, scale_x, Wp, gamma, (int)M, \
                                                                      (int)N, (int)K, Y, acc); \
    } while (0)
#define BITNET_GEMV_CASE(S_)                                                                   \
    if (steps <= S_) {                                                                         \
        const bool f = full && steps == S_;                                                    \
        if (f && stage) BITNET_GEMV_LAUNCH(S_, true, true);                                    \
        else if (f) BITNET_GEMV_LAUNCH(S_, true, false);                                       \
        else if (stage) BITNET_GEMV_LAUNCH(S_, false, true);                                   \
        else BITNET_GEMV_LAUNCH(S_, false, false);                                             \
        return hipGetLastError();                                                              \
    }
    BITNET_GEMV_CASE(1)
    BITNET_GEMV_CASE(2)
    BITNET_GEMV_CASE(4)
    BITNET_GEMV_CASE(8)
    BITNET_GEMV_CASE(16)
#undef BITNET_GEMV_CASE
#undef BITNET_GEMV_LAUNCH
    return hipErrorInvalidValue;
}

}  // namespace bitnet
