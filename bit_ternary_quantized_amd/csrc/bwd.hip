// Straight-through-estimator backward of the BitLinear layer on gfx950
// bf16 matrix cores.
//
// "BitNet 1.5技术解析：2比特量化在神经网络中的应用与挑战" (2.1, 2.2) writes both
// quantizers with the detach trick and "1.58-bit量化技术突破AI算力与内存墙限制"
// (3.2) returns the incoming gradient unchanged, so the layer's gradients are
// those of a plain linear map at the dequantized operands:
//   grad_x[m][k] = gamma * sum_n gy[m][n] * code[n][k]
//   grad_W[n][k] =         sum_m gy[m][n] * X_deq[m][k],  X_deq = Xq / scale_x
// "BitNet 三元权重量化训练工程" (gradient-clipping section) pairs a bf16
// forward with fp32 gradients: both products run on v_mfma_f32_32x32x16_bf16
// with fp32 accumulation.  gy and the codes are exact in bf16; X_deq is
// rounded to bf16 once (Xq times the correctly rounded 1/scale_x).
//
// Each matrix-core operand wants its contraction index contiguous per lane.
// grad_x reads gy rows as they are; the codes are unpacked from 2 bits
// straight into a [k][n] LDS tile (pairs of rows n, n+1 per 32-bit write).
// grad_W contracts over tokens, so both its tiles are transposed on the way
// into LDS ([n][m] from gy rows, [k][m] from Xq rows, pairs of tokens per
// write).  No operand is copied through HBM.
//
// Tiles are 256 x 256 (512 threads, 2 x 4 waves of 128 x 64) when the output
// has enough of them, else 128 x 128 (256 threads, 2 x 2 waves of 64 x 64);
// when even those are too few, grad_W splits its token range and a second
// kernel adds the fp32 partial tiles in split order (deterministic).
#include "common.h"

namespace bitnet {

namespace {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

constexpr int BK = 32;       // contraction per step (bf16)
constexpr int STRIDE = 80;   // LDS bytes per tile row: 64 data + 16 pad

// 16-byte chunk c of tile row r, XOR-swizzled by bits [S, S+2) of the row so
// that 32-bit writes to rows 8 (S = 3) or 16 (S = 4) apart use distinct banks;
// consecutive rows stay conflict-free for 16-byte reads through the pad.
template <int S>
__device__ __forceinline__ int chunk_off(int r, int c) {
    return r * STRIDE + ((c ^ ((r >> S) & 3)) << 4);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    v2bf v;
    v[0] = (__bf16)lo;
    v[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, v);
}

template <int BM>
constexpr int kThreadsFor = BM == 256 ? 512 : 256;

template <int BM, int BN>
struct Cfg {
    static constexpr int T = kThreadsFor<BM>;
    static constexpr int WAVES_N = BM == 256 ? 4 : 2;
    static constexpr int WTM = BM / 2, WTN = BN / WAVES_N;
    static constexpr int IM = WTM / 32, JN = WTN / 32;
    static constexpr int TILE = BM * STRIDE;  // A and B tiles have equal rows here
};

// Workgroup id -> (tile m, tile n, split), regrouped so that each XCD (ids
// are dealt round-robin over the 8 XCDs) works on a contiguous run.
__device__ __forceinline__ void tile_of(int wg, int tiles_m, int tiles_n, int splits, int& tm,
                                        int& tn, int& sp) {
    const int G = tiles_m * tiles_n * splits;
    const int q = G / 8, r = G % 8;
    const int x = wg % 8, local = wg / 8;
    int id = (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + local;
    sp = id % splits;
    id /= splits;
    tm = id / tiles_n;
    tn = id % tiles_n;
}

// One 32-deep step of the wave's MFMA blocks from the LDS tiles.
template <int BM, int BN, int SA, int SB>
__device__ __forceinline__ void mma_step(const uint8_t* As, const uint8_t* Bs,
                                         v16f (&acc)[Cfg<BM, BN>::IM][Cfg<BM, BN>::JN], int wm,
                                         int wn, int lane) {
    using C = Cfg<BM, BN>;
    const int g = lane >> 5, l32 = lane & 31;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
        v8bf a[C::IM], b[C::JN];
#pragma unroll
        for (int i = 0; i < C::IM; ++i)
            a[i] = *reinterpret_cast<const v8bf*>(As + chunk_off<SA>(wm * C::WTM + i * 32 + l32, 2 * g + kh));
#pragma unroll
        for (int j = 0; j < C::JN; ++j)
            b[j] = *reinterpret_cast<const v8bf*>(Bs + chunk_off<SB>(wn * C::WTN + j * 32 + l32, 2 * g + kh));
#pragma unroll
        for (int i = 0; i < C::IM; ++i)
#pragma unroll
            for (int j = 0; j < C::JN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
}

// Output of one wave: 32x32 block layout, lane holds column l32 and rows
// 8*(r/4) + 4*g + r%4.
template <int BM, int BN, typename F>
__device__ __forceinline__ void for_each_out(const v16f (&acc)[Cfg<BM, BN>::IM][Cfg<BM, BN>::JN],
                                             int wm, int wn, int lane, F&& f) {
    using C = Cfg<BM, BN>;
    const int g = lane >> 5, l32 = lane & 31;
#pragma unroll
    for (int i = 0; i < C::IM; ++i)
#pragma unroll
        for (int j = 0; j < C::JN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                f(wm * C::WTM + i * 32 + 8 * (r >> 2) + 4 * g + (r & 3), wn * C::WTN + j * 32 + l32,
                  acc[i][j][r]);
}

}  // namespace

// ------------------------------------------------------------------ grad_x
// out[m][k] = gamma * sum_n gy[m][n] * code[n][k]; tile BM (m) x BN (k).
template <int BM, int BN, bool OUT_BF16>
__global__ __launch_bounds__(kThreadsFor<BM>) void gradx_kernel(
    const uint16_t* __restrict__ gy, const uint8_t* __restrict__ Wp,
    const float* __restrict__ gamma_p, int M, int N, int K, void* __restrict__ out) {
    using C = Cfg<BM, BN>;
    constexpr int SA = 3, SB = 4;
    __shared__ __align__(16) uint8_t smem[2][2 * C::TILE];
    int tm, tn, sp;
    tile_of(blockIdx.x, (M + BM - 1) / BM, (K + BN - 1) / BN, 1, tm, tn, sp);
    const int m0 = tm * BM, k0 = tn * BN;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    const int KB = K / 4;
    const bool vec = (N % 8) == 0;
    const int nsteps = (N + BK - 1) / BK;

    // A: gy rows, 4 chunks of 8 bf16 per row -> 4*BM chunks, 2 per thread.
    // B: thread t < BN: row pair p = t%16 (n = 2p, 2p+1), 16 codes kc = t/16.
    uint4 pa[2];
    uint32_t pb[2];
    auto load = [&](int st) {
        const int n0 = st * BK;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int c = t + u * C::T;
            const int row = c >> 2, ch = c & 3;
            const int m = m0 + row, n = n0 + ch * 8;
            pa[u] = make_uint4(0, 0, 0, 0);
            if (m < M && n < N) {
                const uint16_t* p = gy + (int64_t)m * N + n;
                if (vec) {
                    pa[u] = *reinterpret_cast<const uint4*>(p);
                } else {
                    uint32_t w[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        w[e] = (n + 2 * e < N ? p[2 * e] : 0u) | ((n + 2 * e + 1 < N ? (uint32_t)p[2 * e + 1] : 0u) << 16);
                    pa[u] = make_uint4(w[0], w[1], w[2], w[3]);
                }
            }
        }
        if (t < BN) {
            const int p = t & 15, kc = t >> 4;
            const int k = k0 + 16 * kc;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int n = n0 + 2 * p + h;
                pb[h] = (n < N && k < K) ? *reinterpret_cast<const uint32_t*>(Wp + (int64_t)n * KB + k / 4) : 0u;
            }
        }
    };
    auto store = [&](int buf) {
        uint8_t* As = smem[buf];
        uint8_t* Bs = smem[buf] + C::TILE;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int c = t + u * C::T;
            *reinterpret_cast<uint4*>(As + chunk_off<SA>(c >> 2, c & 3)) = pa[u];
        }
        if (t < BN) {
            const int p = t & 15, kc = t >> 4;
            // bf16 of a code: lo byte 0x80 if nonzero, hi byte 0x3f / 0xbf
            constexpr uint32_t kHi = 0x00bf3f00u, kLo = 0x00808000u;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const uint32_t c0 = (pb[0] >> (2 * j)) & 3u, c1 = (pb[1] >> (2 * j)) & 3u;
                const uint32_t sel = (c0 | (c1 << 16)) * 0x101u + 0x00040004u;
                const uint32_t v = __builtin_amdgcn_perm(kLo, kHi, sel);
                const int row = 16 * kc + j;
                *reinterpret_cast<uint32_t*>(Bs + chunk_off<SB>(row, p >> 2) + 4 * (p & 3)) = v;
            }
        }
    };

    v16f acc[C::IM][C::JN];
#pragma unroll
    for (int i = 0; i < C::IM; ++i)
#pragma unroll
        for (int j = 0; j < C::JN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    load(0);
    store(0);
    __syncthreads();
    for (int st = 0; st < nsteps; ++st) {
        const int buf = st & 1;
        if (st + 1 < nsteps) load(st + 1);
        mma_step<BM, BN, SA, SB>(smem[buf], smem[buf] + C::TILE, acc, wm, wn, lane);
        if (st + 1 < nsteps) store(buf ^ 1);
        __syncthreads();
    }

    const float gam = *gamma_p;
    for_each_out<BM, BN>(acc, wm, wn, lane, [&](int r, int c, float v) {
        const int m = m0 + r, k = k0 + c;
        if (m < M && k < K) {
            if constexpr (OUT_BF16) {
                static_cast<__bf16*>(out)[(int64_t)m * K + k] = (__bf16)(v * gam);
            } else {
                static_cast<float*>(out)[(int64_t)m * K + k] = v * gam;
            }
        }
    });
}

// ------------------------------------------------------------------ grad_W
// out[n][k] = sum_m gy[m][n] * X_deq[m][k]; tile BM (n) x BN (k); token range
// of split sp: [sp*mper, min(M, (sp+1)*mper)).  With splits > 1 the tile goes
// to part[sp][n][k] (fp32) for the ordered reduction.
template <int BM, int BN>
__global__ __launch_bounds__(kThreadsFor<BM>) void gradw_kernel(
    const uint16_t* __restrict__ gy, const int8_t* __restrict__ Xq,
    const float* __restrict__ scale_x, int M, int N, int K, int splits, int mper,
    float* __restrict__ out) {
    using C = Cfg<BM, BN>;
    constexpr int SA = 3, SB = 3;
    __shared__ __align__(16) uint8_t smem[2][2 * C::TILE];
    int tm, tn, sp;
    tile_of(blockIdx.x, (N + BM - 1) / BM, (K + BN - 1) / BN, splits, tm, tn, sp);
    const int n0 = tm * BM, k0 = tn * BN;
    const int mlo = sp * mper, mhi = min(M, mlo + mper);
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    const bool vec = (N % 8) == 0;
    const int nsteps = (mhi - mlo + BK - 1) / BK;

    // thread -> token pair p = t%16 (m = 2p, 2p+1 of the step), chunk t/16:
    // A: 8 consecutive n of gy rows m, m+1;  B: 8 consecutive k of Xq rows.
    // Threads t < 2*BM load A; threads t < 2*BN load B (here BM == BN).
    const int p = t & 15, ch = t >> 4;
    uint4 ga[2];
    uint2 qb[2];
    float rs[2];
    auto load = [&](int st) {
        const int mb = mlo + st * BK;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int m = mb + 2 * p + h;
            const bool mv = m < mhi;
            const int n = n0 + 8 * ch;
            ga[h] = make_uint4(0, 0, 0, 0);
            if (mv && n < N) {
                const uint16_t* src = gy + (int64_t)m * N + n;
                if (vec) {
                    ga[h] = *reinterpret_cast<const uint4*>(src);
                } else {
                    uint32_t w[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        w[e] = (n + 2 * e < N ? src[2 * e] : 0u) |
                               ((n + 2 * e + 1 < N ? (uint32_t)src[2 * e + 1] : 0u) << 16);
                    ga[h] = make_uint4(w[0], w[1], w[2], w[3]);
                }
            }
            const int k = k0 + 8 * ch;
            qb[h] = (mv && k < K) ? *reinterpret_cast<const uint2*>(Xq + (int64_t)m * K + k) : make_uint2(0, 0);
            rs[h] = mv ? 1.0f / scale_x[m] : 0.0f;
        }
    };
    auto store = [&](int buf) {
        uint8_t* As = smem[buf];
        uint8_t* Bs = smem[buf] + C::TILE;
        const int cp = p >> 2, off = 4 * (p & 3);
        {   // A: pairs (gy[m][n+i], gy[m+1][n+i]) -> row n+i
            const uint32_t a0[4] = {ga[0].x, ga[0].y, ga[0].z, ga[0].w};
            const uint32_t a1[4] = {ga[1].x, ga[1].y, ga[1].z, ga[1].w};
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t v = (i & 1) ? __builtin_amdgcn_perm(a1[i >> 1], a0[i >> 1], 0x07060302u)
                                           : __builtin_amdgcn_perm(a1[i >> 1], a0[i >> 1], 0x05040100u);
                *reinterpret_cast<uint32_t*>(As + chunk_off<SA>(8 * ch + i, cp) + off) = v;
            }
        }
        {   // B: pairs (Xq[m][k+j]/s[m], Xq[m+1][k+j]/s[m+1]) -> row k+j
            const uint32_t q0[2] = {qb[0].x, qb[0].y};
            const uint32_t q1[2] = {qb[1].x, qb[1].y};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float f0 = (float)(int8_t)(q0[j >> 2] >> (8 * (j & 3))) * rs[0];
                const float f1 = (float)(int8_t)(q1[j >> 2] >> (8 * (j & 3))) * rs[1];
                *reinterpret_cast<uint32_t*>(Bs + chunk_off<SB>(8 * ch + j, cp) + off) = pack_bf16x2(f0, f1);
            }
        }
    };

    v16f acc[C::IM][C::JN];
#pragma unroll
    for (int i = 0; i < C::IM; ++i)
#pragma unroll
        for (int j = 0; j < C::JN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    if (nsteps > 0) {
        load(0);
        store(0);
    }
    __syncthreads();
    for (int st = 0; st < nsteps; ++st) {
        const int buf = st & 1;
        if (st + 1 < nsteps) load(st + 1);
        mma_step<BM, BN, SA, SB>(smem[buf], smem[buf] + C::TILE, acc, wm, wn, lane);
        if (st + 1 < nsteps) store(buf ^ 1);
        __syncthreads();
    }

    float* dst = splits > 1 ? out + (int64_t)sp * N * K : out;
    for_each_out<BM, BN>(acc, wm, wn, lane, [&](int r, int c, float v) {
        const int n = n0 + r, k = k0 + c;
        if (n < N && k < K) dst[(int64_t)n * K + k] = v;
    });
}

// out[i] = sum over s = 0..splits-1 of part[s][i], in that order.
__global__ __launch_bounds__(256) void split_reduce_kernel(const float* __restrict__ part,
                                                           int splits, int64_t count,
                                                           float* __restrict__ out) {
    const int64_t i4 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i4 >= count) return;
    if (i4 + 4 <= count && (count % 4) == 0) {
        float4 s = reinterpret_cast<const float4*>(part + i4)[0];
        for (int p = 1; p < splits; ++p) {
            const float4 v = reinterpret_cast<const float4*>(part + (int64_t)p * count + i4)[0];
            s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
        }
        reinterpret_cast<float4*>(out + i4)[0] = s;
    } else {
        for (int64_t i = i4; i < i4 + 4 && i < count; ++i) {
            float s = part[i];
            for (int p = 1; p < splits; ++p) s += part[(int64_t)p * count + i];
            out[i] = s;
        }
    }
}

// ------------------------------------------------------------------ plans
namespace {

struct Plan {
    bool big;     // 256 x 256 tiles
    int splits;   // token splits (grad_W only)
    int mper;     // tokens per split (multiple of BK)
    int64_t tiles;
};

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Enough workgroups to cover the 256 CUs at least twice, else smaller tiles,
// else (grad_W) split the token range.
Plan plan_for(int64_t rows, int64_t cols, int64_t depth, bool allow_split) {
    Plan p{true, 1, (int)depth, ceil_div(rows, 256) * ceil_div(cols, 256)};
    if (p.tiles >= 512) return p;
    p.big = false;
    p.tiles = ceil_div(rows, 128) * ceil_div(cols, 128);
    if (!allow_split || p.tiles >= 256) return p;
    int64_t s = ceil_div(512, p.tiles);
    const int64_t max_s = std::max<int64_t>(1, depth / (4 * BK));  // >= 4 steps per split
    s = std::min(s, max_s);
    int64_t mper = ceil_div(ceil_div(depth, s), BK) * BK;
    s = ceil_div(depth, mper);
    p.splits = (int)s;
    p.mper = (int)mper;
    return p;
}

size_t align256(size_t b) { return (b + 255) / 256 * 256; }

}  // namespace

size_t bwd_ws_bytes(int64_t M, int64_t N, int64_t K) {
    const Plan p = plan_for(N, K, M, true);
    return p.splits > 1 ? align256((size_t)p.splits * N * K * 4) : 0;
}

hipError_t launch_bwd_ste(const uint16_t* gy, const int8_t* Xq, const float* scale_x,
                          const uint8_t* Wp, const float* gamma, int64_t M, int64_t N, int64_t K,
                          void* grad_x, bool gx_bf16, float* grad_W, void* ws, hipStream_t s) {
    const int m = (int)M, n = (int)N, k = (int)K;
    if (grad_x) {
        const Plan p = plan_for(M, K, N, false);
        if (p.big) {
            if (gx_bf16) gradx_kernel<256, 256, true><<<(unsigned)p.tiles, 512, 0, s>>>(gy, Wp, gamma, m, n, k, grad_x);
            else gradx_kernel<256, 256, false><<<(unsigned)p.tiles, 512, 0, s>>>(gy, Wp, gamma, m, n, k, grad_x);
        } else {
            if (gx_bf16) gradx_kernel<128, 128, true><<<(unsigned)p.tiles, 256, 0, s>>>(gy, Wp, gamma, m, n, k, grad_x);
            else gradx_kernel<128, 128, false><<<(unsigned)p.tiles, 256, 0, s>>>(gy, Wp, gamma, m, n, k, grad_x);
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (grad_W) {
        const Plan p = plan_for(N, K, M, true);
        float* dst = p.splits > 1 ? static_cast<float*>(ws) : grad_W;
        const unsigned grid = (unsigned)(p.tiles * p.splits);
        if (p.big)
            gradw_kernel<256, 256><<<grid, 512, 0, s>>>(gy, Xq, scale_x, m, n, k, p.splits, p.mper, dst);
        else
            gradw_kernel<128, 128><<<grid, 256, 0, s>>>(gy, Xq, scale_x, m, n, k, p.splits, p.mper, dst);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        if (p.splits > 1) {
            const int64_t count = N * K;
            split_reduce_kernel<<<(unsigned)ceil_div(ceil_div(count, 4), 256), 256, 0, s>>>(
                static_cast<const float*>(ws), p.splits, count, grad_W);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

}  // namespace bitnet
