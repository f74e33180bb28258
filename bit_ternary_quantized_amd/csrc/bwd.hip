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
// grad_x reads gy rows as they are; the codes are unpacked from 2 bits into
// a natural [n][k] LDS tile.  grad_W contracts over tokens, so both of its
// tiles ([m][n] from gy, [m][k] from Xq) are natural too.  Tiles stored with
// the contraction index as their row are read transposed by gfx950's
// ds_read_b64_tr_b16, so every LDS write is a 16-byte store.  No operand is
// copied through HBM.
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
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

constexpr int BK = 64;  // contraction per step: 4 MFMA sub-steps of 16

// LDS tiles come in two layouts.
//  "rows": one row per output index, its 64 contraction values contiguous
//          (128 B + 16 pad); MFMA operands are plain 16-byte reads.
//  "cols": one row per contraction index, the output indices contiguous
//          (pitch = 2*width + 64 B, i.e. 64 B mod 256, so that the transposing
//          reads below hit 64 distinct banks); written with 16-byte stores
//          straight from the source rows, read transposed with
//          ds_read_b64_tr_b16.
constexpr int ROWS_STRIDE = 144;
template <int W>
constexpr int cols_pitch() { return 2 * W + 64; }

// Transposing read (gfx950 ds_read_b64_tr_b16).  Within each 16-lane group,
// lane j supplies the address of 4 consecutive bf16; output lane 4a+b then
// holds element b of the chunks of lanes a, 4+a, 8+a, 12+a.  So if lane
// j = 4e + a points at contraction row c0+e, columns x0+4a..x0+4a+3, output
// lane i holds column x0+i at rows c0..c0+3.
__device__ __forceinline__ v4s lds_read_tr16(const uint8_t* tile, int byte_off) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4s*)((__attribute__((address_space(3))) const char*)tile + byte_off));
}

// Matrix-core operand (8 contraction values for output index x0 + lane%32)
// from a "cols" tile: two transposing reads give contraction rows
// c0 + 8*(lane/32) + 0..3 and + 4..7.
template <int PITCH>
__device__ __forceinline__ v8bf cols_operand(const uint8_t* tile, int c0, int x0, int lane) {
    const int G = lane >> 4, j = lane & 15, e = j >> 2, a = j & 3;
    const int row = c0 + 8 * (G >> 1) + e, col = x0 + 16 * (G & 1) + 4 * a;
    const v4s lo = lds_read_tr16(tile, row * PITCH + 2 * col);
    const v4s hi = lds_read_tr16(tile, (row + 4) * PITCH + 2 * col);
    v8bf r;
    const uint2 l = __builtin_bit_cast(uint2, lo), h = __builtin_bit_cast(uint2, hi);
    r = __builtin_bit_cast(v8bf, make_uint4(l.x, l.y, h.x, h.y));
    return r;
}

// Matrix-core operand from a "rows" tile: contraction values
// c0 + 8*(lane/32) + 0..7 of output row x0 + lane%32.
__device__ __forceinline__ v8bf rows_operand(const uint8_t* tile, int c0, int x0, int lane) {
    return *reinterpret_cast<const v8bf*>(tile + (x0 + (lane & 31)) * ROWS_STRIDE +
                                          2 * (c0 + 8 * (lane >> 5)));
}

template <int BM>
constexpr int kThreadsFor = BM == 256 ? 512 : 256;

template <int BM, int BN>
struct Cfg {
    static constexpr int T = kThreadsFor<BM>;
    static constexpr int WAVES_N = BM == 256 ? 4 : 2;
    static constexpr int WTM = BM / 2, WTN = BN / WAVES_N;
    static constexpr int IM = WTM / 32, JN = WTN / 32;
    static constexpr int MFMAS = IM * JN * 4;  // per wave and step
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

// Interleave hint for one step: each MFMA followed by a few VALU and LDS ops.
template <int N_MFMA>
__device__ __forceinline__ void interleave_hint() {
#pragma unroll
    for (int q = 0; q < N_MFMA; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // up to four VALU
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // up to two LDS reads
        __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // up to one LDS write
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

// 8 bf16 of row `r` from column `c` (zero past `cols` or past `rows`);
// branch-free: out-of-range reads go to a clamped, valid address.
__device__ __forceinline__ uint4 load8_bf16(const uint16_t* P, int rows, int cols, int r, int c,
                                            bool vec) {
    const bool rv = r < rows;
    const uint16_t* p = P + (int64_t)(rv ? r : 0) * cols;
    if (vec) {
        const bool v = rv && c < cols;
        const uint4 x = *reinterpret_cast<const uint4*>(p + (v ? c : 0));
        return v ? x : make_uint4(0, 0, 0, 0);
    }
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const bool v0 = rv && c + 2 * e < cols, v1 = rv && c + 2 * e + 1 < cols;
        const uint32_t lo = p[v0 ? c + 2 * e : 0], hi = p[v1 ? c + 2 * e + 1 : 0];
        w[e] = (v0 ? lo : 0u) | ((v1 ? hi : 0u) << 16);
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// 16 ternary codes (one packed dword, columns k..k+15) -> 16 bf16 in natural
// column order (8 dwords, two codes each).  bf16 of a code: low byte 0x80 if
// nonzero, high byte 0x3f (+1) or 0xbf (-1).
__device__ __forceinline__ void codes16_to_bf16(uint32_t w, uint32_t (&o)[8]) {
    constexpr uint32_t kHi = 0x00bf3f00u, kLo = 0x00808000u;
    const uint32_t ev = w & 0x33333333u;          // codes 0,2 of every byte (bits 0-1, 4-5)
    const uint32_t od = (w >> 2) & 0x33333333u;   // codes 1,3 of every byte
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        // [ev.b, ev.b, od.b, od.b]: codes 4b (low nibble) and 4b+1, then 4b+2 and 4b+3 (high)
        const uint32_t pb = __builtin_amdgcn_perm(od, ev, (uint32_t)(b | b << 8 | (b + 4) << 16 | (b + 4) << 24));
        const uint32_t s0 = (pb & 0x03030303u) + 0x00040004u;
        const uint32_t s1 = ((pb >> 4) & 0x03030303u) + 0x00040004u;
        o[2 * b] = __builtin_amdgcn_perm(kLo, kHi, s0);
        o[2 * b + 1] = __builtin_amdgcn_perm(kLo, kHi, s1);
    }
}

}  // namespace

// ------------------------------------------------------------------ grad_x
// out[m][k] = gamma * sum_n gy[m][n] * code[n][k]; tile BM (m) x BN (k).
// A tile ("rows"): gy rows m as they are.  B tile ("cols"): codes of rows n
// unpacked to bf16 in natural order ([n][k]), read transposed.
template <int BM, int BN, bool OUT_BF16>
__global__ __launch_bounds__(kThreadsFor<BM>) void gradx_kernel(
    const uint16_t* __restrict__ gy, const uint8_t* __restrict__ Wp,
    const float* __restrict__ gamma_p, int M, int N, int K, void* __restrict__ out) {
    using C = Cfg<BM, BN>;
    constexpr int A_BYTES = BM * ROWS_STRIDE;
    constexpr int BP = cols_pitch<BN>();
    constexpr int B_BYTES = BK * BP;
    constexpr int kAPer = BM * 8 / C::T;             // 16-byte A chunks per thread
    constexpr int kBPer = BK * (BN / 16) / C::T;     // 16-code B items per thread
    __shared__ __align__(16) uint8_t smem[2][A_BYTES + B_BYTES];
    int tm, tn, sp;
    tile_of(blockIdx.x, (M + BM - 1) / BM, (K + BN - 1) / BN, 1, tm, tn, sp);
    const int m0 = tm * BM, k0 = tn * BN;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    const int KB = K / 4;
    const bool vec = (N % 8) == 0;
    const int nsteps = (N + BK - 1) / BK;
    constexpr int kcN = BN / 16;

    struct Stage {
        uint4 a[kAPer];
        uint32_t b[kBPer];
    };
    auto load = [&](int st, Stage& f) {
        const int n0 = st * BK;
#pragma unroll
        for (int u = 0; u < kAPer; ++u) {
            const int c = t + u * C::T;
            f.a[u] = load8_bf16(gy, M, N, m0 + c / 8, n0 + 8 * (c % 8), vec);
        }
#pragma unroll
        for (int u = 0; u < kBPer; ++u) {  // item: row n0 + e / kcN, codes 16*(e % kcN)
            const int e = t + u * C::T;
            const int n = n0 + e / kcN, k = k0 + 16 * (e % kcN);
            const bool v = n < N && k < K;
            const uint32_t w = *reinterpret_cast<const uint32_t*>(Wp + (int64_t)(v ? n : 0) * KB + (v ? k / 4 : 0));
            f.b[u] = v ? w : 0u;
        }
    };
    auto store = [&](int buf, const Stage& f) {
        uint8_t* As = smem[buf];
        uint8_t* Bs = smem[buf] + A_BYTES;
#pragma unroll
        for (int u = 0; u < kAPer; ++u) {
            const int c = t + u * C::T;
            *reinterpret_cast<uint4*>(As + (c / 8) * ROWS_STRIDE + 16 * (c % 8)) = f.a[u];
        }
#pragma unroll
        for (int u = 0; u < kBPer; ++u) {
            const int e = t + u * C::T;
            uint32_t o[8];
            codes16_to_bf16(f.b[u], o);
            uint4* d = reinterpret_cast<uint4*>(Bs + (e / kcN) * BP + 32 * (e % kcN));
            d[0] = make_uint4(o[0], o[1], o[2], o[3]);
            d[1] = make_uint4(o[4], o[5], o[6], o[7]);
        }
    };

    v16f acc[C::IM][C::JN];
#pragma unroll
    for (int i = 0; i < C::IM; ++i)
#pragma unroll
        for (int j = 0; j < C::JN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // two steps of global loads in flight; past the end of N the loads are
    // zero-filled from clamped addresses, so the step body has no branch
    Stage s0, nxt;
    load(0, s0);
    load(1, nxt);
    store(0, s0);
    __syncthreads();
    for (int st = 0; st < nsteps; ++st) {
        const int buf = st & 1;
        Stage cur;
        load(st + 2, cur);
        const uint8_t* As = smem[buf];
        const uint8_t* Bs = smem[buf] + A_BYTES;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            v8bf a[C::IM], b[C::JN];
#pragma unroll
            for (int i = 0; i < C::IM; ++i) a[i] = rows_operand(As, 16 * q, wm * C::WTM + i * 32, lane);
#pragma unroll
            for (int j = 0; j < C::JN; ++j) b[j] = cols_operand<BP>(Bs, 16 * q, wn * C::WTN + j * 32, lane);
#pragma unroll
            for (int i = 0; i < C::IM; ++i)
#pragma unroll
                for (int j = 0; j < C::JN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        store(buf ^ 1, nxt);
        interleave_hint<C::MFMAS>();
        __syncthreads();
        nxt = cur;
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
// to part[sp][n][k] (fp32) for the ordered reduction.  Both tiles are "cols"
// tiles: gy rows m as they are, and Xq rows m converted to bf16(Xq / s[m]);
// both are read transposed.
template <int BM, int BN>
__global__ __launch_bounds__(kThreadsFor<BM>) void gradw_kernel(
    const uint16_t* __restrict__ gy, const int8_t* __restrict__ Xq,
    const float* __restrict__ scale_x, int M, int N, int K, int splits, int mper,
    float* __restrict__ out) {
    using C = Cfg<BM, BN>;
    constexpr int AP = cols_pitch<BM>(), BP = cols_pitch<BN>();
    constexpr int A_BYTES = BK * AP, B_BYTES = BK * BP;
    constexpr int kAPer = BK * (BM / 8) / C::T;  // 8-wide gy pieces per thread
    constexpr int kBPer = BK * (BN / 8) / C::T;  // 8-wide Xq pieces per thread
    __shared__ __align__(16) uint8_t smem[2][A_BYTES + B_BYTES];
    int tm, tn, sp;
    tile_of(blockIdx.x, (N + BM - 1) / BM, (K + BN - 1) / BN, splits, tm, tn, sp);
    const int n0 = tm * BM, k0 = tn * BN;
    const int mlo = sp * mper, mhi = min(M, mlo + mper);
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    const bool vec = (N % 8) == 0;
    const int nsteps = (mhi - mlo + BK - 1) / BK;

    struct Stage {
        uint4 a[kAPer];
        uint2 b[kBPer];
        float rs[kBPer];
    };
    auto load = [&](int st, Stage& f) {
        const int mb = mlo + st * BK;
#pragma unroll
        for (int u = 0; u < kAPer; ++u) {  // piece: token mb + c / (BM/8), n 8*(c % (BM/8))
            const int c = t + u * C::T;
            const int m = mb + c / (BM / 8);
            f.a[u] = load8_bf16(gy, m < mhi ? M : 0, N, m, n0 + 8 * (c % (BM / 8)), vec);
        }
#pragma unroll
        for (int u = 0; u < kBPer; ++u) {
            const int c = t + u * C::T;
            const int m = mb + c / (BN / 8), k = k0 + 8 * (c % (BN / 8));
            const bool mv = m < mhi, v = mv && k < K;
            const uint2 q = *reinterpret_cast<const uint2*>(Xq + (int64_t)(v ? m : 0) * K + (v ? k : 0));
            f.b[u] = v ? q : make_uint2(0, 0);
            const float sx = scale_x[mv ? m : 0];
            f.rs[u] = mv ? 1.0f / sx : 0.0f;
        }
    };
    auto store = [&](int buf, const Stage& f) {
        uint8_t* As = smem[buf];
        uint8_t* Bs = smem[buf] + A_BYTES;
#pragma unroll
        for (int u = 0; u < kAPer; ++u) {
            const int c = t + u * C::T;
            *reinterpret_cast<uint4*>(As + (c / (BM / 8)) * AP + 16 * (c % (BM / 8))) = f.a[u];
        }
#pragma unroll
        for (int u = 0; u < kBPer; ++u) {
            const int c = t + u * C::T;
            const uint32_t q[2] = {f.b[u].x, f.b[u].y};
            uint32_t o[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float x0 = (float)(int8_t)(q[j >> 1] >> (16 * (j & 1))) * f.rs[u];
                const float x1 = (float)(int8_t)(q[j >> 1] >> (16 * (j & 1) + 8)) * f.rs[u];
                typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
                v2bf pr;
                pr[0] = (__bf16)x0;
                pr[1] = (__bf16)x1;
                o[j] = __builtin_bit_cast(uint32_t, pr);
            }
            *reinterpret_cast<uint4*>(Bs + (c / (BN / 8)) * BP + 16 * (c % (BN / 8))) =
                make_uint4(o[0], o[1], o[2], o[3]);
        }
    };

    v16f acc[C::IM][C::JN];
#pragma unroll
    for (int i = 0; i < C::IM; ++i)
#pragma unroll
        for (int j = 0; j < C::JN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    Stage s0, nxt;
    load(0, s0);
    load(1, nxt);
    store(0, s0);
    __syncthreads();
    for (int st = 0; st < nsteps; ++st) {
        const int buf = st & 1;
        Stage cur;
        load(st + 2, cur);
        const uint8_t* As = smem[buf];
        const uint8_t* Bs = smem[buf] + A_BYTES;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            v8bf a[C::IM], b[C::JN];
#pragma unroll
            for (int i = 0; i < C::IM; ++i) a[i] = cols_operand<AP>(As, 16 * q, wm * C::WTM + i * 32, lane);
#pragma unroll
            for (int j = 0; j < C::JN; ++j) b[j] = cols_operand<BP>(Bs, 16 * q, wn * C::WTN + j * 32, lane);
#pragma unroll
            for (int i = 0; i < C::IM; ++i)
#pragma unroll
                for (int j = 0; j < C::JN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        store(buf ^ 1, nxt);
        interleave_hint<C::MFMAS>();
        __syncthreads();
        nxt = cur;
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
