// Quantizers of the BitLinear hot path for gfx950.
//
//   act_quant    RMSNorm (unit gain) + per-token absmax int8
//                ("BitNet 1.5技术解析" 2.2 and 3.1; "BitNet 三元权重量化训练工程",
//                straight-through-estimator section: eps = 1e-5, 127/max|x|)
//   weight_quant absmean ternary codes + 2-bit packing
//                ("BitNet 1.5技术解析" 2.1; "1.58-bit量化技术突破AI算力与内存墙限制"
//                2.2 and 4.1)
//   pack_ternary pre-quantized codes -> 2-bit packing (same page, 4.1)
//
// All three are HBM-bound streams.  Every operation that decides an integer
// is a single correctly rounded binary32 operation (built with contraction
// off), and every sum uses the library's canonical tree order, so the int8
// activations, the codes, gamma and scale_x are reproducible bit for bit.
#include "common.h"

namespace bitnet {

// ================================== act_quant: RMSNorm + per-token absmax int8
// One wave per token row.  Block b of the row is the 64*E elements
// [b*64E, (b+1)*64E); lane l holds elements b*64E + l*E .. +E-1 (one 16-byte
// load, so each wave load is a fully coalesced 1 KiB).  The sum of squares is
// the tree over the row: in-lane tree over E, butterfly over the lanes, then
// the tree over blocks.  NB > 0: the row (at most NB blocks) stays in
// registers between the two passes.  NB == 0: any length; the row is
// streamed twice.

constexpr int kAqWaves = 4;

template <typename T, int NB>
__global__ __launch_bounds__(kAqWaves * kWave) void act_quant_kernel(
    const T* __restrict__ X, int64_t M, int64_t K, float eps, int8_t* __restrict__ Q,
    float* __restrict__ S) {
    constexpr int E = Vec16<T>::E;
    constexpr int BLK = kWave * E;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t row = (int64_t)blockIdx.x * kAqWaves + (threadIdx.x >> 6);
    if (row >= M) return;  // uniform per wave
    const T* x = X + row * K;
    int8_t* q = Q + row * K;
    const int64_t nblk = (K + BLK - 1) / BLK;
    const bool vec_ok = (K % E) == 0;  // rows start 16-byte aligned

    auto load_block = [&](int64_t b, float (&v)[E]) {
        const int64_t k0 = b * BLK + (int64_t)lane * E;
        if (vec_ok && k0 + E <= K) {
            Vec16<T>::load(x + k0, v);
        } else {
#pragma unroll
            for (int e = 0; e < E; ++e) v[e] = (k0 + e < K) ? load_elem(x, k0 + e) : 0.0f;
        }
    };
    auto block_sq_sum = [&](const float (&v)[E]) {
        float sq[E];
#pragma unroll
        for (int e = 0; e < E; ++e) sq[e] = v[e] * v[e];
        return wave_tree_sum(lane_tree<E>(sq));
    };

    // The row cache holds the 16 loaded bytes per block as they are (8 bf16
    // in 4 registers rather than 8 floats), widened to float where used, so
    // twice as many waves fit when the input is bf16.
    auto load_raw = [&](int64_t b) -> uint4 {
        const int64_t k0 = b * BLK + (int64_t)lane * E;
        if (vec_ok && k0 + E <= K) return *reinterpret_cast<const uint4*>(x + k0);
        uint32_t w[4] = {0u, 0u, 0u, 0u};
        if constexpr (sizeof(T) == 4) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (k0 + e < K) w[e] = __float_as_uint(load_elem(x, k0 + e));
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (k0 + e < K) w[e / 2] |= (uint32_t)x[k0 + e] << (16 * (e % 2));
        }
        return make_uint4(w[0], w[1], w[2], w[3]);
    };
    auto widen = [](const uint4& r, float (&v)[E]) {
        const uint32_t w[4] = {r.x, r.y, r.z, r.w};
        if constexpr (sizeof(T) == 4) {
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(w[i]);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[2 * i] = __uint_as_float(w[i] << 16);
                v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
            }
        }
    };

    float amax = 0.0f;
    float ss;
    uint4 cache[NB > 0 ? NB : 1];
    if constexpr (NB > 0) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            if (b < nblk) cache[b] = load_raw(b);
        }
        float bs[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            if (b < nblk) {
                float v[E];
                widen(cache[b], v);
                bs[b] = block_sq_sum(v);
#pragma unroll
                for (int e = 0; e < E; ++e) amax = fmaxf(amax, fabsf(v[e]));
            } else {
                bs[b] = 0.0f;
            }
        }
        ss = lane_tree<NB>(bs);  // blocks beyond the row are +0 (exact padding)
    } else {
        PairwiseStack st;
        for (int64_t b = 0; b < nblk; ++b) {
            float v[E];
            load_block(b, v);
            st.push(block_sq_sum(v));
#pragma unroll
            for (int e = 0; e < E; ++e) amax = fmaxf(amax, fabsf(v[e]));
        }
        ss = st.total();
    }
    amax = wave_max(amax);

    const float ms = ss / (float)K;
    const float d = sqrtf(ms + eps);
    const float inv = 1.0f / d;
    // max|x * inv| == max|x| * inv: rounding is monotone, inv > 0
    const float a = amax * inv;
    const float scale = 127.0f / fmaxf(a, 1e-5f);
    if (lane == 0) S[row] = scale;

    auto quant_store = [&](int64_t b, const float (&v)[E]) {
        const int64_t k0 = b * BLK + (int64_t)lane * E;
        int8_t qv[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const float n = v[e] * inv;
            float r = rintf(n * scale);
            r = fminf(fmaxf(r, -128.0f), 127.0f);
            qv[e] = (int8_t)(int)r;
        }
        if (vec_ok && k0 + E <= K) {
            if constexpr (E == 8) {
                uint2 pk;
                pk.x = (uint32_t)(uint8_t)qv[0] | ((uint32_t)(uint8_t)qv[1] << 8) |
                       ((uint32_t)(uint8_t)qv[2] << 16) | ((uint32_t)(uint8_t)qv[3] << 24);
                pk.y = (uint32_t)(uint8_t)qv[4] | ((uint32_t)(uint8_t)qv[5] << 8) |
                       ((uint32_t)(uint8_t)qv[6] << 16) | ((uint32_t)(uint8_t)qv[7] << 24);
                if ((K % 8) == 0) {
                    *reinterpret_cast<uint2*>(q + k0) = pk;
                } else {
#pragma unroll
                    for (int e = 0; e < E; ++e) q[k0 + e] = qv[e];
                }
            } else {
                const uint32_t pk = (uint32_t)(uint8_t)qv[0] | ((uint32_t)(uint8_t)qv[1] << 8) |
                                    ((uint32_t)(uint8_t)qv[2] << 16) |
                                    ((uint32_t)(uint8_t)qv[3] << 24);
                *reinterpret_cast<uint32_t*>(q + k0) = pk;
            }
        } else {
#pragma unroll
            for (int e = 0; e < E; ++e)
                if (k0 + e < K) q[k0 + e] = qv[e];
        }
    };

    if constexpr (NB > 0) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            // an empty register constraint: the compiler cannot reuse the
            // floats widened for the sums (which would keep all of them live)
            asm volatile("" : "+v"(cache[b].x), "+v"(cache[b].y), "+v"(cache[b].z), "+v"(cache[b].w));
            if (b < nblk) {
                float v[E];
                widen(cache[b], v);
                quant_store(b, v);
            }
        }
    } else {
        for (int64_t b = 0; b < nblk; ++b) {
            float v[E];
            load_block(b, v);
            quant_store(b, v);
        }
    }
}

// Rows of exactly NB whole blocks (K == NB * 64E): each wave walks rows
// wave, wave + W, ... (W = waves in the grid), with the next row's loads in
// flight while it reduces, quantizes and stores the current one, so the HBM
// read and write streams overlap instead of running as two phases.  Two
// named register sets alternate (no copies); every load is an unconditional
// buffer load (past the last row: an out-of-range offset, which reads zeros),
// so no branch splits the wait counters.  Same arithmetic as above.
constexpr int kAqMaxGroups = 1024;  // workgroups of the row-walking grid (measured: 512-2048 within 3%)

// The body takes its workgroup index and the number of workgroups walking
// the rows, so a combined launch can run it on part of its grid.
template <typename T, int NB>
__device__ __forceinline__ void act_quant_rows_body(const T* __restrict__ X, int64_t M, int64_t K, float eps,
                                                    int8_t* __restrict__ Q, float* __restrict__ S, int bid,
                                                    int nblocks) {
    constexpr int E = Vec16<T>::E;
    constexpr int BLK = kWave * E;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t wave_id = (int64_t)bid * kAqWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t nwaves = (int64_t)nblocks * kAqWaves;
    if (wave_id >= M) return;  // uniform per wave

    auto load_row = [&](int64_t row, bool valid, uint4 (&c)[NB]) {
        const __amdgpu_buffer_rsrc_t rsrc = make_buf(X + row * K);
#pragma unroll
        for (int b = 0; b < NB; ++b)
            c[b] = buf_load16(rsrc, valid ? (uint32_t)((b * BLK + lane * E) * (int)sizeof(T)) : kBufOOB);
    };
    auto widen = [](const uint4& r, float (&v)[E]) {
        const uint32_t w[4] = {r.x, r.y, r.z, r.w};
        if constexpr (sizeof(T) == 4) {
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(w[i]);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[2 * i] = __uint_as_float(w[i] << 16);
                v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
            }
        }
    };
    auto finish_row = [&](int64_t row, uint4 (&c)[NB]) {
        float amax = 0.0f;
        float bs[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            float v[E], sq[E];
            widen(c[b], v);
#pragma unroll
            for (int e = 0; e < E; ++e) {
                sq[e] = v[e] * v[e];
                amax = fmaxf(amax, fabsf(v[e]));
            }
            bs[b] = wave_tree_sum(lane_tree<E>(sq));
        }
        const float ss = lane_tree<NB>(bs);
        amax = wave_max(amax);
        const float ms = ss / (float)K;
        const float d = sqrtf(ms + eps);
        const float inv = 1.0f / d;
        const float a = amax * inv;  // max|x * inv| == max|x| * inv
        const float scale = 127.0f / fmaxf(a, 1e-5f);
        if (lane == 0) S[row] = scale;
        int8_t* q = Q + row * K;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            // an empty register constraint: the floats widened for the sums
            // are not kept live until here
            asm volatile("" : "+v"(c[b].x), "+v"(c[b].y), "+v"(c[b].z), "+v"(c[b].w));
            float v[E];
            widen(c[b], v);
            uint32_t pk[E / 4];
#pragma unroll
            for (int i = 0; i < E / 4; ++i) {
                uint32_t w = 0;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float r = rintf((v[4 * i + e] * inv) * scale);
                    r = fminf(fmaxf(r, -128.0f), 127.0f);
                    w |= (uint32_t)(uint8_t)(int8_t)(int)r << (8 * e);
                }
                pk[i] = w;
            }
            const int64_t k0 = b * BLK + lane * E;
            if constexpr (E == 8) *reinterpret_cast<uint2*>(q + k0) = make_uint2(pk[0], pk[1]);
            else *reinterpret_cast<uint32_t*>(q + k0) = pk[0];
        }
    };
    uint4 ca[NB], cb[NB];
    load_row(wave_id, true, ca);
    for (int64_t row = wave_id;;) {
        const int64_t r1 = row + nwaves;
        load_row(r1 < M ? r1 : row, r1 < M, cb);
        finish_row(row, ca);
        if (r1 >= M) break;
        const int64_t r2 = r1 + nwaves;
        load_row(r2 < M ? r2 : r1, r2 < M, ca);
        finish_row(r1, cb);
        if (r2 >= M) break;
        row = r2;
    }
}

template <typename T, int NB>
__global__ __launch_bounds__(kAqWaves * kWave) void act_quant_rows_kernel(
    const T* __restrict__ X, int64_t M, int64_t K, float eps, int8_t* __restrict__ Q,
    float* __restrict__ S) {
    act_quant_rows_body<T, NB>(X, M, K, eps, Q, S, blockIdx.x, gridDim.x);
}

template <typename T>
static hipError_t act_quant_dispatch(const T* X, int64_t M, int64_t K, float eps, int8_t* Q,
                                     float* S, hipStream_t s) {
    constexpr int E = Vec16<T>::E;
    const int64_t nblk = (K + kWave * E - 1) / (kWave * E);
    const int64_t groups = (M + kAqWaves - 1) / kAqWaves;
    const dim3 grid((unsigned)groups), block(kAqWaves * kWave);
    if (K == nblk * kWave * E) {  // whole blocks: the row-walking kernel
        const dim3 g((unsigned)std::min<int64_t>(groups, kAqMaxGroups));
        switch (nblk) {
            case 1: act_quant_rows_kernel<T, 1><<<g, block, 0, s>>>(X, M, K, eps, Q, S); return hipGetLastError();
            case 2: act_quant_rows_kernel<T, 2><<<g, block, 0, s>>>(X, M, K, eps, Q, S); return hipGetLastError();
            case 4: act_quant_rows_kernel<T, 4><<<g, block, 0, s>>>(X, M, K, eps, Q, S); return hipGetLastError();
            case 8: act_quant_rows_kernel<T, 8><<<g, block, 0, s>>>(X, M, K, eps, Q, S); return hipGetLastError();
            case 16: act_quant_rows_kernel<T, 16><<<g, block, 0, s>>>(X, M, K, eps, Q, S); return hipGetLastError();
            default: break;
        }
    }
    if (nblk <= 1)
        act_quant_kernel<T, 1><<<grid, block, 0, s>>>(X, M, K, eps, Q, S);
    else if (nblk <= 2)
        act_quant_kernel<T, 2><<<grid, block, 0, s>>>(X, M, K, eps, Q, S);
    else if (nblk <= 4)
        act_quant_kernel<T, 4><<<grid, block, 0, s>>>(X, M, K, eps, Q, S);
    else if (nblk <= 8)
        act_quant_kernel<T, 8><<<grid, block, 0, s>>>(X, M, K, eps, Q, S);
    else if (nblk <= 16)
        act_quant_kernel<T, 16><<<grid, block, 0, s>>>(X, M, K, eps, Q, S);
    else
        act_quant_kernel<T, 0><<<grid, block, 0, s>>>(X, M, K, eps, Q, S);
    return hipGetLastError();
}

hipError_t launch_act_quant(const void* X, bool x_bf16, int64_t M, int64_t K, float eps,
                            int8_t* Xq, float* scale_x, hipStream_t s) {
    if (x_bf16)
        return act_quant_dispatch(static_cast<const uint16_t*>(X), M, K, eps, Xq, scale_x, s);
    return act_quant_dispatch(static_cast<const float*>(X), M, K, eps, Xq, scale_x, s);
}

// ============================ weight_quant: absmean ternary codes, 2-bit packed
// Pass 1: one wave per weight row -> tree sum of |w| over the row.
// Pass 2: the tree over the row sums, gamma = max(S/(N*K), 1e-5), and the
//         code threshold (below): one workgroup for large N, else every
//         workgroup of pass 3 redundantly (one launch fewer).
// Pass 3: each thread turns kPackU groups of 4 weights into packed bytes.
//
// Code decision without a per-element division.  code != 0 exactly when
// rint(fl(|w| / gamma)) >= 1, i.e. when fl(|w| / gamma) > 0.5.  With a
// correctly rounded quotient that holds iff |w| / gamma > 0.5 + 2^-25 (the
// rounding boundary above 0.5; a quotient exactly on it rounds to the even
// neighbour 0.5), i.e. iff |w| > t with t = gamma * (0.5 + 2^-25).  t has at
// most 49 significant bits, so it is exact in binary64, and for a binary32
// |w| the test |w| > t equals |w| >= thr, thr = the least float above t.

constexpr int kWqWaves = 4;

template <typename T>
__device__ __forceinline__ void wq_row_abs_sum_body(const T* __restrict__ W, int64_t N, int64_t K,
                                                    float* __restrict__ row_sums, int bid) {
    constexpr int E = Vec16<T>::E;
    constexpr int BLK = kWave * E;
    constexpr int G = 8;  // loads in flight per lane
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t row = (int64_t)bid * kWqWaves + (threadIdx.x >> 6);
    if (row >= N) return;
    const T* w = W + row * K;
    const int64_t nblk = (K + BLK - 1) / BLK;
    const bool vec_ok = (K % E) == 0;
    PairwiseStack st;
    for (int64_t b0 = 0; b0 < nblk; b0 += G) {
        float v[G][E];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int64_t k0 = (b0 + g) * BLK + (int64_t)lane * E;
            if (b0 + g < nblk && vec_ok && k0 + E <= K) {
                Vec16<T>::load(w + k0, v[g]);
            } else {
#pragma unroll
                for (int e = 0; e < E; ++e)
                    v[g][e] = (b0 + g < nblk && k0 + e < K) ? load_elem(w, k0 + e) : 0.0f;
            }
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            if (b0 + g < nblk) {
                float a[E];
#pragma unroll
                for (int e = 0; e < E; ++e) a[e] = fabsf(v[g][e]);
                st.push(wave_tree_sum(lane_tree<E>(a)));
            }
        }
    }
    if (lane == 0) row_sums[row] = st.total();
}

template <typename T>
__global__ __launch_bounds__(kWqWaves * kWave) void wq_row_abs_sum_kernel(
    const T* __restrict__ W, int64_t N, int64_t K, float* __restrict__ row_sums) {
    wq_row_abs_sum_body<T>(W, N, K, row_sums, blockIdx.x);
}

// Pass 2: the tree over the N row sums.  With P = N rounded up to a power of
// two and L = max(256, P/W), wave w of W sums the aligned range [w*L,
// (w+1)*L) as a tree and the W partial sums are combined as a tree (ranges
// beyond N are +0).  Every W gives the same bits: it is the canonical tree
// over the row sums padded with zeros, and extra zero padding adds exact
// zeros.
template <int W>
__device__ __forceinline__ void gamma_and_thr(const float* __restrict__ row_sums, int64_t N,
                                              int64_t K, float* part, float& g, float& thr) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x >> 6;
    constexpr int E = 4;
    constexpr int BLK = kWave * E;
    int64_t P = 1;
    while (P < N) P *= 2;
    const int64_t L = P / W > BLK ? P / W : BLK;
    const int64_t lo = (int64_t)wv * L;
    const int64_t nblk = L / BLK;
    PairwiseStack st;
    for (int64_t b0 = 0; b0 < nblk; b0 += 8) {
        float v[8][E];
#pragma unroll
        for (int gi = 0; gi < 8; ++gi) {
            const int64_t k0 = lo + (b0 + gi) * BLK + (int64_t)lane * E;
#pragma unroll
            for (int e = 0; e < E; ++e)
                v[gi][e] = (b0 + gi < nblk && k0 + e < N) ? row_sums[k0 + e] : 0.0f;
        }
#pragma unroll
        for (int gi = 0; gi < 8; ++gi)
            if (b0 + gi < nblk) st.push(wave_tree_sum(lane_tree<E>(v[gi])));
    }
    if (lane == 0) part[wv] = st.total();
    __syncthreads();
    float pw[W];
#pragma unroll
    for (int i = 0; i < W; ++i) pw[i] = part[i];
    const float total = lane_tree<W>(pw);
    const float mean = total / (float)(N * K);
    g = fmaxf(mean, 1e-5f);
    const double t = (double)g * (0.5 + 0x1p-25);
    thr = (float)t;
    if ((double)thr <= t) thr = __uint_as_float(__float_as_uint(thr) + 1u);
}

constexpr int kGammaWaves = 16;

__global__ __launch_bounds__(kGammaWaves * kWave) void wq_gamma_kernel(
    const float* __restrict__ row_sums, int64_t N, int64_t K, float* __restrict__ gamma,
    float* __restrict__ thr_out) {
    __shared__ float part[kGammaWaves];
    float g, thr;
    gamma_and_thr<kGammaWaves>(row_sums, N, K, part, g, thr);
    if (threadIdx.x == 0) {
        gamma[0] = g;
        thr_out[0] = thr;
    }
}

__device__ __forceinline__ uint32_t code_bits(float w, float thr) {
    // 01 = +1, 10 = -1, 00 = 0
    return fabsf(w) >= thr ? (w > 0.0f ? 1u : 2u) : 0u;
}

constexpr int kPackU = 4;  // groups of 4 weights per thread (loads in flight)
// When (rows x pack workgroups) is at most this, every pack workgroup
// evaluates gamma and the threshold itself from the row sums (one launch
// fewer, for small matrices); otherwise a single workgroup does and the pack
// kernel reads the threshold.
constexpr int64_t kFusedGammaMaxWork = (int64_t)1 << 22;

// FUSED: the threshold is computed here from the row sums (block 0 also
// writes gamma); otherwise it is read from thr_p.
template <typename T, bool FUSED>
__global__ __launch_bounds__(256) void wq_pack_kernel(const T* __restrict__ W, int64_t total4,
                                                      const float* __restrict__ thr_p,
                                                      const float* __restrict__ row_sums,
                                                      int64_t N, int64_t K, float* __restrict__ gamma,
                                                      uint8_t* __restrict__ out) {
    const int64_t base = (int64_t)blockIdx.x * (256 * kPackU) + threadIdx.x;
    float v[kPackU][4];
#pragma unroll
    for (int u = 0; u < kPackU; ++u) {
        const int64_t i = base + u * 256;
        if (i < total4) {
            if constexpr (sizeof(T) == 4) {
                const float4 q = reinterpret_cast<const float4*>(W)[i];
                v[u][0] = q.x; v[u][1] = q.y; v[u][2] = q.z; v[u][3] = q.w;
            } else {
                const uint2 q = reinterpret_cast<const uint2*>(W)[i];
                v[u][0] = __uint_as_float(q.x << 16);
                v[u][1] = __uint_as_float(q.x & 0xffff0000u);
                v[u][2] = __uint_as_float(q.y << 16);
                v[u][3] = __uint_as_float(q.y & 0xffff0000u);
            }
        }
    }
    float thr;
    if constexpr (FUSED) {
        __shared__ float part[4];
        float g;
        gamma_and_thr<4>(row_sums, N, K, part, g, thr);
        if (blockIdx.x == 0 && threadIdx.x == 0) gamma[0] = g;
    } else {
        thr = *thr_p;
    }
#pragma unroll
    for (int u = 0; u < kPackU; ++u) {
        const int64_t i = base + u * 256;
        if (i < total4) {
            uint32_t byte = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) byte |= code_bits(v[u][j], thr) << (2 * j);
            out[i] = (uint8_t)byte;
        }
    }
}

// ===================================================== per-row weight quant
// The per-output-channel variant ("BitNet量化感知训练中的梯度传播优化",
// section on the BitLinear implementation, 1: one scale per output row; the
// zyxy.net STE lecture: the mean of |w| along each row): gamma_n =
// max(T(|w_n|) / K, 1e-5) from the per-row tree sums of pass 1, each row's
// code threshold from its own gamma (the rule above), and the pack with the
// threshold of the row a byte belongs to.
__device__ __forceinline__ float code_threshold(float g) {
    const double t = (double)g * (0.5 + 0x1p-25);
    float thr = (float)t;
    if ((double)thr <= t) thr = __uint_as_float(__float_as_uint(thr) + 1u);
    return thr;
}

__global__ __launch_bounds__(256) void wq_rows_gamma_kernel(const float* __restrict__ row_sums, int64_t N,
                                                            int64_t K, float* __restrict__ gamma,
                                                            float* __restrict__ thr) {
    const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (n >= N) return;
    const float mean = row_sums[n] / (float)K;
    const float g = fmaxf(mean, 1e-5f);
    gamma[n] = g;
    thr[n] = code_threshold(g);
}

template <typename T>
__global__ __launch_bounds__(256) void wq_pack_rows_kernel(const T* __restrict__ W, int64_t total4, int64_t KB,
                                                           const float* __restrict__ thr,
                                                           uint8_t* __restrict__ out) {
    const int64_t base = (int64_t)blockIdx.x * (256 * kPackU) + threadIdx.x;
#pragma unroll
    for (int u = 0; u < kPackU; ++u) {
        const int64_t i = base + u * 256;  // packed byte: 4 weights of row i / KB
        if (i < total4) {
            float v[4];
            if constexpr (sizeof(T) == 4) {
                const float4 q = reinterpret_cast<const float4*>(W)[i];
                v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
            } else {
                const uint2 q = reinterpret_cast<const uint2*>(W)[i];
                v[0] = __uint_as_float(q.x << 16);
                v[1] = __uint_as_float(q.x & 0xffff0000u);
                v[2] = __uint_as_float(q.y << 16);
                v[3] = __uint_as_float(q.y & 0xffff0000u);
            }
            const float t = thr[i / KB];
            uint32_t byte = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) byte |= code_bits(v[j], t) << (2 * j);
            out[i] = (uint8_t)byte;
        }
    }
}

size_t weight_quant_rows_ws_bytes(int64_t N) {
    // row sums, then the row thresholds, each 256-byte aligned
    return (size_t)(2 * ((N * 4 + 255) / 256) * 256);
}

hipError_t launch_weight_quant_rows(const void* W, bool w_bf16, int64_t N, int64_t K, uint8_t* W_packed,
                                    float* gamma, void* ws, hipStream_t s) {
    float* row_sums = static_cast<float*>(ws);
    float* thr = reinterpret_cast<float*>(static_cast<char*>(ws) + ((N * 4 + 255) / 256) * 256);
    const dim3 g1((unsigned)((N + kWqWaves - 1) / kWqWaves)), b1(kWqWaves * kWave);
    if (w_bf16)
        wq_row_abs_sum_kernel<uint16_t><<<g1, b1, 0, s>>>(static_cast<const uint16_t*>(W), N, K, row_sums);
    else
        wq_row_abs_sum_kernel<float><<<g1, b1, 0, s>>>(static_cast<const float*>(W), N, K, row_sums);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    wq_rows_gamma_kernel<<<(unsigned)((N + 255) / 256), 256, 0, s>>>(row_sums, N, K, gamma, thr);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t total4 = N * K / 4;
    const unsigned g3 = (unsigned)((total4 + 256 * kPackU - 1) / (256 * kPackU));
    if (w_bf16)
        wq_pack_rows_kernel<uint16_t><<<g3, 256, 0, s>>>(static_cast<const uint16_t*>(W), total4, K / 4, thr,
                                                         W_packed);
    else
        wq_pack_rows_kernel<float><<<g3, 256, 0, s>>>(static_cast<const float*>(W), total4, K / 4, thr, W_packed);
    return hipGetLastError();
}

size_t weight_quant_ws_bytes(int64_t N) {
    // row sums, then the threshold float, 256-byte aligned
    return (size_t)(((N * 4 + 255) / 256) * 256 + 256);
}

static unsigned stream_grid(int64_t work_items, int per_block) {
    int64_t g = (work_items + per_block - 1) / per_block;
    const int64_t cap = 256 * 32;  // enough resident waves to saturate HBM
    if (g > cap) g = cap;
    if (g < 1) g = 1;
    return (unsigned)g;
}

// ============================================================ code counts
// Counts of the packed codes (00 = 0, 01 = +1, 10 = -1, 11 unused) for the
// zero-ratio and polarity monitoring of the quantized weights
// ("BitNet 1.5技术解析" 6, item 3; "BitNet量化感知训练中的梯度传播优化",
// section on convergence monitoring).  Pass 1: a bounded grid; each thread
// counts 16-byte chunks with population counts over the low and high bit of
// every 2-bit field, each workgroup sums its threads and writes its four
// partial counts.  Pass 2: one workgroup adds the partials in workgroup
// order.  Integers throughout, no atomics: exact and deterministic.
constexpr int kCountGroups = 1024;  // pass-1 workgroups at most

__device__ __forceinline__ uint32_t block_sum_u32(uint32_t v, uint32_t* red) {  // 256 threads
#pragma unroll
    for (int m = 1; m < kWave; m *= 2) v += __shfl_xor(v, m, kWave);
    if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    const uint32_t t = red[0] + red[1] + red[2] + red[3];
    __syncthreads();
    return t;
}

__global__ __launch_bounds__(256) void code_counts_kernel(const uint8_t* __restrict__ P, int64_t nbytes,
                                                          uint32_t* __restrict__ partial) {
    __shared__ uint32_t red[4];
    uint32_t c[4] = {0u, 0u, 0u, 0u};  // zeros, +1, -1, 11
    auto count_fields = [&](uint32_t w, uint32_t field_mask) {  // one bit per 2-bit field
        const uint32_t lo = w & field_mask, hi = (w >> 1) & field_mask;
        c[0] += __builtin_popcount(~(lo | hi) & field_mask);
        c[1] += __builtin_popcount(lo & ~hi);
        c[2] += __builtin_popcount(hi & ~lo);
        c[3] += __builtin_popcount(lo & hi);
    };
    const int64_t nvec = nbytes / 16;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nvec; i += (int64_t)gridDim.x * 256) {
        const uint4 v = reinterpret_cast<const uint4*>(P)[i];
        count_fields(v.x, 0x55555555u);
        count_fields(v.y, 0x55555555u);
        count_fields(v.z, 0x55555555u);
        count_fields(v.w, 0x55555555u);
    }
    if (blockIdx.x == 0 && threadIdx.x < nbytes - nvec * 16) count_fields(P[nvec * 16 + threadIdx.x], 0x55u);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t t = block_sum_u32(c[j], red);
        if (threadIdx.x == 0) partial[4 * blockIdx.x + j] = t;
    }
}

__global__ __launch_bounds__(256) void code_counts_final_kernel(const uint32_t* __restrict__ partial,
                                                                int groups,
                                                                unsigned long long* __restrict__ counts) {
    __shared__ unsigned long long red[4][4];
    unsigned long long c[4] = {0ull, 0ull, 0ull, 0ull};
    for (int b = threadIdx.x; b < groups; b += 256)
#pragma unroll
        for (int j = 0; j < 4; ++j) c[j] += partial[4 * b + j];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        unsigned long long v = c[j];
#pragma unroll
        for (int m = 1; m < kWave; m *= 2) v += __shfl_xor(v, m, kWave);
        if ((threadIdx.x & (kWave - 1)) == 0) red[j][threadIdx.x >> 6] = v;
    }
    __syncthreads();
    if (threadIdx.x < 4) {
        const int j = threadIdx.x;
        counts[j] = red[j][0] + red[j][1] + red[j][2] + red[j][3];
    }
}

size_t code_counts_ws_bytes() { return (size_t)kCountGroups * 4 * sizeof(uint32_t); }

hipError_t launch_code_counts(const uint8_t* W_packed, int64_t nbytes, uint64_t* counts, void* ws,
                              hipStream_t s) {
    const int64_t need = (nbytes / 16 + 255) / 256;
    const int groups = (int)std::max<int64_t>(1, std::min<int64_t>(need, kCountGroups));
    uint32_t* partial = static_cast<uint32_t*>(ws);
    code_counts_kernel<<<groups, 256, 0, s>>>(W_packed, nbytes, partial);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    code_counts_final_kernel<<<1, 256, 0, s>>>(partial, groups, reinterpret_cast<unsigned long long*>(counts));
    return hipGetLastError();
}

// ============================================================ weight clamp
// The clamp of the master weights after an update to [lo, hi]
// ("BitNet量化感知训练中的梯度传播优化", section on the BitLinear
// implementation: weight.data.clamp_(-1, 1)).  In place, 16 bytes per thread
// and step; an unclamped weight keeps its bits, a bound bf16 cannot hold is
// rounded to nearest even.
template <typename T>
__global__ __launch_bounds__(256) void weight_clamp_kernel(T* __restrict__ W, int64_t count, float lo,
                                                           float hi) {
    constexpr int E = 16 / (int)sizeof(T);
    const int64_t nvec = count / E;
    const int64_t stride = (int64_t)gridDim.x * 256;
    auto clamp_bits = [&](uint32_t bits) -> uint32_t {  // one element's bits
        if constexpr (sizeof(T) == 4) {
            const float v = __uint_as_float(bits);
            return v < lo ? __float_as_uint(lo) : v > hi ? __float_as_uint(hi) : bits;
        } else {
            const float v = bf16_bits_to_f32(bits);
            if (v < lo) return __builtin_bit_cast(uint16_t, (__bf16)lo);
            if (v > hi) return __builtin_bit_cast(uint16_t, (__bf16)hi);
            return bits;
        }
    };
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nvec; i += stride) {
        uint4 v = reinterpret_cast<const uint4*>(W)[i];
        uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            if constexpr (sizeof(T) == 4) {
                w[d] = clamp_bits(w[d]);
            } else {
                w[d] = clamp_bits(w[d] & 0xffffu) | (clamp_bits(w[d] >> 16) << 16);
            }
        }
        reinterpret_cast<uint4*>(W)[i] = make_uint4(w[0], w[1], w[2], w[3]);
    }
    // the last count % E elements
    if (blockIdx.x == 0 && threadIdx.x < count - nvec * E) {
        const int64_t i = nvec * E + threadIdx.x;
        if constexpr (sizeof(T) == 4) {
            uint32_t* p = reinterpret_cast<uint32_t*>(W) + i;
            *p = clamp_bits(*p);
        } else {
            uint16_t* p = reinterpret_cast<uint16_t*>(W) + i;
            *p = (uint16_t)clamp_bits(*p);
        }
    }
}

hipError_t launch_weight_clamp(void* W, bool w_bf16, int64_t count, float lo, float hi, hipStream_t s) {
    const int64_t per = w_bf16 ? 8 : 4;
    const unsigned grid = stream_grid((count / per + 1), 256);
    if (w_bf16)
        weight_clamp_kernel<uint16_t><<<grid, 256, 0, s>>>(static_cast<uint16_t*>(W), count, lo, hi);
    else
        weight_clamp_kernel<float><<<grid, 256, 0, s>>>(static_cast<float*>(W), count, lo, hi);
    return hipGetLastError();
}


// Passes 2 and 3 (gamma, threshold, packing) from the row sums in ws.
static hipError_t weight_quant_pack(const void* W, bool w_bf16, int64_t N, int64_t K, uint8_t* W_packed,
                                    float* gamma, void* ws, hipStream_t s) {
    float* row_sums = static_cast<float*>(ws);
    float* thr = reinterpret_cast<float*>(static_cast<char*>(ws) + ((N * 4 + 255) / 256) * 256);
    hipError_t e;
    const int64_t total4 = N * K / 4;
    const unsigned g3 = (unsigned)((total4 + 256 * kPackU - 1) / (256 * kPackU));
    const uint16_t* Wb = static_cast<const uint16_t*>(W);
    const float* Wf = static_cast<const float*>(W);
    if (N * (int64_t)g3 <= kFusedGammaMaxWork) {
        if (w_bf16)
            wq_pack_kernel<uint16_t, true><<<g3, 256, 0, s>>>(Wb, total4, thr, row_sums, N, K, gamma, W_packed);
        else
            wq_pack_kernel<float, true><<<g3, 256, 0, s>>>(Wf, total4, thr, row_sums, N, K, gamma, W_packed);
        return hipGetLastError();
    }
    wq_gamma_kernel<<<1, kGammaWaves * kWave, 0, s>>>(row_sums, N, K, gamma, thr);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (w_bf16)
        wq_pack_kernel<uint16_t, false><<<g3, 256, 0, s>>>(Wb, total4, thr, row_sums, N, K, gamma, W_packed);
    else
        wq_pack_kernel<float, false><<<g3, 256, 0, s>>>(Wf, total4, thr, row_sums, N, K, gamma, W_packed);
    return hipGetLastError();
}

hipError_t launch_weight_quant(const void* W, bool w_bf16, int64_t N, int64_t K,
                               uint8_t* W_packed, float* gamma, void* ws, hipStream_t s) {
    float* row_sums = static_cast<float*>(ws);
    const dim3 g1((unsigned)((N + kWqWaves - 1) / kWqWaves)), b1(kWqWaves * kWave);
    if (w_bf16)
        wq_row_abs_sum_kernel<uint16_t><<<g1, b1, 0, s>>>(static_cast<const uint16_t*>(W), N, K,
                                                           row_sums);
    else
        wq_row_abs_sum_kernel<float><<<g1, b1, 0, s>>>(static_cast<const float*>(W), N, K,
                                                        row_sums);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return weight_quant_pack(W, w_bf16, N, K, W_packed, gamma, ws, s);
}

// ============================================= both quantizers, one launch fewer
// Launch 1 runs act_quant's row-walking kernel on workgroups [0, A) and the
// weight row sums on [A, A + ceil(N/4)): two independent streams of HBM
// reads in one grid, with no launch boundary between them.  Launch 2 (and
// the gamma kernel for large N) is weight_quant's.  Same bodies, same
// arithmetic: the outputs are bit-identical to the two separate calls.
template <typename TX, int NB, typename TW>
__global__ __launch_bounds__(kAqWaves * kWave) void quant_operands_kernel(
    const TX* __restrict__ X, int64_t M, int64_t K, float eps, int8_t* __restrict__ Q, float* __restrict__ S,
    int act_blocks, const TW* __restrict__ W, int64_t N, float* __restrict__ row_sums) {
    static_assert(kAqWaves == kWqWaves, "one workgroup shape for both bodies");
    const int b = blockIdx.x;  // uniform
    if (b < act_blocks) act_quant_rows_body<TX, NB>(X, M, K, eps, Q, S, b, act_blocks);
    else wq_row_abs_sum_body<TW>(W, N, K, row_sums, b - act_blocks);
}

namespace {
template <typename TX, typename TW>
hipError_t quant_operands_pass1(const TX* X, int64_t M, int64_t K, float eps, int8_t* Q, float* S, const TW* W,
                                int64_t N, float* row_sums, int nblk, hipStream_t s) {
    const int64_t groups = (M + kAqWaves - 1) / kAqWaves;
    const int act_blocks = (int)std::min<int64_t>(groups, kAqMaxGroups);
    const int64_t wq_blocks = (N + kWqWaves - 1) / kWqWaves;
    const dim3 grid((unsigned)(act_blocks + wq_blocks)), block(kAqWaves * kWave);
    switch (nblk) {
        case 1: quant_operands_kernel<TX, 1, TW><<<grid, block, 0, s>>>(X, M, K, eps, Q, S, act_blocks, W, N, row_sums); break;
        case 2: quant_operands_kernel<TX, 2, TW><<<grid, block, 0, s>>>(X, M, K, eps, Q, S, act_blocks, W, N, row_sums); break;
        case 4: quant_operands_kernel<TX, 4, TW><<<grid, block, 0, s>>>(X, M, K, eps, Q, S, act_blocks, W, N, row_sums); break;
        case 8: quant_operands_kernel<TX, 8, TW><<<grid, block, 0, s>>>(X, M, K, eps, Q, S, act_blocks, W, N, row_sums); break;
        case 16: quant_operands_kernel<TX, 16, TW><<<grid, block, 0, s>>>(X, M, K, eps, Q, S, act_blocks, W, N, row_sums); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}
template <typename TX>
hipError_t quant_operands_w(const TX* X, int64_t M, int64_t K, float eps, int8_t* Q, float* S, const void* W,
                            bool w_bf16, int64_t N, float* row_sums, int nblk, hipStream_t s) {
    if (w_bf16) return quant_operands_pass1(X, M, K, eps, Q, S, static_cast<const uint16_t*>(W), N, row_sums, nblk, s);
    return quant_operands_pass1(X, M, K, eps, Q, S, static_cast<const float*>(W), N, row_sums, nblk, s);
}
}  // namespace

hipError_t launch_quant_operands(const void* X, bool x_bf16, int64_t M, int64_t K, float eps, int8_t* Xq,
                                 float* scale_x, const void* W, bool w_bf16, int64_t N, uint8_t* W_packed,
                                 float* gamma, void* ws, hipStream_t s) {
    const int64_t E = x_bf16 ? 8 : 4;
    const int64_t nblk = (K + kWave * E - 1) / (kWave * E);
    const bool rows = K == nblk * kWave * E && (nblk == 1 || nblk == 2 || nblk == 4 || nblk == 8 || nblk == 16);
    hipError_t e;
    if (!rows) {  // act_quant's general kernel: the two calls' launches in order
        e = launch_act_quant(X, x_bf16, M, K, eps, Xq, scale_x, s);
        if (e != hipSuccess) return e;
        return launch_weight_quant(W, w_bf16, N, K, W_packed, gamma, ws, s);
    }
    float* row_sums = static_cast<float*>(ws);
    e = x_bf16 ? quant_operands_w(static_cast<const uint16_t*>(X), M, K, eps, Xq, scale_x, W, w_bf16, N, row_sums,
                                  (int)nblk, s)
               : quant_operands_w(static_cast<const float*>(X), M, K, eps, Xq, scale_x, W, w_bf16, N, row_sums,
                                  (int)nblk, s);
    if (e != hipSuccess) return e;
    return weight_quant_pack(W, w_bf16, N, K, W_packed, gamma, ws, s);
}

// ============================================================ pack helper
__global__ __launch_bounds__(256) void pack_codes_kernel(const int8_t* __restrict__ codes,
                                                         int64_t total4,
                                                         uint8_t* __restrict__ out) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total4; i += stride) {
        const uint32_t c4 = reinterpret_cast<const uint32_t*>(codes)[i];
        uint32_t byte = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int8_t c = (int8_t)(c4 >> (8 * j));
            byte |= (c > 0 ? 1u : (c < 0 ? 2u : 0u)) << (2 * j);
        }
        out[i] = (uint8_t)byte;
    }
}

hipError_t launch_pack_ternary(const int8_t* codes, int64_t N, int64_t K, uint8_t* W_packed,
                               hipStream_t s) {
    const int64_t total4 = N * K / 4;
    pack_codes_kernel<<<stream_grid(total4, 256), 256, 0, s>>>(codes, total4, W_packed);
    return hipGetLastError();
}

}  // namespace bitnet
