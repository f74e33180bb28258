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
    const int64_t row = (int64_t)blockIdx.x * kAqWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
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
    const __amdgpu_buffer_rsrc_t rx = make_buf(x);
    auto load_raw = [&](int64_t b) -> uint4 {
        const int64_t k0 = b * BLK + (int64_t)lane * E;
        // rows of whole vectors: an unconditional buffer load (past the row it
        // reads zeros), so the loads of a row are in flight together
        if (vec_ok) return buf_load16(rx, k0 < K ? (uint32_t)(k0 * (int64_t)sizeof(T)) : kBufOOB);
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
            for (int i = 0; i < E / 4; ++i)
                pk[i] = q8x4((v[4 * i] * inv) * scale, (v[4 * i + 1] * inv) * scale, (v[4 * i + 2] * inv) * scale,
                             (v[4 * i + 3] * inv) * scale);
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
// Pass 1: one wave per weight row -> tree sum of |w| over the row; each
//         workgroup (4 rows) also writes the tree node over its rows.
// Pass 2: the tree over those nodes (the tree over the row sums), gamma =
//         max(S/(N*K), 1e-5), and the code threshold (below), evaluated in
//         the pack launch: by its workgroup 0, which publishes the threshold
//         to the others, for large matrices; by every workgroup for small
//         ones.
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

// quad_sums (when non-null): the workgroup also writes the tree node over
// its kWqWaves = 4 rows, (r0 + r1) + (r2 + r3) with rows past N as +0: the
// canonical tree over the row sums is the tree over these aligned 4-row
// nodes (the row sums are >= +0, so the zero padding changes no bit), and
// gamma is evaluated from N/4 values instead of N.
// gate (when non-null): the pack launch's threshold word, cleared here by
// workgroup 0 (this pass always runs first in the call, so the pack launch
// never sees a ready mark left by an earlier call).
__device__ __forceinline__ float code_threshold(float g);

// row_gamma / row_thr (when non-null): the per-output-channel variant's
// gamma_n = max(S_n / K, 1e-5) and its code threshold, written with the row sum.
template <typename T>
__device__ __forceinline__ void wq_row_abs_sum_body(const T* __restrict__ W, int64_t N, int64_t K,
                                                    float* __restrict__ row_sums, int bid,
                                                    float* __restrict__ quad_sums,
                                                    uint64_t* __restrict__ gate,
                                                    float* __restrict__ row_gamma = nullptr,
                                                    float* __restrict__ row_thr = nullptr,
                                                    uint64_t* __restrict__ counts_clear = nullptr) {
    if (gate && bid == 0 && threadIdx.x == 0) *gate = 0;
    // the counted call's four counts, added into by its last launch
    if (counts_clear && bid == 0 && threadIdx.x < 4) counts_clear[threadIdx.x] = 0;
    constexpr int E = Vec16<T>::E;
    constexpr int BLK = kWave * E;
    constexpr int G = 8;  // loads in flight per lane
    __shared__ float quad[kWqWaves];
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: the row base stays scalar
    const int64_t row = (int64_t)bid * kWqWaves + wv;
    const T* w = W + (row < N ? row : 0) * K;
    const int64_t nblk = row < N ? (K + BLK - 1) / BLK : 0;  // uniform in the wave
    PairwiseStack st;
    auto push_block = [&](const float (&v)[E]) {
        float a[E];
#pragma unroll
        for (int e = 0; e < E; ++e) a[e] = fabsf(v[e]);
        st.push(wave_tree_sum(lane_tree<E>(a)));
    };
    if ((K % E) == 0) {  // uniform: rows of whole 16-byte vectors (the usual case)
        // unconditional buffer loads (a vector past the row reads zeros), so
        // the G loads of a round are in flight together
        const __amdgpu_buffer_rsrc_t rw = make_buf(w);
        for (int64_t b0 = 0; b0 < nblk; b0 += G) {
            uint4 raw[G];
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const int64_t k0 = (b0 + g) * BLK + (int64_t)lane * E;
                raw[g] = buf_load16(rw, b0 + g < nblk && k0 < K ? (uint32_t)(k0 * (int64_t)sizeof(T)) : kBufOOB);
            }
#pragma unroll
            for (int g = 0; g < G; ++g) {
                if (b0 + g < nblk) {
                    float v[E];
                    widen16<T>(raw[g], v);
                    push_block(v);
                }
            }
        }
    } else {
        for (int64_t b0 = 0; b0 < nblk; b0 += G) {
            float v[G][E];
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const int64_t k0 = (b0 + g) * BLK + (int64_t)lane * E;
#pragma unroll
                for (int e = 0; e < E; ++e)
                    v[g][e] = (b0 + g < nblk && k0 + e < K) ? load_elem(w, k0 + e) : 0.0f;
            }
#pragma unroll
            for (int g = 0; g < G; ++g)
                if (b0 + g < nblk) push_block(v[g]);
        }
    }
    const float total = row < N ? st.total() : 0.0f;
    if (lane == 0 && row < N) {
        row_sums[row] = total;
        if (row_gamma) {  // uniform: a kernel argument
            const float g = fmaxf(total / (float)K, 1e-5f);
            row_gamma[row] = g;
            row_thr[row] = code_threshold(g);
        }
    }
    if (quad_sums) {  // uniform: a kernel argument
        if (lane == 0) quad[wv] = total;
        __syncthreads();
        if (threadIdx.x == 0) quad_sums[bid] = (quad[0] + quad[1]) + (quad[2] + quad[3]);
    }
}

template <typename T>
__global__ __launch_bounds__(kWqWaves * kWave) void wq_row_abs_sum_kernel(
    const T* __restrict__ W, int64_t N, int64_t K, float* __restrict__ row_sums, float* __restrict__ quad_sums,
    uint64_t* __restrict__ gate, float* __restrict__ row_gamma, float* __restrict__ row_thr,
    uint64_t* __restrict__ counts_clear = nullptr) {
    wq_row_abs_sum_body<T>(W, N, K, row_sums, blockIdx.x, quad_sums, gate, row_gamma, row_thr, counts_clear);
}

// Pass 2: the tree over the n = ceil(N/4) four-row nodes of pass 1 (the
// tree over the N row sums).  With P = n rounded up to a power of two and L
// = max(256, P/W), wave w of W sums the aligned range [w*L, (w+1)*L) as a
// tree and the W partial sums are combined as a tree (ranges beyond n are
// +0).  Every W gives the same bits: it is the canonical tree over the nodes
// padded with zeros, and extra zero padding adds exact zeros.
template <int W>
__device__ __forceinline__ void gamma_and_thr(const float* __restrict__ nodes, int64_t n, int64_t N,
                                              int64_t K, float* part, float& g, float& thr) {
    const float* __restrict__ row_sums = nodes;
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = W == 1 ? 0 : threadIdx.x >> 6;
    constexpr int E = 4;
    constexpr int BLK = kWave * E;
    int64_t P = 1;
    while (P < n) P *= 2;
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
                v[gi][e] = (b0 + gi < nblk && k0 + e < n) ? row_sums[k0 + e] : 0.0f;
        }
#pragma unroll
        for (int gi = 0; gi < 8; ++gi)
            if (b0 + gi < nblk) st.push(wave_tree_sum(lane_tree<E>(v[gi])));
    }
    float total;
    if constexpr (W == 1) {  // one wave (any wave of the workgroup), no barrier; part unused
        total = st.total();
    } else {
        if (lane == 0) part[wv] = st.total();
        __syncthreads();
        float pw[W];
#pragma unroll
        for (int i = 0; i < W; ++i) pw[i] = part[i];
        total = lane_tree<W>(pw);
    }
    const float mean = total / (float)(N * K);
    g = fmaxf(mean, 1e-5f);
    const double t = (double)g * (0.5 + 0x1p-25);
    thr = (float)t;
    if ((double)thr <= t) thr = __uint_as_float(__float_as_uint(thr) + 1u);
}


__device__ __forceinline__ uint32_t code_bits(float w, float thr) {
    // 01 = +1, 10 = -1, 00 = 0
    return fabsf(w) >= thr ? (w > 0.0f ? 1u : 2u) : 0u;
}

// Adds the 2-bit fields of w (one bit per field in field_mask) to the counts
// of zeros, +1 (01), -1 (10) and the unused pattern 11.
__device__ __forceinline__ void count_code_fields(uint32_t w, uint32_t field_mask, uint32_t (&c)[4]) {
    const uint32_t lo = w & field_mask, hi = (w >> 1) & field_mask;
    c[0] += __builtin_popcount(~(lo | hi) & field_mask);
    c[1] += __builtin_popcount(lo & ~hi);
    c[2] += __builtin_popcount(hi & ~lo);
    c[3] += __builtin_popcount(lo & hi);
}

constexpr int kPackU = 4;  // groups of 4 weights per thread (loads in flight)
// with the published threshold, groups per thread: with the fifth wave, 128
// bytes of weights per thread (16 groups of bf16, 8 of fp32), so that at
// 4096 x 4096 bf16 the whole matrix is requested by one round of resident
// workgroups (1024 of five waves; a CU holds six) and its loads stream while
// workgroup 0 evaluates gamma; else 8 groups (16 fp32 groups per thread
// measured slower at 28672 x 8192: 362 against 335 us)
template <typename T, bool POLLER>
constexpr int pack_u_pub() { return POLLER ? 128 / (4 * (int)sizeof(T)) : 8; }
constexpr int kPollerGroupsPerCu = 6;  // five-wave workgroups a CU holds (32 wave slots)
// When (rows x pack workgroups) is at most this, every pack workgroup
// evaluates gamma and the threshold itself from the four-row nodes (for
// small matrices; the weight loads are issued first, so the evaluation hides
// under them).  Above it workgroup 0 evaluates them once and publishes the
// threshold to the others (below).  Measured at 4096 x 4096 bf16, the call:
// gamma in a launch of its own 21.8 us; published 20.0 us; every workgroup
// evaluating it 23.0 us.
constexpr int64_t kFusedGammaMaxWork = (int64_t)1 << 22;
// reads of the published threshold before a workgroup evaluates it itself
// (set_gate_polls changes it for later calls: tests use 0 to run that path)
constexpr int kGatePolls = 32;
static int g_gate_polls = kGatePolls;
int set_gate_polls(int n) {
    const int prev = g_gate_polls;
    g_gate_polls = n;
    return prev;
}

// The pack of a group of 4 weights into one byte of codes, and the counts of
// the codes written (COUNT: +1 codes in the low half of cnt, -1 codes in the
// high half).
template <typename T, bool COUNT>
__device__ __forceinline__ void pack_group(const uint4& raw, float thr, int64_t i, uint8_t* __restrict__ out,
                                           uint32_t& cnt) {
    float v[4];
    if constexpr (sizeof(T) == 4) {
        v[0] = __uint_as_float(raw.x);
        v[1] = __uint_as_float(raw.y);
        v[2] = __uint_as_float(raw.z);
        v[3] = __uint_as_float(raw.w);
    } else {
        v[0] = __uint_as_float(raw.x << 16);
        v[1] = __uint_as_float(raw.x & 0xffff0000u);
        v[2] = __uint_as_float(raw.y << 16);
        v[3] = __uint_as_float(raw.y & 0xffff0000u);
    }
    uint32_t byte = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) byte |= code_bits(v[j], thr) << (2 * j);
    out[i] = (uint8_t)byte;
    if constexpr (COUNT) {
        const uint32_t lo = byte & 0x55u, hi = (byte >> 1) & 0x55u;
        cnt += __builtin_popcount(lo & ~hi) + (__builtin_popcount(hi & ~lo) << 16);
    }
}

// The weights of a workgroup's NT U groups of 4 (NT threads), thread t taking
// groups t, t + NT, ...: one buffer descriptor at the workgroup's first
// group, every load unconditional (past total4 an out-of-range offset reads
// zeros), so all U loads are in flight together and nothing waits for them
// before the threshold is known.
template <typename T, int U, int NT>
__device__ __forceinline__ void load_groups(const T* __restrict__ W, int64_t g0, int64_t total4, int t,
                                            uint4 (&raw)[U]) {
    const __amdgpu_buffer_rsrc_t rw = make_buf(W + g0 * 4);
    constexpr uint32_t kGroupBytes = 4 * sizeof(T);
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t off = g0 + t + u * NT < total4 ? (t + u * NT) * kGroupBytes : kBufOOB;
        if constexpr (sizeof(T) == 4) {
            raw[u] = buf_load16(rw, off);
        } else {
            const uint2 q = buf_load8(rw, off);
            raw[u] = make_uint4(q.x, q.y, 0u, 0u);
        }
    }
}

// COUNT (the pack bodies): the workgroup also counts the codes it writes.
// Each thread keeps its +1 and -1 counts in the two halves of one word (at
// most 4U codes a thread, at most 256 * 64 = 16384 a workgroup: inside 16
// bits), each wave adds its 64 words with DPP row moves (wave_sum_u32), and
// after one barrier thread 0 stores the workgroup's pair (+1, -1) in slot
// `slot` (the pack workgroup's index) of count_partial: a plain store, every
// slot written once per call, nothing to clear.
// (Device-scope atomics into shared slots instead were measured slower: at
// 4096 x 4096 bf16 the counting pack took 12.2 us with one set of atomics per
// workgroup, 13.8 us with one per wave, against 11.6 us with stores.)
// counted_sum_kernel then adds the pairs: the monitoring counts without a
// second read of the packed weights.
static_assert(256 * 4 * 16 < 65536, "per-workgroup code counts fit 16 bits");
// sum over the 64 lanes (every lane active) with row moves, returned to
// every lane (integers: exact in any order).  (Lane exchanges through
// ds_bpermute instead: the counting pack at 28672 x 8192 fp32 took 184 us,
// the plain one 173.5 us.)
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xf, 0xf, false);
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
    v += dpp_u32<kDppXor1>(v);
    v += dpp_u32<kDppXor2>(v);
    v += dpp_u32<kDppHalfMirror>(v);
    v += dpp_u32<kDppMirror>(v);
    return (__builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16)) +
           (__builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48));
}
template <bool COUNT, int NW>
__device__ __forceinline__ void store_group_counts(uint32_t cnt, uint32_t* __restrict__ count_partial,
                                                   int slot) {
    if constexpr (COUNT) {
        __shared__ uint32_t red[NW];
        cnt = wave_sum_u32(cnt);
        if ((threadIdx.x & (kWave - 1)) == 0 && (threadIdx.x >> 6) < NW) red[threadIdx.x >> 6] = cnt;
        __syncthreads();
        if (threadIdx.x == 0) {
            uint32_t t = 0;
#pragma unroll
            for (int w = 0; w < NW; ++w) t += red[w];
            reinterpret_cast<uint2*>(count_partial)[slot] = make_uint2(t & 0xffffu, t >> 16);
        }
    }
}

// Small matrices: every workgroup computes gamma and the threshold from the
// four-row nodes (its weight loads issued first, so the evaluation hides
// under them); block 0 also writes gamma.
// (The pack bodies take their workgroup index `bid`, so that a launch can
// also run other work on other workgroups.)
template <typename T, int U, bool COUNT>
__device__ __forceinline__ void wq_pack_body(const T* __restrict__ W, int64_t total4,
                                             const float* __restrict__ nodes, int64_t N, int64_t K,
                                             float* __restrict__ gamma, uint8_t* __restrict__ out,
                                             uint32_t* __restrict__ count_partial, int bid) {
    const int64_t g0 = (int64_t)bid * (256 * U);
    uint4 raw[U];
    load_groups<T, U, 256>(W, g0, total4, threadIdx.x, raw);
    float thr, g;
    __shared__ float part[4];
    gamma_and_thr<4>(nodes, (N + 3) / 4, N, K, part, g, thr);
    if (bid == 0 && threadIdx.x == 0) gamma[0] = g;
    uint32_t cnt = 0u;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t i = g0 + threadIdx.x + u * 256;
        if (i < total4) pack_group<T, COUNT>(raw[u], thr, i, out, cnt);
    }
    store_group_counts<COUNT, 4>(cnt, count_partial, bid);
}
template <typename T, int U, bool COUNT = false>
__global__ __launch_bounds__(256) void wq_pack_kernel(const T* __restrict__ W, int64_t total4,
                                                      const float* __restrict__ nodes,
                                                      int64_t N, int64_t K, float* __restrict__ gamma,
                                                      uint8_t* __restrict__ out,
                                                      uint32_t* __restrict__ count_partial = nullptr) {
    wq_pack_body<T, U, COUNT>(W, total4, nodes, N, K, gamma, out, count_partial, blockIdx.x);
}

// Large matrices: the threshold is evaluated once, by workgroup 0, and
// published in `gate`, one 64-bit word holding the threshold bits and a
// ready mark, written with a single store (cleared by pass 1 of the same
// call).  Every other workgroup reads that word until the mark is there, at
// most `polls` times (kGatePolls unless a test lowers it) a short sleep
// apart, and then evaluates the threshold itself from the four-row nodes (the
// same bits).  No workgroup waits on another's progress beyond that bounded
// number of reads.  Waves 0-3 load and pack the weights (256 U groups of 4 a
// workgroup).
// POLLER: a fifth wave, with no weight loads, does the reading (or, in
// workgroup 0, evaluates gamma and the threshold: one wave, the same tree,
// so the same bits) and hands the threshold to waves 0-3 through LDS and one
// barrier.  A wave's reads wait for all of its earlier loads, so reads
// issued by a loading wave return only after its weights: when the whole
// matrix is requested in one round of resident workgroups, the threshold is
// on the critical path (4096 x 4096 bf16: 17.2 us for the call with thread 0
// reading, 14.6 us with the fifth wave, 15.6 us with the wait taken out
// altogether).  Over many rounds of workgroups the mark is there at the
// first read, and the fifth wave only leaves a CU fewer loading waves
// (28672 x 8192 fp32: 349 against 335 us), so there thread 0 reads the word
// after issuing its weight loads (workgroup 0: all four waves evaluate).
template <bool POLLER>
constexpr int pub_threads() { return POLLER ? 5 * kWave : 4 * kWave; }
// The four-wave form, as a body of the workgroup index `bid` (its role:
// workgroup 0 evaluates the threshold; its count slot) and of the block of
// groups `dbid` it packs.
template <typename T, int U, bool COUNT>
__device__ __forceinline__ void wq_pack_pub4_body(const T* __restrict__ W, int64_t total4,
                                                  uint64_t* __restrict__ gate, const float* __restrict__ nodes,
                                                  int64_t N, int64_t K, float* __restrict__ gamma,
                                                  uint8_t* __restrict__ out, int polls,
                                                  uint32_t* __restrict__ count_partial, int bid, int dbid) {
    const int64_t g0 = (int64_t)dbid * (256 * U);
    __shared__ float pub_thr;
    __shared__ int pub_ok;
    __shared__ float part[4];
    uint4 raw[U];
    float thr = 0.0f;
    load_groups<T, U, 256>(W, g0, total4, threadIdx.x, raw);
    if (bid == 0) {  // uniform
        float g;
        gamma_and_thr<4>(nodes, (N + 3) / 4, N, K, part, g, thr);
        if (threadIdx.x == 0) {
            gamma[0] = g;
            __hip_atomic_store(gate, ((uint64_t)1 << 32) | __float_as_uint(thr), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
    } else {
        if (threadIdx.x == 0) {
            int ok = 0;
            float t = 0.0f;
            for (int i = 0; i < polls; ++i) {
                const uint64_t word = __hip_atomic_load(gate, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if ((uint32_t)(word >> 32) == 1u) {
                    ok = 1;
                    t = __uint_as_float((uint32_t)word);
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
            }
            pub_ok = ok;
            pub_thr = t;
        }
        __syncthreads();
        if (pub_ok) {  // uniform: one LDS value for the workgroup
            thr = pub_thr;
        } else {
            float g;
            gamma_and_thr<4>(nodes, (N + 3) / 4, N, K, part, g, thr);
        }
    }
    uint32_t cnt = 0u;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t i = g0 + threadIdx.x + u * 256;
        if (i < total4) pack_group<T, COUNT>(raw[u], thr, i, out, cnt);
    }
    store_group_counts<COUNT, 4>(cnt, count_partial, bid);
}

template <typename T, int U, bool POLLER, bool COUNT = false>
__global__ __launch_bounds__(pub_threads<POLLER>()) void wq_pack_pub_kernel(
    const T* __restrict__ W, int64_t total4, uint64_t* __restrict__ gate, const float* __restrict__ nodes,
    int64_t N, int64_t K, float* __restrict__ gamma, uint8_t* __restrict__ out, int polls,
    uint32_t* __restrict__ count_partial = nullptr) {
    if constexpr (!POLLER) {
        // the groups in reverse order: the first workgroups read the end of W,
        // which the row-sum pass read last (the part of a matrix larger than
        // the Infinity Cache that it may still hold)
        wq_pack_pub4_body<T, U, COUNT>(W, total4, gate, nodes, N, K, gamma, out, polls, count_partial, blockIdx.x,
                                       (int)gridDim.x - 1 - (int)blockIdx.x);
    } else {
        const int64_t g0 = (int64_t)blockIdx.x * (256 * U);
        __shared__ float pub_thr;
        uint4 raw[U];
        float thr = 0.0f;
        const bool loader = threadIdx.x < 256;  // uniform in each wave
        if (loader) {
            load_groups<T, U, 256>(W, g0, total4, threadIdx.x, raw);
        } else {
            float g;
            bool ok = false;
            if (blockIdx.x == 0) {
                gamma_and_thr<1>(nodes, (N + 3) / 4, N, K, nullptr, g, thr);
                if (threadIdx.x == 256) {
                    gamma[0] = g;
                    __hip_atomic_store(gate, ((uint64_t)1 << 32) | __float_as_uint(thr), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                }
                ok = true;
            } else {
                for (int i = 0; i < polls; ++i) {
                    // every lane reads the same word: the wave's decision is uniform
                    const uint64_t word = __hip_atomic_load(gate, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    if ((uint32_t)(word >> 32) == 1u) {
                        ok = true;
                        thr = __uint_as_float((uint32_t)word);
                        break;
                    }
                    __builtin_amdgcn_s_sleep(2);
                }
            }
            if (!ok) gamma_and_thr<1>(nodes, (N + 3) / 4, N, K, nullptr, g, thr);
            if (threadIdx.x == 256) pub_thr = thr;
        }
        __syncthreads();
        thr = pub_thr;
        uint32_t cnt = 0u;
        if (threadIdx.x < 256) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t i = g0 + threadIdx.x + u * 256;
                if (i < total4) pack_group<T, COUNT>(raw[u], thr, i, out, cnt);
            }
        }
        store_group_counts<COUNT, 4>(cnt, count_partial, blockIdx.x);
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

// The weights of each thread come in with unconditional buffer loads (past
// the end an out-of-range offset reads zeros), all in flight together, then
// the thresholds of their rows (L2-resident after the first reads).
template <typename T>
__global__ __launch_bounds__(256) void wq_pack_rows_kernel(const T* __restrict__ W, int64_t total4, int64_t KB,
                                                           const float* __restrict__ thr,
                                                           uint8_t* __restrict__ out) {
    const int64_t g0 = (int64_t)blockIdx.x * (256 * kPackU);
    const int64_t base = g0 + threadIdx.x;
    const __amdgpu_buffer_rsrc_t rw = make_buf(W + g0 * 4);
    constexpr uint32_t kGroupBytes = 4 * sizeof(T);
    uint4 raw[kPackU];
#pragma unroll
    for (int u = 0; u < kPackU; ++u) {
        const uint32_t off = base + u * 256 < total4 ? (threadIdx.x + u * 256) * kGroupBytes : kBufOOB;
        if constexpr (sizeof(T) == 4) {
            raw[u] = buf_load16(rw, off);
        } else {
            const uint2 q = buf_load8(rw, off);
            raw[u] = make_uint4(q.x, q.y, 0u, 0u);
        }
    }
#pragma unroll
    for (int u = 0; u < kPackU; ++u) {
        const int64_t i = base + u * 256;  // packed byte: 4 weights of row i / KB
        if (i < total4) {
            float v[4];
            if constexpr (sizeof(T) == 4) {
                v[0] = __uint_as_float(raw[u].x);
                v[1] = __uint_as_float(raw[u].y);
                v[2] = __uint_as_float(raw[u].z);
                v[3] = __uint_as_float(raw[u].w);
            } else {
                v[0] = __uint_as_float(raw[u].x << 16);
                v[1] = __uint_as_float(raw[u].x & 0xffff0000u);
                v[2] = __uint_as_float(raw[u].y << 16);
                v[3] = __uint_as_float(raw[u].y & 0xffff0000u);
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
        wq_row_abs_sum_kernel<uint16_t><<<g1, b1, 0, s>>>(static_cast<const uint16_t*>(W), N, K, row_sums,
                                                           nullptr, nullptr, gamma, thr);
    else
        wq_row_abs_sum_kernel<float><<<g1, b1, 0, s>>>(static_cast<const float*>(W), N, K, row_sums, nullptr,
                                                        nullptr, gamma, thr);
    hipError_t e = hipGetLastError();
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

size_t weight_quant_ws_bytes(int64_t N) { return weight_quant_ws_size(N); }

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

__global__ __launch_bounds__(256) void code_counts_kernel(const uint8_t* __restrict__ P, int64_t nbytes,
                                                          uint32_t* __restrict__ partial) {
    __shared__ uint32_t red[4][4];
    uint32_t c[4] = {0u, 0u, 0u, 0u};  // zeros, +1, -1, 11
    auto count_fields = [&](uint32_t w, uint32_t field_mask) { count_code_fields(w, field_mask, c); };
    const int64_t nvec = nbytes / 16;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nvec; i += (int64_t)gridDim.x * 256) {
        const uint4 v = reinterpret_cast<const uint4*>(P)[i];
        count_fields(v.x, 0x55555555u);
        count_fields(v.y, 0x55555555u);
        count_fields(v.z, 0x55555555u);
        count_fields(v.w, 0x55555555u);
    }
    if (blockIdx.x == 0 && threadIdx.x < nbytes - nvec * 16) count_fields(P[nvec * 16 + threadIdx.x], 0x55u);
    // the four sums: each wave adds its lanes, one barrier, four threads add
    // the four waves
#pragma unroll
    for (int j = 0; j < 4; ++j) c[j] = wave_sum_u32(c[j]);
    if ((threadIdx.x & (kWave - 1)) == 0)
#pragma unroll
        for (int j = 0; j < 4; ++j) red[j][threadIdx.x >> 6] = c[j];
    __syncthreads();
    if (threadIdx.x < 4)
        partial[4 * blockIdx.x + threadIdx.x] =
            red[threadIdx.x][0] + red[threadIdx.x][1] + red[threadIdx.x][2] + red[threadIdx.x][3];
}

// slots of 4 partial counts per thread of the final kernel: it adds at most
// 256 * kFinalSlotsPerThread slots
constexpr int kFinalSlotsPerThread = 4;
static_assert(kCountGroups <= 256 * kFinalSlotsPerThread,
              "code_counts_final_kernel adds at most 256 * kFinalSlotsPerThread slots");

// partial: `groups` slots of 4 counts, slot b at word b * stride_words
__global__ __launch_bounds__(256) void code_counts_final_kernel(const uint32_t* __restrict__ partial,
                                                                int groups, int stride_words,
                                                                unsigned long long* __restrict__ counts) {
    __shared__ unsigned long long red[4][4];
    unsigned long long c[4] = {0ull, 0ull, 0ull, 0ull};
    // every slot of the thread requested at once (16 bytes each; past
    // `groups` an out-of-range offset reads zeros)
    const __amdgpu_buffer_rsrc_t rp = make_buf(partial);
    uint4 v[kFinalSlotsPerThread];
#pragma unroll
    for (int r = 0; r < kFinalSlotsPerThread; ++r) {
        const int b = threadIdx.x + 256 * r;
        v[r] = buf_load16(rp, b < groups ? (uint32_t)(b * stride_words) * 4u : kBufOOB);
    }
#pragma unroll
    for (int r = 0; r < kFinalSlotsPerThread; ++r) {
        c[0] += v[r].x;
        c[1] += v[r].y;
        c[2] += v[r].z;
        c[3] += v[r].w;
    }
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
    code_counts_final_kernel<<<1, 256, 0, s>>>(partial, groups, 4, reinterpret_cast<unsigned long long*>(counts));
    return hipGetLastError();
}

// The counted weight quant's last step: adds the (+1, -1) pairs of the pack
// workgroups (`pairs` pairs of uint32, pair p from the pack workgroup that
// wrote groups of 4 weights [p * gpw, (p + 1) * gpw) of `total4`) into the
// four counts, which pass 1 of the same call zeroed.  One pass: workgroup b
// adds pairs [4096 b, 4096 b + 4096), each thread 16 of them requested at
// once through a buffer descriptor (past `pairs` an out-of-range offset
// reads zeros), and thread 0 adds the workgroup's +1, -1 and zero counts
// into counts[1], [2], [0] with 64-bit integer atomics (exact in any order).
// Every code that pack writes is 00, 01 or 10, so a workgroup's zeros are the
// codes its pairs cover minus their nonzero ones, and counts[3] (pattern 11)
// stays 0.  (One workgroup in dependent passes instead: 7.5 us for the 57344
// pairs of 28672 x 8192 fp32.)
constexpr int kCountedPairsPerThread = 16;
constexpr int kCountedPairsPerGroup = 256 * kCountedPairsPerThread;

__global__ __launch_bounds__(256) void counted_sum_kernel(const uint2* __restrict__ partial, int64_t pairs,
                                                          int64_t gpw, int64_t total4,
                                                          unsigned long long* __restrict__ counts) {
    const int64_t p0 = (int64_t)blockIdx.x * kCountedPairsPerGroup;
    const __amdgpu_buffer_rsrc_t rp = make_buf(partial + p0);
    uint2 v[kCountedPairsPerThread];
#pragma unroll
    for (int r = 0; r < kCountedPairsPerThread; ++r) {
        const int b = threadIdx.x + 256 * r;
        v[r] = buf_load8(rp, p0 + b < pairs ? (uint32_t)b * 8u : kBufOOB);
    }
    // at most 4096 pairs of at most 16384 codes: 2^26, inside 32 bits
    uint32_t plus = 0u, minus = 0u;
#pragma unroll
    for (int r = 0; r < kCountedPairsPerThread; ++r) {
        plus += v[r].x;
        minus += v[r].y;
    }
    plus = wave_sum_u32(plus);
    minus = wave_sum_u32(minus);
    __shared__ uint32_t red[4][2];
    if ((threadIdx.x & (kWave - 1)) == 0) {
        red[threadIdx.x >> 6][0] = plus;
        red[threadIdx.x >> 6][1] = minus;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned long long p = (unsigned long long)red[0][0] + red[1][0] + red[2][0] + red[3][0];
        const unsigned long long m = (unsigned long long)red[0][1] + red[1][1] + red[2][1] + red[3][1];
        const int64_t p1 = p0 + kCountedPairsPerGroup < pairs ? p0 + kCountedPairsPerGroup : pairs;
        const int64_t g_end = p1 * gpw < total4 ? p1 * gpw : total4;
        const unsigned long long codes = 4ull * (unsigned long long)(g_end - p0 * gpw);
        atomicAdd(&counts[0], codes - p - m);
        atomicAdd(&counts[1], p);
        atomicAdd(&counts[2], m);
    }
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


// Workspace of weight_quant: row sums | threshold | four-row nodes
// (weight_quant_ws_size in common.h).
// the 64-bit threshold word of the pack launch, in the 256-byte slot after the row sums
static uint64_t* ws_gate(void* ws, int64_t N) {
    return reinterpret_cast<uint64_t*>(static_cast<char*>(ws) + ((N * 4 + 255) / 256) * 256);
}
static float* ws_nodes(void* ws, int64_t N) {
    return reinterpret_cast<float*>(static_cast<char*>(ws) + ((N * 4 + 255) / 256) * 256 + 256);
}

// Passes 2 and 3 (gamma, threshold, packing) from the four-row nodes in ws,
// in one launch.
// counts (when non-null): the pack launch also writes per-workgroup code
// counts to `count_partial` and one workgroup adds them into counts[4].
static hipError_t weight_quant_pack(const void* W, bool w_bf16, int64_t N, int64_t K, uint8_t* W_packed,
                                    float* gamma, void* ws, hipStream_t s, uint64_t* counts = nullptr,
                                    uint32_t* count_partial = nullptr) {
    uint64_t* gate = ws_gate(ws, N);
    const float* nodes = ws_nodes(ws, N);
    const int64_t total4 = N * K / 4;
    const unsigned g3 = (unsigned)((total4 + 256 * kPackU - 1) / (256 * kPackU));
    const bool fused = N * (int64_t)g3 <= kFusedGammaMaxWork;
    // the fifth-wave reader when one round of resident workgroups covers the matrix
    const int up5 = w_bf16 ? pack_u_pub<uint16_t, true>() : pack_u_pub<float, true>();
    const int64_t g5 = (total4 + 256 * up5 - 1) / (256 * up5);
    int dev = 0, cus = 0;
    hipError_t e = hipSuccess;
    if (!fused) {
        e = hipGetDevice(&dev);
        if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
    }
    const bool poller = g5 <= (int64_t)kPollerGroupsPerCu * cus;
    const int up = poller ? up5 : pack_u_pub<float, false>();
    const unsigned g3p = (unsigned)((total4 + 256 * up - 1) / (256 * up));
    const uint16_t* Wb = static_cast<const uint16_t*>(W);
    const float* Wf = static_cast<const float*>(W);
#define BITNET_PACK(T_, W_, C_)                                                                              \
    do {                                                                                                     \
        if (fused)                                                                                           \
            wq_pack_kernel<T_, kPackU, C_><<<g3, 256, 0, s>>>(W_, total4, nodes, N, K, gamma, W_packed,        \
                                                               count_partial);                               \
        else if (poller)                                                                                     \
            wq_pack_pub_kernel<T_, pack_u_pub<T_, true>(), true, C_><<<g3p, pub_threads<true>(), 0, s>>>(     \
                W_, total4, gate, nodes, N, K, gamma, W_packed, g_gate_polls, count_partial);                \
        else                                                                                                 \
            wq_pack_pub_kernel<T_, pack_u_pub<T_, false>(), false, C_><<<g3p, pub_threads<false>(), 0, s>>>(  \
                W_, total4, gate, nodes, N, K, gamma, W_packed, g_gate_polls, count_partial);                \
    } while (0)
    if (counts) {
        if (w_bf16) BITNET_PACK(uint16_t, Wb, true);
        else BITNET_PACK(float, Wf, true);
    } else {
        if (w_bf16) BITNET_PACK(uint16_t, Wb, false);
        else BITNET_PACK(float, Wf, false);
    }
#undef BITNET_PACK
    e = hipGetLastError();
    if (e != hipSuccess || !counts) return e;
    const int64_t pairs = fused ? g3 : g3p;
    const int64_t gpw = 256 * (int64_t)(fused ? kPackU : up);  // groups of 4 weights a pack workgroup
    counted_sum_kernel<<<(unsigned)((pairs + kCountedPairsPerGroup - 1) / kCountedPairsPerGroup), 256, 0, s>>>(
        reinterpret_cast<const uint2*>(count_partial), pairs, gpw, total4,
        reinterpret_cast<unsigned long long*>(counts));
    return hipGetLastError();
}

// the counted call's (+1, -1) pairs, one per pack workgroup, after
// weight_quant's workspace (sized for the larger of the two pack grids)
static size_t weight_quant_counted_slots_offset(int64_t N) { return weight_quant_ws_size(N); }
size_t weight_quant_counted_ws_bytes(int64_t N, int64_t K) {
    const int64_t groups = (N * K / 4 + 256 * kPackU - 1) / (256 * kPackU);
    return weight_quant_ws_size(N) + (size_t)((groups * 8 + 255) / 256 * 256);
}

hipError_t launch_weight_quant(const void* W, bool w_bf16, int64_t N, int64_t K,
                               uint8_t* W_packed, float* gamma, void* ws, hipStream_t s) {
    float* row_sums = static_cast<float*>(ws);
    float* nodes = ws_nodes(ws, N);
    uint64_t* gate = ws_gate(ws, N);
    const dim3 g1((unsigned)((N + kWqWaves - 1) / kWqWaves)), b1(kWqWaves * kWave);
    if (w_bf16)
        wq_row_abs_sum_kernel<uint16_t><<<g1, b1, 0, s>>>(static_cast<const uint16_t*>(W), N, K,
                                                           row_sums, nodes, gate, nullptr, nullptr);
    else
        wq_row_abs_sum_kernel<float><<<g1, b1, 0, s>>>(static_cast<const float*>(W), N, K,
                                                        row_sums, nodes, gate, nullptr, nullptr);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return weight_quant_pack(W, w_bf16, N, K, W_packed, gamma, ws, s);
}

// weight_quant plus the code counts, written by the pack launch's workgroups
// as they pack (no second read of the packed weights)
hipError_t launch_weight_quant_counted(const void* W, bool w_bf16, int64_t N, int64_t K, uint8_t* W_packed,
                                       float* gamma, uint64_t* counts, void* ws, hipStream_t s) {
    float* row_sums = static_cast<float*>(ws);
    float* nodes = ws_nodes(ws, N);
    uint64_t* gate = ws_gate(ws, N);
    uint32_t* slots =
        reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + weight_quant_counted_slots_offset(N));
    const dim3 g1((unsigned)((N + kWqWaves - 1) / kWqWaves)), b1(kWqWaves * kWave);
    if (w_bf16)
        wq_row_abs_sum_kernel<uint16_t><<<g1, b1, 0, s>>>(static_cast<const uint16_t*>(W), N, K,
                                                           row_sums, nodes, gate, nullptr, nullptr, counts);
    else
        wq_row_abs_sum_kernel<float><<<g1, b1, 0, s>>>(static_cast<const float*>(W), N, K,
                                                        row_sums, nodes, gate, nullptr, nullptr, counts);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return weight_quant_pack(W, w_bf16, N, K, W_packed, gamma, ws, s, counts, slots);
}

// ============================================ both quantizers, one launch fewer
// Two launches either way, the activation stream beside one of the two
// weight passes; same bodies, same arithmetic, so the outputs are
// bit-identical to the two separate calls.
//  - activation bytes >= weight bytes and a matrix large enough for the
//    published threshold (the 7B prefill layer): launch 1 is weight_quant's
//    pass 1 (row sums and nodes); launch 2 runs act_quant's row-walking body
//    on workgroups [0, A) and the weight pack on [A, A + P), so the pack's
//    second read of W streams beside the activations instead of alone, and
//    gamma's nodes are complete before launch 2 starts.  8192 x 4096 x 4096
//    bf16: 30.0 us against 32.3 us the other way; with the pack's workgroups
//    first in the grid 34.1 us (they take every slot and the activation
//    workgroups queue behind them).
//  - otherwise: launch 1 runs act_quant on [0, A) and the row sums on
//    [A, A + ceil(N/4)); launch 2 is weight_quant's pack.  A weight matrix
//    far larger than the activations (4096 x 28672 x 8192, fp32 W): 362 us
//    against 366 us the other way; a small layer (8192 x 1376 x 512): the
//    call alone 9.4 against 9.15 us, but the forward step (the call and the
//    product) 30.8-31.5 against 31.8-32.0 us.
template <typename TX, int NB, typename TW>
__global__ __launch_bounds__(kAqWaves * kWave) void quant_operands_kernel(
    const TX* __restrict__ X, int64_t M, int64_t K, float eps, int8_t* __restrict__ Q, float* __restrict__ S,
    int act_blocks, const TW* __restrict__ W, int64_t N, float* __restrict__ row_sums,
    float* __restrict__ nodes, uint64_t* __restrict__ gate) {
    static_assert(kAqWaves == kWqWaves, "one workgroup shape for both bodies");
    const int b = blockIdx.x;  // uniform
    if (b < act_blocks) act_quant_rows_body<TX, NB>(X, M, K, eps, Q, S, b, act_blocks);
    else wq_row_abs_sum_body<TW>(W, N, K, row_sums, b - act_blocks, nodes, gate);
}

template <typename TX, int NB, typename TW>
__global__ __launch_bounds__(kAqWaves * kWave) void act_pack_kernel(
    const TX* __restrict__ X, int64_t M, int64_t K, float eps, int8_t* __restrict__ Q, float* __restrict__ S,
    int act_blocks, const TW* __restrict__ W, int64_t total4, uint64_t* __restrict__ gate,
    const float* __restrict__ nodes, int64_t N, float* __restrict__ gamma, uint8_t* __restrict__ out,
    int polls) {
    static_assert(kAqWaves == 4, "one workgroup shape for both bodies");
    const int b = blockIdx.x;  // uniform
    if (b < act_blocks) {
        act_quant_rows_body<TX, NB>(X, M, K, eps, Q, S, b, act_blocks);
    } else {
        wq_pack_pub4_body<TW, pack_u_pub<TW, false>(), false>(W, total4, gate, nodes, N, K, gamma, out, polls,
                                                              nullptr, b - act_blocks, b - act_blocks);
    }
}

namespace {
template <typename TX, typename TW, int NB>
hipError_t act_pack_launch(const TX* X, int64_t M, int64_t K, float eps, int8_t* Q, float* S, const TW* W,
                           int64_t N, uint8_t* W_packed, float* gamma, void* ws, hipStream_t s) {
    float* row_sums = static_cast<float*>(ws);
    float* nodes = ws_nodes(ws, N);
    uint64_t* gate = ws_gate(ws, N);
    const int act_blocks = (int)std::min<int64_t>((M + kAqWaves - 1) / kAqWaves, kAqMaxGroups);
    const int64_t total4 = N * K / 4;
    const int64_t g3 = (total4 + 256 * kPackU - 1) / (256 * kPackU);
    const bool fused = N * g3 <= kFusedGammaMaxWork;
    if (fused || M * K * (int64_t)sizeof(TX) < N * K * (int64_t)sizeof(TW)) {  // act_quant beside the row sums
        const int64_t wq_blocks = (N + kWqWaves - 1) / kWqWaves;
        const dim3 grid((unsigned)(act_blocks + wq_blocks)), block(kAqWaves * kWave);
        quant_operands_kernel<TX, NB, TW><<<grid, block, 0, s>>>(X, M, K, eps, Q, S, act_blocks, W, N, row_sums,
                                                                 nodes, gate);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        return weight_quant_pack(W, sizeof(TW) == 2, N, K, W_packed, gamma, ws, s);
    }
    const dim3 g1((unsigned)((N + kWqWaves - 1) / kWqWaves)), b1(kWqWaves * kWave);
    wq_row_abs_sum_kernel<TW><<<g1, b1, 0, s>>>(W, N, K, row_sums, nodes, gate, nullptr, nullptr);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    constexpr int up = pack_u_pub<TW, false>();
    const int pack_blocks = (int)((total4 + 256 * up - 1) / (256 * up));
    const dim3 grid((unsigned)(pack_blocks + act_blocks)), block(kAqWaves * kWave);
    act_pack_kernel<TX, NB, TW><<<grid, block, 0, s>>>(X, M, K, eps, Q, S, act_blocks, W, total4, gate, nodes, N,
                                                       gamma, W_packed, g_gate_polls);
    return hipGetLastError();
}
template <typename TX, typename TW>
hipError_t act_pack_nb(const TX* X, int64_t M, int64_t K, float eps, int8_t* Q, float* S, const TW* W, int64_t N,
                       uint8_t* W_packed, float* gamma, void* ws, int nblk, hipStream_t s) {
    switch (nblk) {
        case 1: return act_pack_launch<TX, TW, 1>(X, M, K, eps, Q, S, W, N, W_packed, gamma, ws, s);
        case 2: return act_pack_launch<TX, TW, 2>(X, M, K, eps, Q, S, W, N, W_packed, gamma, ws, s);
        case 4: return act_pack_launch<TX, TW, 4>(X, M, K, eps, Q, S, W, N, W_packed, gamma, ws, s);
        case 8: return act_pack_launch<TX, TW, 8>(X, M, K, eps, Q, S, W, N, W_packed, gamma, ws, s);
        case 16: return act_pack_launch<TX, TW, 16>(X, M, K, eps, Q, S, W, N, W_packed, gamma, ws, s);
        default: return hipErrorInvalidValue;
    }
}
template <typename TX>
hipError_t act_pack_w(const TX* X, int64_t M, int64_t K, float eps, int8_t* Q, float* S, const void* W,
                      bool w_bf16, int64_t N, uint8_t* W_packed, float* gamma, void* ws, int nblk, hipStream_t s) {
    if (w_bf16)
        return act_pack_nb(X, M, K, eps, Q, S, static_cast<const uint16_t*>(W), N, W_packed, gamma, ws, nblk, s);
    return act_pack_nb(X, M, K, eps, Q, S, static_cast<const float*>(W), N, W_packed, gamma, ws, nblk, s);
}
}  // namespace

hipError_t launch_quant_operands(const void* X, bool x_bf16, int64_t M, int64_t K, float eps, int8_t* Xq,
                                 float* scale_x, const void* W, bool w_bf16, int64_t N, uint8_t* W_packed,
                                 float* gamma, void* ws, hipStream_t s) {
    const int64_t E = x_bf16 ? 8 : 4;
    const int64_t nblk = (K + kWave * E - 1) / (kWave * E);
    const bool rows = K == nblk * kWave * E && (nblk == 1 || nblk == 2 || nblk == 4 || nblk == 8 || nblk == 16);
    if (!rows) {  // act_quant's general kernel: the two calls' launches in order
        hipError_t e = launch_act_quant(X, x_bf16, M, K, eps, Xq, scale_x, s);
        if (e != hipSuccess) return e;
        return launch_weight_quant(W, w_bf16, N, K, W_packed, gamma, ws, s);
    }
    return x_bf16 ? act_pack_w(static_cast<const uint16_t*>(X), M, K, eps, Xq, scale_x, W, w_bf16, N, W_packed,
                               gamma, ws, (int)nblk, s)
                  : act_pack_w(static_cast<const float*>(X), M, K, eps, Xq, scale_x, W, w_bf16, N, W_packed, gamma,
                               ws, (int)nblk, s);
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
