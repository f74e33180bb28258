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
// column order unpack16 produces; tokens >= M are zero).  With K <= 4096 the
// token rows come in as coalesced 16-byte loads, are byte-transposed and
// written to an LDS tile, all before the first weight load is issued (with
// the weight stream already in flight the activation lines return behind
// it), and every lane then reads its operand from the tile.  The row factors
// gamma / scale_x are requested at the start as well.  Then every packed
// weight byte of the pass is requested with no branch in front of the loads;
// all row groups are computed before one reduction of the 16 partial int32
// tiles in LDS.
//
// Fused decode variant (TX = bf16 bits or float): the activations come in
// unquantized and every workgroup quantizes them itself, so a decode step is
// one launch instead of two.  The quantization is act_quant's, operation for
// operation: act_quant's blocks (64 lanes x one 16-byte chunk, lane l holding
// elements 64E*b + E*l .. +E-1 of block b) are the work items, shared out
// over the 16 waves; each item's block sum of squares (in-lane tree, then the
// lane tree) and block max go to LDS; each row's scale comes from its
// partials in block order (the pairwise tree over blocks, missing blocks +0,
// which leaves the value unchanged) with the same binary32 steps; then each
// item's q goes to the LDS activation tile in natural order, byte-transposed
// in registers as it is read.  So q and scale_x are bit-identical to
// act_quant's and Y to act_quant followed by this GEMV.  Every workgroup
// quantizes all M*K activations (all of K feeds its row groups), about 11
// VALU operations per element: cheap for a few tokens, more than the
// separate act_quant launch it saves from about 8 tokens of 4096 on.
#include <type_traits>

#include "common.h"

namespace bitnet {

namespace {
typedef int v4i __attribute__((ext_vector_type(4)));
constexpr int kWaves = 16;
constexpr int kThreads = kWaves * 64;
constexpr int kMaxGroups = 4;  // row groups per pass when S <= 4
// fused decode: at most this many (token row, block) items per wave, so the
// raw X chunks (4 registers each) stay in registers with no spill
constexpr int kDecodeMaxItems = 8;
}  // namespace

// S: MFMA steps (64 columns) per wave, Kw = 64*S; FULL: K == 16*Kw, so every
// lane's column range lies inside the row and loads are 16-byte vectors.
// STAGE: the activations come in with coalesced 16-byte loads through an LDS
// tile (M > 8: 16 token rows would otherwise be fetched as scattered pieces
// by every lane); without it each lane loads its own chunks (few tokens).
constexpr int kStageMaxK = 4096;  // LDS activation tile bound
constexpr int kStageStride = kStageMaxK + 16;

// CH: gamma_p holds one scale per output channel (see the GEMM).
// DL: Wp is in the decode layout (pack_decode_kernel below), else row-major.
// TX: int8_t, Xin = Xq and scale_x given; uint16_t (bf16) or float, Xin = X
// unquantized, quantized here with eps (K <= kStageMaxK), scale_x unused,
// and workgroup 0 writes q and the scales to xq_out / sx_out when non-null.
template <int S, bool FULL, bool STAGE, bool CH, typename TX = int8_t, int IT = 1, bool DL = false>
__global__ __launch_bounds__(kThreads) void gemv_t2_kernel(
    const void* __restrict__ Xin, const float* __restrict__ scale_x,
    const uint8_t* __restrict__ Wp, const float* __restrict__ gamma_p, int M, int N, int K,
    float* __restrict__ Y, int32_t* __restrict__ acc_out, float eps, int8_t* __restrict__ xq_out,
    float* __restrict__ sx_out) {
    constexpr bool QX = !std::is_same<TX, int8_t>::value;
    const int8_t* __restrict__ Xq = static_cast<const int8_t*>(Xin);
    // row groups per pass: weight (G*S) and activation (4*S) registers stay
    // within the budget of 4 waves per SIMD
    constexpr int G = S >= 16 ? 1 : (S >= 8 ? 2 : kMaxGroups);
    __shared__ int red[G][kWaves][256];
    __shared__ __align__(16) uint8_t As[STAGE || QX ? 16 * kStageStride : 16];
    __shared__ float tok_scale[QX ? 16 : 1], tok_inv[QX ? 16 : 1];
    // the row factor of each token: gamma / scale_x (1 / scale_x with a
    // scale per channel), requested before anything else so that the
    // epilogue does not wait for it
    __shared__ float row_rs[QX ? 1 : 16];
    // fused: per token row and block, the block's sum of squares and max |x|
    constexpr int QE = Vec16<std::conditional_t<QX, TX, float>>::E;
    constexpr int QBLK = kWave * QE;
    constexpr int QNB = QX ? kStageMaxK / QBLK : 1;  // blocks of the longest row
    __shared__ float blk_sq[QX ? 16 : 1][QNB], blk_max[QX ? 16 : 1][QNB];
    constexpr int Kw = 64 * S;
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);  // uniform in the wave
    const int col = lane & 15, g = lane >> 4;
    const int kb = wave * Kw + g * (Kw / 4);  // first column of this lane
    const int KB = K / 4;
    const int ngroups = (N + 15) / 16;

    // ---- activation operand: token col, columns kb + 16 s
    uint4 av[S];
    constexpr int kAPer = STAGE ? (16 * kStageMaxK / 16) / kThreads : 1;
    uint4 ac[kAPer];  // coalesced chunks for the LDS tile (STAGE)
    // 16-byte chunks per row: a constant when the row is whole steps (FULL:
    // K = 1024 S), so the staging index math has no runtime division
    const int kch = FULL ? 64 * S : K / 16;
    // fused: work item i = (token row i / nblk, block i % nblk); wave w takes
    // items w, w + 16, ...  Their raw X chunks are requested first, with
    // unconditional buffer loads (offsets past the rows read zeros, as
    // act_quant pads), so that the wait for them is not a wait for the
    // weight stream that follows.
    uint4 xc[QX ? IT : 1];
    const int qnblk = (K + QBLK - 1) / QBLK;
    if constexpr (QX) {
        static_assert(S <= kStageMaxK / (16 * 64), "fused rows fit the LDS tile");
        const __amdgpu_buffer_rsrc_t rx = make_buf(Xin);
#pragma unroll
        for (int j = 0; j < IT; ++j) {
            const int it = wave + kWaves * j;
            const int row = it / qnblk, blk = it - row * qnblk;
            // K % 16 == 0: a lane's QE elements are all inside the row or all past it
            const int k0 = blk * QBLK + lane * QE;
            const bool v = row < M && k0 < K;
            xc[j] = buf_load16(rx, v ? (uint32_t)(((int64_t)row * K + k0) * (int)sizeof(TX)) : kBufOOB);
        }
    } else if constexpr (STAGE) {
        if (t < 16) row_rs[t] = t < M ? (CH ? 1.0f / scale_x[t] : *gamma_p / scale_x[t]) : 0.0f;
#pragma unroll
        for (int i = 0; i < kAPer; ++i) {
            const int c = t + i * kThreads;
            const int tok = c / kch;
            ac[i] = make_uint4(0, 0, 0, 0);
            if (c < 16 * kch && tok < M)
                ac[i] = *reinterpret_cast<const uint4*>(Xq + (int64_t)tok * K + 16 * (c - tok * kch));
        }
        // The tile is written before any weight load is issued: staged while
        // the weight stream is already in flight, the activation lines came
        // back behind it (measured at N = 11008, K = 4096, 16 tokens: 6.5 us
        // with the weight loads first, 5.2 us this way).
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < kAPer; ++i) {
            const int c = t + i * kThreads;
            if (c < 16 * kch) {
                const int tok = c / kch, kc = c - tok * kch;
                const uint32_t a[4] = {ac[i].x, ac[i].y, ac[i].z, ac[i].w};
                uint32_t o[4];
                transpose4x4_bytes(a, o);
                *reinterpret_cast<uint4*>(As + tok * kStageStride + 16 * kc) = make_uint4(o[0], o[1], o[2], o[3]);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    } else {
        if (t < 16) row_rs[t] = t < M ? (CH ? 1.0f / scale_x[t] : *gamma_p / scale_x[t]) : 0.0f;
        const bool tv = col < M;
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const int k = kb + 16 * s;
            av[s] = make_uint4(0, 0, 0, 0);
            if (tv && (FULL || k < K)) av[s] = *reinterpret_cast<const uint4*>(Xq + (int64_t)col * K + k);
        }
    }

    // ---- weights for up to G row groups of the pass at `base`, all loads in flight
    auto load_weights = [&](int base, uint32_t (&wq)[G][S]) {
#pragma unroll
        for (int r = 0; r < G; ++r) {
            const int grp = base + r * gridDim.x;
            const int n = grp * 16 + col;
            const bool nv = grp < ngroups && n < N;
            const int nc = nv ? n : 0;  // clamped address, value dropped below
            const uint8_t* src = Wp + (int64_t)nc * KB + kb / 4;
            if constexpr (DL) {
                // decode layout: this wave's pieces of the row group are S/4
                // contiguous kilobytes, one per load instruction, in lane order
                static_assert(FULL && S % 4 == 0, "the decode layout holds whole 16-byte pieces");
                const int gc = grp < ngroups ? grp : 0;
                const uint8_t* blk = Wp + ((int64_t)gc * kWaves + wave) * (S / 4) * 1024 + lane * 16;
#pragma unroll
                for (int s = 0; s < S; s += 4) {
                    const uint4 v = *reinterpret_cast<const uint4*>(blk + (s / 4) * 1024);
                    wq[r][s] = nv ? v.x : 0u;
                    wq[r][s + 1] = nv ? v.y : 0u;
                    wq[r][s + 2] = nv ? v.z : 0u;
                    wq[r][s + 3] = nv ? v.w : 0u;
                }
            } else if constexpr (FULL && S % 4 == 0) {
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
    };

    // ---- products of every row group of the pass, then one reduction
    auto products = [&](int base, const uint32_t (&wq)[G][S]) {
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
                    const float rs = QX ? 1.0f / tok_scale[tk] : row_rs[tk];
                    Y[(int64_t)tk * N + nn] = ((float)sum * rs) * gamma_p[nn];
                } else {
                    const float rs = QX ? *gamma_p / tok_scale[tk] : row_rs[tk];
                    Y[(int64_t)tk * N + nn] = (float)sum * rs;
                }
                if (acc_out) acc_out[(int64_t)tk * N + nn] = sum;
            }
        }
        __syncthreads();
    };

    if constexpr (QX) {
        // ---- fused: the first pass is peeled so that the X loads, the first
        // weight loads and the quantization are straight-line code (a wait
        // for X then counts only the weight loads issued after it)
        constexpr int E = QE, BLK = QBLK, NBX = QNB;
        using TW = std::conditional_t<QX, TX, float>;
        int base = blockIdx.x;  // < ngroups: the grid has at most ngroups workgroups
        // X first, alone: requested behind the weight stream it arrives late
        // (every workgroup reads the same few lines); then the weight loads,
        // and the quantization runs while they stream in
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
        __builtin_amdgcn_sched_barrier(0);
        uint32_t wq[G][S];
        load_weights(base, wq);
        // 1) per item: act_quant's block partials (in-lane tree, lane tree;
        //    lane maxima, wave max)
#pragma unroll
        for (int j = 0; j < IT; ++j) {
            const int it = wave + kWaves * j;
            const int row = it / qnblk, blk = it - row * qnblk;
            if (row < M) {
                float v[E], sq[E], amax = 0.0f;
                widen16<TW>(xc[j], v);
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    sq[e] = v[e] * v[e];
                    amax = fmaxf(amax, fabsf(v[e]));
                }
                const float bsum = wave_tree_sum(lane_tree<E>(sq));
                amax = wave_max(amax);
                if (lane == 0) {
                    blk_sq[row][blk] = bsum;
                    blk_max[row][blk] = amax;
                }
            }
        }
        // token rows past M are zeros in the tile
        if (wave >= M)
            for (int k0 = lane * 16; k0 < qnblk * BLK; k0 += kWave * 16)
                *reinterpret_cast<uint4*>(As + wave * kStageStride + k0) = make_uint4(0, 0, 0, 0);
        __syncthreads();
        // 2) wave r < M: row r's 1/RMS and scale from the partials in block
        //    order (missing blocks +0: the same tree value)
        if (wave < M) {
            float bs[NBX], amax = 0.0f;
#pragma unroll
            for (int b = 0; b < NBX; ++b) {
                bs[b] = b < qnblk ? blk_sq[wave][b] : 0.0f;
                amax = fmaxf(amax, b < qnblk ? blk_max[wave][b] : 0.0f);
            }
            const float ss = lane_tree<NBX>(bs);
            const float ms = ss / (float)K;
            const float d = sqrtf(ms + eps);
            const float inv = 1.0f / d;
            const float a = amax * inv;  // max|x * inv| == max|x| * inv
            const float scale = 127.0f / fmaxf(a, 1e-5f);
            if (lane == 0) {
                tok_inv[wave] = inv;
                tok_scale[wave] = scale;
                if (sx_out && blockIdx.x == 0) sx_out[wave] = scale;
            }
        }
        __syncthreads();
        // 3) per item: its block of q into the tile
#pragma unroll
        for (int j = 0; j < IT; ++j) {
            const int it = wave + kWaves * j;
            const int row = it / qnblk, blk = it - row * qnblk;
            if (row < M) {
                const float inv = tok_inv[row], scale = tok_scale[row];
                float v[E];
                widen16<TW>(xc[j], v);
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
                const int k0 = blk * BLK + lane * E;
                uint8_t* qp = As + row * kStageStride + k0;
                if constexpr (E == 8) *reinterpret_cast<uint2*>(qp) = make_uint2(pk[0], pk[1]);
                else *reinterpret_cast<uint32_t*>(qp) = pk[0];
                if (xq_out && blockIdx.x == 0 && k0 < K) {
                    int8_t* qo = xq_out + (int64_t)row * K + k0;
                    if constexpr (E == 8) *reinterpret_cast<uint2*>(qo) = make_uint2(pk[0], pk[1]);
                    else *reinterpret_cast<uint32_t*>(qo) = pk[0];
                }
            }
        }
        __syncthreads();
        // the operand: natural-order q from the tile, byte-transposed
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const int k = kb + 16 * s;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (FULL || k < K) v = *reinterpret_cast<const uint4*>(As + col * kStageStride + k);
            const uint32_t a[4] = {v.x, v.y, v.z, v.w};
            uint32_t o[4];
            transpose4x4_bytes(a, o);
            av[s] = make_uint4(o[0], o[1], o[2], o[3]);
        }
        products(base, wq);
        for (base += gridDim.x * G; base < ngroups; base += gridDim.x * G) {
            uint32_t wq2[G][S];
            load_weights(base, wq2);
            products(base, wq2);
        }
    } else {
        bool transposed = false;
        for (int base = blockIdx.x; base < ngroups; base += gridDim.x * G) {
            uint32_t wq[G][S];
            load_weights(base, wq);
            if (!transposed) {
                if constexpr (STAGE) {
                    __syncthreads();  // the tile written above
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
            products(base, wq);
        }
    }
}

// ------------------------------------------- staged GEMV for whole-step rows
// gemv_t2_kernel's int8 path specialised to K = 1024 S (S = 1, 2, 4): the
// token rows are staged in the LDS tile with compile-time index math, all
// before the first weight load, and the row factors requested first.  Same
// lane mapping, products and reduction, so the same bits.  (Written as its
// own kernel: the identical schedule inside the general template measured
// 0.4 us slower at 16 tokens x 11008 x 4096, 5.66 against 5.25 us.)
// DENSE (more than 4 tokens): every token-row load is an unconditional
// buffer load (rows >= M read zeros), so all of them are in flight together;
// a load under a per-thread condition made the compiler wait after every
// second one (16 tokens: 5.41 -> 5.21 us).  With at most 4 tokens most of
// those loads would read nothing, and the conditional form measured faster
// (2 tokens: 4.99 against 5.07 us).
template <int S, bool CH, bool DENSE>
__global__ __launch_bounds__(kThreads) void gemv_staged_kernel(
    const int8_t* __restrict__ Xq, const float* __restrict__ scale_x, const uint8_t* __restrict__ Wp,
    const float* __restrict__ gamma_p, int M, int N, float* __restrict__ Y, int32_t* __restrict__ acc_out) {
    constexpr int K = 1024 * S, KB = K / 4, Kw = 64 * S, kch = K / 16;
    constexpr int G = S >= 16 ? 1 : (S >= 8 ? 2 : kMaxGroups);
    constexpr int kAPer = 16 * kch / kThreads;  // 16-byte chunks per thread for 16 token rows
    constexpr int kPitch = K + 16;              // LDS row pitch (16-byte skew between rows)
    static_assert(16 * kch % kThreads == 0, "whole chunks per thread");
    __shared__ int red[G][kWaves][256];
    __shared__ __align__(16) uint8_t As[16 * kPitch];
    __shared__ float row_rs[16];
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int col = lane & 15, g = lane >> 4;
    const int kb = wave * Kw + g * (Kw / 4);
    const int ngroups = (N + 15) / 16;
    // the token rows: coalesced 16-byte chunks, waited for, byte-transposed
    // into the tile (rows >= M as zeros) before any weight load is issued;
    // the row factors: gamma / scale_x (1 / scale_x with a scale per channel)
    uint4 ac[kAPer];
    if constexpr (DENSE) {
        const float sxv = __uint_as_float(buf_load4(make_buf(scale_x), t < M ? 4u * t : kBufOOB));
        const __amdgpu_buffer_rsrc_t rx = make_buf(Xq);
#pragma unroll
        for (int i = 0; i < kAPer; ++i) {
            const int c = t + i * kThreads;
            ac[i] = buf_load16(rx, c / kch < M ? (uint32_t)((c / kch) * K + 16 * (c % kch)) : kBufOOB);
        }
        const float rs = t < M ? (CH ? 1.0f / sxv : *gamma_p / sxv) : 0.0f;  // every thread: no sunk load
        if (t < 16) row_rs[t] = rs;
    } else {
        if (t < 16) row_rs[t] = t < M ? (CH ? 1.0f / scale_x[t] : *gamma_p / scale_x[t]) : 0.0f;
#pragma unroll
        for (int i = 0; i < kAPer; ++i) {
            const int c = t + i * kThreads;
            ac[i] = make_uint4(0, 0, 0, 0);
            if (c / kch < M) ac[i] = *reinterpret_cast<const uint4*>(Xq + (int64_t)(c / kch) * K + 16 * (c % kch));
        }
    }
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < kAPer; ++i) {
        const int c = t + i * kThreads;
        const uint32_t a[4] = {ac[i].x, ac[i].y, ac[i].z, ac[i].w};
        uint32_t o[4];
        transpose4x4_bytes(a, o);
        *reinterpret_cast<uint4*>(As + (c / kch) * kPitch + 16 * (c % kch)) = make_uint4(o[0], o[1], o[2], o[3]);
    }
    __builtin_amdgcn_sched_barrier(0);
    uint4 av[S];
    bool first = true;
    for (int base = blockIdx.x; base < ngroups; base += gridDim.x * G) {
        // every packed weight byte of the pass requested at once
        uint32_t wq[G][S];
#pragma unroll
        for (int r = 0; r < G; ++r) {
            const int grp = base + r * gridDim.x;
            const int n = grp * 16 + col;
            const bool nv = grp < ngroups && n < N;
            const uint8_t* src = Wp + (int64_t)(nv ? n : 0) * KB + kb / 4;
#pragma unroll
            for (int s = 0; s < S; s += 4) {
                if constexpr (S >= 4) {
                    const uint4 v = *reinterpret_cast<const uint4*>(src + 4 * s);
                    wq[r][s] = nv ? v.x : 0u;
                    wq[r][s + 1] = nv ? v.y : 0u;
                    wq[r][s + 2] = nv ? v.z : 0u;
                    wq[r][s + 3] = nv ? v.w : 0u;
                }
            }
            if constexpr (S < 4) {
#pragma unroll
                for (int s = 0; s < S; ++s) {
                    const uint32_t v = *reinterpret_cast<const uint32_t*>(src + 4 * s);
                    wq[r][s] = nv ? v : 0u;
                }
            }
        }
        if (first) {
            __syncthreads();  // the tile
#pragma unroll
            for (int s = 0; s < S; ++s) av[s] = *reinterpret_cast<const uint4*>(As + col * kPitch + kb + 16 * s);
            first = false;
        }
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
                if constexpr (CH) Y[(int64_t)tk * N + nn] = ((float)sum * row_rs[tk]) * gamma_p[nn];
                else Y[(int64_t)tk * N + nn] = (float)sum * row_rs[tk];
                if (acc_out) acc_out[(int64_t)tk * N + nn] = sum;
            }
        }
        __syncthreads();
    }
}

// ------------------------------------------------ one token: the row GEMV
// For a single token the matrix cores would multiply fifteen zero rows, and
// gemv_t2_kernel's split of K over sixteen waves needs a reduction through
// LDS.  Here one wave takes kRowRows weight rows with its lanes across K:
// lane l holds the 64-column chunks l, l + 64, ... of each row (16 packed
// bytes per load, so every load instruction reads 1 KB of one row), unpacks
// them with unpack16, multiplies on the VALU with v_dot4 against the token's
// matching byte-transposed activation chunks, and the 64 lane sums are added
// with DPP (the integer sum is exact in any order).  The epilogue is
// gemv_t2_kernel's, operation for operation, so Y and acc are the same bits.
constexpr int kRowRows = 4;   // weight rows per wave
constexpr int kRowWaves = 4;  // waves per workgroup

template <int CTRL>
__device__ __forceinline__ int dpp_read_i32(int v) {
    return __builtin_amdgcn_mov_dpp(v, CTRL, 0xf, 0xf, false);
}
// sum over the 64 lanes (every lane active), returned to every lane
__device__ __forceinline__ int wave_sum_i32(int v) {
    v += dpp_read_i32<kDppXor1>(v);
    v += dpp_read_i32<kDppXor2>(v);
    v += dpp_read_i32<kDppHalfMirror>(v);
    v += dpp_read_i32<kDppMirror>(v);
    return (__builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16)) +
           (__builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48));
}

// CHK: 64-column chunks per lane (K <= 4096 CHK); K % 64 == 0.
// KC: K as a compile-time constant (0: K at run time); the 7B decode row
// length K = 4096 is instantiated so that the chunk bounds fold away.
template <int CHK, bool CH, int KC = 0>
__global__ __launch_bounds__(kRowWaves * kWave) void gemv_row_kernel(
    const int8_t* __restrict__ Xq, const float* __restrict__ scale_x, const uint8_t* __restrict__ Wp,
    const float* __restrict__ gamma_p, int N, int K_, float* __restrict__ Y, int32_t* __restrict__ acc_out) {
    const int K = KC ? KC : K_;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int row0 = (blockIdx.x * kRowWaves + wave) * kRowRows;
    if (row0 >= N) return;  // uniform in the wave
    const int KB = K / 4, nch = K / 64;
    // the row factor first (its latency hides under the loads)
    const float rs = CH ? 1.0f / scale_x[0] : *gamma_p / scale_x[0];
    // the weight rows first
    const __amdgpu_buffer_rsrc_t rw = make_buf(Wp + (int64_t)row0 * KB);
    uint4 w[kRowRows][CHK];
#pragma unroll
    for (int r = 0; r < kRowRows; ++r)
#pragma unroll
        for (int c = 0; c < CHK; ++c) {
            const int ch = lane + kWave * c;
            w[r][c] = buf_load16(rw, row0 + r < N && ch < nch ? (uint32_t)(r * KB + 16 * ch) : kBufOOB);
        }
    // the token's chunks after them (in flight together; the products start
    // once all have arrived: measured at 1 x 11008 x 4096, 4.68 us against
    // 4.75 us with the token's chunks requested first)
    const __amdgpu_buffer_rsrc_t rx = make_buf(Xq);
    uint4 xr[CHK][4];
#pragma unroll
    for (int c = 0; c < CHK; ++c) {
        const int ch = lane + kWave * c;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            xr[c][q] = buf_load16(rx, ch < nch ? (uint32_t)(64 * ch + 16 * q) : kBufOOB);
    }
    uint32_t xa[CHK][16];
#pragma unroll
    for (int c = 0; c < CHK; ++c)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t a[4] = {xr[c][q].x, xr[c][q].y, xr[c][q].z, xr[c][q].w};
            uint32_t o[4];
            transpose4x4_bytes(a, o);
#pragma unroll
            for (int i = 0; i < 4; ++i) xa[c][4 * q + i] = o[i];
        }
    int acc[kRowRows];
#pragma unroll
    for (int r = 0; r < kRowRows; ++r) {
        acc[r] = 0;
#pragma unroll
        for (int c = 0; c < CHK; ++c) {
            const uint32_t wd[4] = {w[r][c].x, w[r][c].y, w[r][c].z, w[r][c].w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                uint32_t b[4];
                unpack16(wd[q], b);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[r] = __builtin_amdgcn_sdot4((int)xa[c][4 * q + i], (int)b[i], acc[r], false);
            }
        }
    }
#pragma unroll
    for (int r = 0; r < kRowRows; ++r) acc[r] = wave_sum_i32(acc[r]);
    if (lane < kRowRows) {
        int sum = acc[0];
#pragma unroll
        for (int r = 1; r < kRowRows; ++r) sum = lane == r ? acc[r] : sum;
        const int n = row0 + lane;
        if (n < N) {
            if constexpr (CH) Y[n] = ((float)sum * rs) * gamma_p[n];
            else Y[n] = (float)sum * rs;
            if (acc_out) acc_out[n] = sum;
        }
    }
}

// One token from the unquantized activations (the fused decode forward at
// M = 1): act_quant's arithmetic on the row, then gemv_row_kernel's products.  The
// kRowDecWaves waves of a workgroup share the row: wave w reduces act_quant
// blocks w, w + kRowDecWaves, ... (one 16-byte chunk per lane each), the
// block partials meet in LDS, every wave forms the same 1/RMS and scale from
// them in block order, quantizes its blocks into an LDS copy of q, and after
// a barrier each lane reads its 64-column chunk.  The row is requested first
// and waited for alone; the weight loads follow and stream in while the row
// is quantized.
constexpr int kRowDecWaves = 8;
constexpr int kRowDecMaxK = 64 * 64;  // one chunk per lane

template <typename TX>
__global__ __launch_bounds__(kRowDecWaves * kWave) void gemv_row_decode_kernel(
    const TX* __restrict__ X, const uint8_t* __restrict__ Wp, const float* __restrict__ gamma_p, int N, int K,
    float eps, float* __restrict__ Y, int8_t* __restrict__ xq_out, float* __restrict__ sx_out) {
    constexpr int E = Vec16<TX>::E;         // elements per 16-byte chunk
    constexpr int BLK = kWave * E;          // an act_quant block
    constexpr int NBX = kRowDecMaxK / BLK;  // blocks of the longest row (power of two)
    constexpr int IT = (NBX + kRowDecWaves - 1) / kRowDecWaves;  // blocks per wave
    __shared__ float blk_sq[NBX], blk_max[NBX];
    __shared__ __align__(16) uint8_t qrow[kRowDecMaxK];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int row0 = (blockIdx.x * kRowDecWaves + wave) * kRowRows;  // may pass N: such waves still quantize
    const int KB = K / 4, nch = K / 64;
    const int nblk = (K + BLK - 1) / BLK;
    // 1) the row: block b = wave + kRowDecWaves j, this lane's E elements
    //    (K % 64 == 0: all of them inside the row or all past it)
    const __amdgpu_buffer_rsrc_t rx = make_buf(X);
    uint4 xc[IT];
#pragma unroll
    for (int j = 0; j < IT; ++j) {
        const int b = wave + kRowDecWaves * j;
        const int k0 = b * BLK + lane * E;
        xc[j] = buf_load16(rx, b < nblk && k0 < K ? (uint32_t)(k0 * (int)sizeof(TX)) : kBufOOB);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __builtin_amdgcn_sched_barrier(0);
    // 2) this wave's weight rows, all in flight
    const __amdgpu_buffer_rsrc_t rw = make_buf(Wp + (int64_t)(row0 < N ? row0 : 0) * KB);
    uint4 w[kRowRows];
#pragma unroll
    for (int r = 0; r < kRowRows; ++r)
        w[r] = buf_load16(rw, row0 + r < N && lane < nch ? (uint32_t)(r * KB + 16 * lane) : kBufOOB);
    // 3) block partials: in-lane tree and lane tree of the squares, max |x|
#pragma unroll
    for (int j = 0; j < IT; ++j) {
        const int b = wave + kRowDecWaves * j;
        if (b < nblk) {
            float v[E], sq[E], amax = 0.0f;
            widen16<TX>(xc[j], v);
#pragma unroll
            for (int e = 0; e < E; ++e) {
                sq[e] = v[e] * v[e];
                amax = fmaxf(amax, fabsf(v[e]));
            }
            const float bsum = wave_tree_sum(lane_tree<E>(sq));
            amax = wave_max(amax);
            if (lane == 0) {
                blk_sq[b] = bsum;
                blk_max[b] = amax;
            }
        }
    }
    __syncthreads();
    // 4) 1/RMS and the scale from the partials in block order (missing
    //    blocks add +0, which leaves the tree's value unchanged)
    float bs[NBX], amax = 0.0f;
#pragma unroll
    for (int b = 0; b < NBX; ++b) {
        bs[b] = b < nblk ? blk_sq[b] : 0.0f;
        amax = fmaxf(amax, b < nblk ? blk_max[b] : 0.0f);
    }
    const float ss = lane_tree<NBX>(bs);
    const float ms = ss / (float)K;
    const float d = sqrtf(ms + eps);
    const float inv = 1.0f / d;
    const float a = amax * inv;  // max|x * inv| == max|x| * inv
    const float scale = 127.0f / fmaxf(a, 1e-5f);
    if (sx_out && blockIdx.x == 0 && threadIdx.x == 0) sx_out[0] = scale;
    // 5) this wave's blocks of q into the row copy
#pragma unroll
    for (int j = 0; j < IT; ++j) {
        const int b = wave + kRowDecWaves * j;
        if (b < nblk) {
            float v[E];
            widen16<TX>(xc[j], v);
            uint32_t pk[E / 4];
#pragma unroll
            for (int i = 0; i < E / 4; ++i) {
                uint32_t u = 0;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float r = rintf((v[4 * i + e] * inv) * scale);
                    r = fminf(fmaxf(r, -128.0f), 127.0f);
                    u |= (uint32_t)(uint8_t)(int8_t)(int)r << (8 * e);
                }
                pk[i] = u;
            }
            const int k0 = b * BLK + lane * E;
            if constexpr (E == 8) *reinterpret_cast<uint2*>(qrow + k0) = make_uint2(pk[0], pk[1]);
            else *reinterpret_cast<uint32_t*>(qrow + k0) = pk[0];
            if (xq_out && blockIdx.x == 0 && k0 < K) {
                if constexpr (E == 8) *reinterpret_cast<uint2*>(xq_out + k0) = make_uint2(pk[0], pk[1]);
                else *reinterpret_cast<uint32_t*>(xq_out + k0) = pk[0];
            }
        }
    }
    __syncthreads();
    // 6) the lane's 64 columns of q, byte-transposed for unpack16's order
    uint32_t xa[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (lane < nch) v = *reinterpret_cast<const uint4*>(qrow + 64 * lane + 16 * q);
        const uint32_t a4[4] = {v.x, v.y, v.z, v.w};
        uint32_t o[4];
        transpose4x4_bytes(a4, o);
#pragma unroll
        for (int i = 0; i < 4; ++i) xa[4 * q + i] = o[i];
    }
    // 7) gemv_row_kernel's products, lane sums and epilogue
    int acc[kRowRows];
#pragma unroll
    for (int r = 0; r < kRowRows; ++r) {
        acc[r] = 0;
        const uint32_t wd[4] = {w[r].x, w[r].y, w[r].z, w[r].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint32_t b[4];
            unpack16(wd[q], b);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[r] = __builtin_amdgcn_sdot4((int)xa[4 * q + i], (int)b[i], acc[r], false);
        }
    }
#pragma unroll
    for (int r = 0; r < kRowRows; ++r) acc[r] = wave_sum_i32(acc[r]);
    if (lane < kRowRows) {
        int sum = acc[0];
#pragma unroll
        for (int r = 1; r < kRowRows; ++r) sum = lane == r ? acc[r] : sum;
        const int n = row0 + lane;
        if (n < N) {
            const float rs = *gamma_p / scale;
            Y[n] = (float)sum * rs;
        }
    }
}

bool gemv_supported(int64_t M, int64_t K) { return M <= kGemvMaxM && K <= 16 * 64 * 16; }

hipError_t launch_gemv_t2(const int8_t* Xq, const float* scale_x, const uint8_t* Wp,
                          const float* gamma, int64_t M, int64_t N, int64_t K, float* Y,
                          int32_t* acc, hipStream_t s, bool channel) {
    if (!gemv_supported(M, K)) return hipErrorInvalidValue;
    if (M == 1 && K % 64 == 0 && K <= 2 * 64 * 64) {  // one token: the row GEMV
        const unsigned rgrid = (unsigned)((N + kRowRows * kRowWaves - 1) / (kRowRows * kRowWaves));
        constexpr unsigned kRowThreads = kRowWaves * kWave;
        if (K == 64 * 64) {
            if (channel) gemv_row_kernel<1, true, 4096><<<rgrid, kRowThreads, 0, s>>>(Xq, scale_x, Wp, gamma, (int)N, (int)K, Y, acc);
            else gemv_row_kernel<1, false, 4096><<<rgrid, kRowThreads, 0, s>>>(Xq, scale_x, Wp, gamma, (int)N, (int)K, Y, acc);
        } else if (K <= 64 * 64) {
            if (channel) gemv_row_kernel<1, true><<<rgrid, kRowThreads, 0, s>>>(Xq, scale_x, Wp, gamma, (int)N, (int)K, Y, acc);
            else gemv_row_kernel<1, false><<<rgrid, kRowThreads, 0, s>>>(Xq, scale_x, Wp, gamma, (int)N, (int)K, Y, acc);
        } else {
            if (channel) gemv_row_kernel<2, true><<<rgrid, kRowThreads, 0, s>>>(Xq, scale_x, Wp, gamma, (int)N, (int)K, Y, acc);
            else gemv_row_kernel<2, false><<<rgrid, kRowThreads, 0, s>>>(Xq, scale_x, Wp, gamma, (int)N, (int)K, Y, acc);
        }
        return hipGetLastError();
    }
    const int64_t ngroups = (N + 15) / 16;
    const unsigned grid = (unsigned)std::min<int64_t>(ngroups, 256);
    const int64_t steps = (K + 16 * 64 - 1) / (16 * 64);  // MFMA steps per wave
    const bool full = K % (16 * 64) == 0;
    if (full && (steps == 1 || steps == 2 || steps == 4)) {  // K = 1024, 2048, 4096: the staged kernel
#define BITNET_STAGED(S_)                                                                                  \
        if (steps == S_) {                                                                                 \
            if (channel && M > 4)                                                                          \
                gemv_staged_kernel<S_, true, true><<<grid, kThreads, 0, s>>>(Xq, scale_x, Wp, gamma, (int)M, (int)N, Y, acc); \
            else if (channel)                                                                              \
                gemv_staged_kernel<S_, true, false><<<grid, kThreads, 0, s>>>(Xq, scale_x, Wp, gamma, (int)M, (int)N, Y, acc); \
            else if (M > 4)                                                                                \
                gemv_staged_kernel<S_, false, true><<<grid, kThreads, 0, s>>>(Xq, scale_x, Wp, gamma, (int)M, (int)N, Y, acc); \
            else                                                                                           \
                gemv_staged_kernel<S_, false, false><<<grid, kThreads, 0, s>>>(Xq, scale_x, Wp, gamma, (int)M, (int)N, Y, acc); \
            return hipGetLastError();                                                                      \
        }
        BITNET_STAGED(1)
        BITNET_STAGED(2)
        BITNET_STAGED(4)
#undef BITNET_STAGED
    }
    // measured at N = 11008, K = 4096: the LDS tile (written before the
    // weight loads) beats direct per-lane loads at every token count
    const bool stage = K <= kStageMaxK;
#define BITNET_GEMV_LAUNCH(S_, F_, G_)                                                          \
    do {                                                                                       \
        if (channel)                                                                           \
            gemv_t2_kernel<S_, F_, G_, true><<<grid, kThreads, 0, s>>>(Xq, scale_x, Wp, gamma, (int)M, \
                                                                     (int)N, (int)K, Y, acc, 0.0f, \
                                                                     nullptr, nullptr);         \
        else                                                                                   \
            gemv_t2_kernel<S_, F_, G_, false><<<grid, kThreads, 0, s>>>(Xq, scale_x, Wp, gamma, (int)M, \
                                                                      (int)N, (int)K, Y, acc, 0.0f, \
                                                                      nullptr, nullptr);         \
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

namespace {

template <typename TX, int IT>
hipError_t decode_launch(const TX* X, const uint8_t* Wp, const float* gamma, int64_t M, int64_t N,
                         int64_t K, float eps, float* Y, int8_t* xq_out, float* sx_out, hipStream_t s,
                         bool decode_layout) {
    const int64_t ngroups = (N + 15) / 16;
    const unsigned grid = (unsigned)std::min<int64_t>(ngroups, 256);
    const int64_t steps = (K + 16 * 64 - 1) / (16 * 64);
    const bool full = K % (16 * 64) == 0;
    if (decode_layout) {
        if (!decode_layout_supported(K)) return hipErrorInvalidValue;
        gemv_t2_kernel<4, true, false, false, TX, IT, true><<<grid, kThreads, 0, s>>>(
            X, nullptr, Wp, gamma, (int)M, (int)N, (int)K, Y, nullptr, eps, xq_out, sx_out);
        return hipGetLastError();
    }
#define BITNET_DECODE_CASE(S_)                                                                  \
    if (steps <= S_) {                                                                          \
        if (full && steps == S_)                                                                \
            gemv_t2_kernel<S_, true, false, false, TX, IT><<<grid, kThreads, 0, s>>>(           \
                X, nullptr, Wp, gamma, (int)M, (int)N, (int)K, Y, nullptr, eps, xq_out, sx_out); \
        else                                                                                    \
            gemv_t2_kernel<S_, false, false, false, TX, IT><<<grid, kThreads, 0, s>>>(          \
                X, nullptr, Wp, gamma, (int)M, (int)N, (int)K, Y, nullptr, eps, xq_out, sx_out); \
        return hipGetLastError();                                                               \
    }
    BITNET_DECODE_CASE(1)
    BITNET_DECODE_CASE(2)
    BITNET_DECODE_CASE(4)
#undef BITNET_DECODE_CASE
    return hipErrorInvalidValue;
}

template <typename TX>
hipError_t decode_dispatch(const TX* X, const uint8_t* Wp, const float* gamma, int64_t M, int64_t N,
                           int64_t K, float eps, float* Y, int8_t* xq_out, float* sx_out, hipStream_t s,
                           bool dl) {
    // work items (token row, block) per wave
    constexpr int64_t blk = kWave * Vec16<TX>::E;
    const int64_t per_wave = (M * ((K + blk - 1) / blk) + kWaves - 1) / kWaves;
    if (per_wave <= 1) return decode_launch<TX, 1>(X, Wp, gamma, M, N, K, eps, Y, xq_out, sx_out, s, dl);
    if (per_wave <= 2) return decode_launch<TX, 2>(X, Wp, gamma, M, N, K, eps, Y, xq_out, sx_out, s, dl);
    if (per_wave <= 4) return decode_launch<TX, 4>(X, Wp, gamma, M, N, K, eps, Y, xq_out, sx_out, s, dl);
    if (per_wave <= 8) return decode_launch<TX, 8>(X, Wp, gamma, M, N, K, eps, Y, xq_out, sx_out, s, dl);
    return hipErrorInvalidValue;
}

}  // namespace

bool gemv_decode_fits(bool x_bf16, int64_t M, int64_t K) {
    const int64_t blk = kWave * (x_bf16 ? 8 : 4);
    return M >= 1 && M <= kGemvMaxM && K >= 1 && K <= kStageMaxK &&
           M * ((K + blk - 1) / blk) <= kDecodeMaxItems * kWaves;
}

hipError_t launch_gemv_decode(const void* X, bool x_bf16, const uint8_t* Wp, const float* gamma,
                              int64_t M, int64_t N, int64_t K, float eps, float* Y, int8_t* xq_out,
                              float* sx_out, hipStream_t s, bool decode_layout) {
    if (!gemv_decode_fits(x_bf16, M, K) || K % 16 != 0) return hipErrorInvalidValue;
    if (M == 1 && !decode_layout && K % 64 == 0 && K <= kRowDecMaxK) {  // one token: the row GEMV
        const unsigned grid = (unsigned)((N + kRowRows * kRowDecWaves - 1) / (kRowRows * kRowDecWaves));
        constexpr unsigned kThreadsDec = kRowDecWaves * kWave;
        if (x_bf16)
            gemv_row_decode_kernel<uint16_t><<<grid, kThreadsDec, 0, s>>>(
                static_cast<const uint16_t*>(X), Wp, gamma, (int)N, (int)K, eps, Y, xq_out, sx_out);
        else
            gemv_row_decode_kernel<float><<<grid, kThreadsDec, 0, s>>>(
                static_cast<const float*>(X), Wp, gamma, (int)N, (int)K, eps, Y, xq_out, sx_out);
        return hipGetLastError();
    }
    if (x_bf16)
        return decode_dispatch(static_cast<const uint16_t*>(X), Wp, gamma, M, N, K, eps, Y, xq_out, sx_out, s,
                               decode_layout);
    return decode_dispatch(static_cast<const float*>(X), Wp, gamma, M, N, K, eps, Y, xq_out, sx_out, s,
                           decode_layout);
}

// ------------------------------------------------------- the decode layout
// K = 1024 S: wave v of the GEMV loads row group grp (rows 16 grp .. +15) with
// S/4 instructions of 16 bytes per lane; lane l = 16 g + c takes row
// 16 grp + c, packed bytes 16 S v + 4 S g + 16 i in instruction i.  The
// decode layout stores exactly those pieces in that order: the 1 KB block of
// (grp, v, i) at ((grp * 16 + v) * S/4 + i) * 1024, lane l's piece at + 16 l,
// the rows past N as zeros.  A row-major W gives every instruction sixteen
// 64-byte pieces of sixteen rows; here it reads one contiguous kilobyte.
// Defined for the shape the fused decode call takes: K = 4096 (S = 4).
bool decode_layout_supported(int64_t K) { return K == 4096; }
int64_t decode_layout_bytes(int64_t N, int64_t K) { return (N + 15) / 16 * 16 * (K / 4); }

__global__ __launch_bounds__(256) void pack_decode_kernel(const uint8_t* __restrict__ Wp, int64_t N, int64_t K,
                                                          uint8_t* __restrict__ Wd) {
    const int64_t S = K / 1024, S4 = S / 4, KB = K / 4;
    const int64_t pieces = (N + 15) / 16 * 16 * KB / 16;  // 16-byte pieces of Wd
    for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < pieces;
         c += (int64_t)gridDim.x * blockDim.x) {
        const int l = (int)(c & 63);
        const int64_t rest = c >> 6;  // (grp * 16 + v) * S4 + i
        const int64_t i = rest % S4, v = (rest / S4) % kWaves, grp = rest / S4 / kWaves;
        const int64_t row = grp * 16 + (l & 15);
        const int64_t byte = 16 * S * v + 4 * S * (l >> 4) + 16 * i;
        uint4 val = make_uint4(0, 0, 0, 0);
        if (row < N) val = *reinterpret_cast<const uint4*>(Wp + row * KB + byte);
        reinterpret_cast<uint4*>(Wd)[c] = val;
    }
}

hipError_t launch_pack_decode(const uint8_t* Wp, int64_t N, int64_t K, uint8_t* Wd, hipStream_t s) {
    if (!decode_layout_supported(K) || N < 1) return hipErrorInvalidValue;
    const int64_t pieces = decode_layout_bytes(N, K) / 16;
    const unsigned grid = (unsigned)std::min<int64_t>((pieces + 255) / 256, 8192);
    pack_decode_kernel<<<grid, 256, 0, s>>>(Wp, N, K, Wd);
    return hipGetLastError();
}

}  // namespace bitnet
