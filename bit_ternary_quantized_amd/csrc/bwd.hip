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
// rounded to bf16 once (Xq times 1/scale_x).
//
// One kernel template serves both products.  Output tile BM x BN per
// 512-thread workgroup, BK of the contraction per step.  Two wave groups
// (waves 0-3: tile rows 0 .. BM/2-1, waves 4-7: the rest) put one wave on
// each SIMD and run the same loop one barrier apart (ping-pong): while one
// wave per SIMD issues its MFMAs, the other does its memory phase (operand
// reads, LDS writes of the next tile, global loads two steps ahead).
//
// Operands.  A matrix-core operand wants 8 contraction values per lane.
//   grad_x: A = gy rows as they are ("rows" tile, 16-byte reads); B = the
//     codes, unpacked from 2 bits to bf16 +-1/0 in their natural [n][k]
//     order ("cols" tile).
//   grad_W: A = gy [m][n] and B = X_deq [m][k], both "cols" tiles.
// A "cols" tile has the contraction index as its row; gfx950's transposing
// read ds_read_b64_tr_b16 turns four rows x four columns per lane group into
// the operand layout, so every LDS write is a 16-byte store of loaded (or
// converted) data.  The A tile is private to its group; the B tile is shared:
// each group fills half of it.  The ping-pong barrier order makes that safe:
// a tile written in a group's memory phase of step s is read in memory phases
// s + 1 of both groups, and its buffer is rewritten only at step s + 2.
//
// Small outputs (fewer than 256 large tiles) use 128 x 128 tiles (grad_W with
// the contraction split between the wave groups, see Tile); grad_W then also
// splits its token range over workgroups, and a second kernel adds the fp32
// partial tiles in split order (deterministic).
#include <type_traits>

#include "common.h"

namespace bitnet {

namespace {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

// kGradWT: grad_W with its B operand read from X_deq^T (see xdeq_t_kernel)
enum { kGradX = 0, kGradW = 1, kGradWT = 2 };
constexpr int kThreads = 512;
constexpr int kGroupThreads = 256;

// Tile shapes.  The workgroup's two wave groups either split the output
// rows (each group: BM/2 rows, its four waves side by side along the
// columns; the B tile is shared, each group staging half of it), or, with
// KSPLIT, split the contraction: group g takes every other step, covers the
// whole BM x BN tile with its four waves as 2 x 2, stages its own tiles, and
// the two partial tiles are added once at the end.  The latter gives each
// wave a square 64 x 64 accumulator block, which needs a quarter fewer LDS
// bytes per MFMA than a 64 x 32 one.
template <int BM_, int BN_, int BK_, bool KSPLIT_, int WAVES_M_ = (KSPLIT_ ? 2 : 1)>
struct Tile {
    static constexpr int BM = BM_, BN = BN_, BK = BK_;
    static constexpr bool KSPLIT = KSPLIT_;
    static constexpr int GROWS = KSPLIT ? BM : BM / 2;   // output rows of a group
    static constexpr int GBCOLS = KSPLIT ? BN : BN / 2;  // B columns a group stages
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = 4 / WAVES_M;  // a group's waves
    static constexpr int WTM = GROWS / WAVES_M;          // wave tile rows
    static constexpr int WTN = BN / WAVES_N;             // wave tile columns
    static constexpr int IM = WTM / 32, JN = WTN / 32;
    static constexpr int KQ = BK / 16;  // MFMA k-steps per step
    static constexpr int MFMAS = IM * JN * KQ;
    // "rows" tile: GROWS rows x BK bf16 (2*BK bytes), 16-byte chunks swizzled
    static constexpr int CPR = 2 * BK / 16;
    static constexpr int ROWS_BYTES = GROWS * 2 * BK;
    // staged per thread and step: A chunks (8 elements) and B items (8 columns)
    static constexpr int NA = GROWS * BK / 8 / 256;
    static constexpr int NB = BK * (GBCOLS / 8) / 256;
    // "cols" tile of width W: BK rows, pitch 2W + 64 bytes (64 or 192 mod
    // 256, so the 32 8-byte pieces of each transposing read hit 32 distinct
    // bank pairs)
    static constexpr int pitch(int W) { return 2 * W + 64; }
    static constexpr int cols_bytes(int W) { return BK * pitch(W); }
};
using TileL = Tile<256, 256, 32, false>;
using TileS = Tile<128, 128, 64, false>;   // small outputs, grad_x
using TileSK = Tile<128, 128, 64, true>;  // small outputs, grad_W (measured faster)
// grad_W from X_deq^T: the group's four waves as 2 x 2 (64 x 128 wave tiles),
// so a wave makes 8 transposing reads of its gy operand and 8 plain 16-byte
// reads of X_deq^T per step instead of 16 and 4
using TileLW = Tile<256, 256, 32, false, 2>;

// Chunk c of row r of a "rows" tile: each 256-byte bank window holds 16/CPR
// rows; XOR-ing the chunk index with the window index gives every 16-lane
// group (16 rows, same chunk; or 16/CPR rows, all chunks) distinct banks.
template <class T>
__device__ __forceinline__ int rows_slot(int r, int c) {
    constexpr int RPW = 16 / T::CPR;  // rows per 256-byte window
    return r * (2 * T::BK) + 16 * (c ^ ((r / RPW) % T::CPR));
}

// Transposing read (gfx950 ds_read_b64_tr_b16).  Within each 16-lane group,
// lane j supplies the address of 4 consecutive bf16; output lane 4a+b then
// holds element b of the chunks of lanes a, 4+a, 8+a, 12+a.  So if lane
// j = 4e + a points at contraction row c0+e, columns x0+4a..x0+4a+3, output
// lane i holds column x0+i at rows c0..c0+3.
__device__ __forceinline__ uint2 lds_read_tr16(const uint8_t* tile, int byte_off) {
    const v4s v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4s*)((__attribute__((address_space(3))) const char*)tile + byte_off));
    return __builtin_bit_cast(uint2, v);
}

// Operand (8 contraction values c0 + 8*(lane/32) + 0..7 for output index
// x0 + lane%32) from a "cols" tile: two transposing reads, rows +0..3, +4..7.
template <int PITCH>
__device__ __forceinline__ v8bf cols_operand(const uint8_t* tile, int c0, int x0, int lane) {
    const int G = lane >> 4, j = lane & 15, e = j >> 2, a = j & 3;
    const int row = c0 + 8 * (G >> 1) + e, col = x0 + 16 * (G & 1) + 4 * a;
    const uint2 lo = lds_read_tr16(tile, row * PITCH + 2 * col);
    const uint2 hi = lds_read_tr16(tile, (row + 4) * PITCH + 2 * col);
    return __builtin_bit_cast(v8bf, make_uint4(lo.x, lo.y, hi.x, hi.y));
}

// Operand from a "rows" tile: contraction values 16*kq + 8*(lane/32) + 0..7
// of row x0 + lane%32.
template <class T>
__device__ __forceinline__ v8bf rows_operand(const uint8_t* tile, int kq, int x0, int lane) {
    return *reinterpret_cast<const v8bf*>(tile + rows_slot<T>(x0 + (lane & 31), 2 * kq + (lane >> 5)));
}

// 8 ternary codes (the low 16 bits of w: columns k..k+7) -> 8 bf16 in natural
// column order (4 dwords, two codes each).  bf16 of a code: low byte 0x80 if
// nonzero, high byte 0x3f (+1) or 0xbf (-1).
// kHi / kLo: high / low byte of the bf16 value of code 0, +1, -1 in bytes
// 0, 1, 2 (the defaults give 0, +1.0, -1.0).
__device__ __forceinline__ uint4 codes8_to_bf16(uint32_t w, uint32_t kHi = 0x00bf3f00u,
                                                uint32_t kLo = 0x00808000u) {
    const uint32_t ev = w & 0x33333333u;         // codes 0, 2 of every byte
    const uint32_t od = (w >> 2) & 0x33333333u;  // codes 1, 3 of every byte
    uint32_t r[4];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        // [ev.b, ev.b, od.b, od.b]: codes 4b, 4b+2 (low / high nibble of ev.b), 4b+1, 4b+3
        const uint32_t pb = __builtin_amdgcn_perm(od, ev, (uint32_t)(b | b << 8 | (b + 4) << 16 | (b + 4) << 24));
        const uint32_t s0 = (pb & 0x03030303u) + 0x00040004u;
        const uint32_t s1 = ((pb >> 4) & 0x03030303u) + 0x00040004u;
        r[2 * b] = __builtin_amdgcn_perm(kLo, kHi, s0);
        r[2 * b + 1] = __builtin_amdgcn_perm(kLo, kHi, s1);
    }
    return make_uint4(r[0], r[1], r[2], r[3]);
}

// 8 ternary codes times a per-row scale s: codes -> 0, +bf16(s), -bf16(s)
// (s rounded to bf16 once, to nearest even)
__device__ __forceinline__ uint4 codes8_to_bf16_scaled(uint32_t w, float s) {
    const uint32_t b = __builtin_bit_cast(uint16_t, (__bf16)s);
    const uint32_t hi = b >> 8, lo = b & 0xffu;
    return codes8_to_bf16(w, ((hi ^ 0x80u) << 16) | (hi << 8), (lo << 16) | (lo << 8));
}

// 8 int8 (2 dwords) times rs -> 8 bf16 (4 dwords)
__device__ __forceinline__ uint4 int8x8_to_bf16(uint2 q, float rs) {
    const uint32_t w[2] = {q.x, q.y};
    uint32_t r[4];
#pragma unroll
    for (int d = 0; d < 2; ++d) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            v2bf p;
            p[0] = (__bf16)((float)(int8_t)(w[d] >> (16 * h)) * rs);
            p[1] = (__bf16)((float)(int8_t)(w[d] >> (16 * h + 8)) * rs);
            r[2 * d + h] = __builtin_bit_cast(uint32_t, p);
        }
    }
    return make_uint4(r[0], r[1], r[2], r[3]);
}

// Workgroup id -> (tile row, tile column, split), regrouped so that each XCD
// (ids are dealt round-robin over the 8 XCDs) works on a contiguous run of
// an order in which the split is slowest, and inside a split the tiles come
// in bands of kBandRows tile rows, column by column.  The split slowest: the
// B operand of a token range (its q rows) is read by the one or two XCDs
// holding that split's tiles, not by all eight (grad_W at 1376 x 512 from
// 8192 tokens: 35 MB fetched instead of 59).  The bands: the 32 workgroups
// an XCD runs at once cover 4 tile rows x 8 columns instead of 1 x 32, so
// they share 4 A and 8 B operands instead of 1 and 32 (grad_W at 28672 x
// 8192 from 4096 tokens re-fetched all of X once per tile row; measured:
// grad_x at that shape 1458 -> 1420 us, the others within 1%).
constexpr int kBandRows = 4;
__device__ __forceinline__ void tile_of(int wg, int tiles_m, int tiles_n, int splits, int& tm,
                                        int& tn, int& sp) {
    const int G = tiles_m * tiles_n * splits;
    const int q = G / 8, r = G % 8;
    const int x = wg % 8, local = wg / 8;
    int id = (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + local;
    const int per_split = tiles_m * tiles_n;
    sp = __builtin_amdgcn_readfirstlane(id / per_split);
    id -= sp * per_split;
    const int band = id / (kBandRows * tiles_n);
    const int rows = min(kBandRows, tiles_m - band * kBandRows);  // the last band may be short
    const int in = id - band * kBandRows * tiles_n;
    tn = __builtin_amdgcn_readfirstlane(in / rows);
    tm = __builtin_amdgcn_readfirstlane(band * kBandRows + in % rows);
}

// Staged data of one step (per thread): NA 16-byte A chunks as loaded; NB
// B items (8 output columns of one contraction row each) as loaded (braw: 8
// packed codes, or 8 int8 with their row's scale_x, 0 past the token range)
// and converted to 8 bf16 (bcv) in a compute phase.  Nothing loaded is used
// in the phase that loads it (1/scale_x included), so no wait there.
template <int MODE, int NA, int NB>
struct Stage;
template <int NA, int NB>
struct Stage<kGradX, NA, NB> {
    uint4 a[NA];
    uint32_t braw[NB];
    float sn[NB];  // per-channel scale of the item's row (channel variant only)
    uint4 bcv[NB];
};
template <int NA, int NB>
struct Stage<kGradW, NA, NB> {
    uint4 a[NA];
    uint2 braw[NB];
    float sx[NB];
    uint4 bcv[NB];
};
template <int NA, int NB>
struct Stage<kGradWT, NA, NB> {
    uint4 a[NA];
    uint4 b[NB];  // 8 bf16 of X_deq^T, stored as loaded
};

}  // namespace

// MODE kGradX: out [M][K] (fp32, or bf16 if OUT_BF16) = gamma * gy . codes,
//   rows m, columns k, contraction n.  `second` = packed codes, `aux` = gamma.
// MODE kGradW: out [N][K] fp32 = gy^T . X_deq, rows n, columns k, contraction
//   m over the split's token range; with splits > 1 the tile goes to
//   out + sp*N*K (partials).  `second` = Xq, `aux` = scale_x.
// MODE kGradWT: kGradW with `second` = X_deq^T [K][Mp] bf16 (Mp = M rounded
//   up to 8, zero past M; written by xdeq_t_kernel with the same rounding as
//   kGradW's conversion, so the two modes give the same bits).  Its B tile is
//   a "rows" tile read with plain 16-byte reads: no transposing B reads and no
//   conversion in the loop.  `aux` unused.
// VEC: N % 8 == 0 (gy rows 16-byte aligned, 8-element chunks all in or out);
// otherwise gy is read element by element.  GATED (grad_W, one split only):
// the master-weight range gate `gate` applied as the tile is written.
// CH (grad_x): `aux` holds one scale per output channel n (W_deq[n][k] =
// aux[n] * code), folded into the bf16 codes; else aux is the one gamma.
template <int MODE, class T, bool VEC, bool OUT_BF16, bool GATED = false, bool CH = false>
__global__ __launch_bounds__(kThreads) void bwd_kernel(
    const uint16_t* __restrict__ gy, const void* __restrict__ second, const float* __restrict__ aux,
    int M, int N, int K, int splits, int kper, void* __restrict__ out, SteGate gate) {
    constexpr int BK = T::BK, GROWS = T::GROWS, IM = T::IM, JN = T::JN, KQ = T::KQ;
    constexpr int NA = T::NA, NB = T::NB;
    constexpr bool KS = T::KSPLIT;
    // persistent tile loop (without it the registers the ragged element-wise
    // loads need push the big tile over the register file)
    constexpr bool PERS = !KS && VEC;
    constexpr bool GW = MODE != kGradX;   // a grad_W product
    constexpr bool BT = MODE == kGradWT;  // its B operand from X_deq^T rows
    constexpr int PB = T::pitch(T::BN);  // B tile ("cols")
    constexpr int PA = T::pitch(GROWS);  // grad_W A tile
    constexpr int A_BYTES = MODE == kGradX ? T::ROWS_BYTES : T::cols_bytes(GROWS);
    constexpr int B_BYTES = BT ? T::BN * 2 * BK : T::cols_bytes(T::BN);
    constexpr int CPA = GROWS / 8;       // grad_W: 8-element gy chunks per A row
    constexpr int NBUF_B = KS ? 2 : 1;   // B tiles per buffer: per group, or one shared
    __shared__ __align__(16) uint8_t smem_a[2][2][A_BYTES];       // [group][buffer]
    __shared__ __align__(16) uint8_t smem_b[NBUF_B][2][B_BYTES];  // [group or 0][buffer]

    // grad_W A chunk c -> (token row, 8-column chunk).  Rows of 16 chunks:
    // 16 lanes per row.  Rows of 8 chunks (pitch 192): each 16-lane group
    // takes chunks 0-3 or 4-7 of four consecutive rows, whose 16-byte slots
    // (row offsets 0, 12, 8, 4 slots mod 16) are then all distinct.
    auto a_chunk = [](int c, int& row, int& ch) {
        if constexpr (CPA >= 16) {
            row = c / CPA;
            ch = c % CPA;
        } else {
            static_assert(CPA == 8, "grad_W A rows of 8 or 16 chunks");
            const int q = c >> 4, l = c & 15;
            row = 4 * (q >> 1) + (l >> 2);
            ch = 4 * (q & 1) + (l & 3);
        }
    };
    const int R = GW ? N : M;  // output rows
    const int C = K;           // output columns
    const int KC = GW ? M : N; // contraction length
    // Persistent without a contraction split between the wave groups and
    // with 16-byte rows of the contraction operand: the grid is at most one
    // workgroup per CU and workgroup b takes tiles b, b + grid, ... (tile v
    // on the XCD a one-tile-per-workgroup launch gives it when the grid is a
    // multiple of 8).  Otherwise one tile a workgroup.
    const int nwg = ((R + T::BM - 1) / T::BM) * ((C + T::BN - 1) / T::BN) * splits;
    for (int wgi = blockIdx.x; wgi < nwg; wgi += gridDim.x) {
    int tm, tn, sp;
    tile_of(wgi, (R + T::BM - 1) / T::BM, (C + T::BN - 1) / T::BN, splits, tm, tn, sp);
    const int r0 = tm * T::BM, c0 = tn * T::BN;
    const int klo = sp * kper, khi = min(KC, klo + kper);
    const int nsteps = (khi - klo + BK - 1) / BK;
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wm = wave >> 2, wn = wave & 3;  // wm: the wave group
    const int tg = t & (kGroupThreads - 1);
    const int KB = K / 4;
    const int rg = r0 + (KS ? 0 : wm * GROWS);    // first output row of the group
    const int cb = c0 + (KS ? 0 : wm * T::GBCOLS);  // first column the group stages
    const int wr = (wn / T::WAVES_N) * T::WTM;      // wave tile origin in the group
    const int wc = (wn % T::WAVES_N) * T::WTN;
    // the group's steps: all of them, or (KSPLIT) every other one
    const int nsteps_g = KS ? (nsteps + 1 - wm) / 2 : nsteps;
    auto kstep = [&](int i) { return KS ? 2 * i + wm : i; };
    uint8_t* const smem_bg = &smem_b[KS ? wm : 0][0][0];
    auto bbuf = [&](int i) { return smem_bg + (i & 1) * B_BYTES; };

    // ---- per-thread staging geometry; offsets are relative to the step's
    // base address (which moves by BK along the contraction)
    // A chunks u (c = tg + 256 u): 8 consecutive gy elements.
    //   grad_x: row rg + c / CPR, contraction 8 * (c % CPR) of the step
    //   grad_W: token row of the step, columns rg + 8 * ch (a_chunk)
    uint32_t aoff[NA];
    int a_k[NA];    // contraction index of the chunk's first element (in the step)
    int a_lim[NA];  // grad_W: columns left in the row
    bool a_ok[NA];
#pragma unroll
    for (int u = 0; u < NA; ++u) {
        const int c = tg + u * kGroupThreads;
        if constexpr (MODE == kGradX) {
            const int row = c / T::CPR, ch = c % T::CPR;
            a_k[u] = 8 * ch;
            a_ok[u] = rg + row < R;
            a_lim[u] = 8;
            aoff[u] = (uint32_t)((row * N + 8 * ch) * 2);
        } else {
            int row, ch;
            a_chunk(c, row, ch);
            a_k[u] = row;
            a_lim[u] = R - (rg + 8 * ch);  // columns of this chunk inside the row
            a_ok[u] = a_lim[u] > 0;
            aoff[u] = (uint32_t)((row * N + 8 * ch) * 2);
        }
    }
    // B: NB items per thread, 8 output columns of one contraction row each;
    // consecutive lanes take consecutive 8-column pieces of a row, so every
    // 16-byte LDS store instruction writes contiguous runs (no bank conflict).
    //   grad_x: 8 packed codes (2 bytes) of row bk;  grad_W: 8 int8 of token bk
    constexpr int IPR = T::GBCOLS / 8;            // items per staged row
    constexpr int RPP = kGroupThreads / IPR;      // rows per pass over the group
    static_assert(BK == NB * RPP, "B items cover the step");
    const int bk = tg / IPR, bj = tg % IPR;       // rows bk + h * RPP
    const int bcol = (cb - c0) + 8 * bj;          // first output column in the tile
    const bool b_ok = cb + 8 * bj < C;
    const uint32_t boff = MODE == kGradX ? (uint32_t)(bk * KB + 2 * bj) : (uint32_t)(bk * K + 8 * bj);
    const uint32_t bstep = MODE == kGradX ? (uint32_t)(RPP * KB) : (uint32_t)(RPP * K);
    // BT: B chunks c = tg + 256 h, 8 tokens each: X_deq^T row (output column)
    // c / CPR of the group's staged columns, token chunk c % CPR (the same for
    // every h, since 256 is a multiple of CPR); rows past K read zeros.
    static_assert(!BT || NB * kGroupThreads == T::GBCOLS * T::CPR, "X_deq^T chunks cover the step");
    const int Mp = (M + 7) & ~7;           // X_deq^T row pitch (elements)
    const int btc = tg % T::CPR;           // token chunk of this thread
    const int btrow = tg / T::CPR;         // first staged row, + h * 256 / CPR
    uint32_t btoff[BT ? NB : 1];
#pragma unroll
    for (int h = 0; h < (BT ? NB : 1); ++h) {
        const int row = btrow + h * (kGroupThreads / T::CPR);
        btoff[h] = cb + row < C ? (uint32_t)((row * Mp + 8 * btc) * 2) : kBufOOB;
    }
    (void)Mp;

    auto load_a = [&](int kb, const __amdgpu_buffer_rsrc_t& ra, int u) -> uint4 {
        // kb: contraction base of the step
        if constexpr (VEC) {
            const bool v = a_ok[u] && kb + a_k[u] < khi;
            return buf_load16(ra, v ? aoff[u] : kBufOOB);
        } else {
            uint32_t w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                bool v0, v1;
                if constexpr (MODE == kGradX) {
                    v0 = a_ok[u] && kb + a_k[u] + 2 * e < khi;
                    v1 = a_ok[u] && kb + a_k[u] + 2 * e + 1 < khi;
                } else {
                    v0 = kb + a_k[u] < khi && 2 * e < a_lim[u];
                    v1 = kb + a_k[u] < khi && 2 * e + 1 < a_lim[u];
                }
                const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(ra, v0 ? aoff[u] + 4 * e : kBufOOB, 0, 0);
                const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(ra, v1 ? aoff[u] + 4 * e + 2 : kBufOOB, 0, 0);
                w[e] = (lo & 0xffffu) | (hi << 16);
            }
            return make_uint4(w[0], w[1], w[2], w[3]);
        }
    };
    using StageT = Stage<MODE, NA, NB>;
    // i: the group's step index
    auto load_global = [&](int i, StageT& p) {
        const int kb = klo + kstep(i) * BK;
        if constexpr (MODE == kGradX) {
            const __amdgpu_buffer_rsrc_t ra = make_buf(gy + (int64_t)rg * N + kb);
#pragma unroll
            for (int u = 0; u < NA; ++u) p.a[u] = load_a(kb, ra, u);
            const __amdgpu_buffer_rsrc_t rb =
                make_buf(static_cast<const uint8_t*>(second) + (int64_t)kb * KB + cb / 4);
#pragma unroll
            for (int h = 0; h < NB; ++h) {
                const bool bv = b_ok && kb + bk + h * RPP < khi;
                p.braw[h] = __builtin_amdgcn_raw_buffer_load_b16(rb, bv ? boff + h * bstep : kBufOOB, 0, 0);
            }
            if constexpr (CH) {
                const __amdgpu_buffer_rsrc_t rsn = make_buf(aux + kb);
#pragma unroll
                for (int h = 0; h < NB; ++h) {
                    const bool tv = kb + bk + h * RPP < khi;
                    p.sn[h] = __builtin_bit_cast(float, buf_load4(rsn, tv ? (uint32_t)(4 * (bk + h * RPP)) : kBufOOB));
                }
            }
        } else if constexpr (BT) {
            const __amdgpu_buffer_rsrc_t ra = make_buf(gy + (int64_t)kb * N + rg);
#pragma unroll
            for (int u = 0; u < NA; ++u) p.a[u] = load_a(kb, ra, u);
            const __amdgpu_buffer_rsrc_t rb =
                make_buf(static_cast<const uint16_t*>(second) + (int64_t)cb * Mp + kb);
            const bool tv = kb + 8 * btc < khi;
#pragma unroll
            for (int h = 0; h < NB; ++h) p.b[h] = buf_load16(rb, tv ? btoff[h] : kBufOOB);
        } else {
            const __amdgpu_buffer_rsrc_t ra = make_buf(gy + (int64_t)kb * N + rg);
#pragma unroll
            for (int u = 0; u < NA; ++u) p.a[u] = load_a(kb, ra, u);
            const __amdgpu_buffer_rsrc_t rb =
                make_buf(static_cast<const int8_t*>(second) + (int64_t)kb * K + cb);
            const __amdgpu_buffer_rsrc_t rs = make_buf(aux + kb);
#pragma unroll
            for (int h = 0; h < NB; ++h) {
                const bool tv = kb + bk + h * RPP < khi;
                p.braw[h] = buf_load8(rb, b_ok && tv ? boff + h * bstep : kBufOOB);
                p.sx[h] = __builtin_bit_cast(
                    float, buf_load4(rs, tv ? (uint32_t)(4 * (bk + h * RPP)) : kBufOOB));
            }
        }
    };
    auto convert = [&](StageT& p) {
        if constexpr (!BT) {  // (BT: stored as loaded)
#pragma unroll
            for (int h = 0; h < NB; ++h) {
                if constexpr (MODE == kGradX && CH) p.bcv[h] = codes8_to_bf16_scaled(p.braw[h], p.sn[h]);
                else if constexpr (MODE == kGradX) p.bcv[h] = codes8_to_bf16(p.braw[h]);
                else p.bcv[h] = int8x8_to_bf16(p.braw[h], p.sx[h] > 0.0f ? __builtin_amdgcn_rcpf(p.sx[h]) : 0.0f);
            }
        }
    };
    auto store_lds = [&](int i, const StageT& p) {
        uint8_t* As = smem_a[wm][i & 1];
        uint8_t* Bs = bbuf(i);
#pragma unroll
        for (int u = 0; u < NA; ++u) {
            const int c = tg + u * kGroupThreads;
            if constexpr (MODE == kGradX)
                *reinterpret_cast<uint4*>(As + rows_slot<T>(c / T::CPR, c % T::CPR)) = p.a[u];
            else {
                int row, ch;
                a_chunk(c, row, ch);
                *reinterpret_cast<uint4*>(As + row * PA + 16 * ch) = p.a[u];
            }
        }
        if constexpr (BT) {
#pragma unroll
            for (int h = 0; h < NB; ++h)
                *reinterpret_cast<uint4*>(Bs + rows_slot<T>((cb - c0) + btrow + h * (kGroupThreads / T::CPR), btc)) =
                    p.b[h];
        } else {
#pragma unroll
            for (int h = 0; h < NB; ++h)
                *reinterpret_cast<uint4*>(Bs + (bk + h * RPP) * PB + 2 * bcol) = p.bcv[h];
        }
    };

    v16f acc[IM][JN];
#pragma unroll
    for (int i = 0; i < IM; ++i)
#pragma unroll
        for (int j = 0; j < JN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    v8bf a[KQ][IM], b[KQ][JN];
    auto read_operands = [&](int i) {
        const uint8_t* As = smem_a[wm][i & 1];
        const uint8_t* Bs = bbuf(i);
#pragma unroll
        for (int kq = 0; kq < KQ; ++kq) {
#pragma unroll
            for (int j = 0; j < JN; ++j) {
                if constexpr (BT) b[kq][j] = rows_operand<T>(Bs, kq, wc + j * 32, lane);
                else b[kq][j] = cols_operand<PB>(Bs, 16 * kq, wc + j * 32, lane);
            }
#pragma unroll
            for (int ii = 0; ii < IM; ++ii) {
                if constexpr (MODE == kGradX) a[kq][ii] = rows_operand<T>(As, kq, wr + ii * 32, lane);
                else a[kq][ii] = cols_operand<PA>(As, 16 * kq, wr + ii * 32, lane);
            }
        }
    };
    auto barrier = [] {
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
    };
    // Barrier between the phases of the loop.  With KSPLIT each group stages
    // and reads only its own tiles, and a tile written in a memory phase is
    // read no earlier than the group's next memory phase, two barriers later:
    // the LDS fence is then needed only where a compute phase ends, where each
    // wave first waits for its own LDS operations (lgkmcnt 0), long complete
    // by then; the barrier that ends a memory phase does not wait for its LDS
    // writes.  Without KSPLIT the groups read each other's B columns one
    // barrier after they are written, so every barrier keeps the fence.
    auto phase_barrier = [&](bool drain_lds) {
        if constexpr (KS) {
            __builtin_amdgcn_sched_barrier(0);
            if (drain_lds) __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
        } else {
            barrier();
        }
    };

    // One step of the group (its i-th): memory phase = operands of step i,
    // step i + 1 (loaded two steps ago, converted since) into LDS, loads of
    // step i + 3 into the freed staging set; compute phase = the MFMAs, with
    // the conversion of the other staging set (stored next step) between
    // them.  The memory phase runs at raised wave priority: it sets the step
    // time while the other group's MFMAs run.  Past the group's last step the
    // loads read zeros, which add nothing.
    auto step = [&](int i, StageT& cur, StageT& nx) {
        __builtin_amdgcn_s_setprio(1);
        read_operands(i);
        store_lds(i + 1, cur);
        load_global(i + 3, cur);
        __builtin_amdgcn_s_setprio(0);
        phase_barrier(false);
#pragma unroll
        for (int kq = 0; kq < KQ; ++kq)
#pragma unroll
            for (int ii = 0; ii < IM; ++ii)
#pragma unroll
                for (int j = 0; j < JN; ++j)
                    acc[ii][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kq][ii], b[kq][j], acc[ii][j], 0, 0, 0);
        convert(nx);
        phase_barrier(true);
    };

    // Prologue: the group's step 0 in LDS buffer 0, steps 1 and 2 loading.
    // Group 1 then waits one extra barrier, which puts it a phase behind
    // group 0.  Both groups run the same number of loop steps (a group with
    // fewer real steps runs zero tiles), so every wave passes the same number
    // of barriers.
    StageT s0, s1;
    {
        StageT p0;
        load_global(0, p0);
        convert(p0);
        store_lds(0, p0);
    }
    load_global(1, s1);
    load_global(2, s0);
    convert(s1);
    barrier();
    if (wm == 1) barrier();
    const int nloop = KS ? (nsteps + 1) / 2 : nsteps;  // the larger group's step count
    (void)nsteps_g;
    for (int i = 0; i < nloop; i += 2) {
        step(i, s1, s0);
        step(i + 1, s0, s1);
    }
    if (wm == 0) barrier();

    // ---- KSPLIT: group 1 hands its partial tile to group 0 through LDS
    // (the A buffers, no longer read), lane-contiguous so the accesses are
    // conflict-free; group 0 adds (fixed order: own + other).
    const int g = lane >> 5, l32 = lane & 31;
    if constexpr (KS) {
        static_assert(IM * JN * 16 * 64 * 4 * 4 <= sizeof(smem_a), "partial tiles fit the A buffers");
        float* xfer = reinterpret_cast<float*>(&smem_a[0][0][0]);
        float* mine = xfer + wn * (IM * JN * 16 * 64);
        if (wm == 1) {
#pragma unroll
            for (int ii = 0; ii < IM; ++ii)
#pragma unroll
                for (int j = 0; j < JN; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mine[((ii * JN + j) * 16 + r) * 64 + lane] = acc[ii][j][r];
        }
        barrier();
        if (wm == 1) return;  // uniform per wave; no barrier follows
#pragma unroll
        for (int ii = 0; ii < IM; ++ii)
#pragma unroll
            for (int j = 0; j < JN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[ii][j][r] += mine[((ii * JN + j) * 16 + r) * 64 + lane];
    }

    // ---- epilogue: 32x32 block layout, lane holds column l32 and rows
    // 8*(r/4) + 4*g + r%4
    const float scale = MODE == kGradX && !CH ? *aux : 1.0f;
    float* outf = static_cast<float*>(out);
    // this lane's row and column offsets inside the tile, opaque per tile so
    // that the stores' offsets built from them are not hoisted out of the
    // tile loop (they would stay live across it)
    int lrow = wr + 4 * g, lcol = wc + l32;
    if constexpr (PERS) asm volatile("" : "+v"(lrow), "+v"(lcol));
    if constexpr (GW) outf += (int64_t)sp * N * K;
#pragma unroll
    for (int ii = 0; ii < IM; ++ii) {
        // gated: the master weights of this 32-row block first (clamped
        // indices, so every load is unconditional and they all fly together)
        float wv[GATED ? 16 : 1][GATED ? JN : 1];
        if constexpr (GATED) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = min(rg + lrow + ii * 32 + 8 * (r >> 2) + (r & 3), R - 1);
#pragma unroll
                for (int j = 0; j < JN; ++j) {
                    const int64_t idx = (int64_t)row * C + min(c0 + lcol + j * 32, C - 1);
                    wv[r][j] = gate.bf16 ? bf16_bits_to_f32(static_cast<const uint16_t*>(gate.w)[idx])
                                         : static_cast<const float*>(gate.w)[idx];
                }
            }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = rg + lrow + ii * 32 + 8 * (r >> 2) + (r & 3);
            if (row < R) {
#pragma unroll
                for (int j = 0; j < JN; ++j) {
                    const int col = c0 + lcol + j * 32;
                    if (col < C) {
                        const int64_t idx = (int64_t)row * C + col;
                        float v = acc[ii][j][r] * scale;
                        if constexpr (GATED) v = (gate.lo <= wv[r][j] && wv[r][j] <= gate.hi) ? v : 0.0f;
                        // streaming (non-temporal) stores: the output is not read again here
                        if constexpr (MODE == kGradX && OUT_BF16)
                            __builtin_nontemporal_store((__bf16)v, &static_cast<__bf16*>(out)[idx]);
                        else
                            __builtin_nontemporal_store(v, &outf[idx]);
                    }
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (!PERS) break;  // one tile a workgroup: no back edge
    __syncthreads();  // the next tile rewrites the LDS tiles
    }
}

// out[i] = sum over s = 0..splits-1 of part[s][i], in that order (then the
// master-weight range gate when gate.w is set).
__global__ __launch_bounds__(256) void split_reduce_kernel(const float* __restrict__ part,
                                                           int splits, int64_t count,
                                                           float* __restrict__ out, SteGate gate) {
    const int64_t i4 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i4 >= count) return;
    auto gated = [&](int64_t i, float v) {
        if (gate.w == nullptr) return v;
        const float w = gate.bf16 ? bf16_bits_to_f32(static_cast<const uint16_t*>(gate.w)[i])
                                  : static_cast<const float*>(gate.w)[i];
        return (gate.lo <= w && w <= gate.hi) ? v : 0.0f;
    };
    if (i4 + 4 <= count && (count % 4) == 0) {
        // the partials of up to kReduceBatch splits are requested together,
        // then added in split order (a load per split, each waited for before
        // the next is issued, costs a memory round trip per split); past the
        // last split the index is clamped, the load repeated and its value
        // not added (a select, not a branch, so the waits stay graded)
        constexpr int kReduceBatch = 8;
        auto load_batch = [&](int p0, float4 (&v)[kReduceBatch]) {
#pragma unroll
            for (int j = 0; j < kReduceBatch; ++j) {
                const int p = min(p0 + j, splits - 1);
                v[j] = reinterpret_cast<const float4*>(part + (int64_t)p * count + i4)[0];
            }
        };
        auto add_batch = [&](int p0, int j0, const float4 (&v)[kReduceBatch], float4& s) {
#pragma unroll
            for (int j = j0; j < kReduceBatch; ++j) {
                const bool use = p0 + j < splits;
                s.x = use ? s.x + v[j].x : s.x;
                s.y = use ? s.y + v[j].y : s.y;
                s.z = use ? s.z + v[j].z : s.z;
                s.w = use ? s.w + v[j].w : s.w;
            }
        };
        float4 v[kReduceBatch];
        load_batch(0, v);
        float4 s = v[0];
        add_batch(0, 1, v, s);
        for (int p0 = kReduceBatch; p0 < splits; p0 += kReduceBatch) {
            load_batch(p0, v);
            add_batch(p0, 0, v, s);
        }
        s.x = gated(i4, s.x);
        s.y = gated(i4 + 1, s.y);
        s.z = gated(i4 + 2, s.z);
        s.w = gated(i4 + 3, s.w);
        reinterpret_cast<float4*>(out + i4)[0] = s;
    } else {
        for (int64_t i = i4; i < i4 + 4 && i < count; ++i) {
            float s = part[i];
            for (int p = 1; p < splits; ++p) s += part[(int64_t)p * count + i];
            out[i] = gated(i, s);
        }
    }
}

// X_deq^T for the grad_W product: XdT[k][m] = bf16(Xq[m][k] * (1/scale_x[m]))
// (the reciprocal and the rounding of int8x8_to_bf16, so kGradWT sees the
// very operand values kGradW converts in its loop), for m < Mp = M rounded up
// to 8, zero for m >= M.  A 64-token x 64-column tile per 256-thread
// workgroup, transposed through LDS: each thread loads 16 int8 of a token row
// (four threads cover 64 contiguous bytes of the row) and writes 16 bf16
// values down a column of the LDS tile; then each thread stores 16 bf16 of an
// X_deq^T row (four threads cover 128 contiguous bytes).  The LDS pitch of 66
// elements (33 dwords) puts the four column groups of a wave's 2-byte writes
// on different banks.
constexpr int kXtTile = 64, kXtPitch = kXtTile + 2;
__global__ __launch_bounds__(256) void xdeq_t_kernel(const int8_t* __restrict__ Xq,
                                                     const float* __restrict__ scale_x, int M, int K,
                                                     int Mp, int tiles_m, uint16_t* __restrict__ XdT) {
    __shared__ uint16_t tile[kXtTile * kXtPitch];
    const int t = threadIdx.x;
    const int tm = blockIdx.x % tiles_m, tk = blockIdx.x / tiles_m;
    const int m0 = tm * kXtTile, k0 = tk * kXtTile;
    {
        const int ml = t >> 2, kl = (t & 3) * 16;
        const int m = m0 + ml, k = k0 + kl;
        uint4 q = make_uint4(0, 0, 0, 0);
        float rs = 0.0f;
        if (m < M && k < K) {  // K % 16 == 0: a 16-column chunk is all in or all out
            q = *reinterpret_cast<const uint4*>(Xq + (int64_t)m * K + k);
            const float sx = scale_x[m];
            rs = sx > 0.0f ? __builtin_amdgcn_rcpf(sx) : 0.0f;
        }
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float v = (float)(int8_t)(w[i >> 2] >> (8 * (i & 3))) * rs;
            tile[(kl + i) * kXtPitch + ml] = __builtin_bit_cast(uint16_t, (__bf16)v);
        }
    }
    __syncthreads();
    const int kl = t >> 2, ml = (t & 3) * 16;
    const int k = k0 + kl, m = m0 + ml;
    if (k >= K) return;
    const uint32_t* src = reinterpret_cast<const uint32_t*>(tile + kl * kXtPitch + ml);  // dword aligned
    uint16_t* dst = XdT + (int64_t)k * Mp + m;
#pragma unroll
    for (int h = 0; h < 2; ++h)  // two 8-element halves; Mp % 8 == 0
        if (m + 8 * h < Mp)
            *reinterpret_cast<uint4*>(dst + 8 * h) =
                make_uint4(src[4 * h], src[4 * h + 1], src[4 * h + 2], src[4 * h + 3]);
}

// ------------------------------------------------------------------ plans
namespace {

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct Plan {
    bool big;       // TileL, else TileS
    int splits;     // contraction splits (grad_W only)
    int kper;       // contraction per split (multiple of the step)
    int64_t tiles;  // output tiles
};

// Large tiles when they give at least one workgroup per CU, else small tiles;
// grad_W (allow_split) then splits its token range so that the grid fills
// the 256 CUs in one wave of workgroups (one workgroup fits per CU), each
// split keeping at least 8 steps.
Plan plan_for(int64_t rows, int64_t cols, int64_t depth, bool allow_split) {
    Plan p{true, 1, (int)depth, ceil_div(rows, TileL::BM) * ceil_div(cols, TileL::BN)};
    if (p.tiles >= 256) return p;
    p.big = false;
    p.tiles = ceil_div(rows, TileS::BM) * ceil_div(cols, TileS::BN);
    if (!allow_split || p.tiles >= 256) return p;
    int64_t s = std::max<int64_t>(1, 256 / p.tiles);
    const int64_t max_s = std::max<int64_t>(1, depth / (8 * TileS::BK));
    s = std::min(s, max_s);
    const int64_t kper = ceil_div(ceil_div(depth, s), TileS::BK) * TileS::BK;
    p.splits = (int)ceil_div(depth, kper);
    p.kper = (int)kper;
    return p;
}

size_t align256(size_t b) { return (b + 255) / 256 * 256; }

// grad_W reads X_deq^T (kGradWT) on the large tiles of a tall output
// (N >= 8192), when its staging offsets fit 32 bits (128 rows of Mp bf16) and
// the transposed copy stays within 2 GiB.  The pass over X costs the same
// for any N (3 bytes an element: about 20 us at 4096 x 8192) while the
// product's saving grows with N (its steps run about 6% faster; measured at
// 28672 x 8192 from 4096 tokens 1751 -> 1663 us for the call, bit-identical;
// at N = 4096 (8192 tokens, K = 4096) 248 -> 255 us, so not used there; on
// the small split tiles the extra pass also costs more than it saves).
bool use_xdt(const Plan& p, int64_t M, int64_t N, int64_t K) {
    const int64_t Mp = (M + 7) / 8 * 8;
    return p.big && N >= 8192 && Mp <= ((int64_t)1 << 22) && K * Mp * 2 <= ((int64_t)1 << 31);
}
size_t xdt_bytes(int64_t M, int64_t K) { return align256((size_t)K * (size_t)((M + 7) / 8 * 8) * 2); }

template <int MODE, class T, bool OUT_BF16>
hipError_t launch_one(const uint16_t* gy, const void* second, const float* aux, int M, int N, int K,
                      const Plan& p, void* out, hipStream_t s, const SteGate& gate = SteGate{},
                      bool channel = false) {
    unsigned grid = (unsigned)(p.tiles * p.splits);
    if (!T::KSPLIT && N % 8 == 0) {  // persistent: at most one workgroup a CU
        int dev = 0, cus = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        grid = (unsigned)std::min<int64_t>(grid, std::max(cus, 1));
    }
    // the gate rides in the tile epilogue only without a token split (with
    // one, split_reduce_kernel applies it)
    const bool gated = MODE != kGradX && gate.w != nullptr && p.splits == 1;
#define BITNET_BWD_LAUNCH(V_, G_)                                                                \
    bwd_kernel<MODE, T, V_, OUT_BF16, G_><<<grid, kThreads, 0, s>>>(gy, second, aux, M, N, K,   \
                                                                   p.splits, p.kper, out, gate)
    if constexpr (MODE != kGradX) {
        if (gated) {
            if (N % 8 == 0) BITNET_BWD_LAUNCH(true, true);
            else BITNET_BWD_LAUNCH(false, true);
            return hipGetLastError();
        }
    } else {
        if (channel) {
            if (N % 8 == 0)
                bwd_kernel<MODE, T, true, OUT_BF16, false, true><<<grid, kThreads, 0, s>>>(
                    gy, second, aux, M, N, K, p.splits, p.kper, out, gate);
            else
                bwd_kernel<MODE, T, false, OUT_BF16, false, true><<<grid, kThreads, 0, s>>>(
                    gy, second, aux, M, N, K, p.splits, p.kper, out, gate);
            return hipGetLastError();
        }
    }
    if (N % 8 == 0) BITNET_BWD_LAUNCH(true, false);
    else BITNET_BWD_LAUNCH(false, false);
#undef BITNET_BWD_LAUNCH
    return hipGetLastError();
}

}  // namespace

// grad_W's workspace: the split partials (if any), then X_deq^T (if used)
size_t bwd_ws_bytes(int64_t M, int64_t N, int64_t K) {
    const Plan p = plan_for(N, K, M, true);
    return (p.splits > 1 ? align256((size_t)p.splits * N * K * 4) : 0) + (use_xdt(p, M, N, K) ? xdt_bytes(M, K) : 0);
}

hipError_t launch_bwd_ste(const uint16_t* gy, const int8_t* Xq, const float* scale_x,
                          const uint8_t* Wp, const float* gamma, int64_t M, int64_t N, int64_t K,
                          void* grad_x, bool gx_bf16, float* grad_W, void* ws, hipStream_t s,
                          const SteGate& gate, bool channel) {
    const int m = (int)M, n = (int)N, k = (int)K;
    if (grad_x) {
        const Plan p = plan_for(M, K, N, false);
        hipError_t e;
        if (p.big)
            e = gx_bf16 ? launch_one<kGradX, TileL, true>(gy, Wp, gamma, m, n, k, p, grad_x, s, SteGate{}, channel)
                        : launch_one<kGradX, TileL, false>(gy, Wp, gamma, m, n, k, p, grad_x, s, SteGate{}, channel);
        else
            e = gx_bf16 ? launch_one<kGradX, TileS, true>(gy, Wp, gamma, m, n, k, p, grad_x, s, SteGate{}, channel)
                        : launch_one<kGradX, TileS, false>(gy, Wp, gamma, m, n, k, p, grad_x, s, SteGate{}, channel);
        if (e != hipSuccess) return e;
    }
    if (grad_W) {
        const Plan p = plan_for(N, K, M, true);
        void* dst = p.splits > 1 ? ws : static_cast<void*>(grad_W);
        hipError_t e;
        if (use_xdt(p, M, N, K)) {
            const size_t part = p.splits > 1 ? align256((size_t)p.splits * N * K * 4) : 0;
            uint16_t* xdt = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + part);
            const int64_t Mp = (M + 7) / 8 * 8;
            const int64_t tiles_m = ceil_div(Mp, kXtTile), tiles = tiles_m * ceil_div(K, kXtTile);
            if (tiles > INT32_MAX) return hipErrorInvalidValue;
            xdeq_t_kernel<<<(unsigned)tiles, 256, 0, s>>>(Xq, scale_x, m, k, (int)Mp, (int)tiles_m, xdt);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
            e = launch_one<kGradWT, TileLW, false>(gy, xdt, nullptr, m, n, k, p, dst, s, gate);
        } else {
            e = p.big ? launch_one<kGradW, TileL, false>(gy, Xq, scale_x, m, n, k, p, dst, s, gate)
                      : launch_one<kGradW, TileSK, false>(gy, Xq, scale_x, m, n, k, p, dst, s, gate);
        }
        if (e != hipSuccess) return e;
        if (p.splits > 1) {
            const int64_t count = N * K;
            split_reduce_kernel<<<(unsigned)ceil_div(ceil_div(count, 4), 256), 256, 0, s>>>(
                static_cast<const float*>(ws), p.splits, count, grad_W, gate);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

}  // namespace bitnet
