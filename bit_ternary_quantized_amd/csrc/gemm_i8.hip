// Ternary x int8 GEMM on gfx950 int8 matrix cores (prefill / training shapes).
//
//   acc[m][n] = sum_k Xq[m][k] * code[n][k]     exact int32
//   Y[m][n]   = acc[m][n] * (gamma / scale_x[m])
//
// The linear layer of "BitNet 1.5技术解析：2比特量化在神经网络中的应用与挑战"
// (3.1) on the integer operands, with the wide accumulator asked for in its
// 5.2; the +1 / -1 / 0 codes are the add / subtract / skip of
// "1.58-bit量化技术突破AI算力与内存墙限制" (3.1), evaluated here as an exact
// int8 dot product on v_mfma_i32_32x32x32_i8.
//
// Tiling: a 256 x 256 output tile per 512-thread workgroup; 8 waves as
// 2 (M) x 4 (N), each owning 128 x 64 (4 x 2 MFMA blocks of 32 x 32, 128
// int32 accumulators).  For outputs with few such tiles, 128 x 256 tiles
// (64 x 64 a wave) at two workgroups a CU.  K advances 64 per step.  Activation chunks are
// staged in LDS byte-transposed 4 x 4; the weight tile stays 2-bit packed in
// LDS (256 x 16 B, a quarter of the int8 bytes) and each wave unpacks its
// operands in registers (unpack16 yields the same transposed column order,
// so every product pairs equal columns; the sum over k is exact and
// order-free).
//
// Schedule: ping-pong of two wave groups.  Waves 0-3 (tile rows 0-127) and
// waves 4-7 (rows 128-255) put one wave on each SIMD and run the same loop
// one barrier apart, so on every SIMD one wave issues its 16 MFMAs while the
// other does its memory phase: write the next tile into LDS, issue the
// global loads of the tile after it, read and unpack its operands of the
// current tile into registers.  Each group stages its own activation half
// and its own copy of the weight tile, both double-buffered (32 KB of
// activations and 64 KB of weight codes in all, plus the row scales: 97 KB
// of LDS, one workgroup a CU), so the groups share no LDS data and a
// barrier only orders the phases.  Global
// loads are buffer loads whose tails (rows past M or N, columns past K) read
// zeros, so the loop has no branch.
#include <type_traits>

#include "common.h"

namespace bitnet {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int BN = 256, BK = 64;
constexpr int kThreads = 512;
constexpr int kGroupThreads = 256;  // one wave group: 4 waves, one per SIMD
constexpr int JN = 2;               // 32-column blocks per wave
// Activation tile of one group and step: 128 rows x 64 B.  Weight codes come
// in blocks of 4 steps: 256 rows x 64 B (4 slices of 16 B = 64 codes), so a
// row's load is one 64-byte piece taken by 4 adjacent lanes; each step loads
// a quarter (64 rows) of the block after next.
constexpr int ROW_BYTES = 64;
constexpr int B_BYTES = BN * ROW_BYTES;
constexpr int kStepsPerBlock = 4;
constexpr int kQuarterRows = BN / kStepsPerBlock;
// IM: 32-row blocks per wave.  Tile rows: 32 IM per group, 64 IM in all.
template <int IM>
struct MTile {
    static constexpr int HM = 32 * IM;  // tile rows per group
    static constexpr int BM = 2 * HM;
    static constexpr int A_BYTES = HM * ROW_BYTES;
    static constexpr int kAPer = HM * (ROW_BYTES / 16) / kGroupThreads;  // 16-byte activation chunks per thread
};
// LDS rows are unpadded and XOR-swizzled so that the 16-byte writes of the
// staging threads and the operand reads of the waves both hit distinct banks
// in every 16-lane group: 16-byte chunk c of row r sits at slot
// c ^ ((r >> 2) & 3); inside a weight slice, 8-byte half h at
// h ^ ((r >> 4) & 1) ^ ((r >> 5) & 1).  The row-bit-5 term keeps the two
// reads of rows r and r + 32 (which the compiler may merge into one
// ds_read2_b64) on different banks.
__device__ __forceinline__ int row_slot(int r, int c) { return r * ROW_BYTES + 16 * (c ^ ((r >> 2) & 3)); }
__device__ __forceinline__ int half_swap(int r) { return ((r >> 4) ^ (r >> 5)) & 1; }

// Workgroup id -> tile, XCD-aware: consecutive ids go round-robin over the
// 8 XCDs, so ids are regrouped to give each XCD a contiguous run of tiles
// (row-major over tiles), which then share A rows in that XCD's L2.
__device__ __forceinline__ void tile_of(int wg, int tiles_m, int tiles_n, int& tm, int& tn) {
    const int G = tiles_m * tiles_n;
    const int q = G / 8, r = G % 8;
    const int x = wg % 8, local = wg / 8;
    const int id = (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + local;
    // uniform values; readfirstlane keeps them (and the addresses built
    // from them) in scalar registers after the division's VALU expansion
    tm = __builtin_amdgcn_readfirstlane(id / tiles_n);
    tn = __builtin_amdgcn_readfirstlane(id % tiles_n);
}

template <int KA>
struct Stage {
    uint4 a[KA];  // 16-byte activation chunks of the group's half (tile t)
    uint4 b;      // one 16-byte weight slice (quarter t + 3), halves in slot order
};

}  // namespace

// VECB: K % 64 == 0, so a step's 16 bytes of a packed weight row are all in
// or all out of range (else dword granularity).  CH: one scale per output
// channel, gamma_p[n] (y = acc * (1/scale_x[m]) * gamma_p[n]); else the one
// gamma of the matrix (y = acc * (gamma/scale_x[m])).
template <bool VECB, bool CH = false, int IM = 4>
__global__ __launch_bounds__(kThreads, IM == 4 ? 1 : 4) void gemm_i8t2_kernel(
    const int8_t* __restrict__ Xq, const float* __restrict__ scale_x,
    const uint8_t* __restrict__ Wp, const float* __restrict__ gamma_p, int M, int N, int K,
    float* __restrict__ Y, int32_t* __restrict__ acc_out) {
    constexpr int HM = MTile<IM>::HM, BM = MTile<IM>::BM, A_BYTES = MTile<IM>::A_BYTES;
    constexpr int kAPer = MTile<IM>::kAPer;
    using Stage = bitnet::Stage<kAPer>;
    // LDS: activation tiles [group][buffer], weight tiles [group][block
    // buffer], then (256-row tiles) the row scale table.  128-row tiles keep
    // the table in the first activation buffer instead, written after the K
    // loop, so that two workgroups fit in a CU's 160 KB.
    constexpr int kLdsBytes = 4 * A_BYTES + 4 * B_BYTES + (IM == 4 ? 4 * BM : 0);
    __shared__ __align__(16) uint8_t lds[kLdsBytes];
    auto smem_a = reinterpret_cast<uint8_t(*)[2][A_BYTES]>(lds);
    auto smem_b = reinterpret_cast<uint8_t(*)[2][B_BYTES]>(lds + 4 * A_BYTES);
    float* const row_scale = reinterpret_cast<float*>(IM == 4 ? lds + 4 * A_BYTES + 4 * B_BYTES : lds);

    // Persistent: workgroup b takes tiles b, b + grid, ...  (the grid is at
    // most one workgroup per CU), so the y stores of one tile drain while
    // the next tile's loads and MFMAs run instead of ending every round of
    // workgroups with a write burst.  Tile v maps as workgroup v would in a
    // one-tile-per-workgroup launch (same XCD when the grid is a multiple
    // of 8).  The next tile's first loads are issued before this tile's y
    // stores: a wave's memory operations complete in issue order, so loads
    // issued after 128 stores would wait for all of them.
    const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    const int ntiles = tiles_m * tiles_n;
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);  // uniform in the wave
    const int wm = wave >> 2, wn = wave & 3;                   // wm: the wave group
    const int tg = t & (kGroupThreads - 1);                    // thread inside the group
    const int KB = K / 4;                                      // packed bytes per weight row
    const int nk = (K + BK - 1) / BK;

    // Activations: thread tg stages chunks tg + 256 u (row c / 4, chunk c % 4)
    // of the group's 128 rows; offsets relative to the step's base address.
    int arow[kAPer], acol[kAPer];
#pragma unroll
    for (int u = 0; u < kAPer; ++u) {
        const int c = tg + u * kGroupThreads;
        arow[u] = c >> 2;
        acol[u] = (c & 3) * 16;
    }
    // Weights: in a quarter, thread tg stages slice bc = tg % 4 of row
    // bq = tg / 4 (+ 64 per quarter), both 8-byte halves in slot order.
    const int bq = tg >> 2, bc = tg & 3, bsw = half_swap(bq);
    const uint32_t boff = (uint32_t)(bq * KB + 16 * bc);

    // where a tile's operands start (uniform) and this thread's activation offsets
    struct Geo {
        int m0, n0;
        const int8_t* Xt;
        const uint8_t* Wt;
        uint32_t aoff[kAPer];
    };
    // (live = false: a tile that does not exist, every load of it past the
    // buffer: no memory access, zeros)
    auto geo_of = [&](int tile, bool live) {
        Geo g;
        int tm, tn;
        tile_of(tile, tiles_m, tiles_n, tm, tn);
        g.m0 = tm * BM;
        g.n0 = live ? tn * BN : N;
        const int mh = g.m0 + wm * HM;  // first row of the group's half
#pragma unroll
        for (int u = 0; u < kAPer; ++u)
            g.aoff[u] = live && mh + arow[u] < M ? (uint32_t)(arow[u] * K + acol[u]) : kBufOOB;
        g.Xt = Xq + (int64_t)mh * K;
        g.Wt = Wp + (int64_t)g.n0 * KB;
        return g;
    };

    auto load_a = [&](const Geo& g, int it, uint4 (&a)[kAPer]) {
        const int k0 = it * BK;
        const __amdgpu_buffer_rsrc_t ra = make_buf(g.Xt + k0);
#pragma unroll
        for (int u = 0; u < kAPer; ++u) a[u] = buf_load16(ra, k0 + acol[u] < K ? g.aoff[u] : kBufOOB);
    };
    auto load_b = [&](const Geo& g, int qi, uint4& b) {  // quarter qi: block qi / 4, rows 64 (qi % 4) + bq
        const int blk = qi >> 2, part = qi & 3;
        const int kb0 = blk * kStepsPerBlock * BK;  // first column of the block
        const __amdgpu_buffer_rsrc_t rb = make_buf(g.Wt + (int64_t)part * kQuarterRows * KB + blk * ROW_BYTES);
        const bool rv = g.n0 + part * kQuarterRows + bq < N;
        const int kc = kb0 + bc * BK;  // first column of the slice
        if constexpr (VECB) {
            const bool v = rv && kc < K;
            const uint2 lo = buf_load8(rb, v ? boff + 8 * bsw : kBufOOB);
            const uint2 hi = buf_load8(rb, v ? boff + 8 * (bsw ^ 1) : kBufOOB);
            b = make_uint4(lo.x, lo.y, hi.x, hi.y);
        } else {  // dword d of the slice covers columns kc + 16 d .. + 15
            const int d0 = 2 * bsw, d1 = 2 * (bsw ^ 1);
            b.x = buf_load4(rb, rv && kc + 16 * d0 < K ? boff + 4 * d0 : kBufOOB);
            b.y = buf_load4(rb, rv && kc + 16 * d0 + 16 < K ? boff + 4 * d0 + 4 : kBufOOB);
            b.z = buf_load4(rb, rv && kc + 16 * d1 < K ? boff + 4 * d1 : kBufOOB);
            b.w = buf_load4(rb, rv && kc + 16 * d1 + 16 < K ? boff + 4 * d1 + 4 : kBufOOB);
        }
    };
    // staged activation chunks are byte-transposed in registers (in a
    // compute phase, where the VALU is otherwise idle) and stored as they are
    auto transpose_a = [&](uint4 (&a)[kAPer]) {
#pragma unroll
        for (int u = 0; u < kAPer; ++u) {
            const uint32_t in[4] = {a[u].x, a[u].y, a[u].z, a[u].w};
            uint32_t o[4];
            transpose4x4_bytes(in, o);
            a[u] = make_uint4(o[0], o[1], o[2], o[3]);
        }
    };
    auto store_a = [&](int buf, const uint4 (&a)[kAPer]) {
        uint8_t* As = smem_a[wm][buf];
#pragma unroll
        for (int u = 0; u < kAPer; ++u) {
            const int c = tg + u * kGroupThreads;
            *reinterpret_cast<uint4*>(As + row_slot(c >> 2, c & 3)) = a[u];
        }
    };
    auto store_b = [&](int qi, const uint4& b) {
        uint8_t* Bs = smem_b[wm][(qi >> 2) & 1];
        *reinterpret_cast<uint4*>(Bs + row_slot((qi & 3) * kQuarterRows + bq, bc)) = b;
    };
    // tile t of the activations and quarter t + 3 of the weights
    auto load_global = [&](const Geo& g, int it, Stage& p) {
        load_a(g, it, p.a);
        load_b(g, it + 3, p.b);
    };
    auto store_lds = [&](int it, const Stage& p) {
        store_a(it & 1, p.a);
        store_b(it + 3, p.b);
    };

    const int g = lane >> 5;    // lane group: k chunks 2g, 2g+1 of the step
    const int l32 = lane & 31;  // row (A) / column (B) inside a 32-block

    // Operands of one step: MFMA half kh pairs activation chunk 2g+kh with
    // the same chunk of the codes (one packed dword per half).
    v4i a[2][IM], b[2][JN];
    uint2 bp[JN];
    auto read_codes = [&](int it) {
        const uint8_t* Bs = smem_b[wm][(it >> 2) & 1];
        const int c = it & 3;
#pragma unroll
        for (int j = 0; j < JN; ++j) {
            const int r = wn * 64 + j * 32 + l32;
            bp[j] = *reinterpret_cast<const uint2*>(Bs + row_slot(r, c) + 8 * (g ^ half_swap(r)));
        }
    };
    auto read_acts = [&](int buf) {
        const uint8_t* As = smem_a[wm][buf];
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int i = 0; i < IM; ++i) {
                const uint4 v = *reinterpret_cast<const uint4*>(As + row_slot(i * 32 + l32, 2 * g + kh));
                a[kh][i] = v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
            }
    };
    auto unpack_codes = [&] {
#pragma unroll
        for (int j = 0; j < JN; ++j) {
            uint32_t u[4];
            unpack16(bp[j].x, u);
            b[0][j] = v4i{(int)u[0], (int)u[1], (int)u[2], (int)u[3]};
            unpack16(bp[j].y, u);
            b[1][j] = v4i{(int)u[0], (int)u[1], (int)u[2], (int)u[3]};
        }
    };
    auto barrier = [] {
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
    };

    if ((int)blockIdx.x >= ntiles) return;  // (the grid has at most ntiles workgroups)
    Geo cur = geo_of(blockIdx.x, true);
    // the first tile's prologue loads: weight quarters 0-2, activation tile 0 + quarter 3
    uint4 q0, q1, q2;
    Stage p0;
    load_b(cur, 0, q0);
    load_b(cur, 1, q1);
    load_b(cur, 2, q2);
    load_global(cur, 0, p0);

    for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        const int m0 = cur.m0, n0 = cur.n0;
        float rs_t;  // this thread's entry of the row scale table (t < BM)
        {
            const float gm = CH ? 1.0f : *gamma_p;
            rs_t = (t < BM && m0 + t < M) ? gm / scale_x[m0 + t] : 0.0f;
            if (IM == 4 && t < BM) row_scale[t] = rs_t;
        }
        // per-channel scales of this lane's JN output columns, requested now
        // so their latency hides under the K loop (clamped index: the load is
        // unconditional; columns past N are not stored)
        float sc[CH ? JN : 1];
        if constexpr (CH) {
#pragma unroll
            for (int j = 0; j < JN; ++j) sc[j] = gamma_p[min(n0 + (wave & 3) * 64 + (lane & 31) + j * 32, N - 1)];
        }

        v16i acc[IM][JN];
#pragma unroll
        for (int i = 0; i < IM; ++i)
#pragma unroll
            for (int j = 0; j < JN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

        // One step.  Memory phase: operands of step it (packed codes first, then
        // activations); activation tile it + 1 and weight quarter it + 4 (loaded
        // two steps ago into `st`, transposed since) into LDS; then the loads of
        // tile it + 3 / quarter it + 6 into the freed `st`.  Compute phase: the
        // 16 MFMAs, with the VALU work of the step between them: unpacking the
        // codes just read and byte-transposing the activations of `nx` (loaded a
        // step ago, stored next step).
        //   Buffers: activation tile t in buffer t % 2; weight block t / 4 (steps
        //   4 (t/4) .. + 3) in buffer (t / 4) % 2, written a quarter per step
        //   during the four steps before it is read.  Every buffer is rewritten
        //   only two barriers after its last read.
        //   The memory phase runs at raised wave priority: on each SIMD the
        //   other group's wave is issuing MFMAs meanwhile, and the step time is
        //   set by how soon the memory phase reaches its barrier (measured at
        //   8192 x 4096 x 4096: 131 us with the priority on the compute phase
        //   instead, 123 us this way).
        auto step = [&](int it, Stage& st, Stage& nx) {
            __builtin_amdgcn_s_setprio(1);
            read_codes(it);
            read_acts(it & 1);
            store_lds(it + 1, st);
            load_global(cur, it + 3, st);
            __builtin_amdgcn_s_setprio(0);
            barrier();
            unpack_codes();
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int i = 0; i < IM; ++i)
#pragma unroll
                    for (int j = 0; j < JN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[kh][i], b[kh][j], acc[i][j], 0, 0, 0);
            transpose_a(nx.a);
            barrier();
        };

        // Prologue: activation tile 0 and weight block 0 (quarters 0-3) in LDS
        // (their loads were issued before the previous tile's epilogue, or
        // above for the first tile); tiles 1, 2 and quarters 4, 5 loading.
        // Group 1 then waits one extra barrier, which puts it a phase behind
        // group 0.
        transpose_a(p0.a);
        store_a(0, p0.a);
        store_b(0, q0);
        store_b(1, q1);
        store_b(2, q2);
        store_b(3, p0.b);
        Stage s0, s1;
        load_global(cur, 1, s1);
        load_global(cur, 2, s0);
        transpose_a(s1.a);
        barrier();
        if (wm == 1) barrier();

        // Unrolled by two so that the staging sets alternate by name (no copy);
        // with nk odd the last step runs on zero tiles (loads past K read
        // zeros), which adds nothing to the sums.
        for (int it = 0; it < nk; it += 2) {
            step(it, s1, s0);
            step(it + 1, s0, s1);
        }
        // Group 0 closes with the barrier group 1 took at the start: both
        // groups pass the same barriers in every tile.
        if (wm == 0) barrier();
        if constexpr (IM != 4) {  // the table into the now unread first activation buffer
            if (t < BM) row_scale[t] = rs_t;
            barrier();
        }
        // The next tile's prologue loads, ahead of this tile's stores (its
        // LDS writes wait for the barrier at the end of this tile).  After
        // the last tile they are issued too, all past the buffer: issued on
        // every path, they leave nothing of this tile's prologue live across
        // its K loop.
        {
            const int next = tile + (int)gridDim.x;
            cur = geo_of(min(next, ntiles - 1), next < ntiles);
        }
        load_b(cur, 0, q0);
        load_b(cur, 1, q1);
        load_b(cur, 2, q2);
        load_global(cur, 0, p0);
        // Epilogue.  32x32 block layout: lane holds column l32 and rows
        // 8*(r/4) + 4*g + r%4 for r = 0..15.  Stores address a uniform tile base
        // with 32-bit offsets (a tile spans < 2^31 bytes).
        float* Yt = Y + (int64_t)m0 * N + n0;
        const int mlim = M - m0, nlim = N - n0;
        int rbase = wm * HM + 4 * g, cbase = wn * 64 + l32;
        // opaque per tile, so the 128 store offsets built from them are not
        // hoisted out of the tile loop (they would stay live across it)
        asm volatile("" : "+v"(rbase), "+v"(cbase));
        // Interior tiles store without per-element conditions: a branch per
        // store would let the compiler pull all 256 accumulators into VGPRs at
        // once.  Edge tiles take the guarded loop.
        auto store_tile = [&](auto guarded_tag, auto out, auto value) {
            constexpr bool GUARD = decltype(guarded_tag)::value;
#pragma unroll
            for (int i = 0; i < IM; ++i) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int rloc = rbase + i * 32 + 8 * (r >> 2) + (r & 3);
                    const int roff = rloc * N;
                    const float rs = row_scale[rloc];
#pragma unroll
                    for (int j = 0; j < JN; ++j) {
                        const int cloc = cbase + j * 32;
                        // streaming (non-temporal) stores: the output is not read again here
                        if (!GUARD || (rloc < mlim && cloc < nlim))
                            __builtin_nontemporal_store(value(acc[i][j][r], rs, j), &out[roff + cloc]);
                    }
                }
                // keep the scheduler from pulling later accumulators forward
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        auto yval = [&](int v, float rs, int j) {
            const float y = (float)v * rs;
            if constexpr (CH) return y * sc[j];
            else return y;
        };
        auto aval = [](int v, float, int) { return v; };
        if (mlim >= BM && nlim >= BN) store_tile(std::false_type{}, Yt, yval);
        else store_tile(std::true_type{}, Yt, yval);
        if (acc_out) {
            int32_t* At = acc_out + (int64_t)m0 * N + n0;
            store_tile(std::true_type{}, At, aval);
        }
        // row_scale and the LDS tiles are rewritten by the next tile
        __syncthreads();
    }
}

hipError_t launch_gemm_i8t2(const int8_t* Xq, const float* scale_x, const uint8_t* Wp,
                            const float* gamma, int64_t M, int64_t N, int64_t K, float* Y,
                            int32_t* acc, hipStream_t s, bool channel) {
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    cus = std::max(cus, 1);
    const int64_t tiles_n = (N + BN - 1) / BN;
    const int64_t tiles4 = ((M + MTile<4>::BM - 1) / MTile<4>::BM) * tiles_n;
    if (tiles4 > INT32_MAX) return hipErrorInvalidValue;
    // At most half as many 256-row tiles as CUs (and K % 64 == 0): 128-row
    // tiles, two workgroups a CU (their LDS and registers allow two), so
    // more CUs work and each one's two workgroups overlap their prologues and
    // y stores with the other's K loop.  Otherwise 256-row tiles, one
    // workgroup a CU at most, each walking tiles.  Measured (graphs of 10
    // launches, bit-identical): 512 x 4096 x 4096 43.4 -> 31.6 us, 4096 x
    // 1024 x 4096 44.0 -> 33.1 us, 2048 x 4096 x 4096 46.4 -> 39-41 us,
    // 4096 x 1376 x 512 15.8 -> 12-14 us; with 192 tiles (8192 x 1376 x
    // 512) slower, 16.3 -> 17.0-18.0 us; with K % 64 != 0 the 128-register
    // budget spills inside the K loop.
    const bool half = K % BK == 0 && 2 * tiles4 <= cus;
    const int64_t tiles = half ? ((M + MTile<2>::BM - 1) / MTile<2>::BM) * tiles_n : tiles4;
    const unsigned grid = (unsigned)std::min<int64_t>(tiles, half ? 2 * (int64_t)cus : cus);
#define BITNET_GEMM_LAUNCH(V_, C_, IM_)                                                                  \
    gemm_i8t2_kernel<V_, C_, IM_><<<grid, kThreads, 0, s>>>(Xq, scale_x, Wp, gamma, (int)M, (int)N, (int)K, Y, \
                                                            acc)
    if (half) {
        if (channel) BITNET_GEMM_LAUNCH(true, true, 2);
        else BITNET_GEMM_LAUNCH(true, false, 2);
    } else if (K % BK == 0) {
        if (channel) BITNET_GEMM_LAUNCH(true, true, 4);
        else BITNET_GEMM_LAUNCH(true, false, 4);
    } else {
        if (channel) BITNET_GEMM_LAUNCH(false, true, 4);
        else BITNET_GEMM_LAUNCH(false, false, 4);
    }
#undef BITNET_GEMM_LAUNCH
    return hipGetLastError();
}

}  // namespace bitnet
