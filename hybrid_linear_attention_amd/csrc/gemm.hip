// bf16 GEMM with fp32 accumulation on gfx950 MFMA (v_mfma_f32_16x16x32_bf16),
// for the layer block's projections ("Qwen3.8-27B: from model structure to the
// vLLM inference dataflow", section 01 operator table: [Q0,K0,V0,Z] = U Wqkvz,
// a = U Wa, b = U Wb, Delta_mix = Ogate Wo, Y = X + Delta_mix).
//
//   C[M,N] = A[M,K] * B[N,K]^T (+ R[M,N])
//
// Both operands are K-contiguous, so every MFMA fragment is one 16-byte LDS
// read.  A 256-thread block owns a 128x128 C tile (each wave 64x64 = 4x4 MFMA
// tiles); K advances 32 at a time through a double-buffered LDS stage.
#include "gdn_device.h"
#include "gdn_launch.h"

#include <algorithm>

namespace gdn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

constexpr int GBM = 128, GBN = 128, GBK = 32;
constexpr int GLDS = GBK + 8;  // padded row (80 bytes) spreads rows over LDS banks

template <typename TC, bool RES>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(
    const uint16_t *__restrict__ A, int64_t lda, const uint16_t *__restrict__ B, int64_t ldb,
    TC *__restrict__ C, int64_t ldc, const uint16_t *__restrict__ R, int64_t ldr, int M, int N,
    int K) {
    __shared__ __attribute__((aligned(16))) uint16_t As[2][GBM][GLDS];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][GBN][GLDS];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int m0 = blockIdx.y * GBM, n0 = blockIdx.x * GBN;

    floatx4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};

    // each thread stages 2 x 8 elements of A and of B per K step
    uint4 ra[2], rb[2];
    auto gload = [&](int k0) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int c = tid + h * 256;
            const int row = c >> 2, col = (c & 3) * 8;
            ra[h] = make_uint4(0, 0, 0, 0);
            rb[h] = make_uint4(0, 0, 0, 0);
            if (m0 + row < M && k0 + col < K)
                ra[h] = *reinterpret_cast<const uint4 *>(A + (int64_t)(m0 + row) * lda + k0 + col);
            if (n0 + row < N && k0 + col < K)
                rb[h] = *reinterpret_cast<const uint4 *>(B + (int64_t)(n0 + row) * ldb + k0 + col);
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int c = tid + h * 256;
            const int row = c >> 2, col = (c & 3) * 8;
            *reinterpret_cast<uint4 *>(&As[buf][row][col]) = ra[h];
            *reinterpret_cast<uint4 *>(&Bs[buf][row][col]) = rb[h];
        }
    };

    const int nk = (K + GBK - 1) / GBK;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) gload((kt + 1) * GBK);
        const int kk = 8 * (lane >> 4);
        bf16x8_t af[4], bfr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            af[i] = *reinterpret_cast<const bf16x8_t *>(&As[cur][wm * 64 + i * 16 + (lane & 15)][kk]);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            bfr[j] = *reinterpret_cast<const bf16x8_t *>(&Bs[cur][wn * 64 + j * 16 + (lane & 15)][kk]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        if (kt + 1 < nk) sstore(cur ^ 1);
        __syncthreads();
    }

    // accumulator layout: lane holds rows 4*(lane/16)+r, column lane%16 of each tile
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int col = n0 + wn * 64 + j * 16 + (lane & 15);
            if (col >= N) continue;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = m0 + wm * 64 + i * 16 + 4 * (lane >> 4) + r;
                if (row >= M) continue;
                float val = acc[i][j][r];
                if (RES) val += __uint_as_float(uint32_t(R[(int64_t)row * ldr + col]) << 16);
                st(C + (int64_t)row * ldc + col, val);
            }
        }
}

// ---------------------------------------------------------------------------
// Large-tile variant for K % 64 == 0: a 512-thread block owns a 256x256 C tile
// (8 waves as 4 x 2, each 64 x 128 = 4 x 8 MFMA tiles); K advances 64 at a time
// through a two-stage LDS ring filled by direct-to-LDS 16-byte loads.  LDS rows
// are 128 bytes (64 bf16) with the 16-byte chunk index XOR-swizzled by row
// (chunk j of row r stored at j ^ (r & 7)), so the 16 rows of a fragment read
// fall in different banks; the swizzle is applied on the global side because a
// direct-to-LDS load places lane l's bytes at base + 16 l.
//
// Each 64-deep stage is two 32-deep k-slices, and the one barrier per stage sits
// between them.  Phase A multiplies slice 0 (fragments already in registers)
// while reading slice 1's; the barrier then certifies that the next stage has
// landed and that every wave is done with this one; phase B multiplies slice 1
// while reading the next stage's slice-0 fragments and refilling this stage's
// buffer with the stage after next.  A wave thus leaves the barrier with a full
// slice of MFMAs ready instead of waiting for LDS reads that every wave of the
// block issues at the same moment.  MFMAs run over one B fragment at a time
// (4 tiles) so that the register of the fragment they finish is refilled next.
// ---------------------------------------------------------------------------
constexpr int G2N = 256;
constexpr int G2_THREADS = 512;
constexpr int G2_BK = 64;                          // K per stage (two MFMA k-slices)
constexpr int G2_CPR = G2_BK / 8;                  // 16-byte chunks per LDS row
constexpr int G2_GROUP_M = 4;                      // tile rows per group of the tile order
// tile rows TM (256, or 192 where it quantises the tiles into rounds of the
// chip's CUs better): one operand stage of TM or 256 rows x 64 bf16, two stages
template <int TM> struct G2 {
    static constexpr int MI = TM / 64;                      // 16-row MFMA tiles per wave (4 waves in M)
    static constexpr size_t TILE_A = (size_t)TM * G2_BK * 2;
    static constexpr size_t TILE_B = (size_t)G2N * G2_BK * 2;
    static constexpr size_t STAGE = TILE_A + TILE_B;
    static constexpr size_t SMEM = 2 * STAGE;               // 128 or 112 KiB
    static constexpr int LOADS = (TM + G2N) * G2_CPR / G2_THREADS;  // direct-to-LDS loads per thread per stage
};

// one operand tile of ROWS rows x 64 bf16: rows of 128 bytes, 16-byte chunk j
// of row r stored at chunk j ^ (r & 7)
template <int ROWS>
__device__ __forceinline__ void g2_copy(const uint16_t *__restrict__ X, int64_t ld, int rows_valid,
                                        int row0, int k0, uint8_t *tile, int tid) {
    constexpr int PER_THREAD = ROWS * G2_CPR / G2_THREADS;
    const int wv = tid >> 6, lane = tid & 63;
#pragma unroll
    for (int m = 0; m < PER_THREAD; ++m) {
        const int s = (m * 8 + wv) * 64 + lane;  // wave-contiguous LDS pieces
        const int r = s / G2_CPR;
        const int j = (s % G2_CPR) ^ (r & (G2_CPR - 1));
        const int rr = min(row0 + r, rows_valid - 1);  // rows past the edge load a valid row, never stored
        const uint16_t *src = X + (int64_t)rr * ld + k0 + 8 * j;
        __builtin_amdgcn_global_load_lds(static_cast<const void *>(src),
                                         (__attribute__((address_space(3))) void *)(tile + (size_t)(m * 8 + wv) * 1024),
                                         16, 0, 0);
    }
}

// Tile order.  Workgroups are dealt to the 8 XCDs round-robin (block b on XCD
// b % 8), so XCD x is handed a contiguous run of the linear tile order (its
// share of n, the first n % 8 XCDs one tile more) and the blocks resident on
// one XCD at a time work on neighbouring tiles.  The linear order walks groups
// of G2_GROUP_M tile rows column by column, so the resident blocks of an XCD
// share A row panels and B column panels through its L2.  Both maps are
// bijections (on [0, n) and [0, nbm * nbn)) whatever the hardware's dispatch
// order.
__device__ __forceinline__ int g2_deal(int b, int n) {
    const int x = b % 8, base = n / 8, rem = n % 8;
    return x * base + min(x, rem) + b / 8;
}
__device__ __forceinline__ void g2_order(int t, int nbm, int nbn, int &tm, int &tn) {
    const int gsz = G2_GROUP_M * nbn;
    const int r0 = (t / gsz) * G2_GROUP_M;
    const int gm = min(G2_GROUP_M, nbm - r0);
    const int local = t - (t / gsz) * gsz;
    tm = r0 + local % gm;
    tn = local / gm;
}

// Split tail.  Tiles fill the chip in rounds of one tile per CU; when the last
// round is only partly filled (the last `tail` tiles of the linear order, or
// every tile when there are fewer than CUs), its tiles x stages are dealt out
// evenly to `nblk` blocks instead, as contiguous runs of (tile, stage) units,
// each shorter than a tile: a block covers the end of one tile and the start
// of the next at most.  A run stores its fp32 sums to a 256 x 256 slot of the
// workspace (two per block); gemm_split_reduce_kernel then adds each tile's
// runs in block order (deterministic), adds the residual and writes C.
constexpr int G2_SPLIT_MIN = 4;                          // stages per block at least
constexpr size_t G2_SLOT = (size_t)G2N * G2N;            // floats per run slot
// SPLIT: blocks from `full` on are the split tail's nblk blocks (256-row
// tiles); without it `full` is the tile count.
template <int TM, typename TC, bool RES, bool SPLIT>
__global__ __launch_bounds__(G2_THREADS) void gemm_bf16_v2_kernel(
    const uint16_t *__restrict__ A, int64_t lda, const uint16_t *__restrict__ B, int64_t ldb,
    TC *__restrict__ C, int64_t ldc, const uint16_t *__restrict__ R, int64_t ldr, int M, int N,
    int K, int full, int nblk, float *__restrict__ part) {
    using P = G2<TM>;
    constexpr int MI = P::MI;
    static_assert(!SPLIT || TM == G2N, "the split tail runs on 256 x 256 tiles");
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;  // 4 x 2 waves: rows 16 MI wm, columns 128 wn
    const int lr = lane & 15, lg = lane >> 4;
    const int nbn = (N + G2N - 1) / G2N, nbm = (M + TM - 1) / TM;
    const int nk_all = K / G2_BK;
    // One (tile, stage range) of this block: the K loop over stages kb .. ke - 1
    // and the epilogue, into C or (pslot: a piece of the split tail) into a
    // 256 x 256 fp32 slot.
    auto run = [&](int tm, int tn, int kb, int ke, float *pslot) {
        const int m0 = tm * TM, n0 = tn * G2N;
        floatx4_t acc[MI][8];
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};

        // fragment: row lr of a 16-row tile, logical chunk 4 ks + lg (8 bf16)
        auto frag_a = [&](const uint8_t *At, int ks, int i) {
            const int r = wm * 16 * MI + i * 16 + lr;
            const int pc = (4 * ks + lg) ^ (r & (G2_CPR - 1));
            return *reinterpret_cast<const bf16x8_t *>(At + (size_t)r * (2 * G2_BK) + 16 * pc);
        };
        auto frag_b = [&](const uint8_t *Bt, int ks, int j) {
            const int r = wn * 128 + j * 16 + lr;
            const int pc = (4 * ks + lg) ^ (r & (G2_CPR - 1));
            return *reinterpret_cast<const bf16x8_t *>(Bt + (size_t)r * (2 * G2_BK) + 16 * pc);
        };

        const int nk = ke - kb;  // stages kb .. ke - 1, at K offset kbk on
        const int kbk = kb * G2_BK;
        g2_copy<TM>(A, lda, M, m0, kbk, smem, tid);
        g2_copy<G2N>(B, ldb, N, n0, kbk, smem + P::TILE_A, tid);
        if (nk > 1) {
            g2_copy<TM>(A, lda, M, m0, kbk + G2_BK, smem + P::STAGE, tid);
            g2_copy<G2N>(B, ldb, N, n0, kbk + G2_BK, smem + P::STAGE + P::TILE_A, tid);
            // stage 0 landed (loads complete in order; vmcnt <= one stage's loads,
            // expcnt and lgkmcnt not waited on)
            static_assert(P::LOADS < 16, "vmcnt field");
            __builtin_amdgcn_s_waitcnt(0x0F70 | P::LOADS);
        } else {
            __builtin_amdgcn_s_waitcnt(0);
        }
        __syncthreads();
        bf16x8_t a0[MI], b0[8], a1[MI], b1[8];
#pragma unroll
        for (int i = 0; i < MI; ++i) a0[i] = frag_a(smem, 0, i);
#pragma unroll
        for (int j = 0; j < 8; ++j) b0[j] = frag_b(smem + P::TILE_A, 0, j);

        for (int kt = 0; kt < nk; ++kt) {
            uint8_t *cur = smem + (size_t)(kt & 1) * P::STAGE;
            // phase A: k-slice 0 from registers, slice 1 read meanwhile
#pragma unroll
            for (int i = 0; i < MI; ++i) a1[i] = frag_a(cur, 1, i);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
#pragma unroll
                for (int i = 0; i < MI; ++i)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0[i], b0[j], acc[i][j], 0, 0, 0);
                b1[j] = frag_b(cur + P::TILE_A, 1, j);
            }
            // keep the reads between the MFMAs (mask 0x100: LDS reads, 0x008: MFMA)
            __builtin_amdgcn_sched_group_barrier(0x100, MI, 0);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                __builtin_amdgcn_sched_group_barrier(0x008, MI, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            // the next stage has landed and every wave is done reading this one
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            // phase B: slice 1 from registers; the next stage's slice-0 fragments read
            // (on the last step: stale, in-bounds LDS, never used) and this buffer
            // refilled with the stage after next (near the end: the last stage again,
            // in bounds, never read)
            const uint8_t *nx = smem + (size_t)((kt + 1) & 1) * P::STAGE;
#pragma unroll
            for (int i = 0; i < MI; ++i) a0[i] = frag_a(nx, 0, i);
            const int kc = kbk + min(kt + 2, nk - 1) * G2_BK;
            g2_copy<TM>(A, lda, M, m0, kc, cur, tid);
            g2_copy<G2N>(B, ldb, N, n0, kc, cur + P::TILE_A, tid);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
#pragma unroll
                for (int i = 0; i < MI; ++i)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1[i], b1[j], acc[i][j], 0, 0, 0);
                b0[j] = frag_b(nx + P::TILE_A, 0, j);
            }
            // mask 0x020: the direct-to-LDS loads, two at a time over the first B
            // fragments
            __builtin_amdgcn_sched_group_barrier(0x100, MI, 0);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                __builtin_amdgcn_sched_group_barrier(0x008, MI, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                if (j < P::LOADS / 2) __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);
                else if (j == P::LOADS / 2 && (P::LOADS & 1)) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            }
        }
        __builtin_amdgcn_s_waitcnt(0);  // the last copies land before the block's LDS is reused
        __syncthreads();                 // and every wave is done reading the last stage

        // Epilogue through LDS, one 16-row MFMA tile row (i) at a time: the wave
        // stages its 16 x 128 fp32 sums (accumulator layout: lane holds rows 4 lg +
        // r, column lr of each 16 x 16 tile) in its own padded rows, then each lane
        // takes 8 consecutive columns of a row, so that C (and the residual, and a
        // run's slot) move as 16-byte pieces of whole rows.
        constexpr int ER = 128 + 4;  // padded fp32 staging row
        float *es = reinterpret_cast<float *>(smem) + (size_t)wave * 16 * ER;
#pragma unroll
        for (int i = 0; i < MI; ++i) {
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) es[(4 * lg + r) * ER + 16 * j + lr] = acc[i][j][r];
            __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the wave's LDS writes are done
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int rl = 4 * c + lg, cl = 8 * lr;  // row within the tile row, first column
                const float4 lo = *reinterpret_cast<const float4 *>(es + rl * ER + cl);
                const float4 hi = *reinterpret_cast<const float4 *>(es + rl * ER + cl + 4);
                float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
                const int trow = wm * 16 * MI + i * 16 + rl, tcol = wn * 128 + cl;
                if (SPLIT && pslot != nullptr) {
                    // a run of the split tail: the whole 256 x 256 slot, row-major,
                    // edges included
                    store8(pslot + (size_t)trow * G2N + tcol, v);
                    continue;
                }
                const int row = m0 + trow, col = n0 + tcol;
                if (row >= M || col >= N) continue;  // N % 8 == 0: a piece is all in or all out
                if (RES) {
                    Raw8<bf16> rr;
                    rr.load(reinterpret_cast<const bf16 *>(R + (int64_t)row * ldr + col));
                    float rf[8];
                    rr.get(rf);
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[e] += rf[e];
                }
                store8(C + (int64_t)row * ldc + col, v);
            }
            __builtin_amdgcn_wave_barrier();  // the staging rows are rewritten for the next i
            __builtin_amdgcn_s_waitcnt(0xc07f);
        }
    };

    if (SPLIT && (int)blockIdx.x >= full) {
        // a tail block: units j U / nblk .. (j + 1) U / nblk - 1 of the tail's
        // (tile, stage) order, U = tail tiles x stages; shorter than a tile, so
        // at most the end of one tile and the start of the next
        const int64_t units = (int64_t)(nbm * nbn - full) * nk_all;
        const int j = blockIdx.x - full;
        const int64_t u0 = (int64_t)j * units / nblk, u1 = (int64_t)(j + 1) * units / nblk;
        const int ta = (int)(u0 / nk_all);
        const int64_t end_a = (int64_t)(ta + 1) * nk_all;
        int tm, tn;
        g2_order(full + ta, nbm, nbn, tm, tn);
        run(tm, tn, (int)(u0 - (int64_t)ta * nk_all), (int)(min(u1, end_a) - (int64_t)ta * nk_all),
            part + (size_t)(2 * j) * G2_SLOT);
        if (u1 > end_a) {
            __syncthreads();  // every wave is done with the first run's LDS
            g2_order(full + ta + 1, nbm, nbn, tm, tn);
            run(tm, tn, 0, (int)(u1 - end_a), part + (size_t)(2 * j + 1) * G2_SLOT);
        }
    } else {
        int tm, tn;
        g2_order(g2_deal(blockIdx.x, full), nbm, nbn, tm, tn);
        run(tm, tn, 0, nk_all, nullptr);
    }
}

// The split tail's tiles: the sum of the runs that cover a tile, in block
// order, plus the residual, to C.  Block: 16 rows of one tile; thread: 16
// columns.
template <typename TC, bool RES>
__global__ __launch_bounds__(256) void gemm_split_reduce_kernel(const float *__restrict__ part, int nblk,
                                                                int full, int nbm, int nbn, int nk,
                                                                TC *__restrict__ C, int64_t ldc,
                                                                const uint16_t *__restrict__ R, int64_t ldr,
                                                                int M, int N) {
    const int tt = blockIdx.x / 16;  // tail tile
    int tm, tn;
    g2_order(full + tt, nbm, nbn, tm, tn);
    const int rl = 16 * (blockIdx.x % 16) + (threadIdx.x >> 4), c0 = 16 * (threadIdx.x & 15);
    const int row = tm * G2N + rl;
    if (row >= M) return;
    const int64_t units = (int64_t)(nbm * nbn - full) * nk;
    const int64_t t0 = (int64_t)tt * nk, t1 = t0 + nk;  // the tile's units
    auto ustart = [&](int j) { return (int64_t)j * units / nblk; };
    // the block whose run holds unit t0, then every block that starts before t1
    int j = (int)(t0 * nblk / units);
    while (j > 0 && ustart(j) > t0) --j;
    while (ustart(j + 1) <= t0) ++j;
    float s[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) s[e] = 0.f;
    for (; j < nblk && ustart(j) < t1; ++j) {
        const int sg = ustart(j) / nk == tt ? 0 : 1;  // the tile is block j's first run or its second
        const float4 *q = reinterpret_cast<const float4 *>(part + (size_t)(2 * j + sg) * G2_SLOT +
                                                           (size_t)rl * G2N + c0);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const float4 f = q[v];
            s[4 * v] += f.x;
            s[4 * v + 1] += f.y;
            s[4 * v + 2] += f.z;
            s[4 * v + 3] += f.w;
        }
    }
    // two 8-column pieces (N % 8 == 0: a piece is all in or all out)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int col = tn * G2N + c0 + 8 * h;
        if (col >= N) continue;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = s[8 * h + e];
        if (RES) {
            Raw8<bf16> rr;
            rr.load(reinterpret_cast<const bf16 *>(R + (int64_t)row * ldr + col));
            float rf[8];
            rr.get(rf);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] += rf[e];
        }
        store8(C + (int64_t)row * ldc + col, v);
    }
}

template <int TM, typename TC, bool RES>
static hipError_t launch_gemm_v2(const GemmArgs &a, hipStream_t s) {
    static std::atomic<uint64_t> set{0};
    hipError_t e = set_smem_once(&gemm_bf16_v2_kernel<TM, TC, RES, false>, G2<TM>::SMEM, set);
    if (e != hipSuccess) return e;
    const int nb = ((a.M + TM - 1) / TM) * ((a.N + G2N - 1) / G2N);
    hipLaunchKernelGGL((gemm_bf16_v2_kernel<TM, TC, RES, false>), dim3(nb), dim3(G2_THREADS), G2<TM>::SMEM, s,
                       (const uint16_t *)a.A, a.lda, (const uint16_t *)a.B, a.ldb, (TC *)a.C, a.ldc,
                       (const uint16_t *)a.R, a.ldr, a.M, a.N, a.K, nb, 1, (float *)nullptr);
    return hipGetLastError();
}

// Compute units of the current device (cached per device).
static int device_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Tile rows for a shape: one tile per CU at a time, so the time goes as the
// rounds of tiles times the rows of a tile; 192-row tiles are taken only where
// that product is at least 8% below that of 256-row ones (they reuse each
// fragment read over fewer MFMAs).
static int g2_rows(const GemmArgs &a) {
    const int64_t cus = device_cus();
    const int64_t nbn = (a.N + G2N - 1) / G2N;
    auto cost = [&](int64_t tm) { return (((a.M + tm - 1) / tm) * nbn + cus - 1) / cus * tm; };
    return cost(192) * 100 <= cost(256) * 92 ? 192 : 256;
}

template <typename TC, bool RES>
static hipError_t launch_gemm_v2_any(const GemmArgs &a, hipStream_t s) {
    return g2_rows(a) == 192 ? launch_gemm_v2<192, TC, RES>(a, s) : launch_gemm_v2<256, TC, RES>(a, s);
}

// The split tail of a shape on the current device (256-row tiles): the tiles
// of the last, partly filled round (all tiles when there are fewer than CUs),
// dealt out to nblk blocks of at least G2_SPLIT_MIN stages each; nblk = 0: no
// split (a full last round, or no more blocks than tail tiles).
struct SplitPlan {
    int nbm, nbn, full, tail, nblk;
    size_t bytes;  // workspace: two fp32 run slots per block
};
static SplitPlan split_plan(int M, int N, int K) {
    SplitPlan p{};
    if (M <= 0 || N <= 0 || K <= 0 || K % G2_BK != 0) return p;
    const int cus = device_cus();
    p.nbm = (M + G2N - 1) / G2N;
    p.nbn = (N + G2N - 1) / G2N;
    const int nb = p.nbm * p.nbn, nk = K / G2_BK;
    p.tail = nb >= cus ? nb % cus : nb;
    p.full = nb - p.tail;
    const int64_t units = (int64_t)p.tail * nk;
    p.nblk = (int)std::min<int64_t>(cus, units / G2_SPLIT_MIN);
    if (p.tail == 0 || p.nblk <= p.tail) {
        p.nblk = 0;
        return p;
    }
    p.bytes = 2 * (size_t)p.nblk * G2_SLOT * sizeof(float);
    return p;
}

size_t gemm_bf16_workspace_bytes(int M, int N, int K) { return split_plan(M, N, K).bytes; }

template <typename TC, bool RES>
static hipError_t launch_gemm_split(const GemmArgs &a, const SplitPlan &p, hipStream_t s) {
    static std::atomic<uint64_t> set{0};
    hipError_t e = set_smem_once(&gemm_bf16_v2_kernel<G2N, TC, RES, true>, G2<G2N>::SMEM, set);
    if (e != hipSuccess) return e;
    float *part = static_cast<float *>(a.ws);
    hipLaunchKernelGGL((gemm_bf16_v2_kernel<G2N, TC, RES, true>), dim3(p.full + p.nblk),
                       dim3(G2_THREADS), G2<G2N>::SMEM, s, (const uint16_t *)a.A, a.lda, (const uint16_t *)a.B,
                       a.ldb, (TC *)a.C, a.ldc, (const uint16_t *)a.R, a.ldr, a.M, a.N, a.K, p.full, p.nblk, part);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((gemm_split_reduce_kernel<TC, RES>), dim3(p.tail * 16), dim3(256), 0, s,
                       (const float *)part, p.nblk, p.full, p.nbm, p.nbn, a.K / G2_BK, (TC *)a.C, a.ldc,
                       (const uint16_t *)a.R, a.ldr, a.M, a.N);
    return hipGetLastError();
}

static bool g2_ok(const GemmArgs &a) {
    auto al16 = [](const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
    return a.K > 0 && a.K % G2_BK == 0 && a.M > 0 && a.N > 0 && al16(a.A) && al16(a.B) && a.lda % 8 == 0 &&
           a.ldb % 8 == 0;
}

template <typename TC, bool RES>
static hipError_t launch_gemm_t(const GemmArgs &a, hipStream_t s) {
    dim3 grid((a.N + GBN - 1) / GBN, (a.M + GBM - 1) / GBM);
    hipLaunchKernelGGL((gemm_bf16_kernel<TC, RES>), grid, dim3(256), 0, s,
                       (const uint16_t *)a.A, a.lda, (const uint16_t *)a.B, a.ldb, (TC *)a.C, a.ldc,
                       (const uint16_t *)a.R, a.ldr, a.M, a.N, a.K);
    return hipGetLastError();
}

hipError_t launch_gemm_bf16(const GemmArgs &a, hipStream_t s) {
    if (g2_ok(a) && a.ws != nullptr) {
        const SplitPlan p = split_plan(a.M, a.N, a.K);
        if (p.nblk > 0 && a.ws_bytes >= p.bytes && (reinterpret_cast<uintptr_t>(a.ws) & 255) == 0) {
            if (a.c_bf16) return a.R ? launch_gemm_split<bf16, true>(a, p, s) : launch_gemm_split<bf16, false>(a, p, s);
            return a.R ? launch_gemm_split<float, true>(a, p, s) : launch_gemm_split<float, false>(a, p, s);
        }
    }
    if (g2_ok(a)) {
        if (a.c_bf16) return a.R ? launch_gemm_v2_any<bf16, true>(a, s) : launch_gemm_v2_any<bf16, false>(a, s);
        return a.R ? launch_gemm_v2_any<float, true>(a, s) : launch_gemm_v2_any<float, false>(a, s);
    }
    if (a.c_bf16)
        return a.R ? launch_gemm_t<bf16, true>(a, s) : launch_gemm_t<bf16, false>(a, s);
    return a.R ? launch_gemm_t<float, true>(a, s) : launch_gemm_t<float, false>(a, s);
}

}  // namespace gdn
