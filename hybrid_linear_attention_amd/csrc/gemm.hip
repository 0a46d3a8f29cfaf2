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
// through a two-stage LDS ring filled by direct-to-LDS 16-byte loads.  A wave
// tile of 64 x 128 reads 12 fragments per 32 MFMAs, which keeps the LDS well
// below its bandwidth at full MFMA rate.  LDS rows are 128 bytes (64 bf16) with
// the 16-byte chunk index XOR-swizzled by row (chunk j of row r stored at
// j ^ (r & 7)), so the 16 rows of a fragment read fall in different banks; the
// swizzle is applied on the global side because a direct-to-LDS load places
// lane l's bytes at base + 16 l.
// ---------------------------------------------------------------------------
constexpr int G2M = 256, G2N = 256;
constexpr int G2_THREADS = 512;

// one operand tile of 256 rows x BK bf16: rows of 2 BK bytes, 16-byte chunk j
// of row r stored at chunk j ^ (r & (BK / 8 - 1))
template <int BK>
__device__ __forceinline__ void g2_copy(const uint16_t *__restrict__ X, int64_t ld, int rows_valid,
                                        int row0, int k0, uint8_t *tile, int tid) {
    constexpr int CPR = BK / 8;                      // 16-byte chunks per row
    constexpr int PIECES = G2M * CPR;                // per tile
    constexpr int PER_THREAD = PIECES / G2_THREADS;
    const int wv = tid >> 6, lane = tid & 63;
#pragma unroll
    for (int m = 0; m < PER_THREAD; ++m) {
        const int s = (m * 8 + wv) * 64 + lane;  // wave-contiguous LDS pieces
        const int r = s / CPR;
        const int j = (s % CPR) ^ (r & (CPR - 1));
        const int rr = min(row0 + r, rows_valid - 1);  // rows past the edge load a valid row, never stored
        const uint16_t *src = X + (int64_t)rr * ld + k0 + 8 * j;
        __builtin_amdgcn_global_load_lds(static_cast<const void *>(src),
                                         (__attribute__((address_space(3))) void *)(tile + (size_t)(m * 8 + wv) * 1024),
                                         16, 0, 0);
    }
}

template <typename TC, bool RES, int BK, int NST>
__global__ __launch_bounds__(G2_THREADS) void gemm_bf16_v2_kernel(
    const uint16_t *__restrict__ A, int64_t lda, const uint16_t *__restrict__ B, int64_t ldb,
    TC *__restrict__ C, int64_t ldc, const uint16_t *__restrict__ R, int64_t ldr, int M, int N,
    int K) {
    constexpr int CPR = BK / 8;
    constexpr size_t TILE = (size_t)G2M * BK * 2;
    constexpr size_t STAGE = 2 * TILE;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;  // 4 x 2 waves: rows 64 wm, columns 128 wn
    const int lr = lane & 15, lg = lane >> 4;
    // XCD-aware tile order: the 8 XCDs take contiguous runs of tiles
    const int nbn = (N + G2N - 1) / G2N, nbm = (M + G2M - 1) / G2M;
    const int nb = nbn * nbm;
    int bid = blockIdx.x;
    if (nb % 8 == 0) bid = (bid % 8) * (nb / 8) + bid / 8;
    const int m0 = (bid / nbn) * G2M, n0 = (bid % nbn) * G2N;

    floatx4_t acc[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};

    const int nk = K / BK;
    // NST - 1 k-steps in flight ahead of the one being multiplied
#pragma unroll
    for (int p = 0; p < NST - 1; ++p)
        if (p < nk) {
            g2_copy<BK>(A, lda, M, m0, p * BK, smem + (size_t)p * STAGE, tid);
            g2_copy<BK>(B, ldb, N, n0, p * BK, smem + (size_t)p * STAGE + TILE, tid);
        }
    for (int kt = 0; kt < nk; ++kt) {
        const uint8_t *cur = smem + (size_t)(kt % NST) * STAGE;
        // wait until only the copies of the later NST - 2 k-steps are outstanding
        // (each k-step is BK / 8 load instructions per thread; loads complete in
        // order); near the end fewer are in flight, so wait for all
        constexpr int ALLOWED = (NST - 2) * (BK / 8);
        constexpr int VMCNT_ENC = 0x0F70 | (ALLOWED & 15) | ((ALLOWED >> 4) << 14);  // expcnt, lgkmcnt: no wait
        static_assert(ALLOWED < 64, "vmcnt range");
        if (NST == 2 || kt + NST - 2 >= nk) __builtin_amdgcn_s_waitcnt(0);
        else __builtin_amdgcn_s_waitcnt(VMCNT_ENC);
        __syncthreads();  // stage kt landed; every wave is done with the stage refilled next
        if (kt + NST - 1 < nk) {
            uint8_t *nxt = smem + (size_t)((kt + NST - 1) % NST) * STAGE;
            g2_copy<BK>(A, lda, M, m0, (kt + NST - 1) * BK, nxt, tid);
            g2_copy<BK>(B, ldb, N, n0, (kt + NST - 1) * BK, nxt + TILE, tid);
        }
        const uint8_t *At = cur, *Bt = cur + TILE;
#pragma unroll
        for (int ks = 0; ks < BK / 32; ++ks) {
            // fragment: row lr of a 16-row tile, logical chunk 4 ks + lg (8 bf16)
            bf16x8_t af[4], bfr[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = wm * 64 + i * 16 + lr;
                const int pc = (4 * ks + lg) ^ (r & (CPR - 1));
                af[i] = *reinterpret_cast<const bf16x8_t *>(At + (size_t)r * (2 * BK) + 16 * pc);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int r = wn * 128 + j * 16 + lr;
                const int pc = (4 * ks + lg) ^ (r & (CPR - 1));
                bfr[j] = *reinterpret_cast<const bf16x8_t *>(Bt + (size_t)r * (2 * BK) + 16 * pc);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
    }

    // accumulator layout: lane holds rows 4 lg + r, column lr of each tile
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int col = n0 + wn * 128 + j * 16 + lr;
            if (col >= N) continue;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = m0 + wm * 64 + i * 16 + 4 * lg + r;
                if (row >= M) continue;
                float val = acc[i][j][r];
                if (RES) val += __uint_as_float(uint32_t(R[(int64_t)row * ldr + col]) << 16);
                st(C + (int64_t)row * ldc + col, val);
            }
        }
}

constexpr int G2_BK = 64, G2_NST = 2;  // K step and pipeline stages of the 256 x 256 kernel

template <typename TC, bool RES>
static hipError_t launch_gemm_v2(const GemmArgs &a, hipStream_t s) {
    constexpr size_t smem = (size_t)G2_NST * 2 * G2M * G2_BK * 2;
    static bool set = false;
    if (!set) {
        hipError_t e = hipFuncSetAttribute(
            reinterpret_cast<const void *>(&gemm_bf16_v2_kernel<TC, RES, G2_BK, G2_NST>),
            hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        if (e != hipSuccess) return e;
        set = true;
    }
    const int nb = ((a.M + G2M - 1) / G2M) * ((a.N + G2N - 1) / G2N);
    hipLaunchKernelGGL((gemm_bf16_v2_kernel<TC, RES, G2_BK, G2_NST>), dim3(nb), dim3(G2_THREADS), smem, s,
                       (const uint16_t *)a.A, a.lda, (const uint16_t *)a.B, a.ldb, (TC *)a.C, a.ldc,
                       (const uint16_t *)a.R, a.ldr, a.M, a.N, a.K);
    return hipGetLastError();
}

static bool g2_ok(const GemmArgs &a) {
    auto al16 = [](const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
    return a.K % G2_BK == 0 && a.M > 0 && a.N > 0 && al16(a.A) && al16(a.B) && a.lda % 8 == 0 &&
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
    if (g2_ok(a)) {
        if (a.c_bf16) return a.R ? launch_gemm_v2<bf16, true>(a, s) : launch_gemm_v2<bf16, false>(a, s);
        return a.R ? launch_gemm_v2<float, true>(a, s) : launch_gemm_v2<float, false>(a, s);
    }
    if (a.c_bf16)
        return a.R ? launch_gemm_t<bf16, true>(a, s) : launch_gemm_t<bf16, false>(a, s);
    return a.R ? launch_gemm_t<float, true>(a, s) : launch_gemm_t<float, false>(a, s);
}

}  // namespace gdn
