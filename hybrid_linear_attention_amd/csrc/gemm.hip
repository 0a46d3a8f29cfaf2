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

template <typename TC, bool RES>
static hipError_t launch_gemm_t(const GemmArgs &a, hipStream_t s) {
    dim3 grid((a.N + GBN - 1) / GBN, (a.M + GBM - 1) / GBM);
    hipLaunchKernelGGL((gemm_bf16_kernel<TC, RES>), grid, dim3(256), 0, s,
                       (const uint16_t *)a.A, a.lda, (const uint16_t *)a.B, a.ldb, (TC *)a.C, a.ldc,
                       (const uint16_t *)a.R, a.ldr, a.M, a.N, a.K);
    return hipGetLastError();
}

hipError_t launch_gemm_bf16(const GemmArgs &a, hipStream_t s) {
    if (a.c_bf16)
        return a.R ? launch_gemm_t<bf16, true>(a, s) : launch_gemm_t<bf16, false>(a, s);
    return a.R ? launch_gemm_t<float, true>(a, s) : launch_gemm_t<float, false>(a, s);
}

}  // namespace gdn
