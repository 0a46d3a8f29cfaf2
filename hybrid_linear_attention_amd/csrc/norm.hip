// Row normalisations of the GDN layer block, both HBM-bound single passes.
//
// gated_norm: Ogate = RMSNorm(o) * SiLU(Z) per (token, value head) over d_v
//   ("Qwen3.8-27B: from model structure to the vLLM inference dataflow",
//   section 01 operator table, gated-output row, [T,48,128] -> [T,6144]; the
//   GDN output gate is SiLU applied after the RMSNorm, section 08 evidence
//   matrix).  d_v/2 lanes own one head row, two elements per lane.
// rmsnorm: U = X / sqrt(mean(X^2) + eps) * gamma (operator table, first row),
//   one block per row, 8 elements per 16-byte access.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

template <int D, typename TO, typename TZ, typename TG, typename TY>
__global__ __launch_bounds__(256) void gated_norm_kernel(
    const TO *__restrict__ o, const TZ *__restrict__ z, int64_t z_ld,
    const TG *__restrict__ gamma, float eps, int32_t T, int32_t Hv,
    TY *__restrict__ y) {
    constexpr int LPR = D / 2;
    constexpr int ROWS = 256 / LPR;
    const int l = threadIdx.x % LPR;
    const int row = blockIdx.x * ROWS + threadIdx.x / LPR;  // T * Hv < 2^31
    const bool valid = row < T * Hv;
    const int rr = valid ? row : 0;
    const int t = rr / Hv;
    const int h = rr - t * Hv;
    const int j = 2 * l;
    float2 ov = make_float2(0.f, 0.f), zv = ov;
    if (valid) {
        ov = ld2(o + (int64_t)rr * D + j);
        zv = ld2(z + (int64_t)t * z_ld + h * D + j);
    }
    const float ss = group_sum<LPR>(ov.x * ov.x + ov.y * ov.y);
    const float inv = 1.0f / sqrtf(ss * (1.0f / D) + eps);
    if (valid) {
        const float2 g = ld2(gamma + j);
        st2(y + (int64_t)rr * D + j, ov.x * inv * g.x * silu_f(zv.x), ov.y * inv * g.y * silu_f(zv.y));
    }
}

// Vectorised gated norm: D / 8 lanes per (token, value head) row, 8 elements
// per lane as 16-byte accesses, and R rows per thread whose loads are all issued
// before the first reduction.
template <int D, int R, typename TO, typename TZ, typename TG, typename TY>
__global__ __launch_bounds__(256) void gated_norm_vec_kernel(
    const TO *__restrict__ o, const TZ *__restrict__ z, int64_t z_ld,
    const TG *__restrict__ gamma, float eps, int32_t T, int32_t Hv, TY *__restrict__ y) {
    constexpr int LPR = D / 8;
    constexpr int RPB = 256 / LPR;  // rows per pass of the block
    const int l = threadIdx.x % LPR;
    const int64_t rows = (int64_t)T * Hv;
    const int64_t row0 = (int64_t)blockIdx.x * RPB * R + threadIdx.x / LPR;
    Raw8<TO> ov[R];
    Raw8<TZ> zv[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const int64_t row = row0 + (int64_t)i * RPB;
        if (row < rows) {
            const int64_t t = row / Hv;
            const int h = (int)(row - t * Hv);
            ov[i].load(o + row * D + 8 * l);
            zv[i].load(z + t * z_ld + (int64_t)h * D + 8 * l);
        } else {
            ov[i].zero();
            zv[i].zero();
        }
    }
    float g[8];
    {
        Raw8<TG> gr;
        gr.load(gamma + 8 * l);
        gr.get(g);
    }
#pragma unroll
    for (int i = 0; i < R; ++i) {
        float of[8], zf[8];
        ov[i].get(of);
        zv[i].get(zf);
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += of[e] * of[e];
        ss = group_sum<LPR>(ss);
        const float inv = 1.0f / sqrtf(ss * (1.0f / D) + eps);
        const int64_t row = row0 + (int64_t)i * RPB;
        if (row < rows) {
            float out[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) out[e] = of[e] * inv * g[e] * silu_f(zf[e]);
            store8(y + row * D + 8 * l, out);
        }
    }
}

template <typename T> struct Vec8;
template <> struct Vec8<float> {
    static __device__ __forceinline__ void load(const float *p, float *f) {
        float4 a = ld4(p), b = ld4(p + 4);
        f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
        f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
    }
    static __device__ __forceinline__ void store(float *p, const float *f) {
        *reinterpret_cast<float4 *>(p) = make_float4(f[0], f[1], f[2], f[3]);
        *reinterpret_cast<float4 *>(p + 4) = make_float4(f[4], f[5], f[6], f[7]);
    }
};
template <> struct Vec8<bf16> {
    static __device__ __forceinline__ void load(const bf16 *p, float *f) {
        uint4 u = *reinterpret_cast<const uint4 *>(p);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(w[i] << 16);
            f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
    static __device__ __forceinline__ void store(bf16 *p, const float *f) {
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            w[i] = uint32_t(to_bf16(f[2 * i]).bits) | (uint32_t(to_bf16(f[2 * i + 1]).bits) << 16);
        *reinterpret_cast<uint4 *>(p) = make_uint4(w[0], w[1], w[2], w[3]);
    }
};

constexpr int RMS_THREADS = 256;
constexpr int RMS_MAX_VEC = 8;  // up to 256 * 8 * 8 = 16384 columns

// VEC: 8-element vectors per thread, the fewest that cover the row (the row
// stays in registers between the sum of squares and the scaling, and a smaller
// VEC keeps more blocks resident)
template <typename TX, typename TG, typename TY, int VEC>
__global__ __launch_bounds__(RMS_THREADS) void rmsnorm_kernel(
    const TX *__restrict__ x, const TG *__restrict__ gamma, float eps, int32_t cols,
    TY *__restrict__ y) {
    __shared__ float part[RMS_THREADS / 64];
    const int64_t row = blockIdx.x;
    const int nvec = cols / 8;
    float buf[VEC][8];
    float ss = 0.f;
#pragma unroll
    for (int it = 0; it < VEC; ++it) {
        const int vi = it * RMS_THREADS + threadIdx.x;
        if (vi < nvec) {
            Vec8<TX>::load(x + row * cols + vi * 8, buf[it]);
#pragma unroll
            for (int e = 0; e < 8; ++e) ss += buf[it][e] * buf[it][e];
        }
    }
    ss = group_sum<64>(ss);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < RMS_THREADS / 64; ++w) tot += part[w];
    const float inv = 1.0f / sqrtf(tot / (float)cols + eps);
#pragma unroll
    for (int it = 0; it < VEC; ++it) {
        const int vi = it * RMS_THREADS + threadIdx.x;
        if (vi < nvec) {
            float g[8], out[8];
            Vec8<TG>::load(gamma + vi * 8, g);
#pragma unroll
            for (int e = 0; e < 8; ++e) out[e] = buf[it][e] * inv * g[e];
            Vec8<TY>::store(y + row * cols + vi * 8, out);
        }
    }
}

static bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

template <int D, int R, typename TO, typename TZ, typename TG, typename TY>
static hipError_t launch_gn_vec(const GatedNormArgs &a, hipStream_t s) {
    constexpr int RPB = 256 / (D / 8);
    const int64_t rows = (int64_t)a.T * a.Hv;
    hipLaunchKernelGGL((gated_norm_vec_kernel<D, R, TO, TZ, TG, TY>),
                       dim3((unsigned)((rows + RPB * R - 1) / (RPB * R))), dim3(256), 0, s,
                       (const TO *)a.o, (const TZ *)a.z, a.z_ld, (const TG *)a.gamma, a.eps, a.T,
                       a.Hv, (TY *)a.y);
    return hipGetLastError();
}

template <int D, typename TO, typename TZ, typename TG, typename TY>
static hipError_t launch_gn_t(const GatedNormArgs &a, hipStream_t s) {
    constexpr int ROWS = 256 / (D / 2);
    const int64_t rows = (int64_t)a.T * a.Hv;
    // 16-byte aligned rows take the vectorised kernel (4 rows per thread once
    // there are enough rows to fill the chip)
    if (a.z_ld % (16 / sizeof(TZ)) == 0 && aligned16(a.o) && aligned16(a.z) &&
        aligned16(a.gamma) && aligned16(a.y))
        return rows >= (int64_t)1 << 18 ? launch_gn_vec<D, 4, TO, TZ, TG, TY>(a, s)
                                         : launch_gn_vec<D, 1, TO, TZ, TG, TY>(a, s);
    hipLaunchKernelGGL((gated_norm_kernel<D, TO, TZ, TG, TY>), dim3((unsigned)((rows + ROWS - 1) / ROWS)),
                       dim3(256), 0, s, (const TO *)a.o, (const TZ *)a.z, a.z_ld,
                       (const TG *)a.gamma, a.eps, a.T, a.Hv, (TY *)a.y);
    return hipGetLastError();
}
template <int D, typename TO, typename TZ, typename TG>
static hipError_t launch_gn_y(const GatedNormArgs &a, hipStream_t s) {
    return a.y_bf16 ? launch_gn_t<D, TO, TZ, TG, bf16>(a, s) : launch_gn_t<D, TO, TZ, TG, float>(a, s);
}
template <int D, typename TO, typename TZ>
static hipError_t launch_gn_g(const GatedNormArgs &a, hipStream_t s) {
    return a.gamma_bf16 ? launch_gn_y<D, TO, TZ, bf16>(a, s) : launch_gn_y<D, TO, TZ, float>(a, s);
}
template <int D, typename TO>
static hipError_t launch_gn_z(const GatedNormArgs &a, hipStream_t s) {
    return a.z_bf16 ? launch_gn_g<D, TO, bf16>(a, s) : launch_gn_g<D, TO, float>(a, s);
}
template <int D>
static hipError_t launch_gn_o(const GatedNormArgs &a, hipStream_t s) {
    return a.o_bf16 ? launch_gn_z<D, bf16>(a, s) : launch_gn_z<D, float>(a, s);
}

hipError_t launch_gated_norm(const GatedNormArgs &a, hipStream_t s) {
    switch (a.D) {
        case 16: return launch_gn_o<16>(a, s);
        case 32: return launch_gn_o<32>(a, s);
        case 64: return launch_gn_o<64>(a, s);
        case 128: return launch_gn_o<128>(a, s);
        default: return hipErrorInvalidValue;
    }
}

template <typename TX, typename TG, typename TY, int VEC>
static hipError_t launch_rms_v(const RmsNormArgs &a, hipStream_t s) {
    hipLaunchKernelGGL((rmsnorm_kernel<TX, TG, TY, VEC>), dim3(a.rows), dim3(RMS_THREADS), 0, s,
                       (const TX *)a.x, (const TG *)a.gamma, a.eps, a.cols, (TY *)a.y);
    return hipGetLastError();
}
template <typename TX, typename TG, typename TY>
static hipError_t launch_rms_t(const RmsNormArgs &a, hipStream_t s) {
    const int per = (a.cols / 8 + RMS_THREADS - 1) / RMS_THREADS;  // vectors per thread
    if (per <= 1) return launch_rms_v<TX, TG, TY, 1>(a, s);
    if (per <= 2) return launch_rms_v<TX, TG, TY, 2>(a, s);
    if (per <= 3) return launch_rms_v<TX, TG, TY, 3>(a, s);
    if (per <= 4) return launch_rms_v<TX, TG, TY, 4>(a, s);
    static_assert(RMS_MAX_VEC == 8, "widest row");
    return launch_rms_v<TX, TG, TY, 8>(a, s);
}
template <typename TX, typename TG>
static hipError_t launch_rms_y(const RmsNormArgs &a, hipStream_t s) {
    return a.y_bf16 ? launch_rms_t<TX, TG, bf16>(a, s) : launch_rms_t<TX, TG, float>(a, s);
}
template <typename TX>
static hipError_t launch_rms_g(const RmsNormArgs &a, hipStream_t s) {
    return a.gamma_bf16 ? launch_rms_y<TX, bf16>(a, s) : launch_rms_y<TX, float>(a, s);
}

hipError_t launch_rmsnorm(const RmsNormArgs &a, hipStream_t s) {
    return a.x_bf16 ? launch_rms_g<bf16>(a, s) : launch_rms_g<float>(a, s);
}

}  // namespace gdn
