// Decode step of the gated delta rule: one token per request, the request's
// fp32 state slot streamed from HBM once and written back once.
//
// Update ("Qwen3.8-27B: from model structure to the vLLM inference dataflow",
// section 01 operator table, GDN row; section 08 evidence matrix: the error is
// read from the decayed state):
//   Sbar = alpha S;  e = v - Sbar k;  S' = Sbar + beta e k^T;  o = S' q / sqrt(d)
// Per state row s_i (value channel i) everything follows from two dot products
// taken on the same registers that hold the row:
//   p_i = s_i . k,  r_i = s_i . q
//   e_i = v_i - alpha p_i
//   s_i' = alpha s_i + (beta e_i) k
//   o_i = (alpha r_i + beta e_i (k . q)) / sqrt(d)
// so the kernel is a single read-modify-write pass over the state: HBM-bound at
// 2 * 4 * d * d bytes per (request, value head).
//
// Layout: a row of d fp32 values is owned by d/16 lanes, each holding 16
// columns as four float4 loads strided so that each group of d/16 lanes reads
// whole 128-byte lines per instruction; a thread owns 4 rows so 16 independent
// 16-byte loads are in flight before the first use.  For d = 128 one block of
// 256 threads is exactly one (request, value head) tile (64 KiB).
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

template <int D, typename TA, typename TG, typename TO>
__global__ __launch_bounds__(256) void decode_kernel(
    const TA *__restrict__ q, const TA *__restrict__ k, const TA *__restrict__ v,
    const TG *__restrict__ ga, const TG *__restrict__ gb, int64_t gate_ld,
    float *__restrict__ state, const int32_t *__restrict__ slots, int32_t R,
    int32_t Hk, int32_t Hv, TO *__restrict__ o) {
    constexpr int LPR = D / 16;            // lanes per state row
    constexpr int GROUPS = 256 / LPR;      // rows in flight per pass
    constexpr int RPT = 4;                 // passes (rows per thread)
    constexpr int ROWS_PER_BLOCK = GROUPS * RPT;
    const int l = threadIdx.x % LPR;
    const int grp = threadIdx.x / LPR;
    const int64_t total_rows = (int64_t)R * Hv * D;
    const int64_t row0 = (int64_t)blockIdx.x * ROWS_PER_BLOCK;
    const int group_sz = Hv / Hk;
    const float inv_sqrt_d = 1.0f / sqrtf((float)D);

    f32x4 s[RPT][4];
    int64_t sbase[RPT];
#pragma unroll
    for (int p = 0; p < RPT; ++p) {
        const int64_t g = row0 + (int64_t)p * GROUPS + grp;
        sbase[p] = -1;
#pragma unroll
        for (int m = 0; m < 4; ++m) s[p][m] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (g < total_rows) {
            const int64_t u = g / D;
            const int i = (int)(g % D);
            const int r = (int)(u / Hv);
            const int h = (int)(u % Hv);
            sbase[p] = (((int64_t)slots[r] * Hv + h) * D + i) * D + 4 * l;
#pragma unroll
            for (int m = 0; m < 4; ++m)
                s[p][m] = __builtin_nontemporal_load(
                    reinterpret_cast<const f32x4 *>(state + sbase[p] + 4 * LPR * m));
        }
    }

#pragma unroll
    for (int p = 0; p < RPT; ++p) {
        const int64_t g = row0 + (int64_t)p * GROUPS + grp;
        const bool valid = g < total_rows;
        const int64_t gg = valid ? g : 0;  // keep every lane in the reductions
        const int64_t u = gg / D;
        const int i = (int)(gg % D);
        const int r = (int)(u / Hv);
        const int h = (int)(u % Hv);
        const int kh = h / group_sz;
        const TA *kp = k + ((int64_t)r * Hk + kh) * D + 4 * l;
        const TA *qp = q + ((int64_t)r * Hk + kh) * D + 4 * l;
        float4 kc[4], qc[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            kc[m] = ld4(kp + 4 * LPR * m);
            qc[m] = ld4(qp + 4 * LPR * m);
        }
        float pk = 0.f, pq = 0.f, kq = 0.f;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const f32x4 sv = s[p][m];
            pk += sv.x * kc[m].x + sv.y * kc[m].y + sv.z * kc[m].z + sv.w * kc[m].w;
            pq += sv.x * qc[m].x + sv.y * qc[m].y + sv.z * qc[m].z + sv.w * qc[m].w;
            kq += kc[m].x * qc[m].x + kc[m].y * qc[m].y + kc[m].z * qc[m].z + kc[m].w * qc[m].w;
        }
        pk = group_sum<LPR>(pk);
        pq = group_sum<LPR>(pq);
        kq = group_sum<LPR>(kq);
        const float alpha = gate_alpha(ld(ga + (int64_t)r * gate_ld + h));
        const float beta = gate_beta(ld(gb + (int64_t)r * gate_ld + h));
        const float vi = ld(v + ((int64_t)r * Hv + h) * D + i);
        const float e = vi - alpha * pk;
        const float be = beta * e;
        const float oi = (alpha * pq + be * kq) * inv_sqrt_d;
        if (valid) {
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                f32x4 sv = s[p][m];
                sv.x = alpha * sv.x + be * kc[m].x;
                sv.y = alpha * sv.y + be * kc[m].y;
                sv.z = alpha * sv.z + be * kc[m].z;
                sv.w = alpha * sv.w + be * kc[m].w;
                __builtin_nontemporal_store(
                    sv, reinterpret_cast<f32x4 *>(state + sbase[p] + 4 * LPR * m));
            }
            if (l == 0) st(o + ((int64_t)r * Hv + h) * D + i, oi);
        }
    }
}

template <int D, typename TA, typename TG, typename TO>
static hipError_t launch_decode_t(const DecodeArgs &a, hipStream_t s) {
    constexpr int ROWS_PER_BLOCK = (256 / (D / 16)) * 4;
    const int64_t rows = (int64_t)a.R * a.Hv * D;
    const int64_t blocks = (rows + ROWS_PER_BLOCK - 1) / ROWS_PER_BLOCK;
    hipLaunchKernelGGL((decode_kernel<D, TA, TG, TO>), dim3((unsigned)blocks), dim3(256), 0, s,
                       (const TA *)a.q, (const TA *)a.k, (const TA *)a.v, (const TG *)a.a,
                       (const TG *)a.b, a.gate_ld, a.state, a.slots, a.R, a.Hk, a.Hv,
                       (TO *)a.o);
    return hipGetLastError();
}

template <int D, typename TA, typename TG>
static hipError_t launch_decode_o(const DecodeArgs &a, hipStream_t s) {
    return a.o_bf16 ? launch_decode_t<D, TA, TG, bf16>(a, s) : launch_decode_t<D, TA, TG, float>(a, s);
}
template <int D, typename TA>
static hipError_t launch_decode_g(const DecodeArgs &a, hipStream_t s) {
    return a.gate_bf16 ? launch_decode_o<D, TA, bf16>(a, s) : launch_decode_o<D, TA, float>(a, s);
}
template <int D>
static hipError_t launch_decode_a(const DecodeArgs &a, hipStream_t s) {
    return a.act_bf16 ? launch_decode_g<D, bf16>(a, s) : launch_decode_g<D, float>(a, s);
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t s) {
    switch (a.D) {
        case 16: return launch_decode_a<16>(a, s);
        case 32: return launch_decode_a<32>(a, s);
        case 64: return launch_decode_a<64>(a, s);
        case 128: return launch_decode_a<128>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn
