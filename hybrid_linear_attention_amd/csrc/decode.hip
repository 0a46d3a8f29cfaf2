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
// Layout: a row of d fp32 values is owned by d/8 lanes, each holding 8 columns
// as two float4 loads strided so that each group of d/8 lanes reads whole
// 128-byte lines per instruction; a thread owns one row and a 256-thread block
// 2048/d rows (d = 128: 16 rows of one (request, head) tile, 24576 blocks for
// 64 requests x 48 heads).  State loads and stores are nontemporal: the state
// is touched once per step and must not displace reusable lines.  This shape
// was the fastest of the row/lane/block splits measured on MI355X with a state
// that is not resident in the memory-side cache.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

template <int D, typename TA, typename TG, typename TO>
__global__ __launch_bounds__(256) void decode_kernel(
    const TA *__restrict__ q, const TA *__restrict__ k, const TA *__restrict__ v,
    const TG *__restrict__ ga, const TG *__restrict__ gb, int64_t gate_ld,
    float *__restrict__ state, const int32_t *__restrict__ slots, int32_t R,
    int32_t Hk, int32_t Hv, TO *__restrict__ o) {
    constexpr int LPR = D / 8;             // lanes per state row
    constexpr int NF = 2;                  // float4 per lane per row
    constexpr int ROWS = 256 / LPR;        // rows per block
    // When d is a multiple of the rows per block, every row of a block belongs
    // to one (request, head) unit: derive it from blockIdx alone so the slot and
    // gate lookups are uniform (scalar) loads that issue before the state loads.
    constexpr bool UNIFORM = (D % ROWS) == 0;
    const int l = threadIdx.x % LPR;
    const int64_t g = (int64_t)blockIdx.x * ROWS + threadIdx.x / LPR;  // global row
    const int64_t total_rows = (int64_t)R * Hv * D;
    const bool valid = UNIFORM || g < total_rows;
    int u, i;  // (request, head) unit (R * Hv < 2^31) and row within it
    if constexpr (UNIFORM) {
        const int64_t g0 = (int64_t)blockIdx.x * ROWS;
        u = (int)(g0 / D);
        i = (int)(g0 % D) + threadIdx.x / LPR;
    } else {
        const int64_t gg = valid ? g : 0;  // keep every lane in the reductions
        u = (int)(gg / D);
        i = (int)(gg % D);
    }
    const int r = u / Hv;
    const int h = u - r * Hv;
    const int kh = h / (Hv / Hk);

    const int64_t sbase = (((int64_t)slots[r] * Hv + h) * D + i) * D + 4 * l;
    f32x4 s[NF];
#pragma unroll
    for (int m = 0; m < NF; ++m) {
        s[m] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (valid)
            s[m] = __builtin_nontemporal_load(
                reinterpret_cast<const f32x4 *>(state + sbase + 4 * LPR * m));
    }
    const TA *kp = k + ((int64_t)r * Hk + kh) * D + 4 * l;
    const TA *qp = q + ((int64_t)r * Hk + kh) * D + 4 * l;
    float4 kc[NF], qc[NF];
#pragma unroll
    for (int m = 0; m < NF; ++m) {
        kc[m] = ld4(kp + 4 * LPR * m);
        qc[m] = ld4(qp + 4 * LPR * m);
    }
    const float alpha = gate_alpha(ld(ga + (int64_t)r * gate_ld + h));
    const float beta = gate_beta(ld(gb + (int64_t)r * gate_ld + h));
    const float vi = ld(v + ((int64_t)r * Hv + h) * D + i);

    float pk = 0.f, pq = 0.f, kq = 0.f;
#pragma unroll
    for (int m = 0; m < NF; ++m) {
        const f32x4 sv = s[m];
        pk += sv.x * kc[m].x + sv.y * kc[m].y + sv.z * kc[m].z + sv.w * kc[m].w;
        pq += sv.x * qc[m].x + sv.y * qc[m].y + sv.z * qc[m].z + sv.w * qc[m].w;
        kq += kc[m].x * qc[m].x + kc[m].y * qc[m].y + kc[m].z * qc[m].z + kc[m].w * qc[m].w;
    }
    pk = group_sum<LPR>(pk);
    pq = group_sum<LPR>(pq);
    kq = group_sum<LPR>(kq);
    const float e = vi - alpha * pk;
    const float be = beta * e;
    if (valid) {
#pragma unroll
        for (int m = 0; m < NF; ++m) {
            f32x4 sv = s[m];
            sv.x = alpha * sv.x + be * kc[m].x;
            sv.y = alpha * sv.y + be * kc[m].y;
            sv.z = alpha * sv.z + be * kc[m].z;
            sv.w = alpha * sv.w + be * kc[m].w;
            __builtin_nontemporal_store(sv, reinterpret_cast<f32x4 *>(state + sbase + 4 * LPR * m));
        }
        if (l == 0)
            st(o + ((int64_t)r * Hv + h) * D + i, (alpha * pq + be * kq) * (1.0f / sqrtf((float)D)));
    }
}

template <int D, typename TA, typename TG, typename TO>
static hipError_t launch_decode_t(const DecodeArgs &a, hipStream_t s) {
    constexpr int ROWS_PER_BLOCK = 256 / (D / 8);
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
