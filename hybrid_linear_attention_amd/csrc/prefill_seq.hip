// Sequential-in-time prefill of the gated delta rule for any supported head
// dim: each (request, value head) state lives in registers for the whole
// request and every token applies the decode-step update
//   Sbar = alpha S;  e = v - Sbar k;  S = Sbar + beta e k^T;  o = S q / sqrt(d)
// ("Qwen3.8-27B: from model structure to the vLLM inference dataflow",
// section 01 operator table, GDN row).  Used for d < 128, where a chunked
// tensor-core form would be all padding, and as the reference-shaped path for
// short requests.
//
// A unit of d x d state is owned by d^2/64 threads: d/16 lanes per row, each
// holding 16 columns; each thread owns 4 rows of the unit.  16384/d^2 units
// share a 256-thread block (d = 128: one unit per block).
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

template <int D, typename TA, typename TG, typename TO, typename TS>
__global__ __launch_bounds__(256) void prefill_seq_kernel(
    const TA *__restrict__ q, const TA *__restrict__ k, const TA *__restrict__ v,
    const TG *__restrict__ ga, const TG *__restrict__ gb, int64_t gate_ld,
    TS *__restrict__ state, const int32_t *__restrict__ qsl,
    const int32_t *__restrict__ slots, const uint8_t *__restrict__ has_init, int32_t nreq,
    int32_t Hk, int32_t Hv, TO *__restrict__ o, const int32_t *__restrict__ snap_slots,
    int32_t snap_interval, int32_t max_snaps) {
    constexpr int LPR = D / 16;
    constexpr int RPT = 4;
    constexpr int RG = D / RPT;                   // row groups per unit
    constexpr int TPU = RG * LPR;                 // threads per unit
    constexpr int UPB = 256 / TPU;                // units per block
    const int ul = threadIdx.x / TPU;
    const int w = threadIdx.x % TPU;
    const int l = w % LPR;
    const int rg = w / LPR;
    const int64_t unit = (int64_t)blockIdx.x * UPB + ul;
    if (unit >= (int64_t)nreq * Hv) return;
    const int r = (int)(unit / Hv);
    const int h = (int)(unit % Hv);
    const int kh = h / (Hv / Hk);
    const int t0 = qsl[r], t1 = qsl[r + 1];
    if (t1 <= t0) return;  // empty request: slot untouched
    const bool hi = has_init == nullptr || has_init[r] != 0;
    TS *sp = state + ((int64_t)slots[r] * Hv + h) * D * D;
    const float inv_sqrt_d = 1.0f / sqrtf((float)D);

    float4 s[RPT][4];
#pragma unroll
    for (int p = 0; p < RPT; ++p) {
        const int i = rg + p * RG;
#pragma unroll
        for (int m = 0; m < 4; ++m)
            s[p][m] = hi ? ld4(sp + (int64_t)i * D + 4 * l + 4 * LPR * m)
                         : make_float4(0.f, 0.f, 0.f, 0.f);
    }

    for (int t = t0; t < t1; ++t) {
        const TA *kp = k + ((int64_t)t * Hk + kh) * D + 4 * l;
        const TA *qp = q + ((int64_t)t * Hk + kh) * D + 4 * l;
        float4 kc[4], qc[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            kc[m] = ld4(kp + 4 * LPR * m);
            qc[m] = ld4(qp + 4 * LPR * m);
        }
        float kq = 0.f;
#pragma unroll
        for (int m = 0; m < 4; ++m)
            kq += kc[m].x * qc[m].x + kc[m].y * qc[m].y + kc[m].z * qc[m].z + kc[m].w * qc[m].w;
        kq = group_sum<LPR>(kq);
        const float alpha = gate_alpha(ld(ga + (int64_t)t * gate_ld + h));
        const float beta = gate_beta(ld(gb + (int64_t)t * gate_ld + h));
#pragma unroll
        for (int p = 0; p < RPT; ++p) {
            const int i = rg + p * RG;
            float pk = 0.f, pq = 0.f;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const float4 sv = s[p][m];
                pk += sv.x * kc[m].x + sv.y * kc[m].y + sv.z * kc[m].z + sv.w * kc[m].w;
                pq += sv.x * qc[m].x + sv.y * qc[m].y + sv.z * qc[m].z + sv.w * qc[m].w;
            }
            pk = group_sum<LPR>(pk);
            pq = group_sum<LPR>(pq);
            const float vi = ld(v + ((int64_t)t * Hv + h) * D + i);
            const float e = vi - alpha * pk;
            const float be = beta * e;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                s[p][m].x = alpha * s[p][m].x + be * kc[m].x;
                s[p][m].y = alpha * s[p][m].y + be * kc[m].y;
                s[p][m].z = alpha * s[p][m].z + be * kc[m].z;
                s[p][m].w = alpha * s[p][m].w + be * kc[m].w;
            }
            if (l == 0) st(o + ((int64_t)t * Hv + h) * D + i, (alpha * pq + be * kq) * inv_sqrt_d);
        }
        // prefix-cache snapshot after every snap_interval tokens of the request
        const int done = t - t0 + 1;
        if (snap_slots != nullptr && done % snap_interval == 0 && done / snap_interval <= max_snaps) {
            TS *snp = state + ((int64_t)snap_slots[(int64_t)r * max_snaps + done / snap_interval - 1] * Hv + h) * D * D;
#pragma unroll
            for (int p = 0; p < RPT; ++p)
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    st4(snp + (int64_t)(rg + p * RG) * D + 4 * l + 4 * LPR * m, s[p][m]);
        }
    }
#pragma unroll
    for (int p = 0; p < RPT; ++p) {
        const int i = rg + p * RG;
#pragma unroll
        for (int m = 0; m < 4; ++m)
            st4(sp + (int64_t)i * D + 4 * l + 4 * LPR * m, s[p][m]);
    }
}

template <int D, typename TA, typename TG, typename TO, typename TS>
static hipError_t launch_seq_t(const PrefillArgs &a, hipStream_t s) {
    constexpr int UPB = 16384 / (D * D);
    const int64_t units = (int64_t)a.nreq * a.Hv;
    hipLaunchKernelGGL((prefill_seq_kernel<D, TA, TG, TO, TS>), dim3((unsigned)((units + UPB - 1) / UPB)),
                       dim3(256), 0, s, (const TA *)a.q, (const TA *)a.k, (const TA *)a.v,
                       (const TG *)a.a, (const TG *)a.b, a.gate_ld, (TS *)a.state, a.qsl, a.slots,
                       a.has_init, a.nreq, a.Hk, a.Hv, (TO *)a.o,
                       a.max_snaps > 0 ? a.snap_slots : nullptr, a.max_snaps > 0 ? a.snap_interval : 1,
                       a.max_snaps);
    return hipGetLastError();
}
template <int D, typename TA, typename TG, typename TO>
static hipError_t launch_seq_s(const PrefillArgs &a, hipStream_t s) {
    return a.state_bf16 ? launch_seq_t<D, TA, TG, TO, bf16>(a, s) : launch_seq_t<D, TA, TG, TO, float>(a, s);
}
template <int D, typename TA, typename TG>
static hipError_t launch_seq_o(const PrefillArgs &a, hipStream_t s) {
    return a.o_bf16 ? launch_seq_s<D, TA, TG, bf16>(a, s) : launch_seq_s<D, TA, TG, float>(a, s);
}
template <int D, typename TA>
static hipError_t launch_seq_g(const PrefillArgs &a, hipStream_t s) {
    return a.gate_bf16 ? launch_seq_o<D, TA, bf16>(a, s) : launch_seq_o<D, TA, float>(a, s);
}
template <int D>
static hipError_t launch_seq_a(const PrefillArgs &a, hipStream_t s) {
    return a.act_bf16 ? launch_seq_g<D, bf16>(a, s) : launch_seq_g<D, float>(a, s);
}

hipError_t launch_prefill_seq(const PrefillArgs &a, hipStream_t s) {
    switch (a.D) {
        case 16: return launch_seq_a<16>(a, s);
        case 32: return launch_seq_a<32>(a, s);
        case 64: return launch_seq_a<64>(a, s);
        case 128: return launch_seq_a<128>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn
