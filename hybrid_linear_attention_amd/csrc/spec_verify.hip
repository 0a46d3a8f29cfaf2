// Speculative multi-token verify of the GDN mixer core in one launch: each
// request brings up to 8 tokens (the last accepted token, then drafts) that
// run through conv1d + SiLU, L2 norm, the gated delta rule and the gated
// RMSNorm, and the state and conv history reached after EVERY token are kept
// in a slot of their own so that rejecting drafts rolls the request back by
// choosing a slot.  The pages count extra speculative slots for the conv
// history ("Qwen3.8-27B: from model structure to the vLLM inference
// dataflow", section 01 data-structure table, conv-history row) and pass the
// number of speculative tokens into the state-shape calculator ("How the 64
// layers of Qwen3.8-27B are dispatched in vLLM", step 5); the per-position
// slots are this library's reading of that bookkeeping.
//
// Per token j of request r, value head h (operator table, GDN row):
//   S_j = alpha_j S_{j-1} + beta_j (v_j - alpha_j S_{j-1} k_j) k_j^T
//   o_j = S_j q_j / sqrt(d),   y_j = o_j / rms(o_j) * gamma * SiLU(z_j)
// with S_{-1} read from slot_ids[r] and S_j written to spec_slots[r][j].
//
// One block per (request, key head), as the single-token fused decode: the
// key head's q / k channels and its value heads' v channels are convolved once
// for all tokens (each thread reads its channel's history once and writes the
// history of every position, so the in-place case spec_slots[r][0] ==
// slot_ids[r] is race-free), then each state row is read ONCE and carried
// through the tokens in registers, written out after each of them.  HBM bytes
// per request and key head: rows*d*4 read, n*rows*d*4 written.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

constexpr int SV_THREADS = 1024;
constexpr int SV_BUFFERS = 2;   // state passes whose loads are in flight together
constexpr int SV_DW3 = 0x00020000;
constexpr int SV_NT = 2;        // nontemporal cache policy of the state stream

__device__ __forceinline__ __amdgpu_buffer_rsrc_t sv_rsrc(const void *base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    const uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(((uint64_t)hi << 32) | lo), (short)0,
                                             (int)n, SV_DW3);
}

size_t spec_verify_smem_bytes(int D, int32_t Hk, int32_t Hv, int32_t max_tokens) {
    const int G = Hv / Hk;
    return ((size_t)max_tokens * (2 * D + 2 * G * D + 2 * G + 1) + 64) * sizeof(float);
}

template <int D, int NB, int NT, typename TX, typename TW, typename TY, typename TS>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(8))) void spec_verify_kernel(
    const TX *__restrict__ x, int64_t x_ld, const TX *__restrict__ z, int64_t z_ld,
    const TX *__restrict__ ga, const TX *__restrict__ gb, int64_t gate_ld,
    const TW *__restrict__ w, const TW *__restrict__ gamma, TX *__restrict__ pool,
    TS *__restrict__ state, const int32_t *__restrict__ qsl, const int32_t *__restrict__ slots,
    const int32_t *__restrict__ spec, int32_t max_tokens, const uint8_t *__restrict__ has_init,
    int32_t Hk, int32_t Hv, float l2_eps, float norm_eps, TY *__restrict__ y,
    float *__restrict__ o_out) {
    constexpr int LPR = D / 8;      // lanes per state row
    constexpr int RPP = NT / LPR;   // rows per pass
    constexpr int SB = (int)sizeof(TS);
    using SR = StateRow<TS, LPR>;
    extern __shared__ __attribute__((aligned(16))) float ssm[];
    const int G = Hv / Hk;
    const int rows = G * D;
    const int nmax = max_tokens;
    float *sq = ssm;                  // [nmax][D]   q_j (normalised in place)
    float *sk = sq + nmax * D;        // [nmax][D]   k_j
    float *sv = sk + nmax * D;        // [nmax][rows] v_j of the group's heads
    float *so = sv + nmax * rows;     // [nmax][rows] o_j
    float *sa = so + nmax * rows;     // [nmax][G]   alpha
    float *sb = sa + nmax * G;        // [nmax][G]   beta
    float *skq = sb + nmax * G;       // [nmax]      k_j . q_j
    float *red = skq + nmax;          // [64]        reductions

    const int tid = threadIdx.x;
    const int r = blockIdx.x / Hk;
    const int kh = blockIdx.x - r * Hk;
    const int tok0 = qsl[r];
    // a request longer than max_tokens is cut to it, so that no access leaves
    // the spec-slot table or the LDS arrays (the caller's contract excludes it)
    const int n = min(max(qsl[r + 1] - tok0, 0), nmax);
    if (n == 0) return;  // no tokens: no slot is touched
    const int slot = slots[r];
    const int32_t *sslots = spec + (int64_t)r * nmax;
    const int nq = Hk * D;
    const int C = 2 * nq + Hv * D;
    const int l = tid % LPR;
    const int rg = tid / LPR;
    const int npass = ((rows + RPP - 1) / RPP + NB - 1) / NB * NB;
    const bool hi = has_init == nullptr || has_init[r] != 0;

    // the unit's state rows as buffer resources: loads read zeros without an
    // initial state and past the last row, stores past the last row are dropped
    const uint32_t ubytes = (uint32_t)rows * D * SB;
    const int64_t unit_off = (int64_t)kh * G * D * D;
    const __amdgpu_buffer_rsrc_t rld = sv_rsrc(state + (int64_t)slot * Hv * D * D + unit_off, hi ? ubytes : 0u);
    const uint32_t roff = (uint32_t)rg * D * SB;
    f32x4 buf[NB][2];
    auto load_pass = [&](f32x4 (&dst)[2], int p) {
        SR::template load<SV_NT>(dst, rld, (uint32_t)p * RPP * D * SB + roff, l);
    };
#pragma unroll
    for (int b = 0; b < NB; ++b) load_pass(buf[b], b);

    // conv of the group's channels for all n tokens; window = [h0, h1, h2, x_0 .. x_{n-1}]
    constexpr int WMAX = 8 + 3;
    for (int e = tid; e < (2 + G) * D; e += NT) {
        int c;
        float *dst;
        int dstride;
        if (e < D) {
            c = kh * D + e;
            dst = sq + e;
            dstride = D;
        } else if (e < 2 * D) {
            c = nq + kh * D + (e - D);
            dst = sk + (e - D);
            dstride = D;
        } else {
            c = 2 * nq + kh * G * D + (e - 2 * D);
            dst = sv + (e - 2 * D);
            dstride = rows;
        }
        TX win[WMAX];
        const TX zero = from_f32<TX>(0.f);
        const TX *hp = pool + ((int64_t)slot * C + c) * 3;
        win[0] = hi ? hp[0] : zero;
        win[1] = hi ? hp[1] : zero;
        win[2] = hi ? hp[2] : zero;
#pragma unroll
        for (int j = 0; j < 8; ++j) win[3 + j] = j < n ? x[(int64_t)(tok0 + j) * x_ld + c] : zero;
        const float w0 = ld(w + (int64_t)c * 4), w1 = ld(w + (int64_t)c * 4 + 1);
        const float w2 = ld(w + (int64_t)c * 4 + 2), w3 = ld(w + (int64_t)c * 4 + 3);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (j < n) {
                const float acc = w0 * to_f32(win[j + 3]) + w1 * to_f32(win[j + 2]) +
                                  w2 * to_f32(win[j + 1]) + w3 * to_f32(win[j]);
                dst[j * dstride] = silu_f(acc);
                // history after token j: the window's entries j+1 .. j+3 (raw copies)
                TX *hj = pool + ((int64_t)sslots[j] * C + c) * 3;
                hj[0] = win[j + 1];
                hj[1] = win[j + 2];
                hj[2] = win[j + 3];
            }
        }
    }
    for (int t = tid; t < n * G; t += NT) {
        const int j = t / G, hh = t - j * G;
        const int64_t go = (int64_t)(tok0 + j) * gate_ld + kh * G + hh;
        sa[t] = gate_alpha(ld(ga + go));
        sb[t] = gate_beta(ld(gb + go));
    }
    __syncthreads();

    // |q_j|^2, |k_j|^2 and q_j . k_j, one wave per task
    {
        const int wv = tid >> 6, lane = tid & 63;
        for (int task = wv; task < 3 * n; task += NT / 64) {
            const int j = task / 3, kind = task - 3 * j;
            const float *qj = sq + j * D, *kj = sk + j * D;
            float s = 0.f;
            for (int i = lane; i < D; i += 64)
                s += kind == 0 ? qj[i] * qj[i] : kind == 1 ? kj[i] * kj[i] : qj[i] * kj[i];
            s = group_sum<64>(s);
            if (lane == 0) red[task] = s;
        }
    }
    __syncthreads();
    for (int e = tid; e < n * D; e += NT) {
        const int j = e / D;
        sq[e] *= 1.0f / sqrtf(red[3 * j] + l2_eps);
        sk[e] *= 1.0f / sqrtf(red[3 * j + 1] + l2_eps);
    }
    if (tid < n)
        skq[tid] = red[3 * tid + 2] * (1.0f / sqrtf(red[3 * tid] + l2_eps)) *
                   (1.0f / sqrtf(red[3 * tid + 1] + l2_eps));
    __syncthreads();
    const float inv_sqrt_d = 1.0f / sqrtf((float)D);

    // pass p: the row is read once, then each token updates it in registers
    // and writes it to that token's slot
    auto run_pass = [&](f32x4 (&cur)[2], int p) {
        const int R = p * RPP + rg;
        const bool valid = R < rows;
        const int hh = valid ? R / D : 0;
        const uint32_t off = (uint32_t)p * RPP * D * SB + roff;
        f32x4 s0 = cur[0], s1 = cur[1];
        for (int j = 0; j < n; ++j) {
            const f32x4 k0 = *reinterpret_cast<const f32x4 *>(sk + j * D + SR::col(l, 0));
            const f32x4 k1 = *reinterpret_cast<const f32x4 *>(sk + j * D + SR::col(l, 1));
            const f32x4 q0 = *reinterpret_cast<const f32x4 *>(sq + j * D + SR::col(l, 0));
            const f32x4 q1 = *reinterpret_cast<const f32x4 *>(sq + j * D + SR::col(l, 1));
            float pk = s0.x * k0.x + s0.y * k0.y + s0.z * k0.z + s0.w * k0.w +
                       s1.x * k1.x + s1.y * k1.y + s1.z * k1.z + s1.w * k1.w;
            float pq = s0.x * q0.x + s0.y * q0.y + s0.z * q0.z + s0.w * q0.w +
                       s1.x * q1.x + s1.y * q1.y + s1.z * q1.z + s1.w * q1.w;
            pk = group_sum<LPR>(pk);
            pq = group_sum<LPR>(pq);
            const float alpha = sa[j * G + hh], beta = sb[j * G + hh];
            const float vi = valid ? sv[j * rows + R] : 0.f;
            const float be = beta * (vi - alpha * pk);
            s0 = alpha * s0 + be * k0;
            s1 = alpha * s1 + be * k1;
            const __amdgpu_buffer_rsrc_t rst =
                sv_rsrc(state + (int64_t)sslots[j] * Hv * D * D + unit_off, ubytes);
            SR::template store<SV_NT>(s0, s1, rst, off, l);
            if (valid && l == 0) so[j * rows + R] = (alpha * pq + be * skq[j]) * inv_sqrt_d;
        }
    };
#pragma unroll
    for (int b = 0; b < NB; ++b) run_pass(buf[b], b);
    for (int p = NB; p < npass; p += NB) {
#pragma unroll
        for (int b = 0; b < NB; ++b) load_pass(buf[b], p + b);
#pragma unroll
        for (int b = 0; b < NB; ++b) run_pass(buf[b], p + b);
    }
    __syncthreads();

    // gated RMSNorm of every (token, head) row, NT elements (whole rows) at a time
    const int total = n * rows;
    const int nchunks = (total + NT - 1) / NT;
    for (int ch = 0; ch < nchunks; ++ch) {
        const int e = ch * NT + tid;
        const bool valid = e < total;
        const float ov = valid ? so[e] : 0.f;
        float ss;
        if constexpr (D <= 64) {
            ss = group_sum<D>(ov * ov);
        } else {
            const float part = group_sum<64>(ov * ov);
            if ((tid & 63) == 0) red[(tid >> 6)] = part;
            __syncthreads();
            ss = 0.f;
            const int w0 = (tid >> 6) & ~(D / 64 - 1);
#pragma unroll
            for (int q = 0; q < D / 64; ++q) ss += red[w0 + q];
            __syncthreads();
        }
        if (valid) {
            const int j = e / rows, rem = e - j * rows;
            const int hh = rem / D, i = rem - hh * D;
            const int h = kh * G + hh;
            const int64_t t = tok0 + j;
            const float inv = 1.0f / sqrtf(ss * (1.0f / D) + norm_eps);
            const float zz = ld(z + t * z_ld + (int64_t)h * D + i);
            st(y + (t * Hv + h) * D + i, ov * inv * ld(gamma + i) * silu_f(zz));
            if (o_out) o_out[(t * Hv + h) * D + i] = ov;
        }
    }
}

template <int D, typename TX, typename TW, typename TY, typename TS>
static hipError_t launch_sv_t(const SpecVerifyArgs &a, hipStream_t s) {
    const size_t smem = spec_verify_smem_bytes(D, a.Hk, a.Hv, a.max_tokens);
    hipLaunchKernelGGL((spec_verify_kernel<D, SV_BUFFERS, SV_THREADS, TX, TW, TY, TS>),
                       dim3((unsigned)((int64_t)a.R * a.Hk)), dim3(SV_THREADS), smem, s,
                       (const TX *)a.x, a.x_ld, (const TX *)a.z, a.z_ld, (const TX *)a.a,
                       (const TX *)a.b, a.gate_ld, (const TW *)a.w, (const TW *)a.gamma,
                       (TX *)a.pool, (TS *)a.state, a.qsl, a.slots, a.spec, a.max_tokens, a.has_init,
                       a.Hk, a.Hv, a.l2_eps, a.norm_eps, (TY *)a.y, a.o);
    return hipGetLastError();
}
template <int D, typename TX, typename TW, typename TY>
static hipError_t launch_sv_s(const SpecVerifyArgs &a, hipStream_t s) {
    return a.state_bf16 ? launch_sv_t<D, TX, TW, TY, bf16>(a, s) : launch_sv_t<D, TX, TW, TY, float>(a, s);
}
template <int D, typename TX, typename TW>
static hipError_t launch_sv_y(const SpecVerifyArgs &a, hipStream_t s) {
    return a.y_bf16 ? launch_sv_s<D, TX, TW, bf16>(a, s) : launch_sv_s<D, TX, TW, float>(a, s);
}
template <int D, typename TX>
static hipError_t launch_sv_w(const SpecVerifyArgs &a, hipStream_t s) {
    return a.w_bf16 ? launch_sv_y<D, TX, bf16>(a, s) : launch_sv_y<D, TX, float>(a, s);
}
template <int D>
static hipError_t launch_sv_x(const SpecVerifyArgs &a, hipStream_t s) {
    return a.act_bf16 ? launch_sv_w<D, bf16>(a, s) : launch_sv_w<D, float>(a, s);
}

hipError_t launch_spec_verify(const SpecVerifyArgs &a, hipStream_t s) {
    if (a.max_tokens < 1 || a.max_tokens > 8) return hipErrorInvalidValue;
    switch (a.D) {
        case 16: return launch_sv_x<16>(a, s);
        case 32: return launch_sv_x<32>(a, s);
        case 64: return launch_sv_x<64>(a, s);
        case 128: return launch_sv_x<128>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn
