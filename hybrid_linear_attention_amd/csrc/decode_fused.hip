// One decode step of the GDN mixer core in a single launch: conv1d + SiLU with
// the 3-entry history, L2 norm of q and k, the gated delta rule on the state
// (fp32, or bf16 widened on load and rounded once on store; arithmetic in
// fp32 either way), and the gated RMSNorm of the output.
//
// The step ("Qwen3.8-27B: from model structure to the vLLM inference
// dataflow", section 02, one token's journey through a GDN layer; section 01
// operator table, conv / GDN / gated-output rows) for one token of request r:
//   c = SiLU(w0 x + w1 h2 + w2 h1 + w3 h0)   h <- [h1, h2, x]   (history oldest first)
//   q = c_q / |c_q|,  k = c_k / |c_k|,  v = c_v
//   S' = alpha S + beta (v - alpha S k) k^T,   o = S' q / sqrt(d)
//   y = o / rms(o) * gamma * SiLU(z)           (per value head over d_v)
// with alpha = exp(-softplus(a)), beta = sigmoid(b).
//
// One block per (request, key head): the key head's q and k channels and the v
// channels of the value heads that read it are computed once, their history
// entries are read and rewritten by the same thread (race-free), and the
// block then streams those value heads' state rows (read once, written once,
// nontemporal) and normalises whole heads of o from LDS.  The state rows go
// in groups of DF_BUFFERS passes whose loads are in flight together; the first
// group's loads are issued before the conv so its latency hides under them.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

constexpr int DF_THREADS = 1024;
constexpr int DF_BUFFERS = 3;     // state passes in flight per block
// buffer resource word 3 (raw 32-bit data, range-checked) and the nontemporal
// cache policy of the state's buffer loads and stores
constexpr int BUF_DW3 = 0x00020000;
constexpr int BUF_NT = 2;

// A buffer resource over [base, base + bytes) from wave-uniform values (read
// from the first lane, so the descriptor lives in scalar registers).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void *base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    const uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(((uint64_t)hi << 32) | lo), (short)0,
                                             (int)n, BUF_DW3);
}  // fastest of 256, 512, 1024 threads per group block, measured

template <int D, int NB, int NT, typename TX, typename TW, typename TY, typename TS>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(8))) void decode_fused_kernel(
    const TX *__restrict__ x, int64_t x_ld, const TX *__restrict__ z, int64_t z_ld,
    const TX *__restrict__ ga, const TX *__restrict__ gb, int64_t gate_ld,
    const TW *__restrict__ w, const TW *__restrict__ gamma, TX *__restrict__ pool,
    TS *__restrict__ state, const int32_t *__restrict__ slots,
    const uint8_t *__restrict__ has_init, int32_t Hk, int32_t Hv, float l2_eps,
    float norm_eps, TY *__restrict__ y, float *__restrict__ o_out) {
    constexpr int LPR = D / 8;              // lanes per state row
    constexpr int RPP = NT / LPR;   // rows per pass
    constexpr int SB = (int)sizeof(TS);     // bytes per state element
    using SR = StateRow<TS, LPR>;
    extern __shared__ __attribute__((aligned(16))) float dsm[];
    const int G = Hv / Hk;
    const int rows = G * D;
    float *sq = dsm;            // [D]   q (then normalised)
    float *sk = sq + D;         // [D]   k
    float *sv = sk + D;         // [G*D] v
    float *so = sv + rows;      // [G*D] o
    float *sa = so + rows;      // [G]   alpha
    float *sb = sa + G;         // [G]   beta
    float *red = sb + G;        // [32]  reductions

    const int tid = threadIdx.x;
    const int r = blockIdx.x / Hk;
    const int kh = blockIdx.x - r * Hk;
    const int slot = slots[r];
    const int nq = Hk * D;
    const int C = 2 * nq + Hv * D;
    const int l = tid % LPR;
    const int rg = tid / LPR;
    // passes, rounded up to whole groups of NB (a pass past the last row has
    // no rows)
    const int npass = ((rows + RPP - 1) / RPP + NB - 1) / NB * NB;

    // has_initial = 0: a new request, zero history and zero state
    const bool hi = has_init == nullptr || has_init[r] != 0;

    // The unit's state rows (those of its value heads, contiguous in the slot)
    // as buffer resources: loads read zeros without an initial state and past
    // the last row, where stores are dropped, so no branch guards a state
    // access and every access counts in the memory counters the waits are
    // derived from.  Lane: row rg of a pass, its columns as StateRow lays them out.
    const uint32_t ubytes = (uint32_t)rows * D * SB;
    TS *ubase = state + ((int64_t)slot * Hv + (int64_t)kh * G) * D * D;
    const __amdgpu_buffer_rsrc_t rld = uniform_rsrc(ubase, hi ? ubytes : 0u);
    const __amdgpu_buffer_rsrc_t rst = uniform_rsrc(ubase, ubytes);
    const uint32_t roff = (uint32_t)rg * D * SB;
    f32x4 buf[NB][2];  // pass p lands in buf[p % NB]
    auto load_pass = [&](f32x4 (&dst)[2], int p) {
        SR::template load<BUF_NT>(dst, rld, (uint32_t)p * RPP * D * SB + roff, l);
    };
#pragma unroll
    for (int b = 0; b < NB; ++b) load_pass(buf[b], b);

    // conv of the group's channels: q (D), k (D), v (G D)
    for (int e = tid; e < (2 + G) * D; e += NT) {
        int c;
        float *dst;
        if (e < D) {
            c = kh * D + e;
            dst = sq + e;
        } else if (e < 2 * D) {
            c = nq + kh * D + (e - D);
            dst = sk + (e - D);
        } else {
            c = 2 * nq + kh * G * D + (e - 2 * D);
            dst = sv + (e - 2 * D);
        }
        TX *hp = pool + ((int64_t)slot * C + c) * 3;
        const TX x0 = x[(int64_t)r * x_ld + c];
        TX h0 = from_f32<TX>(0.f), h1 = h0, h2 = h0;
        if (hi) {
            h0 = hp[0];
            h1 = hp[1];
            h2 = hp[2];
        }
        const float acc = ld(w + (int64_t)c * 4) * to_f32(x0) + ld(w + (int64_t)c * 4 + 1) * to_f32(h2) +
                          ld(w + (int64_t)c * 4 + 2) * to_f32(h1) + ld(w + (int64_t)c * 4 + 3) * to_f32(h0);
        *dst = silu_f(acc);
        hp[0] = h1;  // the window slides: raw copies, bit-exact
        hp[1] = h2;
        hp[2] = x0;
    }
    if (tid < G) {
        const int64_t go = (int64_t)r * gate_ld + kh * G + tid;
        sa[tid] = gate_alpha(ld(ga + go));
        sb[tid] = gate_beta(ld(gb + go));
    }
    __syncthreads();

    // |q|^2, |k|^2 and q.k (one wave each)
    {
        const int wv = tid >> 6, lane = tid & 63;
        if (wv < 3) {
            float s = 0.f;
            for (int j = lane; j < D; j += 64)
                s += wv == 0 ? sq[j] * sq[j] : wv == 1 ? sk[j] * sk[j] : sq[j] * sk[j];
            s = group_sum<64>(s);
            if (lane == 0) red[wv] = s;
        }
    }
    __syncthreads();
    const float inv_q = 1.0f / sqrtf(red[0] + l2_eps);
    const float inv_k = 1.0f / sqrtf(red[1] + l2_eps);
    const float kq = red[2] * inv_q * inv_k;
    // q and k normalised in place, then the lane's columns in registers
    for (int e = tid; e < 2 * D; e += NT) dsm[e] *= e < D ? inv_q : inv_k;  // sq, then sk
    __syncthreads();
    const float inv_sqrt_d = 1.0f / sqrtf((float)D);
    float4 kc[2], qc[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        kc[m] = *reinterpret_cast<const float4 *>(sk + SR::col(l, m));
        qc[m] = *reinterpret_cast<const float4 *>(sq + SR::col(l, m));
    }

    // pass p from the registers its load landed in
    auto run_pass = [&](f32x4 (&cur)[2], int p) {
        const int R = p * RPP + rg;
        const bool valid = R < rows;
        const int hh = valid ? R / D : 0;
        const float alpha = sa[hh], beta = sb[hh];
        const float vi = valid ? sv[R] : 0.f;
        float pk = 0.f, pq = 0.f;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const f32x4 s = cur[m];
            pk += s.x * kc[m].x + s.y * kc[m].y + s.z * kc[m].z + s.w * kc[m].w;
            pq += s.x * qc[m].x + s.y * qc[m].y + s.z * qc[m].z + s.w * qc[m].w;
        }
        pk = group_sum<LPR>(pk);
        pq = group_sum<LPR>(pq);
        const float be = beta * (vi - alpha * pk);
        f32x4 sn[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            f32x4 s = cur[m];
            s.x = alpha * s.x + be * kc[m].x;
            s.y = alpha * s.y + be * kc[m].y;
            s.z = alpha * s.z + be * kc[m].z;
            s.w = alpha * s.w + be * kc[m].w;
            sn[m] = s;
        }
        SR::template store<BUF_NT>(sn[0], sn[1], rst, (uint32_t)p * RPP * D * SB + roff, l);
        if (valid && l == 0) so[R] = (alpha * pq + be * kq) * inv_sqrt_d;
    };
    // groups of NB passes: all of a group's loads are in flight together, then
    // its passes are computed and stored (measured faster on this state
    // stream than rotating each freed buffer to the pass NB ahead)
#pragma unroll
    for (int b = 0; b < NB; ++b) run_pass(buf[b], b);
    for (int p = NB; p < npass; p += NB) {
#pragma unroll
        for (int b = 0; b < NB; ++b) load_pass(buf[b], p + b);
#pragma unroll
        for (int b = 0; b < NB; ++b) run_pass(buf[b], p + b);
    }
    __syncthreads();

    // gated RMSNorm of the group's heads, NT elements (whole heads) at a time
    const int nchunks = (rows + NT - 1) / NT;
    for (int ch = 0; ch < nchunks; ++ch) {
        const int e = ch * NT + tid;
        const bool valid = e < rows;
        const float ov = valid ? so[e] : 0.f;
        float ss;
        if constexpr (D <= 64) {
            ss = group_sum<D>(ov * ov);
        } else {
            // a head spans D / 64 waves
            const float part = group_sum<64>(ov * ov);
            if ((tid & 63) == 0) red[4 + (tid >> 6)] = part;
            __syncthreads();
            ss = 0.f;
            const int w0 = (tid >> 6) & ~(D / 64 - 1);
#pragma unroll
            for (int j = 0; j < D / 64; ++j) ss += red[4 + w0 + j];
            __syncthreads();
        }
        if (valid) {
            const int hh = e / D, i = e - hh * D;
            const int h = kh * G + hh;
            const float inv = 1.0f / sqrtf(ss * (1.0f / D) + norm_eps);
            const float zz = ld(z + (int64_t)r * z_ld + (int64_t)h * D + i);
            st(y + ((int64_t)r * Hv + h) * D + i, ov * inv * ld(gamma + i) * silu_f(zz));
            if (o_out) o_out[((int64_t)r * Hv + h) * D + i] = ov;
        }
    }
}

size_t decode_fused_smem_bytes(int D, int32_t Hk, int32_t Hv) {
    const int G = Hv / Hk;
    return (size_t)(2 * D + 2 * G * D + 2 * G + 32) * sizeof(float);
}

template <int D, typename TX, typename TW, typename TY, typename TS>
static hipError_t launch_df_t(const DecodeFusedArgs &a, hipStream_t s) {
    const size_t smem = decode_fused_smem_bytes(D, a.Hk, a.Hv);
    hipLaunchKernelGGL((decode_fused_kernel<D, DF_BUFFERS, DF_THREADS, TX, TW, TY, TS>), dim3((unsigned)((int64_t)a.R * a.Hk)),
                       dim3(DF_THREADS), smem, s, (const TX *)a.x, a.x_ld, (const TX *)a.z, a.z_ld,
                       (const TX *)a.a, (const TX *)a.b, a.gate_ld, (const TW *)a.w,
                       (const TW *)a.gamma, (TX *)a.pool, (TS *)a.state, a.slots, a.has_init, a.Hk, a.Hv,
                       a.l2_eps, a.norm_eps, (TY *)a.y, a.o);
    return hipGetLastError();
}
template <int D, typename TX, typename TW, typename TY>
static hipError_t launch_df_s(const DecodeFusedArgs &a, hipStream_t s) {
    return a.state_bf16 ? launch_df_t<D, TX, TW, TY, bf16>(a, s) : launch_df_t<D, TX, TW, TY, float>(a, s);
}
template <int D, typename TX, typename TW>
static hipError_t launch_df_y(const DecodeFusedArgs &a, hipStream_t s) {
    return a.y_bf16 ? launch_df_s<D, TX, TW, bf16>(a, s) : launch_df_s<D, TX, TW, float>(a, s);
}
template <int D, typename TX>
static hipError_t launch_df_w(const DecodeFusedArgs &a, hipStream_t s) {
    return a.w_bf16 ? launch_df_y<D, TX, bf16>(a, s) : launch_df_y<D, TX, float>(a, s);
}
template <int D>
static hipError_t launch_df_x(const DecodeFusedArgs &a, hipStream_t s) {
    return a.act_bf16 ? launch_df_w<D, bf16>(a, s) : launch_df_w<D, float>(a, s);
}

hipError_t launch_decode_fused(const DecodeFusedArgs &a, hipStream_t s) {
    switch (a.D) {
        case 16: return launch_df_x<16>(a, s);
        case 32: return launch_df_x<32>(a, s);
        case 64: return launch_df_x<64>(a, s);
        case 128: return launch_df_x<128>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn
