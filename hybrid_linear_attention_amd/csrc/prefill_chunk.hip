// Chunkwise-parallel prefill of the gated delta rule on gfx950 MFMA, d = 128.
//
// The recurrence ("Qwen3.8-27B: from model structure to the vLLM inference
// dataflow", section 01 operator table, GDN row)
//   S_t = alpha_t S_{t-1} + beta_t (v_t - alpha_t S_{t-1} k_t) k_t^T,  o_t = S_t q_t / sqrt(d)
// is associative (the page's LM-head notes: GDN's block recurrence is
// parallelised through its associative structure).  Over a chunk of C tokens
// with cumulative log-decay G_t = sum_{u<=t} log alpha_u, gamma_t = e^{G_t}, and
// state S0 entering the chunk, write S_t = gamma_t S0 + sum_{s<=t} e^{G_t-G_s}
// delta_s k_s^T.  The rank-1 "pseudo-values" delta solve a unit lower-triangular
// system:
//   (I + A) Delta = diag(beta) E,   A_ts = beta_t e^{G_t-G_s} k_t.k_s  (s < t)
//   E = V - diag(gamma) K S0^T        (the error against the decayed S0)
// and then
//   O = diag(gamma) Q S0^T + P Delta,  P_ts = e^{G_t-G_s} q_t.k_s  (s <= t)
//   S_C = gamma_C S0 + (diag(e^{G_C-G}) Delta)^T K.
// Only differences G_t - G_s with s <= t are ever exponentiated, so nothing
// overflows however strong the decay.
//
// Precision: every contraction runs on v_mfma_f32_16x16x32_bf16 with both
// operands split into bf16 hi + lo parts (hi = RNE(x), lo = RNE(x - hi)) and
// three products hi*hi + hi*lo + lo*hi accumulated in fp32: ~2^-16 relative per
// operand, which keeps the final state well inside a 1e-3 relative error even
// when the decay is weak.  A single bf16 rounding of k or of Delta would not.
//
// Work split: one 256-thread block per (request, value head, 32-row slice of the
// state).  State rows evolve independently given (k, beta, alpha), so the four
// slices of a head never communicate.  The slice's fp32 state lives in MFMA
// accumulator registers across the whole request; each chunk stages K, Q and
// the gates in LDS as hi/lo planes, then:
//   B: X = K S0^T, OQ = Q S0^T            (wave w: token rows 16w..16w+15)
//   A: K K^T -> A,  Q K^T -> P            (lower-triangular 16x16 tiles, 5 per wave)
//   C: T = (I + A)^-1                     (16x16 diagonal blocks by substitution,
//                                          off-diagonal blocks block-row by block-row)
//   D: Delta = T (beta E)
//   E: O = gamma OQ + P Delta   -> o
//   F: S = gamma_C S + Delta~^T K         (wave w: key columns 32w..32w+31)
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

namespace chunk {

constexpr int D = 128;      // d_k == d_v
constexpr int CH = 64;      // tokens per chunk
constexpr int I = 32;       // state rows (value channels) per block
constexpr int NSL = D / I;  // blocks per (request, head)
constexpr int KP = D + 8;   // padded bf16 row of the K/Q/S planes (272 B, 16-B multiple)
constexpr int TP = CH + 8;  // padded bf16 row of the T/P/E/Delta planes (144 B)
constexpr int AP = CH + 4;  // padded fp32 row of the A/T work matrix

struct Smem {
    uint16_t Kh[CH][KP], Kl[CH][KP];
    union {
        struct { uint16_t h[CH][KP], l[CH][KP]; } Q;
        struct { uint16_t Th[CH][TP], Tl[CH][TP], Dth[I][TP], Dtl[I][TP]; } T;
    } u;
    uint16_t Sh[I][KP], Sl[I][KP];
    float A[CH][AP];
    uint16_t Ph[CH][TP], Pl[CH][TP];
    uint16_t Eh[I][TP], El[I][TP];
    uint16_t Dh[I][TP], Dl[I][TP];
    float G[CH], Gam[CH], Rev[CH], Beta[CH];
};

__device__ __forceinline__ uint16_t bits_of(__bf16 x) { return __builtin_bit_cast(uint16_t, x); }

// x = hi + lo with hi = RNE_bf16(x), lo = RNE_bf16(x - hi).
__device__ __forceinline__ void split(float x, uint16_t &h, uint16_t &l) {
    const __bf16 hb = (__bf16)x;
    const float hf = (float)hb;
    h = bits_of(hb);
    l = bits_of((__bf16)(x - hf));
}

__device__ __forceinline__ void split4_store(float a, float b, float c, float d, uint16_t *ph,
                                             uint16_t *pl) {
    uint16_t h[4], l[4];
    split(a, h[0], l[0]);
    split(b, h[1], l[1]);
    split(c, h[2], l[2]);
    split(d, h[3], l[3]);
    *reinterpret_cast<uint2 *>(ph) = make_uint2(h[0] | (uint32_t(h[1]) << 16), h[2] | (uint32_t(h[3]) << 16));
    *reinterpret_cast<uint2 *>(pl) = make_uint2(l[0] | (uint32_t(l[1]) << 16), l[2] | (uint32_t(l[3]) << 16));
}

__device__ __forceinline__ bf16x8_t frag(const uint16_t *p) {
    return *reinterpret_cast<const bf16x8_t *>(p);
}

__device__ __forceinline__ bf16x8_t frag_strided(const uint16_t *p, int stride) {
    bf16x8_t r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = __builtin_bit_cast(__bf16, p[e * stride]);
    return r;
}

// acc += a * b with a = ah + al, b = bh + bl (the lo*lo term is below fp32 noise).
__device__ __forceinline__ void mma3(floatx4_t &acc, const bf16x8_t &ah, const bf16x8_t &al,
                                     const bf16x8_t &bh, const bf16x8_t &bl) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
}

}  // namespace chunk

template <typename TA, typename TG, typename TO>
__global__ __launch_bounds__(256) void prefill_chunk_kernel(
    const TA *__restrict__ q, const TA *__restrict__ k, const TA *__restrict__ v,
    const TG *__restrict__ ga, const TG *__restrict__ gb, int64_t gate_ld,
    float *__restrict__ state, const int32_t *__restrict__ qsl,
    const int32_t *__restrict__ slots, const uint8_t *__restrict__ has_init, int32_t nreq,
    int32_t Hk, int32_t Hv, TO *__restrict__ o) {
    using namespace chunk;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem_raw[];
    Smem &sm = *reinterpret_cast<Smem *>(smem_raw);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;          // wave 0..3
    const int lr = lane & 15;        // MFMA row/column within a 16-tile
    const int lg = lane >> 4;        // MFMA k-group / accumulator row group

    const int bid = blockIdx.x;
    const int slice = bid % NSL;
    const int unit = bid / NSL;
    const int h = unit % Hv;
    const int r = unit / Hv;
    if (r >= nreq) return;
    const int kh = h / (Hv / Hk);
    const int i0 = slice * I;
    const int tok0 = qsl[r];
    const int L = qsl[r + 1] - tok0;
    if (L <= 0) return;  // empty request: slot untouched
    const bool hi_init = has_init == nullptr || has_init[r] != 0;
    float *sp = state + ((int64_t)slots[r] * Hv + h) * D * D + (int64_t)i0 * D;

    // fp32 master copy of this block's state slice, in accumulator layout:
    // Sm[mi][n][e] = S[16 mi + 4 lg + e][32 w + 16 n + lr]
    floatx4_t Sm[2][2];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * mi + 4 * lg + e;
                const int j = 32 * w + 16 * n + lr;
                const float val = hi_init ? sp[(int64_t)i * D + j] : 0.0f;
                Sm[mi][n][e] = val;
                split(val, sm.Sh[i][j], sm.Sl[i][j]);
            }

    const float inv_sqrt_d = 1.0f / sqrtf((float)D);

    for (int c0 = 0; c0 < L; c0 += CH) {
        const int Lc = min(CH, L - c0);
        const int tb = tok0 + c0;
        __syncthreads();  // previous chunk done with K / T planes; S planes written

        // ---------------- stage K, Q (hi/lo planes) and the gates
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const int idx = tid + 256 * m;  // 0..2047 float4 slots of a 64x128 tile
            const int t = idx >> 5;
            const int c4 = (idx & 31) * 4;
            float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), qv = kv;
            if (t < Lc) {
                const int64_t off = ((int64_t)(tb + t) * Hk + kh) * D + c4;
                kv = ld4(k + off);
                qv = ld4(q + off);
            }
            split4_store(kv.x, kv.y, kv.z, kv.w, &sm.Kh[t][c4], &sm.Kl[t][c4]);
            split4_store(qv.x, qv.y, qv.z, qv.w, &sm.u.Q.h[t][c4], &sm.u.Q.l[t][c4]);
        }
        if (w == 0) {
            float g = 0.f, beta = 0.f;
            if (lane < Lc) {
                const int64_t go = (int64_t)(tb + lane) * gate_ld + h;
                g = gate_log_alpha(ld(ga + go));
                beta = gate_beta(ld(gb + go));
            }
            float G = g;  // inclusive prefix sum over the chunk
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float y = __shfl_up(G, off, 64);
                if (lane >= off) G += y;
            }
            const float Glast = __shfl(G, 63, 64);
            sm.G[lane] = G;
            sm.Gam[lane] = expf(G);
            sm.Rev[lane] = expf(Glast - G);
            sm.Beta[lane] = beta;
        }
        // zero the strictly-upper 16x16 blocks of A and P (never written below)
        for (int idx = tid; idx < 6 * 256; idx += 256) {
            const int blk = idx >> 8;  // (0,1) (0,2) (0,3) (1,2) (1,3) (2,3)
            const int bm = blk < 3 ? 0 : (blk < 5 ? 1 : 2);
            const int bn = blk < 3 ? blk + 1 : (blk < 5 ? blk - 1 : 3);
            const int t = 16 * bm + ((idx >> 4) & 15);
            const int s = 16 * bn + (idx & 15);
            sm.A[t][s] = 0.f;
            sm.Ph[t][s] = 0;
            sm.Pl[t][s] = 0;
        }
        __syncthreads();

        // ---------------- phase B: X = K S0^T, OQ = Q S0^T  (rows 16w.., cols 0..31)
        floatx4_t X[2], OQ[2];
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            X[it] = floatx4_t{0.f, 0.f, 0.f, 0.f};
            OQ[it] = X[it];
        }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int off = 32 * ks + 8 * lg;
            const int row = 16 * w + lr;
            const bf16x8_t kah = frag(&sm.Kh[row][off]), kal = frag(&sm.Kl[row][off]);
            const bf16x8_t qah = frag(&sm.u.Q.h[row][off]), qal = frag(&sm.u.Q.l[row][off]);
#pragma unroll
            for (int it = 0; it < 2; ++it) {
                const bf16x8_t sbh = frag(&sm.Sh[16 * it + lr][off]);
                const bf16x8_t sbl = frag(&sm.Sl[16 * it + lr][off]);
                mma3(X[it], kah, kal, sbh, sbl);
                mma3(OQ[it], qah, qal, sbh, sbl);
            }
        }
        // E = beta (V - gamma X) stored transposed [i][t]; OQ scaled by gamma
        {
            const int t0 = 16 * w + 4 * lg;
#pragma unroll
            for (int it = 0; it < 2; ++it) {
                const int i = 16 * it + lr;
                float ev[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = t0 + e;
                    const float vv = t < Lc ? ld(v + ((int64_t)(tb + t) * Hv + h) * D + i0 + i) : 0.f;
                    ev[e] = sm.Beta[t] * (vv - sm.Gam[t] * X[it][e]);
                    OQ[it][e] *= sm.Gam[t];
                }
                split4_store(ev[0], ev[1], ev[2], ev[3], &sm.Eh[i][t0], &sm.El[i][t0]);
            }
        }

        // ---------------- phase A: K K^T -> A (strict lower), Q K^T -> P (lower)
#pragma unroll 1
        for (int item = w; item < 20; item += 4) {
            const bool isQ = item >= 10;
            int n = isQ ? item - 10 : item;  // lower-triangular tile index
            int tm = 0;
            while (n > tm) { n -= tm + 1; ++tm; }
            const int tn = n;
            floatx4_t acc = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int off = 32 * ks + 8 * lg;
                const bf16x8_t ah = isQ ? frag(&sm.u.Q.h[16 * tm + lr][off]) : frag(&sm.Kh[16 * tm + lr][off]);
                const bf16x8_t al = isQ ? frag(&sm.u.Q.l[16 * tm + lr][off]) : frag(&sm.Kl[16 * tm + lr][off]);
                const bf16x8_t bh = frag(&sm.Kh[16 * tn + lr][off]);
                const bf16x8_t bl = frag(&sm.Kl[16 * tn + lr][off]);
                mma3(acc, ah, al, bh, bl);
            }
            const int s = 16 * tn + lr;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = 16 * tm + 4 * lg + e;
                const float dec = expf(fminf(sm.G[t] - sm.G[s], 0.f));
                if (isQ) {
                    const float val = s <= t ? dec * acc[e] : 0.f;
                    split(val, sm.Ph[t][s], sm.Pl[t][s]);
                } else {
                    sm.A[t][s] = s < t ? sm.Beta[t] * dec * acc[e] : 0.f;
                }
            }
        }
        __syncthreads();

        // ---------------- phase C1: invert the 16x16 diagonal blocks of (I + A)
        {
            const int bb = 16 * w;
            float x[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = (lg + 4 * e == lr) ? 1.f : 0.f;
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                const float xs = __shfl(x[s >> 2], (s & 3) * 16 + lr, 64);  // X[s][lr]
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = lg + 4 * e;
                    if (t > s) x[e] -= sm.A[bb + t][bb + s] * xs;
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) sm.A[bb + lg + 4 * e][bb + lr] = x[e];
        }
        __syncthreads();

        // ---------------- phase C2: off-diagonal blocks, T_bi,w = -T_bi,bi sum_m A_bi,m T_m,w
#pragma unroll 1
        for (int bi = 1; bi < 4; ++bi) {
            float y[4] = {0.f, 0.f, 0.f, 0.f};
            if (w < bi) {
                for (int m = w; m < bi; ++m) {
#pragma unroll 4
                    for (int uu = 0; uu < 16; ++uu) {
                        const float tmu = sm.A[16 * m + uu][16 * w + lr];
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            y[e] += sm.A[16 * bi + lg + 4 * e][16 * m + uu] * tmu;
                    }
                }
            }
            __syncthreads();
            if (w < bi) {
#pragma unroll
                for (int e = 0; e < 4; ++e) sm.A[16 * bi + lg + 4 * e][16 * w + lr] = y[e];
            }
            __syncthreads();
            float tv[4] = {0.f, 0.f, 0.f, 0.f};
            if (w < bi) {
#pragma unroll 4
                for (int uu = 0; uu < 16; ++uu) {
                    const float yu = sm.A[16 * bi + uu][16 * w + lr];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        tv[e] -= sm.A[16 * bi + lg + 4 * e][16 * bi + uu] * yu;
                }
            }
            __syncthreads();
            if (w < bi) {
#pragma unroll
                for (int e = 0; e < 4; ++e) sm.A[16 * bi + lg + 4 * e][16 * w + lr] = tv[e];
            }
            __syncthreads();
        }
        // T (fp32, lower triangle, zeros above) -> hi/lo planes over the dead Q planes
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int idx = tid + 256 * m;  // 1024 groups of 4
            const int t = idx >> 4;
            const int s = (idx & 15) * 4;
            split4_store(sm.A[t][s], sm.A[t][s + 1], sm.A[t][s + 2], sm.A[t][s + 3],
                         &sm.u.T.Th[t][s], &sm.u.T.Tl[t][s]);
        }
        __syncthreads();

        // ---------------- phase D: Delta = T (beta E)  (rows 16w.., cols 0..31)
        const int nks = w >= 2 ? 2 : 1;  // T is lower triangular
        floatx4_t Dacc[2];
#pragma unroll
        for (int it = 0; it < 2; ++it) Dacc[it] = floatx4_t{0.f, 0.f, 0.f, 0.f};
        for (int ks = 0; ks < nks; ++ks) {
            const int off = 32 * ks + 8 * lg;
            const bf16x8_t ah = frag(&sm.u.T.Th[16 * w + lr][off]);
            const bf16x8_t al = frag(&sm.u.T.Tl[16 * w + lr][off]);
#pragma unroll
            for (int it = 0; it < 2; ++it)
                mma3(Dacc[it], ah, al, frag(&sm.Eh[16 * it + lr][off]), frag(&sm.El[16 * it + lr][off]));
        }
        {
            const int t0 = 16 * w + 4 * lg;
#pragma unroll
            for (int it = 0; it < 2; ++it) {
                const int i = 16 * it + lr;
                split4_store(Dacc[it][0], Dacc[it][1], Dacc[it][2], Dacc[it][3], &sm.Dh[i][t0], &sm.Dl[i][t0]);
                split4_store(Dacc[it][0] * sm.Rev[t0], Dacc[it][1] * sm.Rev[t0 + 1],
                             Dacc[it][2] * sm.Rev[t0 + 2], Dacc[it][3] * sm.Rev[t0 + 3],
                             &sm.u.T.Dth[i][t0], &sm.u.T.Dtl[i][t0]);
            }
        }
        __syncthreads();

        // ---------------- phase E: O = gamma Q S0^T + P Delta -> o
        for (int ks = 0; ks < nks; ++ks) {
            const int off = 32 * ks + 8 * lg;
            const bf16x8_t ah = frag(&sm.Ph[16 * w + lr][off]);
            const bf16x8_t al = frag(&sm.Pl[16 * w + lr][off]);
#pragma unroll
            for (int it = 0; it < 2; ++it)
                mma3(OQ[it], ah, al, frag(&sm.Dh[16 * it + lr][off]), frag(&sm.Dl[16 * it + lr][off]));
        }
#pragma unroll
        for (int it = 0; it < 2; ++it)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = 16 * w + 4 * lg + e;
                if (t < Lc)
                    st(o + ((int64_t)(tb + t) * Hv + h) * D + i0 + 16 * it + lr, OQ[it][e] * inv_sqrt_d);
            }

        // ---------------- phase F: S = gamma_C S + Delta~^T K  (cols 32w..32w+31)
        const float gC = sm.Gam[CH - 1];
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
            for (int n = 0; n < 2; ++n) Sm[mi][n] *= gC;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int off = 32 * ks + 8 * lg;
            bf16x8_t bh[2], bl[2];
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                const int j = 32 * w + 16 * n + lr;
                bh[n] = frag_strided(&sm.Kh[off][j], KP);
                bl[n] = frag_strided(&sm.Kl[off][j], KP);
            }
#pragma unroll
            for (int mi = 0; mi < 2; ++mi) {
                const bf16x8_t ah = frag(&sm.u.T.Dth[16 * mi + lr][off]);
                const bf16x8_t al = frag(&sm.u.T.Dtl[16 * mi + lr][off]);
#pragma unroll
                for (int n = 0; n < 2; ++n) mma3(Sm[mi][n], ah, al, bh[n], bl[n]);
            }
        }
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
            for (int n = 0; n < 2; ++n)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = 16 * mi + 4 * lg + e;
                    const int j = 32 * w + 16 * n + lr;
                    split(Sm[mi][n][e], sm.Sh[i][j], sm.Sl[i][j]);
                }
    }

    // final state of the slice back to the slot
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * mi + 4 * lg + e;
                const int j = 32 * w + 16 * n + lr;
                sp[(int64_t)i * D + j] = Sm[mi][n][e];
            }
}

size_t prefill_chunk_smem_bytes() { return sizeof(chunk::Smem); }

template <typename TA, typename TG, typename TO>
static hipError_t launch_chunk_t(const PrefillArgs &a, hipStream_t s) {
    const size_t smem = sizeof(chunk::Smem);
    static bool attr_set = false;  // per instantiation; idempotent if two threads race
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(
            reinterpret_cast<const void *>(&prefill_chunk_kernel<TA, TG, TO>),
            hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int64_t blocks = (int64_t)a.nreq * a.Hv * chunk::NSL;
    hipLaunchKernelGGL((prefill_chunk_kernel<TA, TG, TO>), dim3((unsigned)blocks), dim3(256), smem, s,
                       (const TA *)a.q,
                       (const TA *)a.k, (const TA *)a.v, (const TG *)a.a, (const TG *)a.b,
                       a.gate_ld, a.state, a.qsl, a.slots, a.has_init, a.nreq, a.Hk, a.Hv,
                       (TO *)a.o);
    return hipGetLastError();
}
template <typename TA, typename TG>
static hipError_t launch_chunk_o(const PrefillArgs &a, hipStream_t s) {
    return a.o_bf16 ? launch_chunk_t<TA, TG, bf16>(a, s) : launch_chunk_t<TA, TG, float>(a, s);
}
template <typename TA>
static hipError_t launch_chunk_g(const PrefillArgs &a, hipStream_t s) {
    return a.gate_bf16 ? launch_chunk_o<TA, bf16>(a, s) : launch_chunk_o<TA, float>(a, s);
}

hipError_t launch_prefill_chunk(const PrefillArgs &a, hipStream_t s) {
    if (a.D != chunk::D) return hipErrorInvalidValue;
    return a.act_bf16 ? launch_chunk_g<bf16>(a, s) : launch_chunk_g<float>(a, s);
}

}  // namespace gdn
