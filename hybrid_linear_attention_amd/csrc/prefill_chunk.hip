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
// Chunks are C = 32 tokens: one MFMA k-step spans a chunk, the triangular
// inverse is 32x32, and a chain block's LDS (~68 KB) leaves room for two
// blocks per CU, so one block's waits overlap the other's work.
//
// Three launches:
//   plan   one block: chunk offsets per request (prefix sum of ceil(L/C)), on
//          the device so the host never waits for query_start_loc.
//   prep   one block per (chunk, key head), fully parallel: K K^T and Q K^T once
//          for the key head, then one wave per value head reading it: the
//          gates' cumulative decay, T = (I + A)^-1 and P, written to the
//          workspace as bf16 hi/lo planes (8,448 bytes per chunk and value head).
//   chain  one block per (request, value head, block of 32 or 64 state rows),
//          sequential over the request's chunks: only the state-dependent
//          products.  State rows evolve independently given (k, beta, alpha),
//          so the row blocks of a head never communicate.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

namespace chunk {

constexpr int D = 128;      // d_k == d_v
constexpr int CH = 32;      // tokens per chunk
constexpr int KP = D + 8;   // padded bf16 row of 128-wide planes (272 B)
constexpr int TP = CH + 8;  // padded bf16 row of 32-wide T/P planes (80 B)
constexpr int KTP = CH + 4; // padded bf16 row of the K^T planes (72 B; conflict-free transpose writes)
constexpr int AP = CH + 4;  // padded fp32 row of 32x32 work matrices

// workspace record of one (chunk, value head): T and P as bf16 hi/lo planes
// [32][32], then the cumulative log-decay G and beta of the chunk's tokens
constexpr size_t REC_TH = 0, REC_TL = 2048, REC_PH = 4096, REC_PL = 6144;
constexpr size_t REC_G = 8192, REC_B = REC_G + 128, REC_BYTES = REC_B + 128;  // 8,448

__device__ __forceinline__ uint16_t bits_of(__bf16 x) { return __builtin_bit_cast(uint16_t, x); }

// x = hi + lo with hi = RNE_bf16(x), lo = RNE_bf16(x - hi).
__device__ __forceinline__ void split(float x, uint16_t &h, uint16_t &l) {
    const __bf16 hb = (__bf16)x;
    const float hf = (float)hb;
    h = bits_of(hb);
    l = bits_of((__bf16)(x - hf));
}

__device__ __forceinline__ uint32_t pack2(uint16_t a, uint16_t b) { return a | (uint32_t(b) << 16); }

__device__ __forceinline__ void split4_store(float a, float b, float c, float d, uint16_t *ph,
                                             uint16_t *pl) {
    uint16_t h[4], l[4];
    split(a, h[0], l[0]);
    split(b, h[1], l[1]);
    split(c, h[2], l[2]);
    split(d, h[3], l[3]);
    *reinterpret_cast<uint2 *>(ph) = make_uint2(pack2(h[0], h[1]), pack2(h[2], h[3]));
    *reinterpret_cast<uint2 *>(pl) = make_uint2(pack2(l[0], l[1]), pack2(l[2], l[3]));
}

// eight values (MFMA k-slot order) -> hi/lo operands
__device__ __forceinline__ void split_vals(const float (&x)[8], bf16x8_t &hi, bf16x8_t &lo) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const __bf16 hb = (__bf16)x[e];
        hi[e] = hb;
        lo[e] = (__bf16)(x[e] - (float)hb);
    }
}

__device__ __forceinline__ bf16x8_t frag(const uint16_t *p) {
    return *reinterpret_cast<const bf16x8_t *>(p);
}

// A operand in k-slot order from a bf16 plane row: columns c0 .. c0+3 and
// c0+16 .. c0+19 with c0 = 32 ks + 4 lg (see the chain kernel's layout note)
__device__ __forceinline__ bf16x8_t frag_slots(const uint16_t *row, int c0) {
    const uint2 a = *reinterpret_cast<const uint2 *>(row + c0);
    const uint2 b = *reinterpret_cast<const uint2 *>(row + c0 + 16);
    return __builtin_bit_cast(bf16x8_t, make_uint4(a.x, a.y, b.x, b.y));
}

// acc += a * b with a = ah + al, b = bh + bl (the lo*lo term is below fp32 noise).
__device__ __forceinline__ void mma3(floatx4_t &acc, const bf16x8_t &ah, const bf16x8_t &al,
                                     const bf16x8_t &bh, const bf16x8_t &bl) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
}

// Raw 4-element loads, converted to fp32 only at use, so a prefetch never
// waits on its own load.
template <typename T> struct Raw4;
template <> struct Raw4<float> {
    f32x4 v;
    __device__ __forceinline__ void load(const float *p) { v = *reinterpret_cast<const f32x4 *>(p); }
    __device__ __forceinline__ void zero() { v = f32x4{0.f, 0.f, 0.f, 0.f}; }
    __device__ __forceinline__ float4 get() const { return make_float4(v.x, v.y, v.z, v.w); }
};
template <> struct Raw4<bf16> {
    uint2 v;
    __device__ __forceinline__ void load(const bf16 *p) { v = *reinterpret_cast<const uint2 *>(p); }
    __device__ __forceinline__ void zero() { v = make_uint2(0, 0); }
    __device__ __forceinline__ float4 get() const {
        return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
                           __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u));
    }
};

}  // namespace chunk

// ---------------------------------------------------------------------------
// plan: chunk_off[r] = sum_{r' < r} ceil(L_r' / C)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void prefill_plan_kernel(const int32_t *__restrict__ qsl,
                                                            int32_t nreq,
                                                            int32_t *__restrict__ chunk_off) {
    __shared__ int32_t part[1024];
    const int tid = threadIdx.x;
    const int per = (nreq + 1023) / 1024;
    const int r0 = min(nreq, tid * per), r1 = min(nreq, r0 + per);
    int local = 0;
    for (int r = r0; r < r1; ++r) local += (qsl[r + 1] - qsl[r] + chunk::CH - 1) / chunk::CH;
    part[tid] = local;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {  // inclusive Hillis-Steele scan
        const int add = tid >= off ? part[tid - off] : 0;
        __syncthreads();
        part[tid] += add;
        __syncthreads();
    }
    int run = part[tid] - local;
    if (tid == 0) chunk_off[0] = 0;
    for (int r = r0; r < r1; ++r) {
        run += (qsl[r + 1] - qsl[r] + chunk::CH - 1) / chunk::CH;
        chunk_off[r + 1] = run;
    }
}

// ---------------------------------------------------------------------------
// prep: per (chunk, key head): K K^T and Q K^T, then one wave per value head
// ---------------------------------------------------------------------------
namespace chunk {
struct PrepSmem {
    uint16_t Kh[CH][KP], Kl[CH][KP], Qh[CH][KP], Ql[CH][KP];
    float KK[CH][AP], QK[CH][AP];
    float A[4][CH][AP];   // per-wave work matrix: A, then T = (I + A)^-1
    float G[4][CH], Beta[4][CH];
};
}  // namespace chunk

template <typename TA, typename TG>
__global__ __launch_bounds__(256) void prefill_prep_kernel(
    const TA *__restrict__ q, const TA *__restrict__ k, const TG *__restrict__ ga,
    const TG *__restrict__ gb, int64_t gate_ld, const int32_t *__restrict__ qsl,
    const int32_t *__restrict__ chunk_off, int32_t nreq, int32_t Hk, int32_t Hv,
    uint8_t *__restrict__ records) {
    using namespace chunk;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem_raw[];
    PrepSmem &sm = *reinterpret_cast<PrepSmem *>(smem_raw);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;

    const int c = blockIdx.x / Hk;
    const int kh = blockIdx.x - c * Hk;
    if (c >= chunk_off[nreq]) return;
    const int r = find_request(chunk_off, nreq, c);
    const int tb = qsl[r] + CH * (c - chunk_off[r]);
    const int Lc = min(CH, qsl[r + 1] - tb);
    const int group = Hv / Hk;

    // stage K and Q of the key head as hi/lo planes (1024 four-element slots each)
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int idx = tid + 256 * m;
        const int t = idx >> 5;
        const int c4 = (idx & 31) * 4;
        float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), qv = kv;
        if (t < Lc) {
            const int64_t off = ((int64_t)(tb + t) * Hk + kh) * D + c4;
            kv = ld4(k + off);
            qv = ld4(q + off);
        }
        split4_store(kv.x, kv.y, kv.z, kv.w, &sm.Kh[t][c4], &sm.Kl[t][c4]);
        split4_store(qv.x, qv.y, qv.z, qv.w, &sm.Qh[t][c4], &sm.Ql[t][c4]);
    }
    __syncthreads();

    // K K^T and Q K^T on the three lower-triangular 16x16 tiles of each
    for (int item = w; item < 6; item += 4) {
        const bool isQ = item >= 3;
        const int n = isQ ? item - 3 : item;
        const int tm = n == 0 ? 0 : 1;
        const int tn = n == 2 ? 1 : 0;
        floatx4_t acc = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int off = 32 * ks + 8 * lg;
            const bf16x8_t ah = isQ ? frag(&sm.Qh[16 * tm + lr][off]) : frag(&sm.Kh[16 * tm + lr][off]);
            const bf16x8_t al = isQ ? frag(&sm.Ql[16 * tm + lr][off]) : frag(&sm.Kl[16 * tm + lr][off]);
            mma3(acc, ah, al, frag(&sm.Kh[16 * tn + lr][off]), frag(&sm.Kl[16 * tn + lr][off]));
        }
        float(*dst)[AP] = isQ ? sm.QK : sm.KK;
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[16 * tm + 4 * lg + e][16 * tn + lr] = acc[e];
    }
    __syncthreads();

    // one wave per value head: nothing below crosses waves
    for (int hh = w; hh < group; hh += 4) {
        const int h = kh * group + hh;
        uint8_t *rec = records + ((size_t)c * Hv + h) * REC_BYTES;
        float(*A)[AP] = sm.A[w];
        float *Gw = sm.G[w];
        float *Bw = sm.Beta[w];
        {
            float g = 0.f, beta = 0.f;
            if (lane < Lc) {
                const int64_t go = (int64_t)(tb + lane) * gate_ld + h;
                g = gate_log_alpha(ld(ga + go));
                beta = gate_beta(ld(gb + go));
            }
            float G = g;  // inclusive prefix sum over the chunk; padded rows add nothing
#pragma unroll
            for (int off = 1; off < CH; off <<= 1) {
                const float y = __shfl_up(G, off, 64);
                if (lane >= off) G += y;
            }
            if (lane < CH) {
                Gw[lane] = G;
                Bw[lane] = beta;
                reinterpret_cast<float *>(rec + REC_G)[lane] = G;
                reinterpret_cast<float *>(rec + REC_B)[lane] = beta;
            }
        }
        __builtin_amdgcn_wave_barrier();
        // A = strict-lower(beta_t e^{G_t-G_s} KK), P = lower(e^{G_t-G_s} QK) -> record
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int idx = lane + 64 * m;  // 256 groups of 4 columns
            const int t = idx >> 3;
            const int s0 = (idx & 7) * 4;
            float pv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int s = s0 + e;
                const float dec = expf(fminf(Gw[t] - Gw[s], 0.f));
                A[t][s] = s < t ? Bw[t] * dec * sm.KK[t][s] : 0.f;
                pv[e] = s <= t ? dec * sm.QK[t][s] : 0.f;
            }
            split4_store(pv[0], pv[1], pv[2], pv[3],
                         reinterpret_cast<uint16_t *>(rec + REC_PH) + t * CH + s0,
                         reinterpret_cast<uint16_t *>(rec + REC_PL) + t * CH + s0);
        }
        __builtin_amdgcn_wave_barrier();
        // T = (I + A)^-1: the two 16x16 diagonal blocks by substitution
        // (lane: column lr, rows lg + 4 e), then T10 = -T11 A10 T00
#pragma unroll
        for (int bb = 0; bb < 32; bb += 16) {
            float x[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = (lg + 4 * e == lr) ? 1.f : 0.f;
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                const float xs = __shfl(x[s >> 2], (s & 3) * 16 + lr, 64);  // X[s][lr]
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = lg + 4 * e;
                    if (t > s) x[e] -= A[bb + t][bb + s] * xs;
                }
            }
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int e = 0; e < 4; ++e) A[bb + lg + 4 * e][bb + lr] = x[e];
            __builtin_amdgcn_wave_barrier();
        }
        {
            float y[4] = {0.f, 0.f, 0.f, 0.f};  // Y = A10 T00
#pragma unroll 4
            for (int uu = 0; uu < 16; ++uu) {
                const float tu = A[uu][lr];
#pragma unroll
                for (int e = 0; e < 4; ++e) y[e] += A[16 + lg + 4 * e][uu] * tu;
            }
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int e = 0; e < 4; ++e) A[16 + lg + 4 * e][lr] = y[e];
            __builtin_amdgcn_wave_barrier();
            float tv[4] = {0.f, 0.f, 0.f, 0.f};  // T10 = -T11 Y
#pragma unroll 4
            for (int uu = 0; uu < 16; ++uu) {
                const float yu = A[16 + uu][lr];
#pragma unroll
                for (int e = 0; e < 4; ++e) tv[e] -= A[16 + lg + 4 * e][16 + uu] * yu;
            }
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int e = 0; e < 4; ++e) A[16 + lg + 4 * e][lr] = tv[e];
            __builtin_amdgcn_wave_barrier();
        }
        // T (lower triangle, zeros above) -> record
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int idx = lane + 64 * m;
            const int t = idx >> 3;
            const int s0 = (idx & 7) * 4;
            split4_store(A[t][s0], A[t][s0 + 1], A[t][s0 + 2], A[t][s0 + 3],
                         reinterpret_cast<uint16_t *>(rec + REC_TH) + t * CH + s0,
                         reinterpret_cast<uint16_t *>(rec + REC_TL) + t * CH + s0);
        }
        __builtin_amdgcn_wave_barrier();
    }
}

// ---------------------------------------------------------------------------
// chain: sequential over a request's chunks, per (request, value head, block
// of 16 NW state rows).  Wave w of the NW compute waves owns state rows
// 16 w .. 16 w + 15 of the block for all 32 tokens of a chunk, so the error E,
// the pseudo-values Delta and the state itself never leave its registers:
//   X = K S0^T, OQ = Q S0^T        (A: K / Q rows from LDS, B: state registers)
//   Delta = T (beta E)             (A: T rows from LDS,     B: E registers)
//   O = gamma OQ + P Delta         (A: P rows from LDS,     B: Delta registers)
//   S^T = gamma_C S^T + K^T Delta~ (A: K^T rows from LDS,   B: Delta registers)
// An accumulator lane holds rows 4 lg + e of a 16-row tile; feeding it back
// as the B operand of the next product uses the k-slot order
//   slot (lg, p) -> 32 ks + 16 (p / 4) + 4 lg + p % 4,
// and the A operand is read from LDS in that same order (two 8-byte reads per
// plane), so no register ever crosses lanes.  The block's four waves stage K,
// K^T, Q, T, P and the gates of a chunk in LDS; the next chunk's operands are
// loaded into registers while the current chunk computes.
// ---------------------------------------------------------------------------
namespace chunk {
struct ChainSmem {
    uint16_t Kh[CH][KP], Kl[CH][KP];     // K rows [token][key channel]
    uint16_t KTh[D][KTP], KTl[D][KTP];   // K transposed [key channel][token]
    uint16_t Qh[CH][KP], Ql[CH][KP];
    uint16_t Th[CH][TP], Tl[CH][TP];     // (I + A)^-1 [token][token]
    uint16_t Ph[CH][TP], Pl[CH][TP];     // decayed causal Q K^T
    float Gam[CH], Beta[CH], Rev[CH];
};

// One thread's share of the next chunk.  Thread tid stages K rows 2 tp, 2 tp + 1
// (tp = tid % 16) at columns 8 cg .. 8 cg + 7 (cg = tid / 16): the K^T planes
// are then written as packed token pairs, 16 lanes to one row.
template <typename TA, int RPW> struct ChainPrefetch {
    chunk::Raw4<TA> kr[2][2], qr[2][2];  // [row of the pair][column half]
    uint4 tpr[2];                        // T/P planes: 512 pieces of 16 bytes
    float Gp, Bp;
    float vr[RPW][2][4];

    __device__ __forceinline__ void load(const TA *__restrict__ k, const TA *__restrict__ q,
                                         const TA *__restrict__ v, const uint8_t *__restrict__ records,
                                         int tok0, int L, int cc, int c_first, int Hk, int Hv, int h,
                                         int kh, const int (&irow)[RPW], bool computes, int tid, int lg) {
        using namespace chunk;
        const int tb = tok0 + cc * CH;
        const int Lc = min(CH, L - cc * CH);
        const uint8_t *rec = records + ((size_t)(c_first + cc) * Hv + h) * REC_BYTES;
        const int tp = tid & 15, cg = tid >> 4;
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
            const int t = 2 * tp + rr;
            const int64_t off = ((int64_t)(tb + t) * Hk + kh) * D + 8 * cg;
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                if (t < Lc) {
                    kr[rr][hf].load(k + off + 4 * hf);
                    qr[rr][hf].load(q + off + 4 * hf);
                } else {
                    kr[rr][hf].zero();
                    qr[rr][hf].zero();
                }
            }
        }
#pragma unroll
        for (int m = 0; m < 2; ++m) tpr[m] = reinterpret_cast<const uint4 *>(rec)[tid + 256 * m];
        Gp = 0.f;
        Bp = 0.f;
        if (tid < CH) {
            Gp = reinterpret_cast<const float *>(rec + REC_G)[tid];
            Bp = reinterpret_cast<const float *>(rec + REC_B)[tid];
        }
        if (computes) {
#pragma unroll
            for (int rt = 0; rt < RPW; ++rt)
#pragma unroll
                for (int tau = 0; tau < 2; ++tau)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int t = 16 * tau + 4 * lg + e;
                        vr[rt][tau][e] = t < Lc ? ld(v + ((int64_t)(tb + t) * Hv + h) * D + irow[rt]) : 0.f;
                    }
        }
    }

    __device__ __forceinline__ void stage(chunk::ChainSmem &sm, int tid) const {
        using namespace chunk;
        const int tp = tid & 15, cg = tid >> 4;
        uint16_t kh_[2][8], kl_[2][8];
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
            const int t = 2 * tp + rr;
            const float4 k0 = kr[rr][0].get(), k1 = kr[rr][1].get();
            const float4 q0 = qr[rr][0].get(), q1 = qr[rr][1].get();
            const float kx[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
            const float qx[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
            uint16_t qh_[8], ql_[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                split(kx[e], kh_[rr][e], kl_[rr][e]);
                split(qx[e], qh_[e], ql_[e]);
            }
            *reinterpret_cast<uint4 *>(&sm.Kh[t][8 * cg]) =
                make_uint4(pack2(kh_[rr][0], kh_[rr][1]), pack2(kh_[rr][2], kh_[rr][3]),
                           pack2(kh_[rr][4], kh_[rr][5]), pack2(kh_[rr][6], kh_[rr][7]));
            *reinterpret_cast<uint4 *>(&sm.Kl[t][8 * cg]) =
                make_uint4(pack2(kl_[rr][0], kl_[rr][1]), pack2(kl_[rr][2], kl_[rr][3]),
                           pack2(kl_[rr][4], kl_[rr][5]), pack2(kl_[rr][6], kl_[rr][7]));
            *reinterpret_cast<uint4 *>(&sm.Qh[t][8 * cg]) =
                make_uint4(pack2(qh_[0], qh_[1]), pack2(qh_[2], qh_[3]), pack2(qh_[4], qh_[5]), pack2(qh_[6], qh_[7]));
            *reinterpret_cast<uint4 *>(&sm.Ql[t][8 * cg]) =
                make_uint4(pack2(ql_[0], ql_[1]), pack2(ql_[2], ql_[3]), pack2(ql_[4], ql_[5]), pack2(ql_[6], ql_[7]));
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int j = 8 * cg + e;
            *reinterpret_cast<uint32_t *>(&sm.KTh[j][2 * tp]) = pack2(kh_[0][e], kh_[1][e]);
            *reinterpret_cast<uint32_t *>(&sm.KTl[j][2 * tp]) = pack2(kl_[0][e], kl_[1][e]);
        }
        // T/P planes: piece p = plane (4) x row (32) x 4 groups of 8 columns
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int piece = tid + 256 * m;
            const int plane = piece >> 7;
            const int t = (piece >> 2) & 31;
            const int s8 = (piece & 3) * 8;
            uint16_t *dst = plane == 0 ? &sm.Th[t][s8] : plane == 1 ? &sm.Tl[t][s8]
                          : plane == 2 ? &sm.Ph[t][s8] : &sm.Pl[t][s8];
            *reinterpret_cast<uint4 *>(dst) = tpr[m];
        }
        if (tid < CH) {
            const float Glast = __shfl(Gp, CH - 1, 64);
            sm.Gam[tid] = expf(Gp);
            sm.Rev[tid] = expf(Glast - Gp);
            sm.Beta[tid] = Bp;
        }
    }
};
}  // namespace chunk

template <int NW, int RPW, typename TA, typename TO>
__global__ __launch_bounds__(256, 2) void prefill_chain_kernel(
    const TA *__restrict__ q, const TA *__restrict__ k, const TA *__restrict__ v,
    float *__restrict__ state, const int32_t *__restrict__ qsl,
    const int32_t *__restrict__ slots, const uint8_t *__restrict__ has_init,
    const int32_t *__restrict__ chunk_off, const uint8_t *__restrict__ records, int32_t nreq,
    int32_t Hk, int32_t Hv, TO *__restrict__ o) {
    using namespace chunk;
    constexpr int IB = 16 * RPW * NW;  // state rows per block
    constexpr int NRB = D / IB;        // blocks per (request, head)
    extern __shared__ __attribute__((aligned(16))) uint8_t smem_raw[];
    ChainSmem &sm = *reinterpret_cast<ChainSmem *>(smem_raw);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const bool computes = w < NW;

    // blocks are dealt round-robin to the 8 XCDs: give each XCD a contiguous
    // range of (request, head, row block) so blocks sharing K, Q and the prep
    // records also share an L2
    const int G_ = gridDim.x;
    const int logical = (G_ % 8 == 0) ? (blockIdx.x % 8) * (G_ / 8) + blockIdx.x / 8 : blockIdx.x;
    const int rb = logical % NRB;
    const int unit = logical / NRB;
    const int h = unit % Hv;
    const int r = unit / Hv;
    if (r >= nreq) return;
    const int kh = h / (Hv / Hk);
    const int tok0 = qsl[r];
    const int L = qsl[r + 1] - tok0;
    if (L <= 0) return;  // empty request: slot untouched
    const int nch = (L + CH - 1) / CH;
    const int c_first = chunk_off[r];
    const bool hi_init = has_init == nullptr || has_init[r] != 0;
    int irow[RPW];  // this lane's state rows (value channels)
#pragma unroll
    for (int rt = 0; rt < RPW; ++rt) irow[rt] = IB * rb + 16 * (RPW * w + rt) + lr;
    float *sbase = state + ((int64_t)slots[r] * Hv + h) * D * D;

    // state rows of this lane, transposed accumulator layout:
    // ST[rt][jt][e] = S[irow[rt]][16 jt + 4 lg + e]
    floatx4_t ST[RPW][8];
#pragma unroll
    for (int rt = 0; rt < RPW; ++rt)
#pragma unroll
        for (int jt = 0; jt < 8; ++jt) {
            ST[rt][jt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
            if (computes && hi_init) {
                const float4 s4 = *reinterpret_cast<const float4 *>(sbase + (int64_t)irow[rt] * D + 16 * jt + 4 * lg);
                ST[rt][jt] = floatx4_t{s4.x, s4.y, s4.z, s4.w};
            }
        }
    const float inv_sqrt_d = 1.0f / sqrtf((float)D);

    ChainPrefetch<TA, RPW> pf;
    pf.load(k, q, v, records, tok0, L, 0, c_first, Hk, Hv, h, kh, irow, computes, tid, lg);
    for (int cc = 0; cc < nch; ++cc) {
        const int tb = tok0 + cc * CH;
        const int Lc = min(CH, L - cc * CH);
        __syncthreads();  // every wave is done reading the previous chunk's planes
        pf.stage(sm, tid);
        float vcur[RPW][2][4];
#pragma unroll
        for (int rt = 0; rt < RPW; ++rt)
#pragma unroll
            for (int tau = 0; tau < 2; ++tau)
#pragma unroll
                for (int e = 0; e < 4; ++e) vcur[rt][tau][e] = pf.vr[rt][tau][e];
        __syncthreads();
        // the next chunk's operands load while this one computes
        if (cc + 1 < nch)
            pf.load(k, q, v, records, tok0, L, cc + 1, c_first, Hk, Hv, h, kh, irow, computes, tid, lg);
        if (!computes) continue;

        // ---------------- X = K S0^T and OQ = Q S0^T  (tokens x this wave's rows)
        floatx4_t X[RPW][2], OQ[RPW][2];
#pragma unroll
        for (int rt = 0; rt < RPW; ++rt)
#pragma unroll
            for (int tau = 0; tau < 2; ++tau) {
                X[rt][tau] = floatx4_t{0.f, 0.f, 0.f, 0.f};
                OQ[rt][tau] = X[rt][tau];
            }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            bf16x8_t sbh[RPW], sbl[RPW];
#pragma unroll
            for (int rt = 0; rt < RPW; ++rt) {
                float sv[8];
#pragma unroll
                for (int p = 0; p < 8; ++p) sv[p] = ST[rt][2 * ks + (p >> 2)][p & 3];
                split_vals(sv, sbh[rt], sbl[rt]);
            }
            const int c0 = 32 * ks + 4 * lg;
#pragma unroll
            for (int tau = 0; tau < 2; ++tau) {
                const int row = 16 * tau + lr;
                const bf16x8_t kh_ = frag_slots(sm.Kh[row], c0), kl_ = frag_slots(sm.Kl[row], c0);
                const bf16x8_t qh_ = frag_slots(sm.Qh[row], c0), ql_ = frag_slots(sm.Ql[row], c0);
#pragma unroll
                for (int rt = 0; rt < RPW; ++rt) {
                    mma3(X[rt][tau], kh_, kl_, sbh[rt], sbl[rt]);
                    mma3(OQ[rt][tau], qh_, ql_, sbh[rt], sbl[rt]);
                }
            }
        }
        // E = beta (V - gamma X) (kept in X); OQ scaled by gamma
#pragma unroll
        for (int tau = 0; tau < 2; ++tau)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = 16 * tau + 4 * lg + e;
                const float gm = sm.Gam[t], bt = sm.Beta[t];
#pragma unroll
                for (int rt = 0; rt < RPW; ++rt) {
                    X[rt][tau][e] = bt * (vcur[rt][tau][e] - gm * X[rt][tau][e]);
                    OQ[rt][tau][e] *= gm;
                }
            }

        // ---------------- Delta = T (beta E), then O and the state update
        const int c0 = 4 * lg;  // the chunk is one k-step
        bf16x8_t ebh[RPW], ebl[RPW];
#pragma unroll
        for (int rt = 0; rt < RPW; ++rt) {
            float ev[8];
#pragma unroll
            for (int p = 0; p < 8; ++p) ev[p] = X[rt][p >> 2][p & 3];
            split_vals(ev, ebh[rt], ebl[rt]);
        }
        floatx4_t Dl[RPW][2];
#pragma unroll
        for (int tau = 0; tau < 2; ++tau) {
            const bf16x8_t th_ = frag_slots(sm.Th[16 * tau + lr], c0);
            const bf16x8_t tl_ = frag_slots(sm.Tl[16 * tau + lr], c0);
#pragma unroll
            for (int rt = 0; rt < RPW; ++rt) {
                Dl[rt][tau] = floatx4_t{0.f, 0.f, 0.f, 0.f};
                mma3(Dl[rt][tau], th_, tl_, ebh[rt], ebl[rt]);
            }
        }
        bf16x8_t dbh[RPW], dbl[RPW], tbh[RPW], tbl[RPW];
#pragma unroll
        for (int rt = 0; rt < RPW; ++rt) {
            float dv[8], dtv[8];
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                dv[p] = Dl[rt][p >> 2][p & 3];
                dtv[p] = dv[p] * sm.Rev[16 * (p >> 2) + 4 * lg + (p & 3)];
            }
            split_vals(dv, dbh[rt], dbl[rt]);
            split_vals(dtv, tbh[rt], tbl[rt]);
        }
#pragma unroll
        for (int tau = 0; tau < 2; ++tau) {
            const bf16x8_t ph_ = frag_slots(sm.Ph[16 * tau + lr], c0);
            const bf16x8_t pl_ = frag_slots(sm.Pl[16 * tau + lr], c0);
#pragma unroll
            for (int rt = 0; rt < RPW; ++rt) mma3(OQ[rt][tau], ph_, pl_, dbh[rt], dbl[rt]);
        }
        const float gC = sm.Gam[CH - 1];
#pragma unroll
        for (int jt = 0; jt < 8; ++jt) {
            const bf16x8_t kth = frag_slots(sm.KTh[16 * jt + lr], c0);
            const bf16x8_t ktl = frag_slots(sm.KTl[16 * jt + lr], c0);
#pragma unroll
            for (int rt = 0; rt < RPW; ++rt) {
                ST[rt][jt] *= gC;
                mma3(ST[rt][jt], kth, ktl, tbh[rt], tbl[rt]);
            }
        }
#pragma unroll
        for (int rt = 0; rt < RPW; ++rt)
#pragma unroll
            for (int tau = 0; tau < 2; ++tau)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = 16 * tau + 4 * lg + e;
                    if (t < Lc) st(o + ((int64_t)(tb + t) * Hv + h) * D + irow[rt], OQ[rt][tau][e] * inv_sqrt_d);
                }
    }

    if (computes) {
#pragma unroll
        for (int rt = 0; rt < RPW; ++rt)
#pragma unroll
            for (int jt = 0; jt < 8; ++jt)
                *reinterpret_cast<float4 *>(sbase + (int64_t)irow[rt] * D + 16 * jt + 4 * lg) =
                    make_float4(ST[rt][jt][0], ST[rt][jt][1], ST[rt][jt][2], ST[rt][jt][3]);
    }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

size_t prefill_chunk_workspace_bytes(int32_t Hv, int32_t T, int32_t nreq) {
    const size_t max_chunks = (size_t)T / chunk::CH + (size_t)nreq;
    return align256((size_t)(nreq + 1) * 4) + max_chunks * (size_t)Hv * chunk::REC_BYTES;
}

template <typename K>
static hipError_t set_smem(K kern, size_t bytes, bool &done) {
    if (done) return hipSuccess;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e == hipSuccess) done = true;
    return e;
}

template <int NW, int RPW, typename TA, typename TO>
static hipError_t launch_chain(const PrefillArgs &a, hipStream_t s, const int32_t *chunk_off,
                               const uint8_t *records) {
    using namespace chunk;
    static bool set = false;
    hipError_t e = set_smem(&prefill_chain_kernel<NW, RPW, TA, TO>, sizeof(ChainSmem), set);
    if (e != hipSuccess) return e;
    const int64_t blocks = (int64_t)a.nreq * a.Hv * (D / (16 * NW * RPW));
    hipLaunchKernelGGL((prefill_chain_kernel<NW, RPW, TA, TO>), dim3((unsigned)blocks), dim3(256),
                       sizeof(ChainSmem), s, (const TA *)a.q, (const TA *)a.k, (const TA *)a.v,
                       a.state, a.qsl, a.slots, a.has_init, chunk_off, records, a.nreq, a.Hk, a.Hv,
                       (TO *)a.o);
    return hipGetLastError();
}

template <typename TA, typename TG, typename TO>
static hipError_t launch_chunk_t(const PrefillArgs &a, hipStream_t s) {
    using namespace chunk;
    int32_t *chunk_off = static_cast<int32_t *>(a.ws);
    uint8_t *records = static_cast<uint8_t *>(a.ws) + align256((size_t)(a.nreq + 1) * 4);
    const int64_t max_chunks = (int64_t)a.T / CH + a.nreq;

    hipLaunchKernelGGL(prefill_plan_kernel, dim3(1), dim3(1024), 0, s, a.qsl, a.nreq, chunk_off);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;

    static bool prep_set = false;
    e = set_smem(&prefill_prep_kernel<TA, TG>, sizeof(PrepSmem), prep_set);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((prefill_prep_kernel<TA, TG>), dim3((unsigned)(max_chunks * a.Hk)), dim3(256),
                       sizeof(PrepSmem), s, (const TA *)a.q, (const TA *)a.k, (const TG *)a.a,
                       (const TG *)a.b, a.gate_ld, a.qsl, chunk_off, a.nreq, a.Hk, a.Hv, records);
    e = hipGetLastError();
    if (e != hipSuccess) return e;

    // state rows per chain block: 64 when there are enough (request, head)
    // units to fill the chip, 32 otherwise
    const int64_t units = (int64_t)a.nreq * a.Hv;
    if (units >= 128) return launch_chain<4, 1, TA, TO>(a, s, chunk_off, records);  // 64 rows
    return launch_chain<2, 1, TA, TO>(a, s, chunk_off, records);                    // 32 rows
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
