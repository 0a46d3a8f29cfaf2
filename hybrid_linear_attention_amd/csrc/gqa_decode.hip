// Decode step of the full-attention (GQA) layers over a paged KV cache, gfx950.
//
// The operation ("Qwen3.8-27B: from model structure to the vLLM inference
// dataflow", section 03 GQA / attention lab, section 04 PRECISION & CACHE,
// section 05 PagedAttention card): 24 query heads share 4 key/value heads of
// 256 dims (query head h reads head h / 6); RoPE turns 64 of the 256 dims; the
// attention output is gated by a sigmoid ahead of the output projection; keys
// and values live in fixed-size pages reached through a per-request block
// table.
//
// Two launches:
//  1. attn_split: one block per (request, key/value head, run of 512
//     positions); 4 waves of 128 positions, 16 at a time.  Each block first
//     rotates q of the new token (position L - 1) in fp64 for its group of
//     query heads (one angle per dim, shared by the group) and rounds it to
//     fp32; the block whose run holds position L - 1 also rotates k and stores
//     the rotated k and v into the token's page before it reads any position:
//     rounded once to bf16, or (an fp8 cache) the e4m3 codes nearest to
//     k / k_scale and v / v_scale.  No other block reads that row (another
//     run, request or key/value head reads other rows).  Scores q . K^T on
//     v_mfma_f32_16x16x32_bf16 (rows: the <= 8 query heads of the group, q
//     split into three bf16 terms so that the scores keep fp32 accuracy
//     against the exact bf16 K); an online softmax in base 2 across the 16
//     lanes that hold a head row (DPP), its reference max moved only when a
//     score passes it by 2^8; then P V on v_mfma_f32_16x16x16_bf16 (p as
//     bf16 hi + lo) with both operands taken from row-major LDS tiles by the
//     transposed LDS read.  An fp8 cache is read as e4m3 codes (half the
//     bytes) and widened to bf16 exactly in registers before the MFMAs (the
//     K fragments) or the LDS tile (the V rows); k_scale rides on q and
//     v_scale on the combine.  The block merges its 4 waves and writes one
//     partial (max, sum, unnormalised o) per query head.
//  2. combine: per (request, query head), merges the partials of the
//     request's runs, applies the sigmoid gate and writes y (and o).  (A
//     separate launch: merging in the last block of each group would need a
//     device-scope release per block, which writes back the L2 of every
//     XCD.)
// The cache traffic (every position's K and V read once per key/value head)
// is the bound; the arithmetic all sits on the matrix cores, and the
// loads of the next 16 positions are in flight while a tile computes.
#include <type_traits>

#include "gdn_device.h"
#include "gqa_launch.h"

namespace gdn {
namespace gqa {

constexpr int D = 256;          // head dim
constexpr int SPLIT = 512;      // positions per attention block
constexpr int NWAVE = 4;
constexpr int WKEYS = SPLIT / NWAVE;
constexpr int NTILE = WKEYS / 16;  // 16-position tiles per wave
constexpr int GMAX = 8;         // query heads per key/value head, at most
constexpr int QROW = D + 8;     // padded LDS row of a q term

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

// fp64 -> bf16 nearest-even with a single rounding: truncate to fp32, record
// inexactness in the last mantissa bit (round to odd; fp32 keeps 16 bits more
// than bf16, so the second rounding cannot land on a false tie), then round
// the fp32 pattern to nearest-even bf16.
__device__ __forceinline__ uint16_t bf16_from_f64(double x) {
    const float f = __double2float_rz(x);
    uint32_t u = __float_as_uint(f);
    if ((double)f != x) u |= 1u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return uint16_t(u >> 16);
}

// fp64 -> OCP e4m3 code nearest to x, ties to even, saturated at +-448 (a NaN
// gives code 0).  Every step is exact in fp64: the quantum of x's binade is a
// power of two, so x / quantum is exact and rint rounds it half to even.
__device__ __forceinline__ uint8_t e4m3_from_f64(double x) {
    const uint8_t sign = signbit(x) ? 0x80 : 0;
    const double a = fabs(x);
    if (!(a > 0.0)) return sign;
    int e;
    frexp(a, &e);                                   // a in [2^(e-1), 2^e)
    const double quantum = ldexp(1.0, max(e - 1, -6) - 3);
    const double rq = fmin(rint(a / quantum) * quantum, 448.0);
    if (rq == 0.0) return sign;
    int er;
    const double m = frexp(rq, &er);                // rq = m 2^er, m in [0.5, 1)
    if (er - 1 < -6) return sign | (uint8_t)(rq * 512.0);          // subnormal: k 2^-9
    return sign | (uint8_t)(((er - 1 + 7) << 3) | (int)((m * 2.0 - 1.0) * 8.0));
}

// max over the 16 lanes of a row (same butterfly as group_sum)
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, dpp_f(v, 0));
    v = fmaxf(v, dpp_f(v, 1));
    v = fmaxf(v, dpp_f(v, 2));
    v = fmaxf(v, dpp_f(v, 3));
    return v;
}

__device__ __forceinline__ uint16_t bf16_rne_bits(float x) {
    uint32_t u = __float_as_uint(x);
    u += 0x7fffu + ((u >> 16) & 1u);
    return uint16_t(u >> 16);
}

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// Transposed LDS read (gfx950): within each 16-lane group, lane i receives
// element i % 4 of the 4-element words read by lanes 4j + i / 4, j = 0..3.  With
// lane 4j + q of group kg reading row 4 kg + j, columns 4q .. 4q + 3 of a
// row-major tile of 16-bit values, lane i ends up with rows 4 kg .. 4 kg + 3 of
// column i: the k-major operand layout of v_mfma_f32_16x16x16_bf16.
__device__ __forceinline__ s16x4_t lds_read_tr(const uint8_t *base, uint32_t off) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4_t *)((__attribute__((address_space(3))) uint8_t *)(base) + off));
}

__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Per-wave LDS region: the tile's V rows (16 positions x 256 dims bf16, rows
// padded to VROW bytes so that the transposed reads of 16 rows spread over
// the banks) and its p as bf16 hi / lo terms ([16 positions][16 heads]).
constexpr int VROW = 2 * D + 16;
constexpr int PT_OFF = 16 * VROW;
constexpr int WREG = PT_OFF + 2 * 16 * 16 * 2;
constexpr float RESCALE_LOG2 = 8.f;  // keep p below 2^8 before moving the reference max

// e4m3 -> bf16 for 4 codes: every e4m3 value is exact in bf16, and gfx950's
// scaled fp8 -> bf16 conversion at scale 1 yields those patterns directly, two
// codes per instruction (OCP decoding, NaN codes and signed zeros included,
// checked on all 256 codes)
__device__ __forceinline__ uint2 fp8x4_to_bf16x4(uint32_t w) {
    return make_uint2(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false)),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)));
}

// FP8: the cache holds e4m3 codes (k_scale folded into qscale by the host,
// v_scale applied by the combine); otherwise bf16.
template <int G, bool FP8, typename TA>
__global__ __launch_bounds__(64 * NWAVE) __attribute__((amdgpu_waves_per_eu(2))) void gqa_attn_split_kernel(
    const TA *__restrict__ q, int64_t q_ld, const TA *__restrict__ knew, const TA *__restrict__ vnew,
    int64_t kv_ld, void *__restrict__ kc, void *__restrict__ vc, float k_scale, float v_scale,
    const int32_t *__restrict__ bt, int32_t max_pages, const int32_t *__restrict__ lens, int32_t Hq,
    int32_t Hkv, int32_t rd, int32_t P, int32_t num_pages, int32_t lmax, int32_t nsplit, double theta,
    float qscale, float *__restrict__ po, float2 *__restrict__ pml) {
    static_assert(G >= 1 && G <= GMAX, "query heads per key/value head");
    static_assert(G * D * 4 <= WREG, "the merge reuses a wave's region");
    // q terms (bf16 bits) for all 16 MFMA rows (rows >= G zero); rows padded by
    // 16 bytes so that the 16 rows of a fragment read fall in distinct banks
    __shared__ __attribute__((aligned(16))) uint16_t qf[3][16][QROW];
    __shared__ __attribute__((aligned(16))) uint8_t wreg[NWAVE][WREG];
    __shared__ float2 wml[NWAVE][GMAX];

    const int s = blockIdx.x % nsplit;
    const int rg = blockIdx.x / nsplit;
    const int g = rg % Hkv;
    const int r = rg / Hkv;
    const int L = lens[r];
    if (L < 1 || L > lmax) return;
    const int k0 = s * SPLIT;
    if (k0 >= L) return;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, kg = lane >> 4;
    uint8_t *const vt = wreg[w];
    uint8_t *const pt = wreg[w] + PT_OFF;

    // RoPE of the new token (position L - 1) in fp64: x'_d = x_d cos + sgn
    // x_partner sin over the first rd dims, the angle of dim d shared by every
    // head of the group.  The group's q values are loaded first; the angle and
    // the rotation wait until the first tiles' cache loads are in flight.
    const int pos = L - 1;
    const int half = rd / 2;
    const bool rot = tid < rd;
    const int partner = rot ? (tid < half ? tid + half : tid - half) : tid;
    float qv[G], qp[G];
#pragma unroll
    for (int m = 0; m < G; ++m) {
        const TA *row = q + (int64_t)r * q_ld + (g * G + m) * D;
        qv[m] = to_f32(row[tid]);
        qp[m] = to_f32(row[partner]);
    }
    double cs = 1.0, sn = 0.0;
    auto angle = [&]() {
        if (rot) {
            const int i = tid < half ? tid : tid - half;
            sincos((double)pos * pow(theta, -2.0 * i / rd), &sn, &cs);
        }
    };
    auto rope = [&](float x, float xp) -> double {
        double val = x;
        if (rot) val = tid < half ? val * cs - (double)xp * sn : val * cs + (double)xp * sn;
        return val;
    };
    // the run holding the new token appends its rotated k and its v before it
    // reads any position (the barrier below orders the stores before the loads
    // of every wave)
    const bool appender = s == pos / SPLIT;
    if (appender) {
        angle();
        const int pg = bt[(int64_t)r * max_pages + pos / P];
        if (pg >= 0 && pg < num_pages) {  // else the contract is broken: no append
            const TA *krow = knew + (int64_t)r * kv_ld + g * D;
            const double kval = rope(to_f32(krow[tid]), to_f32(krow[partner]));
            const float vin = to_f32(vnew[(int64_t)r * kv_ld + g * D + tid]);
            const int64_t dst = (((int64_t)pg * Hkv + g) * P + pos % P) * D + tid;
            if constexpr (FP8) {
                static_cast<uint8_t *>(kc)[dst] = e4m3_from_f64(kval / (double)k_scale);
                static_cast<uint8_t *>(vc)[dst] = e4m3_from_f64((double)vin / (double)v_scale);
            } else {
                static_cast<uint16_t *>(kc)[dst] = bf16_from_f64(kval);
                static_cast<uint16_t *>(vc)[dst] = to_bf16(vin).bits;
            }
        }
        __threadfence_block();
    }
    __syncthreads();

    const int wk0 = k0 + w * WKEYS;
    // Mu: reference max (log2 units) of rows 4 kg + i; lsum: this lane's sum of p
    float Mu[4], lsum[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        Mu[i] = -INFINITY;
        lsum[i] = 0.f;
    }
    // O[db]: rows 4 kg + i (query heads), value dim 16 db + n
    floatx4_t O[16];
#pragma unroll
    for (int db = 0; db < 16; ++db) O[db] = floatx4_t{0.f, 0.f, 0.f, 0.f};

    // cache rows of this lane's position in each of the wave's tiles (clamped
    // into the request), fetched once so that no tile waits on a table read
    const int64_t bt0 = (int64_t)r * max_pages;
    uint32_t rows[NTILE];
#pragma unroll
    for (int t = 0; t < NTILE; ++t) {
        const int j = min(wk0 + 16 * t + n, L - 1);
        int pg = bt[bt0 + j / P];
        pg = min(max(pg, 0), num_pages - 1);
        rows[t] = ((uint32_t)pg * (uint32_t)Hkv + (uint32_t)g) * (uint32_t)P + (uint32_t)(j % P);
    }
    // the table reads land here, before any cache load is issued, so that no
    // later wait for them has to count the cache loads in flight behind them
    __builtin_amdgcn_s_waitcnt(0);

    // Every wave runs all its tiles and issues every load: positions past the
    // request read the request's last row again (a cache hit, not HBM
    // traffic) and get p = 0.  No load sits behind a branch, so the compiler's
    // wait counts are exact.  K fragments (B operand of the scores: lane n
    // holds 8 dims of position n) are reloaded once the scores' MFMAs have
    // taken them; V rows (lane l holds dims 4 l .. 4 l + 3 of each of the 16
    // positions) go to LDS at the top of a tile, which frees their registers
    // for the next tile's rows.  Either load thus has most of a tile to land.
    // An fp8 cache moves the same 16-byte pieces with half the loads: K, lane
    // (n, kg) reads dims 64 j + 16 kg .. + 15 of position n for j = 0..3, and
    // the scores' k-step 2 j + b takes its half b (q's fragments are read in
    // the same dim order: any order of the contraction works if A and B agree);
    // V, lanes 0-31 and 32-63 read two positions' rows, 8 dims per lane.  Both
    // are widened to bf16 exactly, at the MFMA and at the LDS tile.
    constexpr int NKL = FP8 ? 4 : 8;   // K loads per tile
    constexpr int NVL = FP8 ? 8 : 16;  // V loads per tile
    // tiles in flight behind the one being computed: the fp8 tiles' registers
    // (32 per tile) leave room for two within two waves per SIMD, bf16 (64) for one
    constexpr int DEPTH = FP8 ? 2 : 1;
    using KRaw = typename std::conditional<FP8, uint4, bf16x8_t>::type;
    KRaw kf[DEPTH][NKL];
    uint2 vraw[DEPTH][NVL];
    const uint8_t *const kc8 = reinterpret_cast<const uint8_t *>(kc);
    const uint8_t *const vc8 = reinterpret_cast<const uint8_t *>(vc);
    auto load_k = [&](int t, int b) {
        if constexpr (FP8) {
            const uint8_t *krow = kc8 + (size_t)rows[t] * D + 16 * kg;
#pragma unroll
            for (int j = 0; j < NKL; ++j) kf[b][j] = *reinterpret_cast<const uint4 *>(krow + 64 * j);
        } else {
            const uint8_t *krow = kc8 + ((size_t)rows[t] * D + 8 * kg) * 2;
#pragma unroll
            for (int ks = 0; ks < NKL; ++ks) kf[b][ks] = *reinterpret_cast<const bf16x8_t *>(krow + 64 * ks);
        }
    };
    auto load_v = [&](int t, int b) {
#pragma unroll
        for (int i = 0; i < NVL; ++i) {
            if constexpr (FP8) {
                const uint32_t ra = __builtin_amdgcn_readlane(rows[t], 2 * i);
                const uint32_t rb = __builtin_amdgcn_readlane(rows[t], 2 * i + 1);
                const uint32_t ri = lane < 32 ? ra : rb;
                vraw[b][i] = *reinterpret_cast<const uint2 *>(vc8 + (size_t)ri * D + 8 * (lane & 31));
            } else {
                const uint32_t ri = __builtin_amdgcn_readlane(rows[t], i);
                vraw[b][i] = *reinterpret_cast<const uint2 *>(vc8 + ((size_t)ri * D + 4 * lane) * 2);
            }
        }
    };
#pragma unroll
    for (int t = 0; t < DEPTH; ++t) {
        load_k(t, t);
        load_v(t, t);
    }
    // the scheduler keeps the phases below in program order: loads issued
    // early stay early, and no wait for a later load lands in front of one
    // for an earlier load (wait counts complete in order)
    __builtin_amdgcn_sched_barrier(0);
    // rotated q of the group (rounded to fp32), scaled by log2(e) / sqrt(D), as
    // hi + mid + lo bf16, while the first tiles land
    if (!appender) angle();
#pragma unroll
    for (int m = 0; m < 16; ++m) {
        const float x = m < G ? (float)rope(qv[m], qp[m]) * qscale : 0.f;
        const uint16_t h0 = bf16_rne_bits(x);
        const float r1 = x - __uint_as_float(uint32_t(h0) << 16);
        const uint16_t h1 = bf16_rne_bits(r1);
        const float r2 = r1 - __uint_as_float(uint32_t(h1) << 16);
        qf[0][m][tid] = h0;
        qf[1][m][tid] = h1;
        qf[2][m][tid] = bf16_rne_bits(r2);
    }
    // p rows of heads 8 .. 15 are never written: zero them once
    for (int e = lane; e < 2 * 16 * 16 / 2; e += 64) reinterpret_cast<uint32_t *>(pt)[e] = 0u;
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    // transposed-read offsets: lane 4j + q of group kg reads row 4 kg + j,
    // columns 4q .. 4q + 3
    const uint32_t tr_row = (uint32_t)(4 * kg + (n >> 2)), tr_col = (uint32_t)(8 * (n & 3));
#pragma unroll
    for (int t = 0; t < NTILE; ++t) {
        const int b = t % DEPTH;
        const int nt = L - (wk0 + 16 * t);  // positions of the tile inside the request (may be <= 0)
        // scores (log2 units): S[i] = row 4 kg + i, position wk0 + 16 t + n; one
        // accumulator per q term keeps three independent MFMA chains of 8 in
        // flight instead of one of 24 (summed smallest first)
        floatx4_t Sp[3];
#pragma unroll
        for (int p = 0; p < 3; ++p) Sp[p] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
            for (int p = 2; p >= 0; --p) {
                const int dim0 = FP8 ? 64 * (ks >> 1) + 16 * kg + 8 * (ks & 1) : 32 * ks + 8 * kg;
                const bf16x8_t a = *reinterpret_cast<const bf16x8_t *>(&qf[p][n][dim0]);
                bf16x8_t bk;
                if constexpr (FP8) {
                    const uint4 w = kf[b][ks >> 1];
                    const uint2 lo = fp8x4_to_bf16x4((ks & 1) ? w.z : w.x);
                    const uint2 hi = fp8x4_to_bf16x4((ks & 1) ? w.w : w.y);
                    bk = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
                } else {
                    bk = kf[b][ks];
                }
                Sp[p] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bk, Sp[p], 0, 0, 0);
            }
        }
        const floatx4_t S = (Sp[2] + Sp[1]) + Sp[0];
        __builtin_amdgcn_sched_barrier(0);
        if (t + DEPTH < NTILE) load_k(t + DEPTH, b);
        __builtin_amdgcn_sched_barrier(0);
        // online softmax with a lazily moved reference max: p = 2^(s - Mu) stays
        // below 2^8; the reference (and with it O and the sums) moves only when a
        // score exceeds it by more than that
        float sc[4], tmax[4];
        bool need = false;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sc[i] = n < nt ? S[i] : -INFINITY;
            tmax[i] = row16_max(sc[i]);
            need |= tmax[i] > Mu[i] + RESCALE_LOG2;
        }
        if (__builtin_amdgcn_ballot_w64(need) != 0) {
            floatx4_t alv;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float mnew = tmax[i] > Mu[i] + RESCALE_LOG2 ? tmax[i] : Mu[i];
                const float al = Mu[i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(Mu[i] - mnew);
                lsum[i] *= al;
                alv[i] = al;
                Mu[i] = mnew;
            }
            // whole accumulators, so that they keep their registers across the branch
#pragma unroll
            for (int db = 0; db < 16; ++db) O[db] *= alv;
        }
        float pr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float mref = Mu[i] == -INFINITY ? 0.f : Mu[i];
            pr[i] = __builtin_amdgcn_exp2f(sc[i] - mref);
            lsum[i] += pr[i];
        }
        // p as bf16 hi + lo at [position n][heads 4 kg .. 4 kg + 3] (heads < 8)
        if (kg < 2) {
            uint32_t hi[2], lo[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const uint16_t h0 = bf16_rne_bits(pr[2 * e]), h1 = bf16_rne_bits(pr[2 * e + 1]);
                const uint16_t l0 = bf16_rne_bits(pr[2 * e] - __uint_as_float(uint32_t(h0) << 16));
                const uint16_t l1 = bf16_rne_bits(pr[2 * e + 1] - __uint_as_float(uint32_t(h1) << 16));
                hi[e] = uint32_t(h0) | (uint32_t(h1) << 16);
                lo[e] = uint32_t(l0) | (uint32_t(l1) << 16);
            }
            *reinterpret_cast<uint2 *>(pt + n * 32 + 8 * kg) = make_uint2(hi[0], hi[1]);
            *reinterpret_cast<uint2 *>(pt + 512 + n * 32 + 8 * kg) = make_uint2(lo[0], lo[1]);
        }
        // V rows of this tile to LDS, then the next tile's rows into the registers
#pragma unroll
        for (int i = 0; i < NVL; ++i) {
            if constexpr (FP8) {
                const uint2 lo = fp8x4_to_bf16x4(vraw[b][i].x), hi = fp8x4_to_bf16x4(vraw[b][i].y);
                *reinterpret_cast<uint4 *>(vt + (2 * i + (lane >> 5)) * VROW + 16 * (lane & 31)) =
                    make_uint4(lo.x, lo.y, hi.x, hi.y);
            } else {
                *reinterpret_cast<uint2 *>(vt + i * VROW + 8 * lane) = vraw[b][i];
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        if (t + DEPTH < NTILE) load_v(t + DEPTH, b);
        __builtin_amdgcn_sched_barrier(0);
        wave_lds_sync();
        // O += P V on the matrix cores: A = p (heads x 16 positions, hi and lo),
        // B = V (16 positions x 16 dims per block), both by transposed reads
        const s16x4_t ph = lds_read_tr(pt, tr_row * 32 + tr_col);
        const s16x4_t pl = lds_read_tr(pt, 512 + tr_row * 32 + tr_col);
#pragma unroll
        for (int db = 0; db < 16; ++db) {
            const s16x4_t vb = lds_read_tr(vt, tr_row * VROW + 32 * db + tr_col);
            O[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pl, vb, O[db], 0, 0, 0);
            O[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ph, vb, O[db], 0, 0, 0);
        }
        wave_lds_sync();
    }

    // the wave's (reference max, sum) per head row, then the block merge
#pragma unroll
    for (int i = 0; i < 4; ++i) lsum[i] = group_sum<16>(lsum[i]);
    if (n == 0 && kg < 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) wml[w][4 * kg + i] = make_float2(Mu[i], lsum[i]);
    }
    __syncthreads();
    // this wave's O rows, scaled to the block's max, into its own region
    float *const ob = reinterpret_cast<float *>(wreg[w]);
    if (kg < 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int h = 4 * kg + i;
            if (h < G) {
                float mb = wml[0][h].x;
#pragma unroll
                for (int u = 1; u < NWAVE; ++u) mb = fmaxf(mb, wml[u][h].x);
                const float scw = wml[w][h].x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(wml[w][h].x - mb);
#pragma unroll
                for (int db = 0; db < 16; ++db) ob[h * D + 16 * db + n] = O[db][i] * scw;
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < G; ++h) {
        float acc = 0.f;
#pragma unroll
        for (int u = 0; u < NWAVE; ++u) acc += reinterpret_cast<const float *>(wreg[u])[h * D + tid];
        const int64_t ph = ((int64_t)r * Hq + g * G + h) * nsplit + s;
        po[ph * D + tid] = acc;
        if (tid == 0) {
            float mb = wml[0][h].x;
#pragma unroll
            for (int u = 1; u < NWAVE; ++u) mb = fmaxf(mb, wml[u][h].x);
            float l = 0.f;
#pragma unroll
            for (int u = 0; u < NWAVE; ++u)
                if (wml[u][h].x != -INFINITY) l += wml[u][h].y * __builtin_amdgcn_exp2f(wml[u][h].x - mb);
            pml[ph] = make_float2(mb, l);
        }
    }
}

template <typename TA, typename TY>
__global__ __launch_bounds__(D) void gqa_combine_kernel(
    const float *__restrict__ po, const float2 *__restrict__ pml, const TA *__restrict__ gate,
    int64_t gate_ld, const int32_t *__restrict__ lens, int32_t Hq, int32_t lmax, int32_t nsplit,
    float v_scale, TY *__restrict__ y, float *__restrict__ o) {
    const int rh = blockIdx.x;
    const int r = rh / Hq, h = rh % Hq;
    const int d = threadIdx.x;
    // the gate and, for up to NSR runs, every partial are loaded together (one
    // round trip after the length instead of three)
    constexpr int NSR = 8;
    const float gt = to_f32(gate[(int64_t)r * gate_ld + h * D + d]);
    const int L = lens[r];
    float out = 0.f;
    if (L >= 1 && L <= lmax) {
        const int ns = (L + SPLIT - 1) / SPLIT;
        const float2 *ml = pml + (int64_t)rh * nsplit;
        const float *pd = po + (int64_t)rh * nsplit * D + d;
        float num = 0.f, den = 0.f;
        if (ns <= NSR) {
            float2 e[NSR];
            float pv[NSR];
#pragma unroll
            for (int s = 0; s < NSR; ++s) {
                e[s] = s < ns ? ml[s] : make_float2(-INFINITY, 0.f);
                pv[s] = s < ns ? pd[(int64_t)s * D] : 0.f;
            }
            float mx = e[0].x;
#pragma unroll
            for (int s = 1; s < NSR; ++s) mx = fmaxf(mx, e[s].x);
#pragma unroll
            for (int s = 0; s < NSR; ++s) {
                if (s < ns) {
                    const float wgt = __builtin_amdgcn_exp2f(e[s].x - mx);
                    den = fmaf(wgt, e[s].y, den);
                    num = fmaf(wgt, pv[s], num);
                }
            }
        } else {
            float mx = -INFINITY;
            for (int s = 0; s < ns; ++s) mx = fmaxf(mx, ml[s].x);
            for (int s = 0; s < ns; ++s) {
                const float2 e = ml[s];
                const float wgt = __builtin_amdgcn_exp2f(e.x - mx);
                den = fmaf(wgt, e.y, den);
                num = fmaf(wgt, pd[(int64_t)s * D], num);
            }
        }
        out = num / den * v_scale;
    }
    if (o != nullptr) o[(int64_t)rh * D + d] = out;
    y[(int64_t)rh * D + d] = from_f32<TY>(out / (1.0f + expf(-gt)));
}

template <int G, bool FP8, typename TA>
static hipError_t launch_attn(const GqaArgs &a, hipStream_t st, int32_t lmax, int32_t nsplit, float2 *pml,
                              float *po) {
    // an fp8 cache: k_scale rides on q (the MFMAs see the codes), v_scale on the combine
    const float qscale = 1.4426950408889634f / sqrtf((float)D) * (FP8 ? a.k_scale : 1.f);
    const int64_t blocks = (int64_t)a.R * a.Hkv * nsplit;
    hipLaunchKernelGGL((gqa_attn_split_kernel<G, FP8, TA>), dim3((unsigned)blocks), dim3(64 * NWAVE), 0, st,
                       (const TA *)a.q, a.q_ld, (const TA *)a.k, (const TA *)a.v, a.kv_ld, a.k_cache, a.v_cache,
                       FP8 ? a.k_scale : 1.f, FP8 ? a.v_scale : 1.f, a.bt, a.max_pages, a.lens, a.Hq, a.Hkv,
                       a.rd, a.P, a.num_pages, lmax, nsplit, a.theta, qscale, po, pml);
    return hipGetLastError();
}

template <bool FP8, typename TA>
static hipError_t launch_attn_g(const GqaArgs &a, hipStream_t st, int32_t lmax, int32_t nsplit, float2 *pml,
                                float *po) {
    switch (a.Hq / a.Hkv) {
        case 1: return launch_attn<1, FP8, TA>(a, st, lmax, nsplit, pml, po);
        case 2: return launch_attn<2, FP8, TA>(a, st, lmax, nsplit, pml, po);
        case 3: return launch_attn<3, FP8, TA>(a, st, lmax, nsplit, pml, po);
        case 4: return launch_attn<4, FP8, TA>(a, st, lmax, nsplit, pml, po);
        case 5: return launch_attn<5, FP8, TA>(a, st, lmax, nsplit, pml, po);
        case 6: return launch_attn<6, FP8, TA>(a, st, lmax, nsplit, pml, po);
        case 7: return launch_attn<7, FP8, TA>(a, st, lmax, nsplit, pml, po);
        default: return launch_attn<8, FP8, TA>(a, st, lmax, nsplit, pml, po);
    }
}

template <typename TA, typename TY>
static hipError_t launch_all(const GqaArgs &a, hipStream_t st) {
    const int64_t lmax64 = std::min<int64_t>(a.max_ctx, (int64_t)a.max_pages * a.P);
    const int32_t lmax = (int32_t)lmax64;
    const int32_t nsplit = (a.max_ctx + SPLIT - 1) / SPLIT;
    float2 *pml = (float2 *)a.ws;
    float *po = (float *)((uint8_t *)pml + gqa_ws_ml_bytes(a.R, a.Hq, nsplit));
    hipError_t e = a.kv_fp8 ? launch_attn_g<true, TA>(a, st, lmax, nsplit, pml, po)
                            : launch_attn_g<false, TA>(a, st, lmax, nsplit, pml, po);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((gqa_combine_kernel<TA, TY>), dim3((unsigned)(a.R * a.Hq)), dim3(D), 0, st, po, pml,
                       (const TA *)a.gate, a.gate_ld, a.lens, a.Hq, lmax, nsplit, a.v_scale, (TY *)a.y, a.o);
    return hipGetLastError();
}

}  // namespace gqa

size_t gqa_ws_ml_bytes(int64_t R, int64_t Hq, int64_t nsplit) {
    return (size_t)((R * Hq * nsplit * 8 + 255) / 256 * 256);
}
size_t gqa_ws_bytes(int64_t R, int64_t Hq, int64_t max_ctx) {
    const int64_t nsplit = (max_ctx + gqa::SPLIT - 1) / gqa::SPLIT;
    return gqa_ws_ml_bytes(R, Hq, nsplit) + (size_t)(R * Hq * nsplit * gqa::D * 4);
}

hipError_t launch_gqa_decode(const GqaArgs &a, hipStream_t s) {
    if (a.act_bf16) return a.y_bf16 ? gqa::launch_all<bf16, bf16>(a, s) : gqa::launch_all<bf16, float>(a, s);
    return a.y_bf16 ? gqa::launch_all<float, bf16>(a, s) : gqa::launch_all<float, float>(a, s);
}

}  // namespace gdn
