// Causal depthwise conv1d (4 taps) + SiLU + per-head L2 norm of q and k, over a
// packed varlen batch, with the per-request conv history in a slot pool.
//
// Operator ("Qwen3.8-27B: from model structure to the vLLM inference
// dataflow", section 01, per-layer operator table, conv row):
//   c_t = SiLU(sum_{i=0..3} w_i * x_{t-i});  q = normalize(q); k = normalize(k)
// and the data-structure table's conv-history row: three past inputs are kept
// per request and layer; the 4-tap window includes the current input.
//
// Work split (HBM-bound: 4 MACs per element read):
//   * one wavefront owns 128 consecutive channels (2 per lane, so bf16 rows are
//     read as 4-byte pairs and a 128-wide head is one wave-local reduction);
//   * a block of 4 waves owns 512 channels for a tile of consecutive tokens,
//     sliding the 3-entry window in registers across the tile;
//   * only a request's first three tokens read its history slot, so those three
//     tokens always belong to the block whose tile holds the request's first
//     token (a tile may run up to two tokens past its end to keep them).  That
//     block, after its tokens, writes the request's new history: the thread that
//     read a history entry is the only one that ever writes it, so one launch
//     is race-free without any grid-wide ordering.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

constexpr int CONV_WAVES = 4;
constexpr int CONV_CH_PER_WAVE = 128;
constexpr int CONV_CH_PER_BLOCK = CONV_WAVES * CONV_CH_PER_WAVE;

// Request holding token t: a direct guess (decode batches have request t at
// token t), else a binary search.
__device__ __forceinline__ int locate_request(const int32_t *__restrict__ qsl, int n, int t) {
    if (t < n && qsl[t] <= t && t < qsl[t + 1]) return t;
    return find_request(qsl, n, t);
}

template <int D, typename TX, typename TW, typename TO>
__global__ __launch_bounds__(256) void conv1d_silu_l2_kernel(
    const TX *__restrict__ x, int64_t x_ld, const TW *__restrict__ w, TX *__restrict__ pool,
    const int32_t *__restrict__ qsl, const int32_t *__restrict__ slots,
    const uint8_t *__restrict__ has_init, int32_t nreq, int32_t T, int32_t C, int32_t nq,
    int32_t tile, float l2_eps, TO *__restrict__ q, TO *__restrict__ k, TO *__restrict__ v) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int c = (blockIdx.y * CONV_WAVES + wave) * CONV_CH_PER_WAVE + 2 * lane;
    const bool active = c < C;  // C is a multiple of D >= 16, so pairs never straddle C
    const int t_begin = blockIdx.x * tile;
    const int t_nom_end = min(T, t_begin + tile);
    const int nqk = 2 * nq;
    const int nv = C - nqk;

    // taps for the two channels: w[c][i] multiplies x[t - i]
    float w0[4], w1[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        w0[i] = active ? ld(w + (int64_t)c * 4 + i) : 0.f;
        w1[i] = active ? ld(w + (int64_t)(c + 1) * 4 + i) : 0.f;
    }

    const int r_first = locate_request(qsl, nreq, t_begin);
    float2 h3 = make_float2(0.f, 0.f), h2 = h3, h1 = h3;  // x_{t-3}, x_{t-2}, x_{t-1}
    bool have_window = false;
    int r = r_first;
    for (int t = t_begin; t < T; ++t) {
        while (t >= qsl[r + 1]) ++r;  // skips empty requests too
        const int p = t - qsl[r];
        if (t >= t_nom_end && (p == 0 || p >= 3)) break;          // past the tile
        if (p >= 1 && p <= 2 && t - p < t_begin) {                // owned by an earlier tile
            have_window = false;
            continue;
        }
        float2 x0 = active ? ld2(x + (int64_t)t * x_ld + c) : make_float2(0.f, 0.f);
        if (!have_window || p == 0) {
            // (re)build the window from the request's own rows and history
            const bool hi = has_init == nullptr || has_init[r] != 0;
            const int64_t hbase = ((int64_t)slots[r] * C + c) * 3;
            float2 hw[3];
#pragma unroll
            for (int lag = 3; lag >= 1; --lag) {
                float2 val = make_float2(0.f, 0.f);
                if (active) {
                    if (p - lag >= 0) {
                        val = ld2(x + (int64_t)(t - lag) * x_ld + c);
                    } else if (hi) {
                        const int j = 3 + p - lag;  // history index, oldest first
                        val = make_float2(ld(pool + hbase + j), ld(pool + hbase + 3 + j));
                    }
                }
                hw[3 - lag] = val;
            }
            h3 = hw[0]; h2 = hw[1]; h1 = hw[2];
            have_window = true;
        }
        float y0 = w0[0] * x0.x + w0[1] * h1.x + w0[2] * h2.x + w0[3] * h3.x;
        float y1 = w1[0] * x0.y + w1[1] * h1.y + w1[2] * h2.y + w1[3] * h3.y;
        y0 = silu_f(y0);
        y1 = silu_f(y1);
        // per-head L2 norm (heads are D channels = D/2 lanes, aligned)
        const float ss = group_sum<D / 2>(y0 * y0 + y1 * y1);
        if (active) {
            if (c < nqk) {
                if (q != nullptr) {  // null: v-only mode
                    const float inv = 1.0f / sqrtf(ss + l2_eps);
                    TO *dst = c < nq ? q + (int64_t)t * nq + c : k + (int64_t)t * nq + (c - nq);
                    st2(dst, y0 * inv, y1 * inv);
                }
            } else {
                st2(v + (int64_t)t * nv + (c - nqk), y0, y1);
            }
        }
        h3 = h2; h2 = h1; h1 = x0;
    }

    // New history of every request whose first token lies in this tile: the
    // last three entries of [old history | request rows].  This thread alone
    // read the old entries above.
    if (!active) return;
    for (int rr = (qsl[r_first] == t_begin ? r_first : r_first + 1);
         rr < nreq && qsl[rr] < t_nom_end; ++rr) {
        const int t0 = qsl[rr];
        const int L = qsl[rr + 1] - t0;
        if (L <= 0) continue;  // empty request: slot untouched
        const bool hi = has_init == nullptr || has_init[rr] != 0;
        TX *hp = pool + ((int64_t)slots[rr] * C + c) * 3;
        TX nv0[3], nv1[3];
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const int m = L + j;  // index into [h0, h1, h2, x0 .. x_{L-1}]
            if (m >= 3) {
                const TX *xp = x + (int64_t)(t0 + m - 3) * x_ld + c;
                nv0[j] = xp[0];
                nv1[j] = xp[1];
            } else if (hi) {
                nv0[j] = hp[m];
                nv1[j] = hp[3 + m];
            } else {
                nv0[j] = from_f32<TX>(0.0f);
                nv1[j] = from_f32<TX>(0.0f);
            }
        }
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            hp[j] = nv0[j];
            hp[3 + j] = nv1[j];
        }
    }
}

// ---------------------------------------------------------------------------
// Vectorised variant for long packed batches: a lane owns 8 consecutive
// channels (16-byte accesses), a wave 512 channels, and a wave loads its whole
// tile of U tokens plus the 3 rows before it and the 2 after it up front, so a
// tile costs one memory latency instead of one per token.  Token ownership and
// the history hand-over are the same as above; the history of 8 channels is 24
// contiguous elements, moved as raw bits so copies stay bit-exact.
// ---------------------------------------------------------------------------
// N consecutive elements held as raw 32-bit words (N * sizeof(TX) a multiple of
// 16 bytes); element access is shifts and masks on registers.
template <typename TX, int N> struct RawVec {
    static constexpr int NV = N * (int)sizeof(TX) / 16;
    uint4 v[NV];
    __device__ __forceinline__ void load(const TX *p) {
#pragma unroll
        for (int i = 0; i < NV; ++i) v[i] = reinterpret_cast<const uint4 *>(p)[i];
    }
    __device__ __forceinline__ void store(TX *p) const {
#pragma unroll
        for (int i = 0; i < NV; ++i) reinterpret_cast<uint4 *>(p)[i] = v[i];
    }
    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int i = 0; i < NV; ++i) v[i] = make_uint4(0, 0, 0, 0);
    }
    __device__ __forceinline__ uint32_t word(int wi) const {
        const uint4 &q = v[wi >> 2];
        return (wi & 3) == 0 ? q.x : (wi & 3) == 1 ? q.y : (wi & 3) == 2 ? q.z : q.w;
    }
    __device__ __forceinline__ void set_word(int wi, uint32_t val) {
        uint4 &q = v[wi >> 2];
        if ((wi & 3) == 0) q.x = val;
        else if ((wi & 3) == 1) q.y = val;
        else if ((wi & 3) == 2) q.z = val;
        else q.w = val;
    }
    // raw bits of element i (bf16: low 16 bits)
    __device__ __forceinline__ uint32_t bits(int i) const {
        if constexpr (sizeof(TX) == 2) return (word(i >> 1) >> (16 * (i & 1))) & 0xffffu;
        else return word(i);
    }
    __device__ __forceinline__ float f(int i) const {
        if constexpr (sizeof(TX) == 2) return __uint_as_float(bits(i) << 16);
        else return __uint_as_float(word(i));
    }
    // set all elements from raw bits
    template <int M> __device__ __forceinline__ void set_bits(const uint32_t (&b)[M]) {
        static_assert(M == N, "element count");
        if constexpr (sizeof(TX) == 2) {
#pragma unroll
            for (int wi = 0; wi < N / 2; ++wi) set_word(wi, b[2 * wi] | (b[2 * wi + 1] << 16));
        } else {
#pragma unroll
            for (int wi = 0; wi < N; ++wi) set_word(wi, b[wi]);
        }
    }
};

constexpr int CV_WAVE_CH = 512;  // 64 lanes x 8 channels
constexpr int CV_WAVES = 4;

// Output of one token for the lane's 8 channels: SiLU of the 4-tap sum, then
// the per-head L2 norm for q and k (a head is D / 8 lanes, aligned).
template <int D, typename TO>
__device__ __forceinline__ void conv_emit(const float (&wt)[4][8], const float (&xw)[4][8], bool active,
                                          int c, int t, int nq, int nqk, int nv, float l2_eps,
                                          TO *__restrict__ q, TO *__restrict__ k, TO *__restrict__ v) {
    float y[8];
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float a = wt[0][e] * xw[0][e] + wt[1][e] * xw[1][e] + wt[2][e] * xw[2][e] +
                        wt[3][e] * xw[3][e];
        y[e] = silu_f(a);
        ss += y[e] * y[e];
    }
    ss = group_sum<D / 8>(ss);
    if (active) {
        if (c < nqk) {
            if (q == nullptr) return;  // v-only mode: q and k are formed elsewhere
            const float inv = 1.0f / sqrtf(ss + l2_eps);
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] *= inv;
            store8(c < nq ? q + (int64_t)t * nq + c : k + (int64_t)t * nq + (c - nq), y);
        } else {
            store8(v + (int64_t)t * nv + (c - nqk), y);
        }
    }
}

template <int D, typename TX, typename TW, typename TO, int U>
__global__ __launch_bounds__(256) void conv1d_vec_kernel(
    const TX *__restrict__ x, int64_t x_ld, const TW *__restrict__ w, TX *__restrict__ pool,
    const int32_t *__restrict__ qsl, const int32_t *__restrict__ slots,
    const uint8_t *__restrict__ has_init, int32_t nreq, int32_t T, int32_t C, int32_t nq,
    float l2_eps, TO *__restrict__ q, TO *__restrict__ k, TO *__restrict__ v) {
    static_assert(U + 4 <= 32, "start mask");
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int c = (blockIdx.y * CV_WAVES + wave) * CV_WAVE_CH + 8 * lane;
    const bool active = c < C;  // C is a multiple of 8 and of D, so a lane never straddles q|k|v
    const int t_begin = blockIdx.x * U;
    const int t_nom_end = min(T, t_begin + U);
    const int nqk = 2 * nq;
    const int nv = C - nqk;
    // v-only mode (q == nullptr): q / k lanes only rewrite their history; heads
    // never straddle the q|k|v boundaries, so every reduction group agrees
    const bool outputs = q != nullptr || c >= nqk;

    // taps: wt[i][e] multiplies x[t - i] in channel c + e (w is [C][4], 32 contiguous elements)
    float wt[4][8];
    {
        RawVec<TW, 32> wr;
        if (active) wr.load(w + (int64_t)c * 4);
        else wr.zero();
#pragma unroll
        for (int e = 0; e < 8; ++e)
#pragma unroll
            for (int i = 0; i < 4; ++i) wt[i][e] = wr.f(4 * e + i);
    }
    // rows t_begin - 3 .. t_begin + U - 1 (xr[m] is row t_begin - 3 + m)
    RawVec<TX, 8> xr[U + 3];
#pragma unroll
    for (int m = 0; m < U + 3; ++m) {
        const int row = t_begin - 3 + m;
        if (outputs && active && row >= 0 && row < T) xr[m].load(x + (int64_t)row * x_ld + c);
        else xr[m].zero();
    }

    // bit b of `starts`: token t_begin - 2 + b is the first token of a non-empty request
    uint32_t starts = 0;
    {
        const int lo = max(t_begin - 2, 0);
        if (lo < T) {
            for (int r = locate_request(qsl, nreq, lo); r < nreq && qsl[r] < t_begin + U + 2; ++r)
                if (qsl[r + 1] > qsl[r] && qsl[r] >= t_begin - 2) starts |= 1u << (qsl[r] - (t_begin - 2));
        }
    }

    // tokens whose 4-token window lies inside their request (no start among t-2 .. t)
#pragma unroll
    for (int j = 0; j < U; ++j) {
        const int t = t_begin + j;
        if (outputs && t < T && ((starts >> j) & 7u) == 0) {  // uniform over each head
            float xw[4][8];  // xw[i] = x[t - i]
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int e = 0; e < 8; ++e) xw[i][e] = xr[j + 3 - i].f(e);
            conv_emit<D>(wt, xw, active, c, t, nq, nqk, nv, l2_eps, q, k, v);
        }
    }

    // each request starting in [t_begin, t_nom_end): its first (up to) three
    // tokens read the request's history, and this lane then writes the new
    // history (it alone read the old entries)
    for (int j = 0; j < U; ++j) {
        if (!((starts >> (j + 2)) & 1u)) continue;
        const int t0 = t_begin + j;
        if (t0 >= t_nom_end) break;
        const int rr = locate_request(qsl, nreq, t0);
        const int L = qsl[rr + 1] - t0;
        const bool hi = has_init == nullptr || has_init[rr] != 0;
        TX *hp = pool + ((int64_t)slots[rr] * C + c) * 3;
        RawVec<TX, 24> oldh;
        if (active && hi) oldh.load(hp);
        else oldh.zero();
#pragma unroll
        for (int m = 0; m < 3; ++m) {
            if (m >= L || !outputs) break;  // uniform over each head
            float xw[4][8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (m >= i) {
                    RawVec<TX, 8> xv;
                    if (active) xv.load(x + (int64_t)(t0 + m - i) * x_ld + c);
                    else xv.zero();
#pragma unroll
                    for (int e = 0; e < 8; ++e) xw[i][e] = xv.f(e);
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) xw[i][e] = oldh.f(3 * e + 3 + m - i);  // oldest first
                }
            }
            conv_emit<D>(wt, xw, active, c, t0 + m, nq, nqk, nv, l2_eps, q, k, v);
        }
        if (active) {
            // new history: the last three entries of [old history | request rows]
            uint32_t nb[24];
#pragma unroll
            for (int jj = 0; jj < 3; ++jj) {
                const int m = L + jj;  // index into [h0, h1, h2, x0 .. x_{L-1}]
                if (m >= 3) {
                    RawVec<TX, 8> xv;
                    xv.load(x + (int64_t)(t0 + m - 3) * x_ld + c);
#pragma unroll
                    for (int e = 0; e < 8; ++e) nb[3 * e + jj] = xv.bits(e);
                } else {
                    // m = L + jj <= 2 (L >= 1): entry jj + 1 or jj + 2 of the old history
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        nb[3 * e + jj] = m == jj + 1 ? oldh.bits(3 * e + jj + 1)
                                                     : oldh.bits(3 * e + (jj + 2 < 3 ? jj + 2 : 2));
                }
            }
            RawVec<TX, 24> newh;
            newh.set_bits(nb);
            newh.store(hp);
        }
    }
}

static bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

template <int D, typename TX, typename TW, typename TO>
static hipError_t launch_conv_t(const ConvArgs &a, hipStream_t s) {
    // long batches with 16-byte aligned rows take the vectorised kernel
    const bool vec_ok = a.x_ld % (16 / sizeof(TX)) == 0 && aligned16(a.x) && aligned16(a.w) &&
                        aligned16(a.pool) && aligned16(a.q) && aligned16(a.k) && aligned16(a.v);  // null is aligned
    if (a.T > 1024 && vec_ok) {
        constexpr int U = sizeof(TX) == 2 ? 16 : 8;
        dim3 grid((a.T + U - 1) / U, (a.C + CV_WAVES * CV_WAVE_CH - 1) / (CV_WAVES * CV_WAVE_CH));
        hipLaunchKernelGGL((conv1d_vec_kernel<D, TX, TW, TO, U>), grid, dim3(256), 0, s,
                           (const TX *)a.x, a.x_ld, (const TW *)a.w, (TX *)a.pool, a.qsl, a.slots,
                           a.has_init, a.nreq, a.T, a.C, a.nq, a.l2_eps, (TO *)a.q, (TO *)a.k,
                           (TO *)a.v);
        return hipGetLastError();
    }
    // short tiles when the batch is small (decode), longer ones for prefill
    const int tile = a.T <= 1024 ? 1 : (a.T <= 16384 ? 8 : 16);
    dim3 grid((a.T + tile - 1) / tile, (a.C + CONV_CH_PER_BLOCK - 1) / CONV_CH_PER_BLOCK);
    hipLaunchKernelGGL((conv1d_silu_l2_kernel<D, TX, TW, TO>), grid, dim3(256), 0, s,
                       (const TX *)a.x, a.x_ld, (const TW *)a.w, (TX *)a.pool, a.qsl, a.slots,
                       a.has_init, a.nreq, a.T, a.C, a.nq, tile, a.l2_eps, (TO *)a.q, (TO *)a.k,
                       (TO *)a.v);
    return hipGetLastError();
}

template <int D, typename TX, typename TW>
static hipError_t launch_conv_o(const ConvArgs &a, hipStream_t s) {
    return a.act_bf16 ? launch_conv_t<D, TX, TW, bf16>(a, s) : launch_conv_t<D, TX, TW, float>(a, s);
}

template <int D, typename TX>
static hipError_t launch_conv_w(const ConvArgs &a, hipStream_t s) {
    return a.w_bf16 ? launch_conv_o<D, TX, bf16>(a, s) : launch_conv_o<D, TX, float>(a, s);
}

template <int D>
static hipError_t launch_conv_x(const ConvArgs &a, hipStream_t s) {
    return a.x_bf16 ? launch_conv_w<D, bf16>(a, s) : launch_conv_w<D, float>(a, s);
}

hipError_t launch_conv1d(const ConvArgs &a, hipStream_t s) {
    switch (a.D) {
        case 16: return launch_conv_x<16>(a, s);
        case 32: return launch_conv_x<32>(a, s);
        case 64: return launch_conv_x<64>(a, s);
        case 128: return launch_conv_x<128>(a, s);
        default: return hipErrorInvalidValue;
    }
}

// Prefix-cache snapshots of the conv history: after the first (j + 1) I tokens
// of request r the history is that prefix's last three conv inputs (I >= 3, so
// rows of x only), copied raw into slot snap_slots[r][j].  One block per
// (request, snapshot), threads over the channels.
template <typename TX>
__global__ __launch_bounds__(256) void snapshot_history_kernel(
    const TX *__restrict__ x, int64_t x_ld, TX *__restrict__ pool, const int32_t *__restrict__ qsl,
    const int32_t *__restrict__ snap_slots, int32_t interval, int32_t max_snaps, int32_t C) {
    const int r = blockIdx.x / max_snaps;
    const int j = blockIdx.x - r * max_snaps;
    const int t0 = qsl[r];
    const int L = qsl[r + 1] - t0;
    const int n = (j + 1) * interval;
    if (n > L) return;  // no such snapshot
    TX *hp = pool + (int64_t)snap_slots[(int64_t)r * max_snaps + j] * C * 3;
    const TX *xr = x + (int64_t)(t0 + n - 3) * x_ld;
    for (int c = threadIdx.x; c < C; c += 256) {
#pragma unroll
        for (int k = 0; k < 3; ++k) hp[(int64_t)c * 3 + k] = xr[(int64_t)k * x_ld + c];
    }
}

hipError_t launch_snapshot_history(const void *x, int64_t x_ld, bool x_bf16, void *pool,
                                   const int32_t *qsl, const int32_t *snap_slots, int32_t interval,
                                   int32_t max_snaps, int32_t nreq, int32_t C, hipStream_t s) {
    const dim3 grid((unsigned)((int64_t)nreq * max_snaps));
    if (x_bf16)
        hipLaunchKernelGGL(snapshot_history_kernel<bf16>, grid, dim3(256), 0, s, (const bf16 *)x, x_ld,
                           (bf16 *)pool, qsl, snap_slots, interval, max_snaps, C);
    else
        hipLaunchKernelGGL(snapshot_history_kernel<float>, grid, dim3(256), 0, s, (const float *)x, x_ld,
                           (float *)pool, qsl, snap_slots, interval, max_snaps, C);
    return hipGetLastError();
}

}  // namespace gdn
