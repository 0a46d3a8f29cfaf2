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
                const float inv = 1.0f / sqrtf(ss + l2_eps);
                TO *dst = c < nq ? q + (int64_t)t * nq + c : k + (int64_t)t * nq + (c - nq);
                st2(dst, y0 * inv, y1 * inv);
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

template <int D, typename TX, typename TW, typename TO>
static hipError_t launch_conv_t(const ConvArgs &a, hipStream_t s) {
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

}  // namespace gdn
