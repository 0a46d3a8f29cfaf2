// Internal launcher interface of the GQA decode kernels (host-side struct,
// validated by the C-ABI layer before use).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

namespace gdn {

struct GqaArgs {
    const void *q; int64_t q_ld;
    const void *gate; int64_t gate_ld;
    const void *k, *v; int64_t kv_ld;
    bool act_bf16;
    void *k_cache, *v_cache;            // bf16 or e4m3 codes [num_pages, Hkv, P, D]
    bool kv_fp8;
    float k_scale, v_scale;             // 1 for a bf16 cache
    const int32_t *bt; int32_t max_pages;
    const int32_t *lens;
    int32_t R, Hq, Hkv, rd, P, num_pages, max_ctx;
    double theta;
    void *y; bool y_bf16;
    float *o;                           // nullable
    void *ws;
};

// workspace: partial (max, sum) per (request, query head, run of positions) |
// partial o (fp32, 256 per partial)
size_t gqa_ws_ml_bytes(int64_t R, int64_t Hq, int64_t nsplit);
size_t gqa_ws_bytes(int64_t R, int64_t Hq, int64_t max_ctx);

hipError_t launch_gqa_decode(const GqaArgs &a, hipStream_t s);

}  // namespace gdn
