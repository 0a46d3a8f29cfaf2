// C-ABI layer of the GQA decode entry points: argument validation (host code,
// before any HIP call) and dispatch.  The contract is in include/gqa.h.
#include "gqa.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <vector>

#include "gqa_launch.h"

namespace {

constexpr int kHeadDim = 256;
constexpr int kMaxGroup = 8;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool act_dtype(gdn_dtype d) { return d == GDN_F32 || d == GDN_BF16; }

gdn_status check_gqa_dims(const gqa_dims *d) {
    if (!d) return GDN_ERR_NULL;
    if (d->num_q_heads <= 0 || d->num_kv_heads <= 0 || d->num_q_heads % d->num_kv_heads != 0) return GDN_ERR_DIMS;
    if (d->num_q_heads / d->num_kv_heads > kMaxGroup) return GDN_ERR_DIMS;
    if (d->head_dim != kHeadDim) return GDN_ERR_DIMS;
    if (d->rotary_dim < 0 || d->rotary_dim > d->head_dim || d->rotary_dim % 2 != 0) return GDN_ERR_DIMS;
    if (d->num_q_heads > 4096) return GDN_ERR_DIMS;
    return GDN_OK;
}

}  // namespace

extern "C" {

size_t gqa_decode_workspace_bytes(const gqa_dims *dims, int32_t num_reqs, int32_t max_context_len) {
    if (check_gqa_dims(dims) != GDN_OK || num_reqs < 0 || max_context_len < 1) return 0;
    return gdn::gqa_ws_bytes(num_reqs, dims->num_q_heads, max_context_len);
}

gdn_status gqa_decode_paged(const gqa_dims *dims, const void *q, int64_t q_ld, const void *gate,
                            int64_t gate_ld, const void *k, const void *v, int64_t kv_ld,
                            gdn_dtype act_dt, void *k_cache, void *v_cache, gdn_dtype cache_dt,
                            float k_scale, float v_scale,
                            const int32_t *block_tables, int32_t max_pages_per_req,
                            const int32_t *context_lens, int32_t num_reqs, int32_t num_pages,
                            int32_t page_size, int32_t max_context_len, double rope_theta, void *y,
                            gdn_dtype y_dt, float *o, void *workspace, size_t workspace_bytes,
                            void *stream) {
    gdn_status st = check_gqa_dims(dims);
    if (st != GDN_OK) return st;
    if (!act_dtype(act_dt) || !act_dtype(y_dt) || (cache_dt != GDN_BF16 && cache_dt != GDN_FP8_E4M3))
        return GDN_ERR_DTYPE;
    const bool fp8 = cache_dt == GDN_FP8_E4M3;
    if (fp8 && !(std::isfinite(k_scale) && k_scale > 0.f && std::isfinite(v_scale) && v_scale > 0.f))
        return GDN_ERR_SHAPE;
    if (num_reqs < 0 || max_pages_per_req < 1 || num_pages < 1 || page_size < 1 || max_context_len < 1)
        return GDN_ERR_SHAPE;
    const int64_t Hq = dims->num_q_heads, Hkv = dims->num_kv_heads, D = dims->head_dim;
    if (q_ld < Hq * D || gate_ld < Hq * D || kv_ld < Hkv * D) return GDN_ERR_SHAPE;
    if ((int64_t)num_pages * Hkv * page_size >= (int64_t(1) << 31)) return GDN_ERR_SHAPE;
    if (dims->rotary_dim > 0 && !(std::isfinite(rope_theta) && rope_theta > 0.0)) return GDN_ERR_SHAPE;
    if (num_reqs == 0) return GDN_OK;
    if (!q || !gate || !k || !v || !k_cache || !v_cache || !block_tables || !context_lens || !y || !workspace)
        return GDN_ERR_NULL;
    if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(workspace)) return GDN_ERR_ALIGN;
    if (workspace_bytes < gdn::gqa_ws_bytes(num_reqs, Hq, max_context_len)) return GDN_ERR_WORKSPACE;
    gdn::GqaArgs a{};
    a.q = q; a.q_ld = q_ld; a.gate = gate; a.gate_ld = gate_ld; a.k = k; a.v = v; a.kv_ld = kv_ld;
    a.act_bf16 = act_dt == GDN_BF16;
    a.k_cache = k_cache; a.v_cache = v_cache; a.kv_fp8 = fp8;
    a.k_scale = fp8 ? k_scale : 1.f; a.v_scale = fp8 ? v_scale : 1.f;
    a.bt = block_tables; a.max_pages = max_pages_per_req; a.lens = context_lens;
    a.R = num_reqs; a.Hq = (int32_t)Hq; a.Hkv = (int32_t)Hkv; a.rd = dims->rotary_dim;
    a.P = page_size; a.num_pages = num_pages; a.max_ctx = max_context_len; a.theta = rope_theta;
    a.y = y; a.y_bf16 = y_dt == GDN_BF16; a.o = o; a.ws = workspace;
    return gdn::launch_gqa_decode(a, (hipStream_t)stream) == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

gdn_status gqa_validate_decode_metadata(const int32_t *block_tables, int32_t max_pages_per_req,
                                        const int32_t *context_lens, int32_t num_reqs,
                                        int32_t num_pages, int32_t page_size,
                                        int32_t max_context_len) {
    if (num_reqs < 0 || max_pages_per_req < 1 || num_pages < 1 || page_size < 1 || max_context_len < 1)
        return GDN_ERR_SHAPE;
    if (num_reqs == 0) return GDN_OK;
    if (!block_tables || !context_lens) return GDN_ERR_NULL;
    const int64_t lmax = std::min<int64_t>(max_context_len, (int64_t)max_pages_per_req * page_size);
    // owner[p] = request that appends into page p (-1: none)
    std::vector<int32_t> owner(num_pages, -1);
    for (int32_t r = 0; r < num_reqs; ++r) {
        const int64_t L = context_lens[r];
        if (L < 1 || L > lmax) return GDN_ERR_METADATA;
        const int64_t npg = (L + page_size - 1) / page_size;
        for (int64_t i = 0; i < npg; ++i) {
            const int32_t p = block_tables[(int64_t)r * max_pages_per_req + i];
            if (p < 0 || p >= num_pages) return GDN_ERR_METADATA;
        }
        const int32_t wp = block_tables[(int64_t)r * max_pages_per_req + (L - 1) / page_size];
        if (owner[wp] != -1) return GDN_ERR_METADATA;
        owner[wp] = r;
    }
    for (int32_t r = 0; r < num_reqs; ++r) {
        const int64_t L = context_lens[r];
        const int64_t npg = (L + page_size - 1) / page_size;
        for (int64_t i = 0; i < npg; ++i) {
            const int32_t p = block_tables[(int64_t)r * max_pages_per_req + i];
            if (owner[p] != -1 && owner[p] != r) return GDN_ERR_METADATA;
        }
    }
    return GDN_OK;
}

}  // extern "C"
