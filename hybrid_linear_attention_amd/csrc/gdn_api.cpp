// C-ABI layer of libgdn: argument validation (pure host code, runs before any
// HIP call) and dispatch to the kernel launchers.  See include/gdn.h for the
// contract of every entry point.
#include "gdn.h"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "gdn_launch.h"

// Static scratch of gdn_prefill_fused_noalloc: each GPU the library runs on
// holds its own copy for the life of the process.  In host code `scratch` only
// names the symbol; its device address on the current GPU comes from
// hipGetSymbolAddress, once per device, and only that address is ever passed
// to a kernel.
static __device__ __align__(256) uint8_t scratch[GDN_NOALLOC_SCRATCH_BYTES];

namespace {

bool valid_dtype(gdn_dtype d) { return d == GDN_F32 || d == GDN_BF16; }
size_t dt_size(gdn_dtype d) { return d == GDN_F32 ? 4 : 2; }
bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

gdn_status check_dims(const gdn_dims *d) {
    if (!d) return GDN_ERR_NULL;
    if (d->num_k_heads <= 0 || d->num_v_heads <= 0 || d->num_v_heads % d->num_k_heads != 0)
        return GDN_ERR_DIMS;
    if (d->head_dim_k != d->head_dim_v) return GDN_ERR_DIMS;
    const int D = d->head_dim_k;
    if (D != 16 && D != 32 && D != 64 && D != 128) return GDN_ERR_DIMS;
    if (d->conv_taps != 4) return GDN_ERR_DIMS;
    if ((int64_t)d->num_v_heads * D > (1 << 20)) return GDN_ERR_DIMS;
    return GDN_OK;
}

gdn_status hip_status(hipError_t e) { return e == hipSuccess ? GDN_OK : GDN_ERR_HIP; }

}  // namespace

extern "C" {

const char *gdn_status_string(gdn_status s) {
    switch (s) {
        case GDN_OK: return "GDN_OK";
        case GDN_ERR_NULL: return "GDN_ERR_NULL: required pointer is NULL";
        case GDN_ERR_DIMS: return "GDN_ERR_DIMS: unsupported head geometry";
        case GDN_ERR_DTYPE: return "GDN_ERR_DTYPE: unsupported dtype";
        case GDN_ERR_SHAPE: return "GDN_ERR_SHAPE: inconsistent counts or strides";
        case GDN_ERR_WORKSPACE: return "GDN_ERR_WORKSPACE: workspace missing or too small";
        case GDN_ERR_ALIGN: return "GDN_ERR_ALIGN: pointer misaligned";
        case GDN_ERR_HIP: return "GDN_ERR_HIP: HIP launch error";
        case GDN_ERR_METADATA: return "GDN_ERR_METADATA: bad query_start_loc or slot ids";
        case GDN_ERR_SCRATCH: return "GDN_ERR_SCRATCH: batch needs more than the library's static scratch";
    }
    return "GDN_ERR_UNKNOWN";
}

const char *gdn_version(void) { return "libgdn 0.1 (gfx950)"; }

gdn_status gdn_conv1d_update(const gdn_dims *dims, const void *x, gdn_dtype x_dt,
                             int64_t x_ld, const void *conv_w, gdn_dtype w_dt,
                             void *conv_pool, gdn_dtype pool_dt,
                             const int32_t *query_start_loc, const int32_t *slot_ids,
                             const uint8_t *has_initial, int32_t num_reqs,
                             int32_t num_tokens, int32_t num_slots, float l2_eps, void *q,
                             void *k, void *v, gdn_dtype act_dt, void *stream) {
    gdn_status st = check_dims(dims);
    if (st != GDN_OK) return st;
    if (!valid_dtype(x_dt) || !valid_dtype(w_dt) || !valid_dtype(pool_dt) || !valid_dtype(act_dt))
        return GDN_ERR_DTYPE;
    if (pool_dt != x_dt) return GDN_ERR_DTYPE;
    const int D = dims->head_dim_k;
    const int32_t nq = dims->num_k_heads * D;
    const int32_t C = 2 * nq + dims->num_v_heads * D;
    if (num_reqs < 0 || num_tokens < 0 || num_slots < 0) return GDN_ERR_SHAPE;
    if (num_reqs > num_slots) return GDN_ERR_SHAPE;
    if (num_tokens > 0 && num_reqs == 0) return GDN_ERR_SHAPE;
    if (x_ld < C) return GDN_ERR_SHAPE;
    if (num_tokens == 0 || num_reqs == 0) return GDN_OK;
    if (!x || !conv_w || !conv_pool || !query_start_loc || !slot_ids || !q || !k || !v)
        return GDN_ERR_NULL;
    if (!(l2_eps >= 0.0f)) return GDN_ERR_SHAPE;
    if (x_ld % 2 != 0 || !aligned(x, 2 * dt_size(x_dt)) || !aligned(conv_w, dt_size(w_dt)) ||
        !aligned(conv_pool, dt_size(pool_dt)) || !aligned(q, 2 * dt_size(act_dt)) ||
        !aligned(k, 2 * dt_size(act_dt)) || !aligned(v, 2 * dt_size(act_dt)) ||
        !aligned(query_start_loc, 4) || !aligned(slot_ids, 4))
        return GDN_ERR_ALIGN;
    gdn::ConvArgs a{D, x, x_ld, x_dt == GDN_BF16, conv_w, w_dt == GDN_BF16, conv_pool,
                    query_start_loc, slot_ids, has_initial, num_reqs, num_tokens, C, nq,
                    l2_eps, q, k, v, act_dt == GDN_BF16};
    return hip_status(gdn::launch_conv1d(a, static_cast<hipStream_t>(stream)));
}

gdn_status gdn_decode_step(const gdn_dims *dims, const void *q, const void *k, const void *v,
                           gdn_dtype act_dt, const void *a, const void *b, gdn_dtype gate_dt,
                           int64_t gate_ld, float *state_pool, const int32_t *slot_ids,
                           int32_t num_reqs, int32_t num_slots, void *o, gdn_dtype o_dt,
                           void *stream) {
    gdn_status st = check_dims(dims);
    if (st != GDN_OK) return st;
    if (!valid_dtype(act_dt) || !valid_dtype(gate_dt) || !valid_dtype(o_dt)) return GDN_ERR_DTYPE;
    if (num_reqs < 0 || num_slots < 0 || num_reqs > num_slots) return GDN_ERR_SHAPE;
    if (gate_ld < dims->num_v_heads) return GDN_ERR_SHAPE;
    if (num_reqs == 0) return GDN_OK;
    if (!q || !k || !v || !a || !b || !state_pool || !slot_ids || !o) return GDN_ERR_NULL;
    const size_t qk_align = act_dt == GDN_F32 ? 16 : 8;
    if (!aligned(state_pool, 16) || !aligned(q, qk_align) || !aligned(k, qk_align) ||
        !aligned(v, dt_size(act_dt)) || !aligned(a, dt_size(gate_dt)) ||
        !aligned(b, dt_size(gate_dt)) || !aligned(o, dt_size(o_dt)) || !aligned(slot_ids, 4))
        return GDN_ERR_ALIGN;
    gdn::DecodeArgs da{dims->head_dim_k, q, k, v, act_dt == GDN_BF16, a, b, gate_ld,
                       gate_dt == GDN_BF16, state_pool, slot_ids, num_reqs,
                       dims->num_k_heads, dims->num_v_heads, o, o_dt == GDN_BF16};
    return hip_status(gdn::launch_decode(da, static_cast<hipStream_t>(stream)));
}

gdn_status gdn_decode_fused(const gdn_dims *dims, const void *x_qkv, int64_t x_ld, const void *z,
                            int64_t z_ld, const void *a, const void *b, int64_t gate_ld,
                            gdn_dtype act_dt, const void *conv_w, const void *gamma,
                            gdn_dtype w_dt, void *conv_pool, void *state_pool,
                            gdn_dtype state_dt, const int32_t *slot_ids,
                            const uint8_t *has_initial, int32_t num_reqs, int32_t num_slots,
                            float l2_eps, float norm_eps, void *y, gdn_dtype y_dt, float *o,
                            void *stream) {
    gdn_status st = check_dims(dims);
    if (st != GDN_OK) return st;
    const int D = dims->head_dim_k;
    if (gdn::decode_fused_smem_bytes(D, dims->num_k_heads, dims->num_v_heads) > 64 * 1024)
        return GDN_ERR_DIMS;
    if (!valid_dtype(act_dt) || !valid_dtype(w_dt) || !valid_dtype(y_dt) || !valid_dtype(state_dt))
        return GDN_ERR_DTYPE;
    const int64_t C = 2 * (int64_t)dims->num_k_heads * D + (int64_t)dims->num_v_heads * D;
    if (num_reqs < 0 || num_slots < 0 || num_reqs > num_slots) return GDN_ERR_SHAPE;
    if (x_ld < C || z_ld < (int64_t)dims->num_v_heads * D || gate_ld < dims->num_v_heads)
        return GDN_ERR_SHAPE;
    if (!(l2_eps >= 0.0f) || !(norm_eps >= 0.0f)) return GDN_ERR_SHAPE;
    if (num_reqs == 0) return GDN_OK;
    if (!x_qkv || !z || !a || !b || !conv_w || !gamma || !conv_pool || !state_pool || !slot_ids ||
        !y)
        return GDN_ERR_NULL;
    const size_t e = dt_size(act_dt);
    if (!aligned(x_qkv, e) || !aligned(z, e) || !aligned(a, e) || !aligned(b, e) ||
        !aligned(conv_pool, e) || !aligned(conv_w, dt_size(w_dt)) || !aligned(gamma, dt_size(w_dt)) ||
        !aligned(state_pool, 16) || !aligned(slot_ids, 4) || !aligned(y, dt_size(y_dt)) ||
        (o && !aligned(o, 4)))
        return GDN_ERR_ALIGN;
    gdn::DecodeFusedArgs da{D, x_qkv, x_ld, z, z_ld, a, b, gate_ld, act_dt == GDN_BF16, conv_w,
                            gamma, w_dt == GDN_BF16, conv_pool, state_pool, state_dt == GDN_BF16,
                            slot_ids, has_initial, num_reqs, dims->num_k_heads, dims->num_v_heads,
                            l2_eps, norm_eps, y, y_dt == GDN_BF16, o};
    return hip_status(gdn::launch_decode_fused(da, static_cast<hipStream_t>(stream)));
}

gdn_status gdn_spec_verify(const gdn_dims *dims, const void *x_qkv, int64_t x_ld, const void *z,
                           int64_t z_ld, const void *a, const void *b, int64_t gate_ld,
                           gdn_dtype act_dt, const void *conv_w, const void *gamma,
                           gdn_dtype w_dt, void *conv_pool, void *state_pool,
                           gdn_dtype state_dt, const int32_t *query_start_loc,
                           const int32_t *slot_ids, const int32_t *spec_slot_ids, int32_t max_tokens,
                           const uint8_t *has_initial, int32_t num_reqs, int32_t num_tokens,
                           int32_t num_slots, float l2_eps, float norm_eps, void *y,
                           gdn_dtype y_dt, float *o, void *stream) {
    gdn_status st = check_dims(dims);
    if (st != GDN_OK) return st;
    const int D = dims->head_dim_k;
    if (max_tokens < 1 || max_tokens > GDN_SPEC_MAX_TOKENS) return GDN_ERR_SHAPE;
    if (gdn::spec_verify_smem_bytes(D, dims->num_k_heads, dims->num_v_heads, max_tokens) > 64 * 1024)
        return GDN_ERR_DIMS;
    if (!valid_dtype(act_dt) || !valid_dtype(w_dt) || !valid_dtype(y_dt) || !valid_dtype(state_dt))
        return GDN_ERR_DTYPE;
    const int64_t C = 2 * (int64_t)dims->num_k_heads * D + (int64_t)dims->num_v_heads * D;
    if (num_reqs < 0 || num_tokens < 0 || num_slots < 0 || num_reqs > num_slots)
        return GDN_ERR_SHAPE;
    if (num_tokens > 0 && num_reqs == 0) return GDN_ERR_SHAPE;
    if ((int64_t)num_tokens > (int64_t)num_reqs * max_tokens) return GDN_ERR_SHAPE;
    if (x_ld < C || z_ld < (int64_t)dims->num_v_heads * D || gate_ld < dims->num_v_heads)
        return GDN_ERR_SHAPE;
    if (!(l2_eps >= 0.0f) || !(norm_eps >= 0.0f)) return GDN_ERR_SHAPE;
    if (num_tokens == 0 || num_reqs == 0) return GDN_OK;
    if (!x_qkv || !z || !a || !b || !conv_w || !gamma || !conv_pool || !state_pool ||
        !query_start_loc || !slot_ids || !spec_slot_ids || !y)
        return GDN_ERR_NULL;
    const size_t e = dt_size(act_dt);
    if (!aligned(x_qkv, e) || !aligned(z, e) || !aligned(a, e) || !aligned(b, e) ||
        !aligned(conv_pool, e) || !aligned(conv_w, dt_size(w_dt)) || !aligned(gamma, dt_size(w_dt)) ||
        !aligned(state_pool, 16) || !aligned(query_start_loc, 4) || !aligned(slot_ids, 4) ||
        !aligned(spec_slot_ids, 4) || !aligned(y, dt_size(y_dt)) || (o && !aligned(o, 4)))
        return GDN_ERR_ALIGN;
    gdn::SpecVerifyArgs sa{D, x_qkv, x_ld, z, z_ld, a, b, gate_ld, act_dt == GDN_BF16, conv_w,
                           gamma, w_dt == GDN_BF16, conv_pool, state_pool, state_dt == GDN_BF16,
                           query_start_loc,
                           slot_ids, spec_slot_ids, max_tokens, has_initial, num_reqs,
                           dims->num_k_heads, dims->num_v_heads, l2_eps, norm_eps, y,
                           y_dt == GDN_BF16, o};
    return hip_status(gdn::launch_spec_verify(sa, static_cast<hipStream_t>(stream)));
}

size_t gdn_prefill_workspace_bytes(const gdn_dims *dims, int32_t num_tokens, int32_t num_reqs) {
    if (check_dims(dims) != GDN_OK || num_tokens < 0 || num_reqs < 0) return 0;
    return gdn::prefill_workspace_bytes(dims->head_dim_k, dims->num_k_heads, dims->num_v_heads,
                                        num_tokens, num_reqs);
}

gdn_status gdn_prefill_varlen(const gdn_dims *dims, const void *q, const void *k, const void *v,
                              gdn_dtype act_dt, const void *a, const void *b, gdn_dtype gate_dt,
                              int64_t gate_ld, float *state_pool,
                              const int32_t *query_start_loc, const int32_t *slot_ids,
                              const uint8_t *has_initial, int32_t num_reqs, int32_t num_tokens,
                              int32_t num_slots, void *o, gdn_dtype o_dt, void *workspace,
                              size_t workspace_bytes, void *stream) {
    gdn_status st = check_dims(dims);
    if (st != GDN_OK) return st;
    if (!valid_dtype(act_dt) || !valid_dtype(gate_dt) || !valid_dtype(o_dt)) return GDN_ERR_DTYPE;
    if (num_reqs < 0 || num_tokens < 0 || num_slots < 0 || num_reqs > num_slots)
        return GDN_ERR_SHAPE;
    if (num_tokens > 0 && num_reqs == 0) return GDN_ERR_SHAPE;
    if (gate_ld < dims->num_v_heads) return GDN_ERR_SHAPE;
    if (num_tokens == 0 || num_reqs == 0) return GDN_OK;
    if (!q || !k || !v || !a || !b || !state_pool || !query_start_loc || !slot_ids || !o)
        return GDN_ERR_NULL;
    const size_t need = gdn::prefill_workspace_bytes(dims->head_dim_k, dims->num_k_heads,
                                                     dims->num_v_heads, num_tokens, num_reqs);
    if (need > 0 && (!workspace || workspace_bytes < need)) return GDN_ERR_WORKSPACE;
    const size_t qk_align = act_dt == GDN_F32 ? 16 : 8;
    if (!aligned(state_pool, 16) || !aligned(q, qk_align) || !aligned(k, qk_align) ||
        !aligned(v, qk_align) || !aligned(a, dt_size(gate_dt)) || !aligned(b, dt_size(gate_dt)) ||
        !aligned(o, dt_size(o_dt)) || !aligned(query_start_loc, 4) || !aligned(slot_ids, 4) ||
        (workspace && !aligned(workspace, 256)))
        return GDN_ERR_ALIGN;
    gdn::PrefillArgs pa{dims->head_dim_k, q, k, v, act_dt == GDN_BF16, a, b, gate_ld,
                        gate_dt == GDN_BF16, state_pool, query_start_loc, slot_ids, has_initial,
                        num_reqs, num_tokens, dims->num_k_heads, dims->num_v_heads, o,
                        o_dt == GDN_BF16, workspace, workspace_bytes};
    return hip_status(gdn::launch_prefill(pa, static_cast<hipStream_t>(stream)));
}

namespace {
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// fused prefill scratch: fp32 q, k, v and o of every token, then the
// workspace of the prefill kernels.  At d = 128 the chunked prefill reads q and
// k only in its prep kernel, before its chain writes o, so q and k share o's
// region (and when the prep kernel forms q and k from x itself, they are not
// used at all); the sequential kernel (d < 128) reads q and k while it writes
// o, so there they have regions of their own.
struct FusedPrefillWs {
    size_t q, k, v, o, pre, total;
    size_t q_off, k_off, v_off, o_off, pre_off;
    FusedPrefillWs(const gdn_dims *d, int32_t T, int32_t nreq) {
        const size_t D = d->head_dim_k;
        q = align256((size_t)T * d->num_k_heads * D * 4);
        k = q;
        // v [T, Hv, D] fp32, or (d = 128 conv mode) the prefill's V images: one
        // 32-token block per chunk and value head, at most T / 32 + nreq chunks
        v = align256(((size_t)T / 32 + (size_t)nreq) * 32 * d->num_v_heads * D * 4);
        o = align256((size_t)T * d->num_v_heads * D * 4);
        pre = align256(gdn::prefill_workspace_bytes(d->head_dim_k, d->num_k_heads, d->num_v_heads, T, nreq));
        if (D == 128) {
            const size_t o_region = o > q + k ? o : q + k;
            o_off = 0;
            q_off = 0;
            k_off = q;
            v_off = o_region;
            pre_off = v_off + v;
        } else {
            q_off = 0;
            k_off = q;
            v_off = q + k;
            o_off = v_off + v;
            pre_off = o_off + o;
        }
        total = pre_off + pre;
    }
};
}  // namespace

size_t gdn_prefill_fused_workspace_bytes(const gdn_dims *dims, int32_t num_tokens, int32_t num_reqs) {
    if (check_dims(dims) != GDN_OK || num_tokens < 0 || num_reqs < 0) return 0;
    return FusedPrefillWs(dims, num_tokens, num_reqs).total;
}

}  // extern "C"

namespace {

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void *scratch_ptr[kMaxDevices];

// The current device's address of `scratch` (looked up on the first call on
// that device).
gdn_status scratch_address(void **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GDN_ERR_HIP;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (scratch_ptr[dev] == nullptr) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
            return GDN_ERR_HIP;
        scratch_ptr[dev] = p;
    }
    *out = scratch_ptr[dev];
    return GDN_OK;
}

// The whole fused prefill step, shared by gdn_prefill_fused (on the caller's
// workspace) and gdn_prefill_fused_noalloc (static_scratch: on the library's
// scratch array, whose address is looked up only after every host check).
gdn_status prefill_fused_impl(const gdn_dims *dims, const void *x_qkv, int64_t x_ld, const void *z,
                              int64_t z_ld, const void *a, const void *b, int64_t gate_ld,
                              gdn_dtype act_dt, const void *conv_w, const void *gamma,
                              gdn_dtype w_dt, void *conv_pool, void *state_pool,
                              gdn_dtype state_dt, const int32_t *query_start_loc,
                              const int32_t *slot_ids, const uint8_t *has_initial,
                              int32_t num_reqs, int32_t num_tokens, int32_t num_slots,
                              const int32_t *snap_slot_ids, int32_t max_snaps,
                              int32_t snap_interval, float l2_eps, float norm_eps, void *y,
                              gdn_dtype y_dt, void *workspace, size_t workspace_bytes,
                              bool static_scratch, void *stream) {
    gdn_status st = check_dims(dims);
    if (st != GDN_OK) return st;
    if (!valid_dtype(act_dt) || !valid_dtype(w_dt) || !valid_dtype(y_dt) || !valid_dtype(state_dt))
        return GDN_ERR_DTYPE;
    const int D = dims->head_dim_k;
    const int32_t nq = dims->num_k_heads * D;
    const int32_t C = 2 * nq + dims->num_v_heads * D;
    if (num_reqs < 0 || num_tokens < 0 || num_slots < 0 || num_reqs > num_slots)
        return GDN_ERR_SHAPE;
    if (num_tokens > 0 && num_reqs == 0) return GDN_ERR_SHAPE;
    if (x_ld < C || z_ld < (int64_t)dims->num_v_heads * D || gate_ld < dims->num_v_heads)
        return GDN_ERR_SHAPE;
    if (!(l2_eps >= 0.0f) || !(norm_eps >= 0.0f)) return GDN_ERR_SHAPE;
    if (max_snaps < 0 || (max_snaps > 0 && (snap_interval <= 0 || snap_interval % GDN_SNAPSHOT_QUANTUM != 0)))
        return GDN_ERR_SHAPE;
    if (num_tokens == 0 || num_reqs == 0) return GDN_OK;
    if (max_snaps > 0 && !snap_slot_ids) return GDN_ERR_NULL;
    if (max_snaps > 0 && !aligned(snap_slot_ids, 4)) return GDN_ERR_ALIGN;
    if (!x_qkv || !z || !a || !b || !conv_w || !gamma || !conv_pool || !state_pool ||
        !query_start_loc || !slot_ids || !y)
        return GDN_ERR_NULL;
    const FusedPrefillWs wl(dims, num_tokens, num_reqs);
    if (static_scratch) {
        if (wl.total > (size_t)GDN_NOALLOC_SCRATCH_BYTES) return GDN_ERR_SCRATCH;
    } else if (!workspace || workspace_bytes < wl.total) {
        return GDN_ERR_WORKSPACE;
    }
    const size_t e = dt_size(act_dt);
    if (x_ld % 2 != 0 || z_ld % 2 != 0 || !aligned(x_qkv, 2 * e) || !aligned(z, 2 * e) ||
        !aligned(a, e) || !aligned(b, e) || !aligned(conv_pool, e) ||
        !aligned(conv_w, dt_size(w_dt)) || !aligned(gamma, 2 * dt_size(w_dt)) ||
        !aligned(state_pool, 16) || !aligned(query_start_loc, 4) || !aligned(slot_ids, 4) ||
        !aligned(y, 2 * dt_size(y_dt)) || (!static_scratch && !aligned(workspace, 256)))
        return GDN_ERR_ALIGN;
    // d = 128 with 16-byte rows: the prefill's prep kernel forms q and k from x
    // itself and its chain forms v, so no conv pass runs
    const bool prep_conv = D == 128 && x_ld % (int64_t)(16 / e) == 0 && aligned(x_qkv, 16) &&
                           aligned(conv_w, 16);
    // a bf16 state at d = 128 needs the prep-conv path (16-byte conv rows)
    if (state_dt == GDN_BF16 && D == 128 && !prep_conv) return GDN_ERR_ALIGN;
    if (static_scratch) {
        const gdn_status sst = scratch_address(&workspace);
        if (sst != GDN_OK) return sst;
    }
    uint8_t *w = static_cast<uint8_t *>(workspace);
    float *q = reinterpret_cast<float *>(w + wl.q_off);
    float *k = reinterpret_cast<float *>(w + wl.k_off);
    float *v = reinterpret_cast<float *>(w + wl.v_off);
    float *o = reinterpret_cast<float *>(w + wl.o_off);
    uint8_t *pre = w + wl.pre_off;
    hipStream_t s = static_cast<hipStream_t>(stream);
    gdn::ConvArgs ca{D, x_qkv, x_ld, act_dt == GDN_BF16, conv_w, w_dt == GDN_BF16, conv_pool,
                     query_start_loc, slot_ids, has_initial, num_reqs, num_tokens, C, nq,
                     l2_eps, q, k, v, false};
    gdn::PrefillArgs pa{D, q, k, v, false, a, b, gate_ld, act_dt == GDN_BF16, state_pool,
                        query_start_loc, slot_ids, has_initial, num_reqs, num_tokens,
                        dims->num_k_heads, dims->num_v_heads, o, false, pre, wl.pre};
    pa.state_bf16 = state_dt == GDN_BF16;
    if (prep_conv) {
        pa.x = x_qkv;
        pa.x_ld = x_ld;
        pa.x_bf16 = act_dt == GDN_BF16;
        pa.conv_w = conv_w;
        pa.w_bf16 = w_dt == GDN_BF16;
        pa.pool = conv_pool;
        pa.l2_eps = l2_eps;
    } else {
        if (gdn::launch_conv1d(ca, s) != hipSuccess) return GDN_ERR_HIP;
    }
    pa.z = z;
    pa.z_ld = z_ld;
    pa.z_bf16 = act_dt == GDN_BF16;
    pa.gamma = gamma;
    pa.gamma_bf16 = w_dt == GDN_BF16;
    pa.norm_eps = norm_eps;
    pa.y = y;
    pa.y_bf16 = y_dt == GDN_BF16;
    pa.snap_slots = max_snaps > 0 ? snap_slot_ids : nullptr;
    pa.snap_interval = snap_interval;
    pa.max_snaps = max_snaps;
    if (gdn::launch_prefill(pa, s) != hipSuccess) return GDN_ERR_HIP;
    if (max_snaps > 0)
        return hip_status(gdn::launch_snapshot_history(x_qkv, x_ld, act_dt == GDN_BF16, conv_pool,
                                                       query_start_loc, snap_slot_ids, snap_interval,
                                                       max_snaps, num_reqs, C, s));
    return GDN_OK;
}

}  // namespace

extern "C" {

gdn_status gdn_prefill_fused(const gdn_dims *dims, const void *x_qkv, int64_t x_ld, const void *z,
                             int64_t z_ld, const void *a, const void *b, int64_t gate_ld,
                             gdn_dtype act_dt, const void *conv_w, const void *gamma,
                             gdn_dtype w_dt, void *conv_pool, void *state_pool,
                             gdn_dtype state_dt, const int32_t *query_start_loc, const int32_t *slot_ids,
                             const uint8_t *has_initial, int32_t num_reqs, int32_t num_tokens,
                             int32_t num_slots, const int32_t *snap_slot_ids, int32_t max_snaps,
                             int32_t snap_interval, float l2_eps, float norm_eps, void *y,
                             gdn_dtype y_dt, void *workspace, size_t workspace_bytes,
                             void *stream) {
    return prefill_fused_impl(dims, x_qkv, x_ld, z, z_ld, a, b, gate_ld, act_dt, conv_w, gamma, w_dt,
                              conv_pool, state_pool, state_dt, query_start_loc, slot_ids,
                              has_initial, num_reqs, num_tokens, num_slots, snap_slot_ids,
                              max_snaps, snap_interval, l2_eps, norm_eps, y, y_dt, workspace,
                              workspace_bytes, false, stream);
}

gdn_status gdn_prefill_fused_noalloc(const gdn_dims *dims, const void *x_qkv, int64_t x_ld,
                                     const void *z, int64_t z_ld, const void *a, const void *b,
                                     int64_t gate_ld, gdn_dtype act_dt, const void *conv_w,
                                     const void *gamma, gdn_dtype w_dt, void *conv_pool,
                                     void *state_pool, gdn_dtype state_dt,
                                     const int32_t *query_start_loc, const int32_t *slot_ids,
                                     const uint8_t *has_initial, int32_t num_reqs,
                                     int32_t num_tokens, int32_t num_slots,
                                     const int32_t *snap_slot_ids, int32_t max_snaps,
                                     int32_t snap_interval, float l2_eps, float norm_eps, void *y,
                                     gdn_dtype y_dt, void *stream) {
    return prefill_fused_impl(dims, x_qkv, x_ld, z, z_ld, a, b, gate_ld, act_dt, conv_w, gamma, w_dt,
                              conv_pool, state_pool, state_dt, query_start_loc, slot_ids,
                              has_initial, num_reqs, num_tokens, num_slots, snap_slot_ids,
                              max_snaps, snap_interval, l2_eps, norm_eps, y, y_dt, nullptr, 0,
                              true, stream);
}

gdn_status gdn_gated_norm(const gdn_dims *dims, const void *o, gdn_dtype o_dt, const void *z,
                          gdn_dtype z_dt, int64_t z_ld, const void *gamma, gdn_dtype gamma_dt,
                          float eps, int32_t num_tokens, void *y, gdn_dtype y_dt, void *stream) {
    gdn_status st = check_dims(dims);
    if (st != GDN_OK) return st;
    if (!valid_dtype(o_dt) || !valid_dtype(z_dt) || !valid_dtype(gamma_dt) || !valid_dtype(y_dt))
        return GDN_ERR_DTYPE;
    const int D = dims->head_dim_v;
    if (num_tokens < 0 || z_ld < (int64_t)dims->num_v_heads * D || !(eps >= 0.0f))
        return GDN_ERR_SHAPE;
    if (num_tokens == 0) return GDN_OK;
    if (!o || !z || !gamma || !y) return GDN_ERR_NULL;
    if (z_ld % 2 != 0 || !aligned(o, 2 * dt_size(o_dt)) || !aligned(z, 2 * dt_size(z_dt)) ||
        !aligned(gamma, 2 * dt_size(gamma_dt)) || !aligned(y, 2 * dt_size(y_dt)))
        return GDN_ERR_ALIGN;
    gdn::GatedNormArgs ga{D, o, o_dt == GDN_BF16, z, z_ld, z_dt == GDN_BF16, gamma,
                          gamma_dt == GDN_BF16, eps, num_tokens, dims->num_v_heads, y,
                          y_dt == GDN_BF16};
    return hip_status(gdn::launch_gated_norm(ga, static_cast<hipStream_t>(stream)));
}

gdn_status gdn_rmsnorm(const void *x, gdn_dtype x_dt, const void *gamma, gdn_dtype gamma_dt,
                       float eps, int32_t rows, int32_t cols, void *y, gdn_dtype y_dt,
                       void *stream) {
    if (!valid_dtype(x_dt) || !valid_dtype(gamma_dt) || !valid_dtype(y_dt)) return GDN_ERR_DTYPE;
    if (rows < 0 || cols <= 0 || cols % 8 != 0 || cols > 16384 || !(eps >= 0.0f))
        return GDN_ERR_SHAPE;
    if (rows == 0) return GDN_OK;
    if (!x || !gamma || !y) return GDN_ERR_NULL;
    if (!aligned(x, 16) || !aligned(gamma, 16) || !aligned(y, 16)) return GDN_ERR_ALIGN;
    gdn::RmsNormArgs ra{x, x_dt == GDN_BF16, gamma, gamma_dt == GDN_BF16, eps, rows, cols,
                        y, y_dt == GDN_BF16};
    return hip_status(gdn::launch_rmsnorm(ra, static_cast<hipStream_t>(stream)));
}

size_t gdn_gemm_bf16_workspace_bytes(int32_t M, int32_t N, int32_t K) {
    if (M <= 0 || N <= 0 || K <= 0) return 0;
    return gdn::gemm_bf16_workspace_bytes(M, N, K);
}

gdn_status gdn_gemm_bf16(const void *A, int64_t lda, const void *B, int64_t ldb, void *C,
                         int64_t ldc, gdn_dtype c_dt, const void *residual, int64_t ldr,
                         int32_t M, int32_t N, int32_t K, void *stream) {
    return gdn_gemm_bf16_ws(A, lda, B, ldb, C, ldc, c_dt, residual, ldr, M, N, K, nullptr, 0, stream);
}

gdn_status gdn_gemm_bf16_ws(const void *A, int64_t lda, const void *B, int64_t ldb, void *C,
                            int64_t ldc, gdn_dtype c_dt, const void *residual, int64_t ldr,
                            int32_t M, int32_t N, int32_t K, void *workspace,
                            size_t workspace_bytes, void *stream) {
    if (!valid_dtype(c_dt)) return GDN_ERR_DTYPE;
    if (M < 0 || N < 0 || K < 0 || N % 8 != 0 || K % 8 != 0) return GDN_ERR_SHAPE;
    if (lda < K || ldb < K || ldc < N || (residual && ldr < N)) return GDN_ERR_SHAPE;
    if (lda % 8 || ldb % 8 || ldc % 8 || (residual && ldr % 8)) return GDN_ERR_SHAPE;
    if (M == 0 || N == 0) return GDN_OK;
    if (!A || !B || !C) return GDN_ERR_NULL;
    if (!aligned(A, 16) || !aligned(B, 16) || !aligned(C, 16) || (residual && !aligned(residual, 16)))
        return GDN_ERR_ALIGN;
    if (workspace && !aligned(workspace, 256)) return GDN_ERR_ALIGN;
    gdn::GemmArgs g{A, lda, B, ldb, C, ldc, c_dt == GDN_BF16, residual, ldr, M, N, K};
    g.ws = workspace;
    g.ws_bytes = workspace ? workspace_bytes : 0;
    return hip_status(gdn::launch_gemm_bf16(g, static_cast<hipStream_t>(stream)));
}

gdn_status gdn_validate_metadata(const int32_t *qsl, const int32_t *slots, int32_t num_reqs,
                                 int32_t num_tokens, int32_t num_slots) {
    if (num_reqs < 0 || num_tokens < 0 || num_slots < 0) return GDN_ERR_SHAPE;
    if (!qsl || (num_reqs > 0 && !slots)) return GDN_ERR_NULL;
    if (qsl[0] != 0 || qsl[num_reqs] != num_tokens) return GDN_ERR_METADATA;
    for (int32_t r = 0; r < num_reqs; ++r) {
        if (qsl[r + 1] < qsl[r]) return GDN_ERR_METADATA;
        if (slots[r] < 0 || slots[r] >= num_slots) return GDN_ERR_METADATA;
    }
    // distinctness: O(n log n) without allocation is awkward in C; use a
    // bitmap on the stack for small pools and a quadratic scan otherwise.
    if (num_slots <= 65536) {
        uint64_t seen[1024] = {0};
        for (int32_t r = 0; r < num_reqs; ++r) {
            const uint32_t s = (uint32_t)slots[r];
            if (seen[s >> 6] & (1ull << (s & 63))) return GDN_ERR_METADATA;
            seen[s >> 6] |= 1ull << (s & 63);
        }
    } else {
        for (int32_t r = 0; r < num_reqs; ++r)
            for (int32_t u = r + 1; u < num_reqs; ++u)
                if (slots[r] == slots[u]) return GDN_ERR_METADATA;
    }
    return GDN_OK;
}

gdn_status gdn_validate_spec_metadata(const int32_t *qsl, const int32_t *slots,
                                      const int32_t *spec, int32_t max_tokens,
                                      int32_t num_reqs, int32_t num_tokens, int32_t num_slots) {
    if (max_tokens < 1 || max_tokens > GDN_SPEC_MAX_TOKENS) return GDN_ERR_SHAPE;
    gdn_status st = gdn_validate_metadata(qsl, slots, num_reqs, num_tokens, num_slots);
    if (st != GDN_OK) return st;
    if (num_reqs > 0 && !spec) return GDN_ERR_NULL;
    // every slot a call writes (spec[r][j] for j < length of r) and every input
    // slot: distinct, except that spec[r][0] may name slot_ids[r] itself
    for (int32_t r = 0; r < num_reqs; ++r) {
        const int32_t len = qsl[r + 1] - qsl[r];
        if (len > max_tokens) return GDN_ERR_METADATA;
        for (int32_t j = 0; j < len; ++j) {
            const int32_t s = spec[(int64_t)r * max_tokens + j];
            if (s < 0 || s >= num_slots) return GDN_ERR_METADATA;
            for (int32_t r2 = 0; r2 < num_reqs; ++r2) {
                if (slots[r2] == s && !(r2 == r && j == 0)) return GDN_ERR_METADATA;
                const int32_t len2 = qsl[r2 + 1] - qsl[r2];
                for (int32_t j2 = 0; j2 < len2; ++j2)
                    if ((r2 != r || j2 != j) && spec[(int64_t)r2 * max_tokens + j2] == s)
                        return GDN_ERR_METADATA;
            }
        }
    }
    return GDN_OK;
}

gdn_status gdn_validate_snapshot_metadata(const int32_t *qsl, const int32_t *slots,
                                          const int32_t *snaps, int32_t max_snaps,
                                          int32_t snap_interval, int32_t num_reqs,
                                          int32_t num_tokens, int32_t num_slots) {
    if (max_snaps < 0 || (max_snaps > 0 && (snap_interval <= 0 || snap_interval % GDN_SNAPSHOT_QUANTUM != 0)))
        return GDN_ERR_SHAPE;
    gdn_status st = gdn_validate_metadata(qsl, slots, num_reqs, num_tokens, num_slots);
    if (st != GDN_OK || max_snaps == 0) return st;
    if (num_reqs > 0 && !snaps) return GDN_ERR_NULL;
    // the slots a call writes: snaps[r][j] for (j + 1) * interval <= length of r
    for (int32_t r = 0; r < num_reqs; ++r) {
        const int32_t n = (qsl[r + 1] - qsl[r]) / snap_interval;
        for (int32_t j = 0; j < n && j < max_snaps; ++j) {
            const int32_t s = snaps[(int64_t)r * max_snaps + j];
            if (s < 0 || s >= num_slots) return GDN_ERR_METADATA;
            for (int32_t r2 = 0; r2 < num_reqs; ++r2) {
                if (slots[r2] == s) return GDN_ERR_METADATA;
                const int32_t n2 = (qsl[r2 + 1] - qsl[r2]) / snap_interval;
                for (int32_t j2 = 0; j2 < n2 && j2 < max_snaps; ++j2)
                    if ((r2 != r || j2 != j) && snaps[(int64_t)r2 * max_snaps + j2] == s)
                        return GDN_ERR_METADATA;
            }
        }
    }
    return GDN_OK;
}

}  // extern "C"
