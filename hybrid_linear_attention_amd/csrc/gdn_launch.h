// Internal launcher interface between the C-ABI layer (gdn_api.cpp) and the
// kernel translation units.  Host-side structs only; validated before use.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

namespace gdn {

struct ConvArgs {
    int D;  // d_k == d_v
    const void *x; int64_t x_ld; bool x_bf16;
    const void *w; bool w_bf16;
    void *pool;
    const int32_t *qsl; const int32_t *slots; const uint8_t *has_init;
    int32_t nreq, T, C, nq;
    float l2_eps;
    void *q, *k, *v; bool act_bf16;
};
hipError_t launch_conv1d(const ConvArgs &a, hipStream_t s);

struct DecodeArgs {
    int D;
    const void *q, *k, *v; bool act_bf16;
    const void *a, *b; int64_t gate_ld; bool gate_bf16;
    float *state; const int32_t *slots;
    int32_t R, Hk, Hv;
    void *o; bool o_bf16;
};
hipError_t launch_decode(const DecodeArgs &a, hipStream_t s);

struct DecodeFusedArgs {
    int D;
    const void *x; int64_t x_ld;
    const void *z; int64_t z_ld;
    const void *a, *b; int64_t gate_ld; bool act_bf16;
    const void *w, *gamma; bool w_bf16;
    void *pool; void *state; bool state_bf16; const int32_t *slots; const uint8_t *has_init;
    int32_t R, Hk, Hv;
    float l2_eps, norm_eps;
    void *y; bool y_bf16; float *o;
};
hipError_t launch_decode_fused(const DecodeFusedArgs &a, hipStream_t s);
size_t decode_fused_smem_bytes(int D, int32_t Hk, int32_t Hv);

struct SpecVerifyArgs {
    int D;
    const void *x; int64_t x_ld;
    const void *z; int64_t z_ld;
    const void *a, *b; int64_t gate_ld; bool act_bf16;
    const void *w, *gamma; bool w_bf16;
    void *pool; void *state; bool state_bf16;
    const int32_t *qsl, *slots, *spec; int32_t max_tokens; const uint8_t *has_init;
    int32_t R, Hk, Hv;
    float l2_eps, norm_eps;
    void *y; bool y_bf16; float *o;
};
hipError_t launch_spec_verify(const SpecVerifyArgs &a, hipStream_t s);
size_t spec_verify_smem_bytes(int D, int32_t Hk, int32_t Hv, int32_t max_tokens);

struct GatedNormArgs {
    int D;
    const void *o; bool o_bf16;
    const void *z; int64_t z_ld; bool z_bf16;
    const void *gamma; bool gamma_bf16;
    float eps;
    int32_t T, Hv;
    void *y; bool y_bf16;
};
hipError_t launch_gated_norm(const GatedNormArgs &a, hipStream_t s);

struct RmsNormArgs {
    const void *x; bool x_bf16;
    const void *gamma; bool gamma_bf16;
    float eps;
    int32_t rows, cols;
    void *y; bool y_bf16;
};
hipError_t launch_rmsnorm(const RmsNormArgs &a, hipStream_t s);

struct PrefillArgs {
    int D;
    const void *q, *k, *v; bool act_bf16;
    const void *a, *b; int64_t gate_ld; bool gate_bf16;
    void *state;  // [slots, Hv, D, D], fp32 (or bf16 with state_bf16, below)
    const int32_t *qsl, *slots; const uint8_t *has_init;
    int32_t nreq, T, Hk, Hv;
    void *o; bool o_bf16;
    void *ws; size_t ws_bytes;
    // optional gated output y = RMSNorm_dv(o) * gamma * SiLU(z) (y == nullptr: o only).
    // With y set, o is scratch the launcher may use ([T, Hv, D] fp32, o_bf16 false).
    const void *z = nullptr; int64_t z_ld = 0; bool z_bf16 = false;
    const void *gamma = nullptr; bool gamma_bf16 = false; float norm_eps = 0.f;
    void *y = nullptr; bool y_bf16 = false;
    // optional conv inputs (d = 128): the prep kernel forms q and k from x, the
    // chain forms v from x and writes the new history of every channel (q, k and
    // v unused; o must be fp32)
    const void *x = nullptr; int64_t x_ld = 0; bool x_bf16 = false;
    const void *conv_w = nullptr; bool w_bf16 = false;
    void *pool = nullptr; float l2_eps = 0.f;
    bool state_bf16 = false;  // bf16 state: widened on load, rounded once (RNE) on store
    // optional prefix-cache snapshots: the state after every snap_interval tokens
    // (a multiple of 32) of request r goes to slot snap_slots[r * max_snaps + j]
    const int32_t *snap_slots = nullptr; int32_t snap_interval = 0, max_snaps = 0;
};
hipError_t launch_snapshot_history(const void *x, int64_t x_ld, bool x_bf16, void *pool,
                                   const int32_t *qsl, const int32_t *snap_slots, int32_t interval,
                                   int32_t max_snaps, int32_t nreq, int32_t C, hipStream_t s);
size_t prefill_workspace_bytes(int D, int32_t Hk, int32_t Hv, int32_t T, int32_t nreq);
hipError_t launch_prefill(const PrefillArgs &a, hipStream_t s);

struct GemmArgs {
    const void *A; int64_t lda;
    const void *B; int64_t ldb;
    void *C; int64_t ldc; bool c_bf16;
    const void *R; int64_t ldr;
    int32_t M, N, K;
    // optional workspace for the split tail (gemm_bf16_workspace_bytes; 256-byte
    // aligned): without it, or when it is too small, no tile is split
    void *ws = nullptr; size_t ws_bytes = 0;
};
hipError_t launch_gemm_bf16(const GemmArgs &a, hipStream_t s);
size_t gemm_bf16_workspace_bytes(int M, int N, int K);  // on the current device; 0: no split

// Raise a kernel's dynamic-LDS limit once per device (the attribute belongs to
// the device the call is made on); `done` records the devices already set, as
// bits of an atomic mask, so concurrent first calls are harmless.
template <typename K>
inline hipError_t set_smem_once(K kern, size_t bytes, std::atomic<uint64_t> &done) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = dev >= 0 && dev < 64 ? uint64_t(1) << dev : 0;
    if (bit != 0 && (done.load(std::memory_order_relaxed) & bit) != 0) return hipSuccess;
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)bytes);
    if (e == hipSuccess && bit != 0) done.fetch_or(bit, std::memory_order_relaxed);
    return e;
}

}  // namespace gdn
