// Prefill dispatch: picks the kernel for the head geometry.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

hipError_t launch_prefill_seq(const PrefillArgs &a, hipStream_t s);
hipError_t launch_prefill_chunk(const PrefillArgs &a, hipStream_t s);
size_t prefill_chunk_workspace_bytes(int32_t Hk, int32_t Hv, int32_t T, int32_t nreq);

// d = 128: chunk offsets and request order, a K image per (chunk, key head)
// and a T image per (chunk, value head).
size_t prefill_workspace_bytes(int D, int32_t Hk, int32_t Hv, int32_t T, int32_t nreq) {
    if (D == 128) return prefill_chunk_workspace_bytes(Hk, Hv, T, nreq);
    return 0;
}

// d = 128 runs the chunkwise MFMA kernel; smaller heads the sequential one,
// followed by the gated norm when y is requested.
hipError_t launch_prefill(const PrefillArgs &a, hipStream_t s) {
    if (a.D == 128) return launch_prefill_chunk(a, s);
    hipError_t e = launch_prefill_seq(a, s);
    if (e != hipSuccess || !a.y) return e;
    GatedNormArgs g{a.D, a.o, a.o_bf16, a.z, a.z_ld, a.z_bf16, a.gamma, a.gamma_bf16, a.norm_eps,
                    a.T, a.Hv, a.y, a.y_bf16};
    return launch_gated_norm(g, s);
}

}  // namespace gdn
