/*
 * gdn.h — C ABI of the MI355X (gfx950) Gated DeltaNet mixer-core library.
 *
 * The method ("Qwen3.8-27B: from model structure to the vLLM inference
 * dataflow", section 01 LAYER-BY-LAYER, per-layer operator table, GDN layer):
 *
 *   [Q0,K0,V0,Z] = U Wqkvz; a = U Wa; b = U Wb
 *   c_t = SiLU(sum_{i=0..3} w_i * QKV0_{t-i});  q = normalize(q); k = normalize(k)
 *   Sbar = alpha S_prev;  e = v - Sbar k;  S = Sbar + beta e k^T;  o = S q / sqrt(d_k)
 *   Ogate = RMSNorm(o) * SiLU(Z);  Delta_mix = Ogate Wo;  Y = X + Delta_mix
 *
 * with the data structures of that section's data-structure table: q/k
 * [T,16,128], v/z [T,48,128], a/b [T,48], recurrent state [R,48,128,128] fp32
 * (3 MiB per sequence per layer), conv history [R,10240,3] (three past inputs;
 * the 4-tap window includes the current one).  A packed batch of requests is
 * delimited by query_start_loc; requests never mix (same table, engine note).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers owned by the caller; the library
 *    never allocates, frees, or keeps them.  Every call is asynchronous: work
 *    is enqueued on `stream` (a hipStream_t; NULL = the null stream) and the
 *    call returns without synchronising.
 *  - Tensors are dense row-major in the shapes given, except where a leading
 *    dimension (`*_ld`, in elements, >= the row width) lets rows be strided.
 *  - Value head h reads key head h / (Hv / Hk): contiguous groups, the layout
 *    the page's 4-way tensor-parallel table implies (key heads 0-3 travel with
 *    value heads 0-11).
 *  - Recurrent state is [num_slots, Hv, d_v, d_k], d_k contiguous, fp32; the
 *    fused entry points (gdn_decode_fused, gdn_prefill_fused, gdn_spec_verify)
 *    also take a bf16 state through their state_dt argument.
 *    Conv history is [num_slots, Cqkv, taps-1], oldest -> newest, where
 *    Cqkv = 2*Hk*d_k + Hv*d_v and channels are ordered q | k | v.
 *  - Slots named in one call must be distinct (a duplicate is a data race).
 *    query_start_loc must be non-decreasing, start at 0 and end at num_tokens,
 *    and slot ids must lie in [0, num_slots): these device-resident contents are
 *    a caller contract (gdn_validate_metadata checks host copies of them).
 *  - Host-checkable faults (null pointers, unsupported dims or dtypes,
 *    negative or inconsistent counts, short workspace, misalignment) return a
 *    status BEFORE anything is enqueued.  A launch failure returns GDN_ERR_HIP.
 *  - Supported dims on the GPU: d_k == d_v in {16, 32, 64, 128},
 *    Hv % Hk == 0, conv_taps == 4.
 *  - Outputs never alias inputs; the state and history pools are updated in
 *    place.  A request of length 0 leaves its slots untouched.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Head geometry: mirrors the inputs of the page's state-shape calculator
 * ("How the 64 layers of Qwen3.8-27B are dispatched in vLLM", step 5:
 * key heads, value heads, key dim, value dim, conv kernel size). */
typedef struct gdn_dims {
    int32_t num_k_heads; /* Hk: 16 (tiny workload: 2)   */
    int32_t num_v_heads; /* Hv: 48 (tiny workload: 6)   */
    int32_t head_dim_k;  /* d_k: 128 (tiny workload: 16) */
    int32_t head_dim_v;  /* d_v: 128 (tiny workload: 16) */
    int32_t conv_taps;   /* 4 */
} gdn_dims;

typedef enum gdn_dtype {
    GDN_F32 = 0,
    GDN_BF16 = 1,
    GDN_FP8_E4M3 = 2 /* OCP e4m3 codes; only the GQA KV cache (gqa.h) takes it */
} gdn_dtype;

typedef enum gdn_status {
    GDN_OK = 0,
    GDN_ERR_NULL = 1,      /* a required pointer is NULL                     */
    GDN_ERR_DIMS = 2,      /* unsupported or inconsistent head geometry      */
    GDN_ERR_DTYPE = 3,     /* unsupported dtype combination                  */
    GDN_ERR_SHAPE = 4,     /* negative or inconsistent counts / strides      */
    GDN_ERR_WORKSPACE = 5, /* workspace missing or too small                 */
    GDN_ERR_ALIGN = 6,     /* pointer not aligned as documented              */
    GDN_ERR_HIP = 7,       /* the HIP runtime reported an error on launch    */
    GDN_ERR_METADATA = 8,  /* gdn_validate_metadata: bad qsl or slot ids     */
    GDN_ERR_SCRATCH = 9    /* gdn_prefill_fused_noalloc: the batch needs more
                              than GDN_NOALLOC_SCRATCH_BYTES of scratch      */
} gdn_status;

/* Human-readable name of a status code (static storage). */
const char *gdn_status_string(gdn_status s);

/* Library version string (static storage). */
const char *gdn_version(void);

/*
 * gdn_conv1d_update — causal depthwise conv1d + SiLU + L2 norm of q and k,
 * over a packed batch, with the per-request conv history read and written in
 * place (operator table, conv row; data-structure table, conv-history row).
 *
 *   x          [num_tokens, x_ld] in x_dt; row t holds the Cqkv conv inputs
 *              q | k | v of token t in its first Cqkv entries.
 *   conv_w     [Cqkv, taps] in w_dt; conv_w[c][i] multiplies x[t - i][c].
 *              No bias.
 *   conv_pool  [num_slots, Cqkv, taps-1] in pool_dt (== x_dt); read for the
 *              first taps-1 tokens of each request (zeros if has_initial[r] is
 *              0), then overwritten with the last taps-1 entries of the window
 *              [history, request rows] — a bit-exact copy of inputs.
 *   query_start_loc [num_reqs + 1] int32 (device), slot_ids [num_reqs] int32
 *              (device), has_initial [num_reqs] uint8 (device; NULL = all 1).
 *   l2_eps     q = q~ / sqrt(|q~|^2 + l2_eps) per (token, key head); same for k.
 *   q, k       [num_tokens, Hk, d_k] in act_dt (outputs, normalised).
 *   v          [num_tokens, Hv, d_v] in act_dt (output, SiLU'd conv output).
 * num_tokens == 0 or num_reqs == 0 enqueues nothing.
 * Alignment: x and conv_w 4-byte aligned, x_ld even; outputs 8-byte aligned.
 */
gdn_status gdn_conv1d_update(const gdn_dims *dims, const void *x, gdn_dtype x_dt,
                             int64_t x_ld, const void *conv_w, gdn_dtype w_dt,
                             void *conv_pool, gdn_dtype pool_dt,
                             const int32_t *query_start_loc,
                             const int32_t *slot_ids, const uint8_t *has_initial,
                             int32_t num_reqs, int32_t num_tokens,
                             int32_t num_slots, float l2_eps, void *q, void *k,
                             void *v, gdn_dtype act_dt, void *stream);

/*
 * gdn_decode_step — one token per request of the gated delta rule, in place
 * on the request's state slot (operator table, GDN row; the error is read from
 * the decayed state, evidence-matrix row citing the Gated DeltaNet paper,
 * eq. 10; decode cost O(Hv d_v d_k) independent of history length, section 01
 * "why compress most layers").
 *
 *   q, k   [num_reqs, Hk, d_k] in act_dt (L2-normalised by the caller's conv).
 *   v      [num_reqs, Hv, d_v] in act_dt.
 *   a, b   [num_reqs, gate_ld] in gate_dt; entries [r][h] for h < Hv are the raw
 *          projections: alpha = exp(-softplus(a)), beta = sigmoid(b).
 *   state_pool [num_slots, Hv, d_v, d_k] fp32, slot slot_ids[r] read once and
 *          written once: S' = alpha S + beta (v - alpha S k) k^T.
 *   o      [num_reqs, Hv, d_v] in o_dt: o = S' q / sqrt(d_k).
 * Alignment: state_pool 16-byte aligned; q, k 16-byte aligned when fp32,
 * 8-byte when bf16.
 */
gdn_status gdn_decode_step(const gdn_dims *dims, const void *q, const void *k,
                           const void *v, gdn_dtype act_dt, const void *a,
                           const void *b, gdn_dtype gate_dt, int64_t gate_ld,
                           float *state_pool, const int32_t *slot_ids,
                           int32_t num_reqs, int32_t num_slots, void *o,
                           gdn_dtype o_dt, void *stream);

/*
 * gdn_decode_fused — one whole decode step of the mixer core in one launch:
 * the conv update of gdn_conv1d_update, the recurrence of gdn_decode_step and
 * the gated norm of gdn_gated_norm, for one token per request (tutorial page,
 * section 02, one token's journey through a GDN layer; section 01 operator
 * table, conv / GDN / gated-output rows).  Results equal the three separate
 * calls up to fp32 rounding order; the history update is the same bit-exact
 * copy.
 *
 *   x_qkv      [num_reqs, x_ld] in act_dt: the q | k | v conv inputs of the token.
 *   z          [num_reqs, z_ld] in act_dt: the output gate, head h at columns
 *              h*d_v .. h*d_v + d_v - 1.
 *   a, b       [num_reqs, gate_ld] in act_dt: raw gate projections.
 *   conv_w     [Cqkv, taps] in w_dt; gamma [d_v] in w_dt (gated-norm gain).
 *   conv_pool  [num_slots, Cqkv, taps-1] in act_dt, updated in place.
 *   state_pool [num_slots, Hv, d_v, d_k] in state_dt, slot slot_ids[r] read once
 *              and written once.  GDN_BF16 is the state-dtype variant (the
 *              engine's `auto` state dtype may resolve away from float32; same
 *              data-structure table, state row): each element is widened exactly,
 *              updated in fp32 and rounded once to nearest-even on store.
 *   has_initial [num_reqs] uint8 (device; NULL = all 1): 0 starts the request
 *              from a zero history and a zero state (its first token).
 *   y          [num_reqs, Hv * d_v] in y_dt: RMSNorm_dv(o) * gamma * SiLU(z).
 *   o          optional [num_reqs, Hv, d_v] fp32 copy of o (NULL = not written).
 * Needs (2 d + 2 (Hv/Hk) d + 2 Hv/Hk + 32) * 4 bytes <= 64 KiB of LDS per
 * (request, key head) block, else GDN_ERR_DIMS.  Alignment: state_pool
 * 16-byte aligned, everything else element-aligned.
 */
gdn_status gdn_decode_fused(const gdn_dims *dims, const void *x_qkv, int64_t x_ld,
                            const void *z, int64_t z_ld, const void *a,
                            const void *b, int64_t gate_ld, gdn_dtype act_dt,
                            const void *conv_w, const void *gamma, gdn_dtype w_dt,
                            void *conv_pool, void *state_pool, gdn_dtype state_dt,
                            const int32_t *slot_ids, const uint8_t *has_initial,
                            int32_t num_reqs, int32_t num_slots, float l2_eps,
                            float norm_eps, void *y, gdn_dtype y_dt, float *o,
                            void *stream);

/*
 * gdn_spec_verify — speculative multi-token verify: a few tokens per request
 * (the last accepted token followed by draft tokens) through the conv update,
 * the recurrence and the gated norm in one launch, keeping the state and the
 * conv history reached after EVERY token in a slot of its own, so that
 * rejecting drafts rolls a request back by choosing the slot of its last
 * accepted token.  The pages count extra speculative slots for the conv
 * history (tutorial page, section 01 data-structure table, conv-history row)
 * and pass the number of speculative tokens into the state-shape calculator
 * (dispatch page, step 5); per-position slots are this library's reading.
 * The outputs equal gdn_prefill_fused over the same tokens; the state and
 * history in spec_slot_ids[r][j] equal those a prefill of the request's
 * first j + 1 tokens would leave.
 *
 *   x_qkv, z, a, b, conv_w, gamma, state_pool, state_dt, l2_eps, norm_eps, y,
 *              y_dt, o: as gdn_decode_fused, with one row per token of the packed
 *              batch (a bf16 state is rounded once per written position).
 *   query_start_loc [num_reqs + 1] int32 (device): request r owns tokens
 *              qsl[r] .. qsl[r+1]-1, at most max_tokens of them (a longer
 *              request is cut to its first max_tokens tokens).
 *   slot_ids   [num_reqs] int32 (device): the slot the request starts from
 *              (state and history), read and not written, unless
 *              spec_slot_ids[r][0] names it.
 *   spec_slot_ids [num_reqs, max_tokens] int32 (device): after token j of
 *              request r, its state goes to state_pool[spec_slot_ids[r][j]] and
 *              its last taps-1 conv inputs to conv_pool[spec_slot_ids[r][j]].
 *              Entries past a request's length are not read.  Every written
 *              slot must be distinct from every other written slot and from
 *              every other request's input slot (gdn_validate_spec_metadata).
 *   max_tokens 1 .. GDN_SPEC_MAX_TOKENS.
 *   has_initial [num_reqs] uint8 (device; NULL = all 1): 0 starts the request
 *              from a zero history and a zero state.
 * Needs max_tokens (2 d + 2 (Hv/Hk) d + 2 Hv/Hk + 1) * 4 + 256 bytes <= 64 KiB
 * of LDS per (request, key head) block, else GDN_ERR_DIMS.  Alignment as
 * gdn_decode_fused.  HBM traffic per request: the state read once, written
 * once per token.
 */
#define GDN_SPEC_MAX_TOKENS 8
gdn_status gdn_spec_verify(const gdn_dims *dims, const void *x_qkv, int64_t x_ld,
                           const void *z, int64_t z_ld, const void *a,
                           const void *b, int64_t gate_ld, gdn_dtype act_dt,
                           const void *conv_w, const void *gamma, gdn_dtype w_dt,
                           void *conv_pool, void *state_pool, gdn_dtype state_dt,
                           const int32_t *query_start_loc, const int32_t *slot_ids,
                           const int32_t *spec_slot_ids, int32_t max_tokens,
                           const uint8_t *has_initial, int32_t num_reqs,
                           int32_t num_tokens, int32_t num_slots, float l2_eps,
                           float norm_eps, void *y, gdn_dtype y_dt, float *o,
                           void *stream);

/*
 * gdn_prefill_workspace_bytes — device workspace gdn_prefill_varlen needs for
 * a batch of at most num_tokens tokens in at most num_reqs requests.
 * Returns 0 for unsupported dims.  The chunk length is not an argument: the
 * chunked prefill (d = 128) always runs 32-token chunks (one MFMA k-step per
 * chunk), and the sequential kernel (d < 128) has none.
 */
size_t gdn_prefill_workspace_bytes(const gdn_dims *dims, int32_t num_tokens,
                                   int32_t num_reqs);

/*
 * gdn_prefill_varlen — the gated delta rule over a packed batch of requests,
 * computed chunkwise in parallel (section 01, LM-head worked example notes:
 * the GDN block recurrence is parallelised through its associative
 * structure).  Exactly the sequential recurrence of gdn_decode_step applied to
 * every token of each request in order, up to rounding.
 *
 *   q, k   [num_tokens, Hk, d_k], v [num_tokens, Hv, d_v] in act_dt.
 *   a, b   [num_tokens, gate_ld] raw gates in gate_dt (as gdn_decode_step).
 *   state_pool [num_slots, Hv, d_v, d_k] fp32: request r starts from slot
 *          slot_ids[r] (or from zero if has_initial[r] == 0; has_initial NULL
 *          = all 1) and its final state is written back to the same slot.
 *   query_start_loc [num_reqs+1], slot_ids [num_reqs] int32, has_initial
 *          [num_reqs] uint8 — device.
 *   o      [num_tokens, Hv, d_v] in o_dt.
 *   workspace  device scratch of at least
 *          gdn_prefill_workspace_bytes(dims, num_tokens, num_reqs) bytes,
 *          256-byte aligned; contents on entry are ignored.
 */
gdn_status gdn_prefill_varlen(const gdn_dims *dims, const void *q,
                              const void *k, const void *v, gdn_dtype act_dt,
                              const void *a, const void *b, gdn_dtype gate_dt,
                              int64_t gate_ld, float *state_pool,
                              const int32_t *query_start_loc,
                              const int32_t *slot_ids,
                              const uint8_t *has_initial, int32_t num_reqs,
                              int32_t num_tokens, int32_t num_slots, void *o,
                              gdn_dtype o_dt, void *workspace,
                              size_t workspace_bytes, void *stream);

/*
 * gdn_prefill_fused_workspace_bytes / gdn_prefill_fused — a whole prefill
 * step of the mixer core over a packed batch: the conv update of
 * gdn_conv1d_update, the recurrence of gdn_prefill_varlen and the gated norm of
 * gdn_gated_norm (tutorial page, section 01 operator table, conv / GDN /
 * gated-output rows), with the intermediate q, k, v and o kept in the
 * workspace.  Arguments follow gdn_decode_fused plus the varlen metadata of
 * gdn_prefill_varlen; has_initial[r] = 0 starts request r from a zero history
 * and a zero state.  state_pool in state_dt as gdn_decode_fused (a bf16 state
 * is widened once on entry and rounded once on exit; at d = 128 it needs x
 * 16-byte aligned with 16-byte rows, else GDN_ERR_ALIGN).  y [num_tokens, Hv *
 * d_v] in y_dt.
 *   Prefix-cache snapshots ("align" mode; the dispatch page shows the hybrid
 *   model asking for --mamba-cache-mode=align): with max_snaps > 0, after the
 *   first (j + 1) * snap_interval tokens of request r (for every such prefix
 *   within the request, j < max_snaps) its state and conv history are also
 *   written to slot snap_slot_ids[r * max_snaps + j] (int32 device table
 *   [num_reqs, max_snaps]), exactly as a prefill of that prefix alone would
 *   leave them; the request's own slot still receives the final state.
 *   snap_interval is a positive multiple of GDN_SNAPSHOT_QUANTUM (the prefill's
 *   chunk), else GDN_ERR_SHAPE; snapshot slots must be distinct and distinct
 *   from every request's slot (gdn_validate_snapshot_metadata).  max_snaps = 0
 *   (snap_slot_ids may be NULL) takes none.  The workspace (at least
 * gdn_prefill_fused_workspace_bytes(dims, num_tokens, num_reqs) bytes,
 * 256-byte aligned) is scratch owned by the caller; nothing in it outlives the
 * call.  Alignment: x_ld and z_ld even, x, z, gamma and y aligned to two
 * elements, state_pool 16-byte aligned.
 */
#define GDN_SNAPSHOT_QUANTUM 32
size_t gdn_prefill_fused_workspace_bytes(const gdn_dims *dims, int32_t num_tokens,
                                         int32_t num_reqs);
gdn_status gdn_prefill_fused(const gdn_dims *dims, const void *x_qkv, int64_t x_ld,
                             const void *z, int64_t z_ld, const void *a,
                             const void *b, int64_t gate_ld, gdn_dtype act_dt,
                             const void *conv_w, const void *gamma, gdn_dtype w_dt,
                             void *conv_pool, void *state_pool, gdn_dtype state_dt,
                             const int32_t *query_start_loc, const int32_t *slot_ids,
                             const uint8_t *has_initial, int32_t num_reqs,
                             int32_t num_tokens, int32_t num_slots,
                             const int32_t *snap_slot_ids, int32_t max_snaps,
                             int32_t snap_interval, float l2_eps, float norm_eps,
                             void *y, gdn_dtype y_dt, void *workspace,
                             size_t workspace_bytes, void *stream);

/*
 * gdn_prefill_fused_noalloc — gdn_prefill_fused without a workspace argument,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  The call
 * allocates nothing: its scratch is a static device array of
 * GDN_NOALLOC_SCRATCH_BYTES in the library, one per GPU the library runs on,
 * held from the first call on that GPU until the process ends.  Arguments,
 * results and alignment are those of gdn_prefill_fused; the same kernels run.
 * A batch whose gdn_prefill_fused_workspace_bytes(dims, num_tokens, num_reqs)
 * exceeds GDN_NOALLOC_SCRATCH_BYTES returns GDN_ERR_SCRATCH before anything is
 * enqueued (at d = 128 a token takes ~86 KiB and a request ~2 MiB more: about
 * 2,900 tokens in 4 requests, or 2,000 tokens in 40).  Every call on one GPU
 * uses that GPU's one array, whose contents need no clearing (each call writes
 * what it reads): calls that overlap on one GPU (several streams, or several
 * host threads) race and must be serialised by the caller.
 */
#define GDN_NOALLOC_SCRATCH_BYTES (256u << 20)
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
                                     gdn_dtype y_dt, void *stream);

/*
 * gdn_gated_norm — Ogate = RMSNorm(o) * SiLU(Z) (operator table, gated-output
 * row: [T,48,128] -> [T,6144]; the GDN output gate is SiLU after RMSNorm,
 * evidence-matrix row on output gates).  Per (token, value head) over d_v:
 *   y[t][h*d_v + j] = o[t][h][j] / sqrt(mean_j o[t][h][j]^2 + eps) * gamma[j]
 *                     * SiLU(z[t][h][j])
 *   o      [num_tokens, Hv, d_v] in o_dt.
 *   z      [num_tokens, z_ld] in z_dt; head h at columns h*d_v .. h*d_v+d_v-1.
 *   gamma  [d_v] in gamma_dt, shared by all heads.
 *   y      [num_tokens, Hv*d_v] in y_dt.
 */
gdn_status gdn_gated_norm(const gdn_dims *dims, const void *o, gdn_dtype o_dt,
                          const void *z, gdn_dtype z_dt, int64_t z_ld,
                          const void *gamma, gdn_dtype gamma_dt, float eps,
                          int32_t num_tokens, void *y, gdn_dtype y_dt,
                          void *stream);

/*
 * gdn_rmsnorm — U = X / sqrt(mean(X^2) + eps) * gamma per row (operator table,
 * first row, [T,5120] -> [T,5120]).
 *   x [rows, cols] in x_dt, gamma [cols] in gamma_dt, y [rows, cols] in y_dt.
 *   cols must be a multiple of 8 and at most 16384.
 */
gdn_status gdn_rmsnorm(const void *x, gdn_dtype x_dt, const void *gamma,
                       gdn_dtype gamma_dt, float eps, int32_t rows, int32_t cols,
                       void *y, gdn_dtype y_dt, void *stream);

/*
 * gdn_gemm_bf16 — C[M,N] = A[M,K] * B[N,K]^T (+ R[M,N]) on bf16 operands with
 * fp32 accumulation, rounded once to c_dt (operator table: the in-projection
 * [Q0,K0,V0,Z] = U Wqkvz and a, b = U Wa, U Wb; and Delta_mix = Ogate Wo
 * followed by the residual Y = X + Delta_mix when `residual` is non-NULL).
 *   A [M, lda] bf16 row-major (activations).
 *   B [N, ldb] bf16 row-major: the weight stored output-major (row n holds the
 *     K inputs of output n), so both operands are contiguous along K.
 *   C [M, ldc] in c_dt; residual [M, ldr] bf16 or NULL (C may not alias it).
 *   K and N multiples of 8; lda, ldb, ldc, ldr multiples of 8 elements;
 *   pointers 16-byte aligned.
 */
gdn_status gdn_gemm_bf16(const void *A, int64_t lda, const void *B, int64_t ldb,
                         void *C, int64_t ldc, gdn_dtype c_dt,
                         const void *residual, int64_t ldr, int32_t M,
                         int32_t N, int32_t K, void *stream);

/*
 * gdn_gemm_bf16_ws — gdn_gemm_bf16 with a workspace (the same operation, the
 * same arguments and checks).  The output tiles of 256 x 256 fill the chip in
 * rounds of one tile per compute unit; when the last round is only partly
 * filled (or there are fewer tiles than compute units), its tiles' K stages
 * are dealt out evenly to up to one block per compute unit, each block taking
 * a contiguous run that covers at most the end of one tile and the start of
 * the next, and a second launch adds each tile's runs in a fixed order (the
 * result is the same on every run; it may differ from the unsplit sum in the
 * last bits).
 *   workspace        device memory of at least
 *                    gdn_gemm_bf16_workspace_bytes(M, N, K) bytes, 256-byte
 *                    aligned (else GDN_ERR_ALIGN), owned by the caller, free
 *                    to reuse once the call's work on `stream` is done; NULL,
 *                    or fewer bytes than asked for: nothing is split.
 * gdn_gemm_bf16_workspace_bytes — the workspace that shape asks for on the
 *   current device (two 256 KiB slots per block: at most 128 MiB on 256
 *   compute units); 0 when nothing of it would be split (K not a multiple of
 *   64, a full last round, or no more blocks of at least 256 of K than tiles).
 */
gdn_status gdn_gemm_bf16_ws(const void *A, int64_t lda, const void *B, int64_t ldb,
                            void *C, int64_t ldc, gdn_dtype c_dt,
                            const void *residual, int64_t ldr, int32_t M,
                            int32_t N, int32_t K, void *workspace,
                            size_t workspace_bytes, void *stream);
size_t gdn_gemm_bf16_workspace_bytes(int32_t M, int32_t N, int32_t K);

/*
 * gdn_validate_metadata — HOST-side check of host copies of the varlen
 * metadata: qsl[0] == 0, qsl non-decreasing, qsl[num_reqs] == num_tokens,
 * slot ids in range and distinct.  Enqueues nothing; GDN_ERR_METADATA on
 * violation.
 */
gdn_status gdn_validate_metadata(const int32_t *query_start_loc_host,
                                 const int32_t *slot_ids_host, int32_t num_reqs,
                                 int32_t num_tokens, int32_t num_slots);

/*
 * gdn_validate_snapshot_metadata — HOST-side check of host copies of
 * gdn_prefill_fused's snapshot metadata: everything gdn_validate_metadata
 * checks, snap_interval a positive multiple of GDN_SNAPSHOT_QUANTUM, and the
 * slots a call writes (snap[r][j] for (j + 1) * snap_interval within request
 * r, j < max_snaps) in range, distinct, and distinct from every request's
 * slot.  Enqueues nothing; GDN_ERR_METADATA on violation.
 */
gdn_status gdn_validate_snapshot_metadata(const int32_t *query_start_loc_host,
                                          const int32_t *slot_ids_host,
                                          const int32_t *snap_slot_ids_host,
                                          int32_t max_snaps, int32_t snap_interval,
                                          int32_t num_reqs, int32_t num_tokens,
                                          int32_t num_slots);

/*
 * gdn_validate_spec_metadata — HOST-side check of host copies of the metadata
 * of gdn_spec_verify: everything gdn_validate_metadata checks, every request at
 * most max_tokens long, and the slots a call writes (spec_slot_ids[r][j] for j
 * below the request's length) in range, distinct, and distinct from the other
 * requests' input slots (spec_slot_ids[r][0] == slot_ids[r] is allowed).
 * Enqueues nothing; GDN_ERR_METADATA on violation.
 */
gdn_status gdn_validate_spec_metadata(const int32_t *query_start_loc_host,
                                      const int32_t *slot_ids_host,
                                      const int32_t *spec_slot_ids_host,
                                      int32_t max_tokens, int32_t num_reqs,
                                      int32_t num_tokens, int32_t num_slots);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
