/*
 * gqa.h — C ABI of the decode core of the full-attention (GQA) layers that
 * alternate with the GDN layers, in the same library as gdn.h.
 *
 * The operation ("Qwen3.8-27B: from model structure to the vLLM inference
 * dataflow", section 03 MEMORY LABS, GQA / attention lab; section 04
 * PRECISION & CACHE; section 05, the PagedAttention card; the glossary's KV
 * page): 24 query heads and 4 key/value heads of 256 dims, query head h
 * reading key/value head h / 6; attention softmax(q k^T / sqrt(256)) v over
 * the request's positions; RoPE on 64 of each head's 256 dims; a sigmoid gate
 * on the attention output ahead of the output projection; K and V held in
 * fixed-size physical pages that a per-request block table maps logical
 * positions onto.
 *
 * One decode step per request r, with context length L = context_lens[r]
 * (the new token included, so the new token sits at position L - 1):
 *   1. q and k of the new token are rotated at position L - 1: over the first
 *      rotary_dim dims, dim i and dim i + rotary_dim/2 (i < rotary_dim/2) turn
 *      together by angle (L - 1) * rope_theta^(-2i/rotary_dim); the other dims
 *      pass through;
 *   2. the rotated k and v are stored at position L - 1 of the cache (k rounded
 *      once to nearest-even from the exact rotation);
 *   3. o[r, h] = sum_j softmax_j(q_h . K_j / sqrt(D)) V_j over j = 0 .. L - 1
 *      of key/value head h / (Hq / Hkv), read through the block table;
 *   4. y[r, h] = o[r, h] * sigmoid(gate[r, h]) (elementwise over the D dims).
 *
 * Conventions are those of gdn.h (device pointers owned by the caller, work
 * enqueued on `stream`, host-checkable faults reported before anything is
 * enqueued).  Supported on the GPU: head_dim 256, 1 <= Hq / Hkv <= 8,
 * rotary_dim even in [0, head_dim], a bf16 or fp8 e4m3 KV cache.
 */
#ifndef GQA_H
#define GQA_H

#include "gdn.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct gqa_dims {
    int32_t num_q_heads;  /* Hq: 24 */
    int32_t num_kv_heads; /* Hkv: 4 */
    int32_t head_dim;     /* D: 256 */
    int32_t rotary_dim;   /* rotated leading dims per head: 64 */
} gqa_dims;

/* Keys one attention block reads; a request's positions are cut into
 * ceil(L / GQA_SPLIT_KEYS) partial softmaxes that a second pass merges. */
#define GQA_SPLIT_KEYS 512

/* Workspace bytes gqa_decode_paged needs for num_reqs requests whose context
 * lengths are at most max_context_len: one partial result (max, sum and
 * unnormalised o) per (request, query head, block of GQA_SPLIT_KEYS
 * positions).  0 for invalid arguments. */
size_t gqa_decode_workspace_bytes(const gqa_dims *dims, int32_t num_reqs, int32_t max_context_len);

/* One decode step of the GQA layer over a paged KV cache (steps 1-4 above).
 *
 *   q, gate    [num_reqs, q_ld] / [num_reqs, gate_ld] in act_dt (bf16 or fp32):
 *              query head h at columns h*D .. h*D + D - 1 of the request's row.
 *   k, v       [num_reqs, kv_ld] in act_dt: key/value head j at columns j*D ...
 *   k_cache, v_cache  [num_pages, Hkv, page_size, D] in cache_dt: position p of
 *              request r lives in page block_tables[r][p / page_size] at offset
 *              p % page_size.  Updated in place at position L - 1 only.
 *              GDN_BF16: the rotated k rounded once to nearest-even, v as given.
 *              GDN_FP8_E4M3 (the server profile's KV dtype, section 04): OCP e4m3
 *              codes; code c of the K cache stands for k_scale * e4m3(c), of the V
 *              cache for v_scale * e4m3(c); the new k and v are stored as the codes
 *              nearest to (rotated k) / k_scale and v / v_scale, ties to even,
 *              saturated at +-448.
 *   k_scale, v_scale  positive finite scales of an fp8 cache (ignored for bf16).
 *   block_tables [num_reqs, max_pages_per_req] int32 (device).
 *   context_lens [num_reqs] int32 (device), new token included.
 *   max_context_len  host bound on every context length (sizes the grid and the
 *              workspace); a request whose length lies outside
 *              [1, min(max_context_len, max_pages_per_req * page_size)] is skipped:
 *              its y and o rows are written as zeros and the cache is untouched.
 *   rope_theta base of the rotation frequencies.
 *   y          [num_reqs, Hq * D] in y_dt (bf16 or fp32).
 *   o          optional [num_reqs, Hq, D] fp32 copy of the attention output
 *              before the gate (NULL = not written).
 *   workspace  device scratch of gqa_decode_workspace_bytes(dims, num_reqs,
 *              max_context_len) bytes, 16-byte aligned.
 * Contract on device-resident metadata (gqa_validate_decode_metadata checks
 * host copies): page ids of the positions 0 .. L - 1 lie in [0, num_pages), and
 * the page receiving a request's new token is read by no other request in the
 * call.  Out-of-range page ids are clamped into the cache (no fault; the result
 * is then meaningless).  Alignment: q, gate, k, v rows and the caches 16-byte
 * aligned (q_ld, gate_ld, kv_ld multiples of 8 elements).
 * An fp8 cache holds NaN codes only if the caller put them there; a NaN input
 * stores code 0 (plus its sign).
 * num_pages * Hkv * page_size must stay below 2^31.
 */
gdn_status gqa_decode_paged(const gqa_dims *dims, const void *q, int64_t q_ld, const void *gate,
                            int64_t gate_ld, const void *k, const void *v, int64_t kv_ld,
                            gdn_dtype act_dt, void *k_cache, void *v_cache, gdn_dtype cache_dt,
                            float k_scale, float v_scale,
                            const int32_t *block_tables, int32_t max_pages_per_req,
                            const int32_t *context_lens, int32_t num_reqs, int32_t num_pages,
                            int32_t page_size, int32_t max_context_len, double rope_theta, void *y,
                            gdn_dtype y_dt, float *o, void *workspace, size_t workspace_bytes,
                            void *stream);

/* Host-side check of a paged decode call's metadata (HOST pointers): every
 * context length in [1, min(max_context_len, max_pages_per_req * page_size)],
 * every page id of positions 0 .. L - 1 in [0, num_pages), and no request's
 * append page among another request's pages.  GDN_OK or GDN_ERR_METADATA
 * (GDN_ERR_NULL / GDN_ERR_SHAPE for bad arguments). */
gdn_status gqa_validate_decode_metadata(const int32_t *block_tables, int32_t max_pages_per_req,
                                        const int32_t *context_lens, int32_t num_reqs,
                                        int32_t num_pages, int32_t page_size,
                                        int32_t max_context_len);

#ifdef __cplusplus
}
#endif

#endif /* GQA_H */
