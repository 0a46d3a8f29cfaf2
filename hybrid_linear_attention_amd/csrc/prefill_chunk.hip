// Chunkwise-parallel prefill of the gated delta rule on gfx950 MFMA, d = 128.
//
// The recurrence ("Qwen3.8-27B: from model structure to the vLLM inference
// dataflow", section 01 operator table, GDN row)
//   S_t = alpha_t S_{t-1} + beta_t (v_t - alpha_t S_{t-1} k_t) k_t^T,  o_t = S_t q_t / sqrt(d)
// is associative (the page's LM-head notes: GDN's block recurrence is
// parallelised through its associative structure).  Over a chunk of C tokens
// with cumulative log-decay G_t = sum_{u<=t} log alpha_u, gamma_t = e^{G_t}, and
// state S0 entering the chunk, write S_t = gamma_t S0 + sum_{s<=t} e^{G_t-G_s}
// delta_s k_s^T.  The rank-1 "pseudo-values" delta solve a unit lower-triangular
// system:
//   (I + A) Delta = diag(beta) E,   A_ts = beta_t e^{G_t-G_s} k_t.k_s  (s < t)
//   E = V - diag(gamma) K S0^T        (the error against the decayed S0)
// and then
//   O = diag(gamma) Q S0^T + P Delta,  P_ts = e^{G_t-G_s} q_t.k_s  (s <= t)
//   S_C = gamma_C S0 + (diag(e^{G_C-G}) Delta)^T K.
// Only differences G_t - G_s with s <= t are ever exponentiated, so nothing
// overflows however strong the decay.
//
// Precision: every contraction runs on v_mfma_f32_16x16x32_bf16 with both
// operands split into bf16 hi + lo parts (hi = RNE(x), lo = RNE(x - hi)) and
// three products hi*hi + hi*lo + lo*hi accumulated in fp32: ~2^-16 relative per
// operand, which keeps the final state well inside a 1e-3 relative error even
// when the decay is weak.  A single bf16 rounding of k or of Delta would not.
//
// Chunks are C = 32 tokens: one MFMA k-step spans a chunk and the triangular
// inverse is 32x32.
//
// Three launches (two for at most 64 requests):
//   plan   one block: chunk offsets per request (prefix sum of ceil(L/C)) and
//          the requests in order of decreasing length, on the device so the
//          host never waits for query_start_loc.  For at most 64 requests the
//          prep and chain waves compute the same figures themselves, in-wave,
//          and the plan launch (and the wait for it) is skipped.
//   prep   one block per (chunk, key head), fully parallel: splits K and Q into
//          hi/lo planes, K K^T and Q K^T on MFMA, then one wave per value head:
//          the gates' cumulative decay, T = (I + A)^-1 and P.  It writes every
//          MFMA A operand the chain needs, already split and in the exact
//          per-lane fragment order, as "images": a 32 KiB K image per (chunk,
//          key head) holding K and Q (the chain reads K^T out of the K planes
//          with the transposed LDS read), and a 9 KiB T image per (chunk, value
//          head) holding T, P and the per-token gamma, e^{G_C-G_t} and beta.
//   chain  sequential over each request's chunks: only the state-dependent
//          products.  Each chunk's images are copied global -> LDS with
//          direct-to-LDS loads (global_load_lds_dwordx4) into a ring of stages
//          while earlier chunks compute; every operand fragment is then one
//          conflict-free 16-byte LDS read.  State rows evolve independently
//          given (k, beta, alpha), so the row blocks of a head never
//          communicate.  Three block layouts: per (request, key head, 64 rows)
//          over the key head's 3 value heads (large batches), per (request,
//          value head, 128 rows) (large batches of other head ratios), and per
//          (request, value head, 32 rows) with the recurrence and the output
//          on separate waves (few requests, where one block's chunk latency is
//          the kernel's time).
#include "gdn_device.h"
#include "gdn_launch.h"

#include <type_traits>

namespace gdn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

namespace chunk {

constexpr int D = 128;      // d_k == d_v
constexpr int CH = 32;      // tokens per chunk
constexpr int KP = D + 8;   // padded bf16 row of the prep kernel's 128-wide planes (272 B)
constexpr int AP = CH + 4;  // padded fp32 row of 32x32 work matrices

// An image is a sequence of fragment blocks: 64 lanes x 16 bytes, lane l at
// byte 16 l, holding the eight bf16 values of one MFMA A operand in k-slot
// order (see the chain kernel's layout note).
constexpr int FRAG = 1024;
// K image: K and Q as (plane hi/lo, row tile tau, k-step ks).  The chain's K^T
// operands are read from the K planes with the transposed LDS read.
constexpr int FK = 0, FQ = 16, KIMG_FRAGS = 32;
// T image: T and P as (plane, tau), then three float[32] token vectors
constexpr int FT = 0, FP = 4, TIMG_FRAGS = 9;
constexpr int T_GAM = 8 * FRAG, T_REV = T_GAM + 128, T_BETA = T_REV + 128;
constexpr size_t KIMG = (size_t)KIMG_FRAGS * FRAG;  // 32,768 bytes
constexpr size_t TIMG = (size_t)TIMG_FRAGS * FRAG;  //  9,216 bytes

constexpr int PLAN_SORT_MAX = 4096;  // longest-first order for up to this many requests

// x = hi + lo with hi = RNE_bf16(x), lo = RNE_bf16(x - hi), two values at a
// time into packed bf16 pairs: one two-value conversion gives both hi parts,
// whose fp32 values are the pair's low half shifted up and its high half
// masked, so each lo costs a subtract and half a conversion (three VALU
// operations per value).
typedef float float2v_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void split2(float x0, float x1, uint32_t &h, uint32_t &l) {
    h = __builtin_bit_cast(uint32_t, __builtin_convertvector(float2v_t{x0, x1}, bf16x2_t));
    const float h0 = __uint_as_float(h << 16), h1 = __uint_as_float(h & 0xffff0000u);
    l = __builtin_bit_cast(uint32_t, __builtin_convertvector(float2v_t{x0 - h0, x1 - h1}, bf16x2_t));
}

__device__ __forceinline__ void split4_store(float a, float b, float c, float d, uint16_t *ph,
                                             uint16_t *pl) {
    uint32_t h0, l0, h1, l1;
    split2(a, b, h0, l0);
    split2(c, d, h1, l1);
    *reinterpret_cast<uint2 *>(ph) = make_uint2(h0, h1);
    *reinterpret_cast<uint2 *>(pl) = make_uint2(l0, l1);
}

// eight values -> two 16-byte hi/lo fragment pieces
__device__ __forceinline__ void split_pack(const float (&x)[8], uint4 &hi, uint4 &lo) {
    uint32_t h[4], l[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) split2(x[2 * p], x[2 * p + 1], h[p], l[p]);
    hi = make_uint4(h[0], h[1], h[2], h[3]);
    lo = make_uint4(l[0], l[1], l[2], l[3]);
}

// eight values (MFMA k-slot order) -> hi/lo operands
__device__ __forceinline__ void split_vals(const float (&x)[8], bf16x8_t &hi, bf16x8_t &lo) {
    uint4 h, l;
    split_pack(x, h, l);
    hi = __builtin_bit_cast(bf16x8_t, h);
    lo = __builtin_bit_cast(bf16x8_t, l);
}

__device__ __forceinline__ bf16x8_t frag(const uint8_t *p) {
    return *reinterpret_cast<const bf16x8_t *>(p);
}

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// Transposed LDS read (gfx950 ds_read_b64_tr_b16): within each 16-lane group,
// lane i receives element i % 4 of the 8-byte words read by lanes 4 j + i / 4,
// j = 0..3, in order of j.
__device__ __forceinline__ s16x4_t lds_read_tr(const uint8_t *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4_t *)((__attribute__((address_space(3))) uint8_t *)(p)));
}

// This lane's byte offset for the K^T reads: lane (lr, lg) supplies the four
// channels 16 jt + 4 (lr % 4) .. + 3 of token 4 lg + lr / 4 (second read: of
// token 16 + 4 lg + lr / 4), which sit in K fragment (tau, ks = jt / 2) at lane
// (token % 16) + 16 (lr % 4), half jt % 2.
__device__ __forceinline__ uint32_t kt_lane_off(int lr, int lg) {
    return 16u * (uint32_t)((4 * lg + (lr >> 2)) + 16 * (lr & 3));
}

// The K^T operand (rows 16 jt + lr of K^T, i.e. channels; k-slots the tokens in
// the chain's slot order) of plane `plane` (0 hi, 1 lo) from the staged K
// image: lane i of 16-lane group lg then holds K[4 lg + j][16 jt + i] for
// j = 0..3 (first read) and K[16 + 4 lg + j][16 jt + i] (second read).
__device__ __forceinline__ bf16x8_t kt_frag(const uint8_t *kimg_lane, int plane, int jt) {
    const uint8_t *p = kimg_lane + ((FK + plane * 8 + (jt >> 1)) * FRAG + 8 * (jt & 1));
    const s16x4_t a = lds_read_tr(p);             // tau = 0: tokens 4 lg + j
    const s16x4_t b = lds_read_tr(p + 4 * FRAG);  // tau = 1: tokens 16 + 4 lg + j
    const s16x4_t ab[2] = {a, b};
    return __builtin_bit_cast(bf16x8_t, ab);
}

// acc += a * b with a = ah + al, b = bh + bl (the lo*lo term is below fp32 noise).
__device__ __forceinline__ void mma3(floatx4_t &acc, const bf16x8_t &ah, const bf16x8_t &al,
                                     const bf16x8_t &bh, const bf16x8_t &bl) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
}

// A scalar load kept in its storage format until use, so that issuing it never
// waits for its own data.
template <typename T> struct Raw1;
template <> struct Raw1<float> {
    float v;
    __device__ __forceinline__ void load(const float *p) { v = *p; }
    __device__ __forceinline__ void zero() { v = 0.f; }
    __device__ __forceinline__ float get() const { return v; }
};
template <> struct Raw1<bf16> {
    uint16_t v;
    __device__ __forceinline__ void load(const bf16 *p) { v = *reinterpret_cast<const uint16_t *>(p); }
    __device__ __forceinline__ void zero() { v = 0; }
    __device__ __forceinline__ float get() const { return __uint_as_float(uint32_t(v) << 16); }
};

// One 16-byte direct-to-LDS copy per lane: lane l's bytes land at LDS address
// lds_frag + 16 l.  Issued as inline assembly (LDS base in M0, the fragment's
// global address in scalar registers, the lane's byte offset 16 l in a vector
// register) rather than through the compiler builtin: the compiler cannot tell
// the two ring stages apart, so after a builtin copy into the next stage it
// waits for every outstanding load before any LDS read of the current stage,
// which stalls each chunk mid-way on the next chunk's copies; and the builtin
// forms each address in vector registers and moves it to M0 through a
// readfirstlane, eight instructions per copy.  Here the copies are invisible to
// the compiler's wait analysis and the chain waits for them itself, once per
// chunk, before the barrier that publishes the stage (vector-memory counts
// complete in order, so the compiler's own waits for other loads stay correct,
// only more conservative).  src_frag and lds_frag must be wave-uniform.
__device__ __forceinline__ void copy_frag(const uint8_t *src_frag, uint32_t lds_frag, uint32_t lane_off) {
    asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(lane_off), "s"(src_frag), "{m0}"(lds_frag) : "memory");
}

// The wave-uniform LDS address of a shared-memory pointer.
__device__ __forceinline__ uint32_t lds_addr(const uint8_t *p) {
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t *)(p));
}

// A buffer resource over [base, base + bytes) from wave-uniform values.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t wave_rsrc(const void *base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    const uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(((uint64_t)hi << 32) | lo), (short)0,
                                             (int)n, 0x00020000);
}

// o of one token and state row through a range-checked buffer store: tokens
// past the chunk's last fall outside the resource and are dropped, so every
// chunk issues the same number of stores and the chunk-top wait can leave
// them in flight.
template <typename TO> __device__ __forceinline__ void store_o(__amdgpu_buffer_rsrc_t r, uint32_t off, float v);
template <> __device__ __forceinline__ void store_o<float>(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, (int)(off * 4), 0, 0);
}
template <> __device__ __forceinline__ void store_o<bf16>(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
    __builtin_amdgcn_raw_buffer_store_b16((unsigned short)to_bf16(v).bits, r, (int)(off * 2), 0, 0);
}

// s_waitcnt immediate: vector-memory count <= vm, LDS/scalar and export counts 0
constexpr int waitcnt_vm(int vm) { return (vm & 15) | ((vm >> 4) << 14); }

}  // namespace chunk

// ---------------------------------------------------------------------------
// plan: chunk_off[r] = sum_{r' < r} ceil(L_r' / C); order = requests by
// decreasing length (ties by index) so the longest chains start first
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void prefill_plan_kernel(const int32_t *__restrict__ qsl,
                                                            int32_t nreq,
                                                            int32_t *__restrict__ chunk_off,
                                                            int32_t *__restrict__ order) {
    __shared__ int32_t part[1024];
    __shared__ int32_t lens[chunk::PLAN_SORT_MAX];
    const int tid = threadIdx.x;
    const int per = (nreq + 1023) / 1024;
    const int r0 = min(nreq, tid * per), r1 = min(nreq, r0 + per);
    int local = 0;
    for (int r = r0; r < r1; ++r) local += (qsl[r + 1] - qsl[r] + chunk::CH - 1) / chunk::CH;
    part[tid] = local;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {  // inclusive Hillis-Steele scan
        const int add = tid >= off ? part[tid - off] : 0;
        __syncthreads();
        part[tid] += add;
        __syncthreads();
    }
    int run = part[tid] - local;
    if (tid == 0) chunk_off[0] = 0;
    for (int r = r0; r < r1; ++r) {
        run += (qsl[r + 1] - qsl[r] + chunk::CH - 1) / chunk::CH;
        chunk_off[r + 1] = run;
    }
    if (nreq <= chunk::PLAN_SORT_MAX) {  // uniform over the block
        for (int r = tid; r < nreq; r += 1024) lens[r] = qsl[r + 1] - qsl[r];
        __syncthreads();
        for (int r = tid; r < nreq; r += 1024) {
            const int L = lens[r];
            int rank = 0;
            for (int r2 = 0; r2 < nreq; ++r2) {
                const int L2 = lens[r2];
                rank += (L2 > L) || (L2 == L && r2 < r);
            }
            order[rank] = r;
        }
    } else {
        for (int r = tid; r < nreq; r += 1024) order[r] = r;
    }
}

// The same plan inside a wave, for at most PLAN_WAVE_MAX requests: the launch
// of the plan kernel and the wait for it cost more than every wave of the
// prep and chain blocks working it out for itself (no LDS, no barrier).  Lane
// t holds request t's length and the inclusive prefix sum of the chunk counts.
constexpr int PLAN_WAVE_MAX = 64;
struct WavePlan {
    int len, incl;
};
__device__ __forceinline__ WavePlan wave_plan(const int32_t *__restrict__ qsl, int nreq, int lane) {
    WavePlan p{0, 0};
    if (lane < nreq) p.len = qsl[lane + 1] - qsl[lane];
    p.incl = (p.len + chunk::CH - 1) / chunk::CH;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int u = __shfl_up(p.incl, off, 64);
        if (lane >= off) p.incl += u;
    }
    return p;
}
// chunk c's request (and its first chunk), as find_request over the offsets;
// total: every request's chunks
__device__ __forceinline__ int wave_plan_chunk(const WavePlan &p, int nreq, int c, int &c_first, int &total) {
    total = __builtin_amdgcn_readfirstlane(__shfl(p.incl, nreq - 1, 64));
    const int r = __builtin_amdgcn_readfirstlane(__popcll(__ballot(p.incl <= c) & (nreq >= 64 ? ~0ull : ((1ull << nreq) - 1))));
    c_first = r > 0 ? __builtin_amdgcn_readfirstlane(__shfl(p.incl, r - 1, 64)) : 0;
    return r;
}
// the request of rank k in the plan's order (longest first, ties by index)
// and its first chunk
__device__ __forceinline__ int wave_plan_rank(const WavePlan &p, int nreq, int lane, int k, int &c_first) {
    int rank = 0;
    for (int u = 0; u < nreq; ++u) {
        const int lu = __shfl(p.len, u, 64);
        rank += (lu > p.len) || (lu == p.len && u < lane);
    }
    const int r = __builtin_amdgcn_readfirstlane(__ffsll((long long)__ballot(lane < nreq && rank == k)) - 1);
    c_first = r > 0 ? __builtin_amdgcn_readfirstlane(__shfl(p.incl, r - 1, 64)) : 0;
    return r;
}

// ---------------------------------------------------------------------------
// prep: per (chunk, key head): the K image, then one wave per value head for
// its T image
// ---------------------------------------------------------------------------
namespace chunk {
constexpr int XR = CH + 3;      // staged conv rows: the 3 tokens before the chunk, then its own
constexpr int XSP = 2 * D + 8;  // padded staged row: q channels, then k channels (bf16)
// One region, three lives: the staged conv input rows (read by the conv, whose
// results wait in registers until every read is done), then the hi / lo planes
// of K and Q (dead once the K image is written and the K K^T / Q K^T tiles,
// which also wait in registers, are formed), then those tiles and the per-wave
// work matrices.  34,816 bytes, so four blocks share a CU.
struct PrepSmem {
    union {
        uint16_t xs[XR][XSP];
        struct { uint16_t Kh[CH][KP], Kl[CH][KP], Qh[CH][KP], Ql[CH][KP]; };
        struct {
            float KK[CH][AP], QK[CH][AP];
            float A[4][CH][AP];   // per-wave work matrix: A, then T = (I + A)^-1
            float G[4][CH], Beta[4][CH];
        };
    };
};
static_assert(sizeof(PrepSmem) == 4 * CH * KP * 2, "the prep kernel's LDS is the K / Q planes' size");
}  // namespace chunk

// Conv inputs of the prep kernel's conv mode: q and k of the chunk are formed
// from x (4-tap causal conv + SiLU + L2 norm, the request's history for rows
// before its start) instead of being read.
struct PrepConvIn {
    const void *x; int64_t x_ld;
    const void *w;
    const void *pool; const int32_t *slots; const uint8_t *has_init;
    int32_t C; float l2_eps;
};

template <typename TA, typename TG, typename TX, typename TW, bool CONV>
__global__ __launch_bounds__(256) void prefill_prep_kernel(
    const TA *__restrict__ q, const TA *__restrict__ k, const TG *__restrict__ ga,
    const TG *__restrict__ gb, int64_t gate_ld, const int32_t *__restrict__ qsl,
    const int32_t *__restrict__ chunk_off, int32_t nreq, int32_t Hk, int32_t Hv,
    uint8_t *__restrict__ kimg, uint8_t *__restrict__ timg, PrepConvIn cv) {
    using namespace chunk;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem_raw[];
    PrepSmem &sm = *reinterpret_cast<PrepSmem *>(smem_raw);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;

    const int c = blockIdx.x / Hk;
    const int kh = blockIdx.x - c * Hk;
    // without chunk offsets (few requests) every wave works out the plan
    int r, c_first;
    if (chunk_off == nullptr) {
        int total;
        r = wave_plan_chunk(wave_plan(qsl, nreq, lane), nreq, c, c_first, total);
        if (c >= total) return;
    } else {
        if (c >= chunk_off[nreq]) return;
        r = find_request(chunk_off, nreq, c);
        c_first = chunk_off[r];
    }
    const int tb = qsl[r] + CH * (c - c_first);
    const int Lc = min(CH, qsl[r + 1] - tb);
    const int group = Hv / Hk;

    // this wave's first value head: its gates load while K and Q are staged
    Raw1<TG> ga0, gb0;
    ga0.zero();
    gb0.zero();
    if (w < group && lane < Lc) {
        const int64_t go = (int64_t)(tb + lane) * gate_ld + kh * group + w;
        ga0.load(ga + go);
        gb0.load(gb + go);
    }

    if constexpr (!CONV) {
        // stage K and Q of the key head as hi/lo planes (1024 four-element slots each)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int idx = tid + 256 * m;
            const int t = idx >> 5;
            const int c4 = (idx & 31) * 4;
            float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), qv = kv;
            if (t < Lc) {
                const int64_t off = ((int64_t)(tb + t) * Hk + kh) * D + c4;
                kv = ld4(k + off);
                qv = ld4(q + off);
            }
            split4_store(kv.x, kv.y, kv.z, kv.w, &sm.Kh[t][c4], &sm.Kl[t][c4]);
            split4_store(qv.x, qv.y, qv.z, qv.w, &sm.Qh[t][c4], &sm.Ql[t][c4]);
        }
    } else {
        // The conv inputs of the chunk are staged in LDS with coalesced 16-byte
        // loads, NCH channels per pass: the key head's q and k channels (bf16:
        // one pass; fp32: q, then k).  Staged row rr holds token tb - 3 + rr;
        // rows before the request start come from its history (zeros without
        // one); rows past the chunk's last token are zeros.  The next pass's
        // rows are loaded while the current pass computes: every lane issues
        // the same loads (out-of-range pieces read a valid address and are
        // zeroed when staged), so the compiler's waits for the pass's taps
        // leave them in flight.
        constexpr int NCH = 512 / (int)sizeof(TX);  // channels per pass (512 bytes a row)
        constexpr int NPASS = 2 * D / NCH;          // q / k passes
        constexpr int EPP = 16 / (int)sizeof(TX);   // channels per 16-byte piece
        constexpr int NCG = NCH / 8;                // 8-channel groups per pass
        constexpr int TPT = CH * NCG / 256;         // tokens per thread
        constexpr int NPIECE = XR * 32;
        constexpr int NM = (NPIECE + 255) / 256;
        const int t0 = qsl[r];
        const TX *x = static_cast<const TX *>(cv.x);
        TX(*xs)[XSP * 2 / (int)sizeof(TX)] = reinterpret_cast<TX(*)[XSP * 2 / (int)sizeof(TX)]>(&sm.xs[0][0]);
        constexpr int npass_all = NPASS;
        // channel of column cq of pass ps (q: 0 .. D-1, k: D .. 2D-1 over the passes)
        auto pass_chan = [&](int ps, int cq) -> int {
            const int c2 = ps * NCH + cq;
            return (c2 >= D ? Hk * D : 0) + kh * D + (c2 & (D - 1));
        };
        auto load_pass = [&](uint4 (&pv)[NM], int ps) {
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                const int pi = tid + 256 * m;
                const int rr = pi >> 5, seg = pi & 31;
                const int tok = tb - 3 + rr;
                const int ch = pass_chan(ps, EPP * seg);
                const bool ok = pi < NPIECE && tok >= t0 && rr - 3 < Lc;
                pv[m] = *reinterpret_cast<const uint4 *>(x + (ok ? (int64_t)tok * cv.x_ld + ch : (int64_t)0));
            }
        };
        auto stage_pass = [&](const uint4 (&pv)[NM], int ps) {
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                const int pi = tid + 256 * m;
                const int rr = pi >> 5, seg = pi & 31;
                const int tok = tb - 3 + rr;
                const bool ok = pi < NPIECE && tok >= t0 && rr - 3 < Lc;
                if (pi < NPIECE && tok >= t0)
                    *reinterpret_cast<uint4 *>(&xs[rr][EPP * seg]) = ok ? pv[m] : make_uint4(0u, 0u, 0u, 0u);
            }
            if (tb == t0) {  // first chunk of its request (uniform over the block)
                const bool hi = cv.has_init == nullptr || cv.has_init[r] != 0;
                const int64_t hbase = (int64_t)cv.slots[r] * cv.C;
                const TX *pool = static_cast<const TX *>(cv.pool);
#pragma unroll
                for (int j = 0; j < (3 * NCH + 255) / 256; ++j) {  // history entry rr = row rr
                    const int idx = tid + 256 * j;
                    const int rr = idx / NCH, cc = idx % NCH;
                    const int ch = pass_chan(ps, cc);
                    if (rr < 3) xs[rr][cc] = hi ? pool[(hbase + ch) * 3 + rr] : TX{};
                }
            }
        };
        // compute mapping: 8 channels (group cgi) of tokens TPT tg .. TPT tg + TPT - 1;
        // the 16 groups of one token's q (or k) are 16 aligned adjacent lanes
        const int tg = tid / NCG, cgi = tid % NCG;
        uint4 pv[NM];
        // normalised q / k of this thread's tokens and channels, per pass, kept
        // until every thread is done reading the staged rows
        float qk[NPASS][TPT][8];
        load_pass(pv, 0);
#pragma unroll
        for (int ps = 0; ps < npass_all; ++ps) {
            if (ps) __syncthreads();  // the previous pass is done with the staged rows
            stage_pass(pv, ps);
            __syncthreads();
            const int ch0 = pass_chan(ps, 8 * cgi);
            float wf[32];  // w[channel + e][i] at 4 e + i
            {
                const TW *wp = static_cast<const TW *>(cv.w) + (int64_t)ch0 * 4;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    Raw8<TW> wr;
                    wr.load(wp + 8 * j);
                    float f8[8];
                    wr.get(f8);
#pragma unroll
                    for (int e = 0; e < 8; ++e) wf[8 * j + e] = f8[e];
                }
            }
            // unconditional (the last pass reloads its own rows, L2-resident) and
            // kept after the taps' loads, so that the wait for the taps never
            // covers these loads
            __builtin_amdgcn_sched_barrier(0);
            load_pass(pv, min(ps + 1, npass_all - 1));
            __builtin_amdgcn_sched_barrier(0);
            float y[TPT][8];
#pragma unroll
            for (int j = 0; j < TPT; ++j)
#pragma unroll
                for (int e = 0; e < 8; ++e) y[j][e] = 0.f;
            // staged row TPT tg + rw is token TPT tg + rw - 3: tap i of token TPT tg + j
#pragma unroll
            for (int rw = 0; rw < TPT + 3; ++rw) {
                Raw8<TX> xr;
                xr.load(&xs[TPT * tg + rw][8 * cgi]);
                float xe[8];
                xr.get(xe);
#pragma unroll
                for (int j = 0; j < TPT; ++j) {
                    const int i = j + 3 - rw;
                    if (i >= 0 && i < 4) {
#pragma unroll
                        for (int e = 0; e < 8; ++e) y[j][e] += wf[4 * e + i] * xe[e];
                    }
                }
            }
            {
                // q or k: SiLU, L2 norm over the head
#pragma unroll
                for (int j = 0; j < TPT; ++j) {
                    const int t = TPT * tg + j;
                    float ss = 0.f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        y[j][e] = t < Lc ? silu_fast(y[j][e]) : 0.f;
                        ss += y[j][e] * y[j][e];
                    }
                    ss = group_sum<16>(ss);
                    const float inv = 1.0f / sqrtf(ss + cv.l2_eps);
#pragma unroll
                    for (int e = 0; e < 8; ++e) qk[ps][j][e] = y[j][e] * inv;
                }
            }
        }
        // every read of the staged rows is done: q and k into their hi / lo planes
        __syncthreads();
#pragma unroll
        for (int ps = 0; ps < npass_all; ++ps) {
            const int cq = ps * NCH + 8 * cgi;
            const bool isk = cq >= D;
            const int col = cq & (D - 1);
#pragma unroll
            for (int j = 0; j < TPT; ++j) {
                const int t = TPT * tg + j;
                uint16_t *ph = isk ? &sm.Kh[t][col] : &sm.Qh[t][col];
                uint16_t *pl = isk ? &sm.Kl[t][col] : &sm.Ql[t][col];
                split4_store(qk[ps][j][0], qk[ps][j][1], qk[ps][j][2], qk[ps][j][3], ph, pl);
                split4_store(qk[ps][j][4], qk[ps][j][5], qk[ps][j][6], qk[ps][j][7], ph + 4, pl + 4);
            }
        }
    }
    __syncthreads();

    // K image: 32 fragment blocks x 64 lanes = 8 pieces per thread, each a
    // coalesced 16-byte store
    {
        uint8_t *kim = kimg + ((size_t)c * Hk + kh) * KIMG;
#pragma unroll 4
        for (int m = 0; m < 8; ++m) {
            const int pi = tid + 256 * m;
            const int f = pi >> 6;
            const int l = pi & 63;
            const int plr = l & 15, plg = l >> 4;
            // K or Q rows 16 tau + lr, channels 32 ks + 4 lg + {0..3, 16..19}
            const int ff = f & 15;
            const int plane = ff >> 3, tau = (ff >> 2) & 1, ks = ff & 3;
            const bool isQ = f >= FQ;
            const uint16_t *row = isQ ? (plane ? sm.Ql[16 * tau + plr] : sm.Qh[16 * tau + plr])
                                      : (plane ? sm.Kl[16 * tau + plr] : sm.Kh[16 * tau + plr]);
            const int c0 = 32 * ks + 4 * plg;
            const uint2 a = *reinterpret_cast<const uint2 *>(row + c0);
            const uint2 b = *reinterpret_cast<const uint2 *>(row + c0 + 16);
            *reinterpret_cast<uint4 *>(kim + (size_t)f * FRAG + 16 * l) = make_uint4(a.x, a.y, b.x, b.y);
        }
    }

    // K K^T and Q K^T on the three lower-triangular 16x16 tiles of each (items
    // w and w + 4 of this wave), kept in registers until every wave is done
    // with the planes, whose space the tiles then take
    floatx4_t kacc[2];
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
        const int item = w + 4 * ii;
        kacc[ii] = floatx4_t{0.f, 0.f, 0.f, 0.f};
        if (item < 6) {
            const bool isQ = item >= 3;
            const int n = isQ ? item - 3 : item;
            const int tm = n == 0 ? 0 : 1;
            const int tn = n == 2 ? 1 : 0;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int off = 32 * ks + 8 * lg;
                const uint16_t *arow_h = isQ ? sm.Qh[16 * tm + lr] : sm.Kh[16 * tm + lr];
                const uint16_t *arow_l = isQ ? sm.Ql[16 * tm + lr] : sm.Kl[16 * tm + lr];
                const bf16x8_t ah = *reinterpret_cast<const bf16x8_t *>(arow_h + off);
                const bf16x8_t al = *reinterpret_cast<const bf16x8_t *>(arow_l + off);
                const bf16x8_t bh = *reinterpret_cast<const bf16x8_t *>(&sm.Kh[16 * tn + lr][off]);
                const bf16x8_t bl = *reinterpret_cast<const bf16x8_t *>(&sm.Kl[16 * tn + lr][off]);
                mma3(kacc[ii], ah, al, bh, bl);
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
        const int item = w + 4 * ii;
        if (item < 6) {
            const bool isQ = item >= 3;
            const int n = isQ ? item - 3 : item;
            const int tm = n == 0 ? 0 : 1;
            const int tn = n == 2 ? 1 : 0;
            float(*dst)[AP] = isQ ? sm.QK : sm.KK;
#pragma unroll
            for (int e = 0; e < 4; ++e) dst[16 * tm + 4 * lg + e][16 * tn + lr] = kacc[ii][e];
        }
    }
    __syncthreads();

    // one wave per value head: nothing below crosses waves
    for (int hh = w; hh < group; hh += 4) {
        const int h = kh * group + hh;
        uint8_t *tim = timg + ((size_t)c * Hv + h) * TIMG;
        float(*A)[AP] = sm.A[w];
        float *Gw = sm.G[w];
        float *Bw = sm.Beta[w];
        {
            float g = 0.f, beta = 0.f;
            if (lane < Lc) {
                if (hh == w) {
                    g = gate_log_alpha(ga0.get());
                    beta = gate_beta(gb0.get());
                } else {
                    const int64_t go = (int64_t)(tb + lane) * gate_ld + h;
                    g = gate_log_alpha(ld(ga + go));
                    beta = gate_beta(ld(gb + go));
                }
            }
            float G = g;  // inclusive prefix sum over the chunk; padded rows add nothing
#pragma unroll
            for (int off = 1; off < CH; off <<= 1) {
                const float y = __shfl_up(G, off, 64);
                if (lane >= off) G += y;
            }
            const float Glast = __shfl(G, CH - 1, 64);
            if (lane < CH) {
                Gw[lane] = G;
                Bw[lane] = beta;
                reinterpret_cast<float *>(tim + T_GAM)[lane] = expf(G);
                reinterpret_cast<float *>(tim + T_REV)[lane] = expf(Glast - G);
                reinterpret_cast<float *>(tim + T_BETA)[lane] = beta;
            }
        }
        __builtin_amdgcn_wave_barrier();
        // A = strict-lower(beta_t e^{G_t-G_s} KK) into the work matrix
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int idx = lane + 64 * m;  // 256 groups of 4 columns
            const int t = idx >> 3;
            const int s0 = (idx & 7) * 4;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int s = s0 + e;
                A[t][s] = s < t ? Bw[t] * __expf(fminf(Gw[t] - Gw[s], 0.f)) * sm.KK[t][s] : 0.f;
            }
        }
        // P = lower(e^{G_t-G_s} QK) straight into its fragments:
        // row t = 16 tau + lr, columns s = 4 lg + {0..3, 16..19}
#pragma unroll
        for (int tau = 0; tau < 2; ++tau) {
            const int t = 16 * tau + lr;
            float pv[8];
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                const int s = 16 * (p >> 2) + 4 * lg + (p & 3);
                pv[p] = s <= t ? __expf(fminf(Gw[t] - Gw[s], 0.f)) * sm.QK[t][s] : 0.f;
            }
            uint4 hi, lo;
            split_pack(pv, hi, lo);
            *reinterpret_cast<uint4 *>(tim + (size_t)(FP + tau) * FRAG + 16 * lane) = hi;
            *reinterpret_cast<uint4 *>(tim + (size_t)(FP + 2 + tau) * FRAG + 16 * lane) = lo;
        }
        __builtin_amdgcn_wave_barrier();
        // T = (I + A)^-1: the two 16x16 diagonal blocks by substitution, then
        // T10 = -T11 (A10 T00).  Lane (lr, lg) holds column lr, rows lg + 4 e of a
        // block; the A rows it needs sit in registers, and columns of earlier
        // results come from other lanes by shuffles.
        float xb[2][4];  // T00 and T11 columns
#pragma unroll
        for (int bi = 0; bi < 2; ++bi) {
            const int bb = 16 * bi;
            float ar[4][16];
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int c4 = 0; c4 < 4; ++c4) {
                    const float4 a4 = *reinterpret_cast<const float4 *>(&A[bb + lg + 4 * e][bb + 4 * c4]);
                    ar[e][4 * c4] = a4.x; ar[e][4 * c4 + 1] = a4.y; ar[e][4 * c4 + 2] = a4.z; ar[e][4 * c4 + 3] = a4.w;
                }
            float x[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = (lg + 4 * e == lr) ? 1.f : 0.f;
#pragma unroll
            for (int s2 = 0; s2 < 16; ++s2) {
                const float xs = __shfl(x[s2 >> 2], (s2 & 3) * 16 + lr, 64);  // X[s2][lr]
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (lg + 4 * e > s2) x[e] -= ar[e][s2] * xs;
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) xb[bi][e] = x[e];
        }
        {
            // Y = A10 T00 (rows 16 + lg + 4 e, column lr)
            float y[4] = {0.f, 0.f, 0.f, 0.f};
            float a10[4][16];
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int c4 = 0; c4 < 4; ++c4) {
                    const float4 a4 = *reinterpret_cast<const float4 *>(&A[16 + lg + 4 * e][4 * c4]);
                    a10[e][4 * c4] = a4.x; a10[e][4 * c4 + 1] = a4.y; a10[e][4 * c4 + 2] = a4.z; a10[e][4 * c4 + 3] = a4.w;
                }
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const float tu = __shfl(xb[0][u >> 2], (u & 3) * 16 + lr, 64);  // T00[u][lr]
#pragma unroll
                for (int e = 0; e < 4; ++e) y[e] += a10[e][u] * tu;
            }
            // T11 rows of this lane: lane (u, lg) holds T11[lg + 4 e][u]
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int e = 0; e < 4; ++e) A[16 + lg + 4 * e][16 + lr] = xb[1][e];
            __builtin_amdgcn_wave_barrier();
            float t11[4][16];
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int c4 = 0; c4 < 4; ++c4) {
                    const float4 a4 = *reinterpret_cast<const float4 *>(&A[16 + lg + 4 * e][16 + 4 * c4]);
                    t11[e][4 * c4] = a4.x; t11[e][4 * c4 + 1] = a4.y; t11[e][4 * c4 + 2] = a4.z; t11[e][4 * c4 + 3] = a4.w;
                }
            float tv[4] = {0.f, 0.f, 0.f, 0.f};  // T10 = -T11 Y
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const float yu = __shfl(y[u >> 2], (u & 3) * 16 + lr, 64);  // Y[u][lr]
#pragma unroll
                for (int e = 0; e < 4; ++e) tv[e] -= t11[e][u] * yu;
            }
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                A[lg + 4 * e][lr] = xb[0][e];
                A[16 + lg + 4 * e][lr] = tv[e];
            }
            __builtin_amdgcn_wave_barrier();
        }
        // T (lower triangle, zeros above) into its fragments
#pragma unroll
        for (int tau = 0; tau < 2; ++tau) {
            const int t = 16 * tau + lr;
            float tv[8];
#pragma unroll
            for (int p = 0; p < 8; ++p) tv[p] = A[t][16 * (p >> 2) + 4 * lg + (p & 3)];
            uint4 hi, lo;
            split_pack(tv, hi, lo);
            *reinterpret_cast<uint4 *>(tim + (size_t)(FT + tau) * FRAG + 16 * lane) = hi;
            *reinterpret_cast<uint4 *>(tim + (size_t)(FT + 2 + tau) * FRAG + 16 * lane) = lo;
        }
        __builtin_amdgcn_wave_barrier();
    }
}

// ---------------------------------------------------------------------------
// chain: sequential over a request's chunks, per (request, value head, block
// of 16 NW state rows).  Wave w owns state rows 16 w .. 16 w + 15 of the block
// for all 32 tokens of a chunk, so the error E, the pseudo-values Delta and the
// state itself never leave its registers:
//   X = K S0^T, OQ = Q S0^T        (A: K / Q fragments, B: state registers)
//   Delta = T (beta E)             (A: T fragments,     B: E registers)
//   O = gamma OQ + P Delta         (A: P fragments,     B: Delta registers)
//   S^T = gamma_C S^T + K^T Delta~ (A: K^T operands,    B: Delta registers)
// An accumulator lane holds rows 4 lg + e of a 16-row tile; feeding it back
// as the B operand of the next product uses the k-slot order
//   slot (lg, p) -> 32 ks + 16 (p / 4) + 4 lg + p % 4,
// and the prep kernel wrote the A fragments in that same order, so no register
// ever crosses lanes.  The K^T operands come from the staged K planes through
// the transposed LDS read (kt_frag).
//
// In the fused prefill (XCONV) the chain also forms v: its rows of state are
// value channels, so each block stages the raw conv inputs of its own v
// channels (35 rows of x per chunk, the 3 before it included) in LDS beside
// the chunk's images, and every lane convolves its channel for its tokens.
//
// Blocks map to (request, key head) groups so that the blocks sharing a K
// image run on one XCD (workgroups are dealt to the 8 XCDs round-robin) and
// the longest requests' groups are dispatched first.
// ---------------------------------------------------------------------------
// Conv inputs of the chain in the fused prefill: x and the conv taps of the v
// channels, and the history pool (read for the v channels' first chunk, then
// rewritten for every channel once the request's last chunk is done: the
// prep kernel has read the q / k history by then).
struct ChainConvIn {
    const void *x; int64_t x_ld;
    const void *w; bool w_bf16;  // conv taps [C, 4]
    void *pool;
    int32_t C;   // conv channels q | k | v
    int32_t nq;  // Hk * D
};

// Prefix-cache snapshots taken by the chain: after every `every` full chunks
// of a request, the state goes to the request's next snapshot slot.
struct ChainSnap {
    const int32_t *slots;  // [nreq, max] snapshot slot table, nullptr: none
    int32_t every;         // chunks between snapshots
    int32_t max;           // snapshots per request at most
};

// v for the tokens a lane holds in the accumulator layout, 16 tau + 4 lg + e
// of a chunk, from v [T, Hv, D] (the unfused prefill): four scalar loads per
// tau, kept raw until the next chunk uses them.
template <int RT, typename TA>
struct ChainVLoads {
    chunk::Raw1<TA> r[RT][2][4];

    __device__ __forceinline__ void load(const TA *v, const int (&irow)[RT], int h, int Hv, int tb, int Lc,
                                         int lane) {
        using namespace chunk;
        const int lg = lane >> 4;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int tau = 0; tau < 2; ++tau)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = 16 * tau + 4 * lg + e;
                    if (t < Lc) r[rt][tau][e].load(v + ((int64_t)(tb + t) * Hv + h) * D + irow[rt]);
                    else r[rt][tau][e].zero();
                }
    }

    __device__ __forceinline__ void get(float (&vc)[RT][2][4]) const {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int tau = 0; tau < 2; ++tau)
#pragma unroll
                for (int e = 0; e < 4; ++e) vc[rt][tau][e] = r[rt][tau][e].get();
    }
};

// The conv inputs a compute wave of a fused chain block stages per chunk: XR
// rows (tokens tb - 3 .. tb + 31) of x over the v channels of its own row
// tiles (16 NT channels), each row followed by one unused 16-byte slot, so
// that lanes reading rows 4 apart (the 4 lane groups of an accumulator) fall
// in different LDS banks.  The wave copies these rows itself, so once its own
// copies have landed it can convolve them without waiting for the block.
template <typename TX, int NT> struct XWave {
    static constexpr int PIECES = 16 * NT * (int)sizeof(TX) / 16;  // 16-byte pieces per row
    static constexpr int ROWB = (PIECES + 1) * 16;
    static constexpr int SLOTS = chunk::XR * (PIECES + 1);
    static constexpr int BYTES = SLOTS * 16;
    static constexpr int NCOPY = (SLOTS + 63) / 64;               // 64-lane copies per chunk
};

// The lane's part of a wave's x-row copies (the same for every chunk, so it
// is decoded once): copy i fills slots 64 i .. + 63 of the wave's rows, slot
// -> (row, piece).  The wave owns nt <= NTMAX tiles (16 nt channels).
template <typename TX, int NTMAX>
struct XCopyPlan {
    static constexpr int NCOPY = XWave<TX, NTMAX>::NCOPY;
    int rr[NCOPY];   // staged row (token tb - 3 + rr), or -1: no copy by this lane
    int col[NCOPY];  // element offset of the piece within a row of x

    // c0: the first of the wave's 16 nt channels
    __device__ __forceinline__ void init(int c0, int nt, int lane) {
        using namespace chunk;
        const int pieces = nt * (int)sizeof(TX);  // 16 nt channels in 16-byte pieces
        const int rs = pieces + 1;                // slots per row
#pragma unroll
        for (int i = 0; i < NCOPY; ++i) {
            const int slot = 64 * i + lane;
            const int row = slot / rs;
            const int pc = slot - row * rs;
            rr[i] = row < XR && pc < pieces ? row : -1;
            col[i] = c0 + pc * (16 / (int)sizeof(TX));
        }
    }

    // Issue the copies of the chunk starting at token tb into the wave's rows at
    // LDS address xs.  Rows past the request's last token repeat it (their v is
    // never used); rows 0..2 of the request's first chunk (first) are not
    // copied: they come from the slot's history.
    __device__ __forceinline__ void issue(uint32_t xs, const ChainConvIn &cv, int tb, int tok_last,
                                          bool first) const {
        const int base_row = first ? tb : tb - 3;
        const uint8_t *base = reinterpret_cast<const uint8_t *>(static_cast<const TX *>(cv.x) +
                                                                  (int64_t)base_row * cv.x_ld);
#pragma unroll
        for (int i = 0; i < NCOPY; ++i) {
            if (rr[i] >= (first ? 3 : 0)) {
                const int grow = min(tb - 3 + rr[i], tok_last);
                const uint32_t off = (uint32_t)(((int64_t)(grow - base_row) * cv.x_ld + col[i]) * (int64_t)sizeof(TX));
                chunk::copy_frag(base, xs + 1024u * (uint32_t)i, off);
            }
        }
    }
};

// The three history rows of one staged channel for the request's first chunk
// (zeros without a history), written by the lane that owns the channel.
template <typename TX>
__device__ __forceinline__ void stage_history(uint8_t *xs_col, int rowb, const ChainConvIn &cv, int c, int slot,
                                              bool hi) {
    const TX *hp = static_cast<const TX *>(cv.pool) + ((int64_t)slot * cv.C + c) * 3;
#pragma unroll
    for (int rr = 0; rr < 3; ++rr) *reinterpret_cast<TX *>(xs_col + rr * rowb) = hi ? hp[rr] : TX{};
}

// The conv taps of channel c, widened to fp32.
__device__ __forceinline__ void load_taps(const ChainConvIn &cv, int c, float (&wt)[4]) {
    if (cv.w_bf16) {
        const float4 f = ld4(static_cast<const bf16 *>(cv.w) + (int64_t)c * 4);
        wt[0] = f.x; wt[1] = f.y; wt[2] = f.z; wt[3] = f.w;
    } else {
        const float4 f = ld4(static_cast<const float *>(cv.w) + (int64_t)c * 4);
        wt[0] = f.x; wt[1] = f.y; wt[2] = f.z; wt[3] = f.w;
    }
}

template <typename TX> __device__ __forceinline__ float lds_x(const uint8_t *p);
template <> __device__ __forceinline__ float lds_x<float>(const uint8_t *p) {
    return *reinterpret_cast<const float *>(p);
}
template <> __device__ __forceinline__ float lds_x<bf16>(const uint8_t *p) {
    return __uint_as_float(uint32_t(*reinterpret_cast<const uint16_t *>(p)) << 16);
}

// v = SiLU(sum_i w_i x_{t-i}) of this lane's channel for its tokens 16 tau +
// 4 lg + e of the chunk (0 past the chunk's last token), from the staged rows
// of its channel (xs_col: row 0 of the channel's column; row rr is token
// tb - 3 + rr, so tap i of token t sits in row t + 3 - i).  The taps are
// summed from the oldest input on, as the other channels' conv does.
template <typename TX>
__device__ __forceinline__ void conv_v(const uint8_t *xs_col, int rowb, const float (&wt)[4], int lg, int Lc,
                                       float (&vc)[2][4]) {
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
        const int t0 = 16 * tau + 4 * lg;
        float xr[7];  // rows t0 .. t0 + 6: tokens t0 - 3 .. t0 + 3
#pragma unroll
        for (int j = 0; j < 7; ++j) xr[j] = lds_x<TX>(xs_col + (t0 + j) * rowb);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float y = 0.f;
#pragma unroll
            for (int i = 3; i >= 0; --i) y += wt[i] * xr[e + 3 - i];
            vc[tau][e] = t0 + e < Lc ? silu_fast(y) : 0.f;
        }
    }
}

// New conv history of channel c: the last 3 entries of the window [history,
// the request's L rows] (raw copies; zeros stand in for a missing history).
// One thread per channel reads all three before writing any.
template <typename TX>
__device__ __forceinline__ void chain_write_history(const ChainConvIn &cv, int c, int slot, bool hi, int tok0, int L) {
    const TX *x = static_cast<const TX *>(cv.x);
    TX *hp = static_cast<TX *>(cv.pool) + ((int64_t)slot * cv.C + c) * 3;
    TX nv[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        const int wi = L + k;  // window index: 0..2 history, 3.. the request's rows
        nv[k] = wi >= 3 ? x[(int64_t)(tok0 + wi - 3) * cv.x_ld + c] : (hi ? hp[wi] : TX{});
    }
#pragma unroll
    for (int k = 0; k < 3; ++k) hp[k] = nv[k];
}

// This wave's copies of one chunk's images, slice `part` of NPART: the slices
// are spread over the previous chunk's MFMA phases so that the wave does not
// stall on a full memory queue in one burst.
constexpr int NPART = 4;
template <int NW>
__device__ __forceinline__ void issue_images(uint32_t stage, const uint8_t *kim, const uint8_t *tim,
                                             int w, int lane, int part) {
    using namespace chunk;
    constexpr int NFRAG = KIMG_FRAGS + TIMG_FRAGS;
    constexpr int PER_WAVE = (NFRAG + NW - 1) / NW;
#pragma unroll
    for (int m = part * PER_WAVE / NPART; m < (part + 1) * PER_WAVE / NPART; ++m) {
        const int f = w + NW * m;
        if (f < NFRAG) {
            const uint8_t *src = f < KIMG_FRAGS ? kim + (size_t)f * FRAG : tim + (size_t)(f - KIMG_FRAGS) * FRAG;
            copy_frag(src, stage + (uint32_t)f * FRAG, 16u * lane);
        }
    }
}

// LDS of one stage of the per-head chain: the chunk's K image, its T image and
// (fused) the compute waves' staged x rows; two stages alternate.
template <int NW, bool XCONV, typename TX>
constexpr size_t chain_stage_bytes() {
    return chunk::KIMG + chunk::TIMG + (XCONV ? (size_t)NW * XWave<TX, 1>::BYTES : 0);
}

// Gated output formed by the per-head chain itself ("Qwen3.8-27B: from model
// structure to the vLLM inference dataflow", section 01 operator table,
// gated-output row: y = o / rms(o) * gamma * SiLU(z), the RMS over the d_v
// channels of one head and token).  A whole-head block holds every channel of
// its head, so the RMS is a reduction inside the block: each chunk's o goes to
// LDS (fp32, one padded row per token), and after the next chunk-top barrier
// every wave normalises 4 of its tokens, a lane 8 channels, with z read and y
// written as 16-byte pieces of whole rows.  z and y are bf16.
struct ChainNorm {
    const bf16 *z; int64_t z_ld;
    const void *gamma; bool gamma_bf16;
    float eps;
    bf16 *y;
};
constexpr int NORM_ROW = chunk::D + 4;  // padded fp32 row of the staged o (528 bytes)
constexpr size_t NORM_BUF = (size_t)chunk::CH * NORM_ROW * 4;  // one chunk's o
// LDS of the per-head chain: two stages, and two chunks' staged o with the
// gated output
template <int NW, bool XCONV, typename TX, bool NORM>
constexpr size_t chain_smem_bytes() {
    return 2 * chain_stage_bytes<NW, XCONV, TX>() + (NORM ? 2 * NORM_BUF : 0);
}

// Every wave computes a 16-row tile and copies its share of the next chunk's
// images (and the x rows of its own channels) while it computes the current.
// NORM (whole-head blocks of the fused prefill): the gated output is formed
// here, one chunk behind, and o is not written.
template <int NW, typename TA, typename TO, bool XCONV, typename TX, typename TS, bool NORM>
__global__ __launch_bounds__(64 * NW) void prefill_chain_kernel(
    const TA *__restrict__ v, TS *__restrict__ state, const int32_t *__restrict__ qsl,
    const int32_t *__restrict__ slots, const uint8_t *__restrict__ has_init,
    const int32_t *__restrict__ chunk_off, const int32_t *__restrict__ order,
    const uint8_t *__restrict__ kimg, const uint8_t *__restrict__ timg, int32_t nreq, int32_t Hk,
    int32_t Hv, TO *__restrict__ o, ChainConvIn cv, ChainSnap snap, ChainNorm nm) {
    using namespace chunk;
    constexpr int IB = 16 * NW;  // state rows per block
    constexpr int NRB = D / IB;  // blocks per (request, head)
    static_assert(!NORM || (NRB == 1 && XCONV), "the gated output needs whole-head blocks of the fused prefill");
    using XW = XWave<TX, 1>;
    constexpr uint32_t XOFF = (uint32_t)(KIMG + TIMG);  // staged x rows within a stage
    constexpr uint32_t STG = (uint32_t)chain_stage_bytes<NW, XCONV, TX>();
    constexpr uint32_t OBASE = 2 * STG;  // (NORM) the two staged o chunks
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t lds0 = lds_addr(smem);
    const int lr = lane & 15, lg = lane >> 4;

    const int group = Hv / Hk;
    const int per_group = group * NRB;
    const int xcd = blockIdx.x & 7;
    const int qd = blockIdx.x >> 3;
    const int gi = 8 * (qd / per_group) + xcd;  // (request rank, key head) group
    const int jj = qd % per_group;
    if (gi >= nreq * Hk) return;
    int c_first;
    const int r = order != nullptr ? order[gi / Hk] : wave_plan_rank(wave_plan(qsl, nreq, lane), nreq, lane, gi / Hk, c_first);
    if (order != nullptr) c_first = chunk_off[r];
    const int kh = gi % Hk;
    const int h = kh * group + jj / NRB;
    const int rb = jj % NRB;
    const int tok0 = qsl[r];
    const int L = qsl[r + 1] - tok0;
    if (L <= 0) return;  // empty request: slot untouched
    const int nch = (L + CH - 1) / CH;
    const bool hi_init = has_init == nullptr || has_init[r] != 0;
    const uint8_t *kim0 = kimg + ((size_t)c_first * Hk + kh) * KIMG;
    const uint8_t *tim0 = timg + ((size_t)c_first * Hv + h) * TIMG;
    const size_t kstep = (size_t)Hk * KIMG, tstep = (size_t)Hv * TIMG;
    const int tok_last = tok0 + L - 1;
    const int cb = 2 * cv.nq + h * D + IB * rb;  // the block's first v channel (fused)
    const int irow = IB * rb + 16 * w + lr;  // this lane's state row (value channel)
    const int irows[1] = {irow};
    const int slot = slots[r];
    TS *sbase = state + ((int64_t)slot * Hv + h) * D * D;

    // state rows of this lane, transposed accumulator layout:
    // ST[jt][e] = S[irow][16 jt + 4 lg + e]
    floatx4_t ST[8];
#pragma unroll
    for (int jt = 0; jt < 8; ++jt) {
        ST[jt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
        if (hi_init) {
            const float4 s4 = ld4(sbase + (int64_t)irow * D + 16 * jt + 4 * lg);
            ST[jt] = floatx4_t{s4.x, s4.y, s4.z, s4.w};
        }
    }
    const float inv_sqrt_d = 1.0f / sqrtf((float)D);
    const uint32_t kt_off = kt_lane_off(lr, lg);
    // this wave's staged x rows (fused) and this lane's column in them
    const uint32_t xw_off = XOFF + (uint32_t)(w * XW::BYTES);
    const int xcol = lr * (int)sizeof(TX);

    float wt[4] = {0.f, 0.f, 0.f, 0.f};
    ChainVLoads<1, TA> vr;
    auto load_v = [&](int cc) { vr.load(v, irows, h, Hv, tok0 + cc * CH, min(CH, L - cc * CH), lane); };
    XCopyPlan<TX, 1> xp;
    float vnext[2][4];  // (fused) v of the next chunk, formed at the end of the current one
    (void)vnext;

    // (NORM) this lane's share of a chunk's gated output: token ntt, channels
    // nc8 .. nc8 + 7 of head h; gamma of those channels; z of the previous
    // chunk (zp) and of the current one (zc, loaded a chunk ahead of its use)
    const int ntt = 4 * w + lg, nc8 = 8 * lr;
    float gmv[8];
    Raw8<bf16> zp, zc;
    uint4 ypk = make_uint4(0, 0, 0, 0);  // the previous chunk's y, stored at the end of this one
    if constexpr (NORM) {
        if (nm.gamma_bf16) {
            Raw8<bf16> g;
            g.load(static_cast<const bf16 *>(nm.gamma) + nc8);
            g.get(gmv);
        } else {
            Raw8<float> g;
            g.load(static_cast<const float *>(nm.gamma) + nc8);
            g.get(gmv);
        }
        zc.zero();
    }
    (void)gmv;
    auto load_z = [&](int tbc, int Lcc) {
        if (ntt < Lcc) zc.load(nm.z + (int64_t)(tbc + ntt) * nm.z_ld + (int64_t)h * D + nc8);
        else zc.zero();
    };
    // y of chunk cn's token ntt from its staged o and z, rounded to bf16
    // (nearest-even).  Straight-line code with the hardware reciprocal square
    // root and reciprocal (about 1 ulp of fp32 each), so that it can be
    // interleaved with the state update's MFMAs.
    auto gated = [&](int cn, const Raw8<bf16> &zr) {
        const float *orow = reinterpret_cast<const float *>(smem + OBASE + (size_t)(cn & 1) * NORM_BUF +
                                                            ((size_t)ntt * NORM_ROW + nc8) * 4);
        const float4 oa = reinterpret_cast<const float4 *>(orow)[0], ob = reinterpret_cast<const float4 *>(orow)[1];
        const float of[8] = {oa.x, oa.y, oa.z, oa.w, ob.x, ob.y, ob.z, ob.w};
        float zf[8];
        zr.get(zf);
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += of[e] * of[e];
        ss = group_sum<16>(ss);
        const float inv = __builtin_amdgcn_rsqf(ss * (1.0f / D) + nm.eps);
        uint32_t pk[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float y0 = of[2 * i] * inv * gmv[2 * i] * silu_fast(zf[2 * i]);
            const float y1 = of[2 * i + 1] * inv * gmv[2 * i + 1] * silu_fast(zf[2 * i + 1]);
            pk[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(float2v_t{y0, y1}, bf16x2_t));
        }
        return make_uint4(pk[0], pk[1], pk[2], pk[3]);
    };
    auto store_y = [&](int tbn, int Lcn, const uint4 &yv) {
        if (ntt < Lcn)
            *reinterpret_cast<uint4 *>(nm.y + ((int64_t)(tbn + ntt) * Hv + h) * D + nc8) = yv;
    };

    if constexpr (XCONV) {
        load_taps(cv, cb + 16 * w + lr, wt);
        xp.init(cb + 16 * w, 1, lane);
        if (lg == 0) stage_history<TX>(smem + xw_off + xcol, XW::ROWB, cv, cb + 16 * w + lr, slot, hi_init);
        xp.issue(lds0 + xw_off, cv, tok0, tok_last, true);
    }
#pragma unroll
    for (int part = 0; part < NPART; ++part) issue_images<NW>(lds0, kim0, tim0, w, lane, part);
    if constexpr (!XCONV) load_v(0);
    // everything above (state rows, chunk 0's copies and v) lands before the
    // loop, so that no wait for the state rows' loads is left inside it
    __builtin_amdgcn_s_waitcnt(0);
    if constexpr (XCONV) conv_v<TX>(smem + xw_off + xcol, XW::ROWB, wt, lg, min(CH, L), vnext);
    for (int cc = 0; cc < nch; ++cc) {
        const int tb = tok0 + cc * CH;
        const int Lc = min(CH, L - cc * CH);
        const uint8_t *stg = smem + (size_t)(cc & 1) * STG;
        const uint32_t nstg = lds0 + (uint32_t)((cc + 1) & 1) * STG;
        const bool more = cc + 1 < nch;  // chunk cc + 1's v loads
        const bool prefetch = more;      // and its copies
        const uint8_t *nkim = kim0 + (cc + 1) * kstep, *ntim = tim0 + (cc + 1) * tstep;
        // this wave's copies and loads of chunk cc have landed (issued before the
        // previous chunk's 8 o stores, which may stay in flight); after the
        // barrier every wave's have, and every wave is done with chunk cc - 1
        if (cc > 0) __builtin_amdgcn_s_waitcnt(waitcnt_vm(8));
        else __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if constexpr (NORM) {
            // z of chunk cc, first: it has long landed when the wait for the
            // next chunk's copies comes
            zp = zc;
            load_z(tb, Lc);
        }
        float vcur[2][4];
        if constexpr (XCONV) {
#pragma unroll
            for (int tau = 0; tau < 2; ++tau)
#pragma unroll
                for (int e = 0; e < 4; ++e) vcur[tau][e] = vnext[tau][e];
            if (more) xp.issue(nstg + xw_off, cv, tb + CH, tok_last, false);
        } else {
            float vcur1[1][2][4];
            vr.get(vcur1);
#pragma unroll
            for (int tau = 0; tau < 2; ++tau)
#pragma unroll
                for (int e = 0; e < 4; ++e) vcur[tau][e] = vcur1[0][tau][e];
        }
        if (prefetch) issue_images<NW>(nstg, nkim, ntim, w, lane, 0);
        const uint8_t *kst = stg + 16 * lane;          // this lane's piece of each K fragment
        const uint8_t *tst = stg + KIMG + 16 * lane;   // and of each T fragment

        // ---------------- X = K S0^T and OQ = Q S0^T  (tokens x this wave's rows)
        // The K / Q fragments of k-step ks + 1 are read while the MFMAs of
        // k-step ks run (scheduling barriers keep the compiler from sinking
        // the reads to their uses, where each MFMA group would wait out a full
        // LDS latency), and the state's bf16 split, plain VALU work on
        // registers, fills the wait for the first k-step's reads.
        floatx4_t X[2], OQ[2];
#pragma unroll
        for (int tau = 0; tau < 2; ++tau) {
            X[tau] = floatx4_t{0.f, 0.f, 0.f, 0.f};
            OQ[tau] = X[tau];
        }
        bf16x8_t kq[2][8];  // [k-step parity][4 tau + (K hi, K lo, Q hi, Q lo)]
        auto read_kq = [&](int ks, bf16x8_t (&f)[8]) {
#pragma unroll
            for (int tau = 0; tau < 2; ++tau) {
                f[4 * tau + 0] = frag(kst + (FK + (0 + tau) * 4 + ks) * FRAG);
                f[4 * tau + 1] = frag(kst + (FK + (2 + tau) * 4 + ks) * FRAG);
                f[4 * tau + 2] = frag(kst + (FQ + (0 + tau) * 4 + ks) * FRAG);
                f[4 * tau + 3] = frag(kst + (FQ + (2 + tau) * 4 + ks) * FRAG);
            }
        };
        read_kq(0, kq[0]);
        bf16x8_t sbh[4], sbl[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            float sv[8];
#pragma unroll
            for (int p = 0; p < 8; ++p) sv[p] = ST[2 * ks + (p >> 2)][p & 3];
            split_vals(sv, sbh[ks], sbl[ks]);
        }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            if (ks + 1 < 4) read_kq(ks + 1, kq[(ks + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
            if (prefetch && ks > 0) issue_images<NW>(nstg, nkim, ntim, w, lane, ks);
            const bf16x8_t(&f)[8] = kq[ks & 1];
#pragma unroll
            for (int tau = 0; tau < 2; ++tau) {
                mma3(X[tau], f[4 * tau + 0], f[4 * tau + 1], sbh[ks], sbl[ks]);
                mma3(OQ[tau], f[4 * tau + 2], f[4 * tau + 3], sbh[ks], sbl[ks]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if (!XCONV && more) load_v(cc + 1);
        // the K^T operands of the state update, read while the LDS is idle
        bf16x8_t kth[8], ktlo[8];
        const uint8_t *ktl = stg + kt_off;
#pragma unroll
        for (int jt = 0; jt < 8; ++jt) {
            kth[jt] = kt_frag(ktl, 0, jt);
            ktlo[jt] = kt_frag(ktl, 1, jt);
        }
        // per-token gamma, e^{G_C - G_t}, beta for this lane's tokens
        const uint8_t *tvec = stg + KIMG;
        float4 gam[2], rev[2], bet[2];
#pragma unroll
        for (int tau = 0; tau < 2; ++tau) {
            const int t0 = 16 * tau + 4 * lg;
            gam[tau] = *reinterpret_cast<const float4 *>(tvec + T_GAM + 4 * t0);
            rev[tau] = *reinterpret_cast<const float4 *>(tvec + T_REV + 4 * t0);
            bet[tau] = *reinterpret_cast<const float4 *>(tvec + T_BETA + 4 * t0);
        }
        const float gC = *reinterpret_cast<const float *>(tvec + T_GAM + 4 * (CH - 1));
        // E = beta (V - gamma X) (kept in X); OQ scaled by gamma
#pragma unroll
        for (int tau = 0; tau < 2; ++tau) {
            const float g4[4] = {gam[tau].x, gam[tau].y, gam[tau].z, gam[tau].w};
            const float b4[4] = {bet[tau].x, bet[tau].y, bet[tau].z, bet[tau].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                X[tau][e] = b4[e] * (vcur[tau][e] - g4[e] * X[tau][e]);
                OQ[tau][e] *= g4[e];
            }
        }

        // ---------------- Delta = T (beta E), then O and the state update
        bf16x8_t ebh, ebl;
        {
            float ev[8];
#pragma unroll
            for (int p = 0; p < 8; ++p) ev[p] = X[p >> 2][p & 3];
            split_vals(ev, ebh, ebl);
        }
        floatx4_t Dl[2];
#pragma unroll
        for (int tau = 0; tau < 2; ++tau) {
            Dl[tau] = floatx4_t{0.f, 0.f, 0.f, 0.f};
            mma3(Dl[tau], frag(tst + (FT + tau) * FRAG), frag(tst + (FT + 2 + tau) * FRAG), ebh, ebl);
        }
        bf16x8_t dbh, dbl, tbh, tbl;
        {
            const float r8[8] = {rev[0].x, rev[0].y, rev[0].z, rev[0].w,
                                 rev[1].x, rev[1].y, rev[1].z, rev[1].w};
            float dv[8], dtv[8];
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                dv[p] = Dl[p >> 2][p & 3];
                dtv[p] = dv[p] * r8[p];
            }
            split_vals(dv, dbh, dbl);
            split_vals(dtv, tbh, tbl);
        }
#pragma unroll
        for (int tau = 0; tau < 2; ++tau)
            mma3(OQ[tau], frag(tst + (FP + tau) * FRAG), frag(tst + (FP + 2 + tau) * FRAG), dbh, dbl);
#pragma unroll
        for (int jt = 0; jt < 8; ++jt) {
            ST[jt] *= gC;
            mma3(ST[jt], kth[jt], ktlo[jt], tbh, tbl);
        }
        // (NORM) the previous chunk's gated output (a full chunk: only the last
        // is ragged) under the state update's MFMAs; on the first chunk it is
        // formed from the other, not yet written, o buffer and never stored
        if constexpr (NORM) ypk = gated(cc - 1, zp);
        if constexpr (XCONV) {
            // v of the next chunk, from this wave's own copies of its rows (landed
            // once its memory counter drains), beside the state update's MFMAs
            // (measured: here, ahead of the o stores, the single-sequence chain
            // is ~3% faster than with it after them; the group chain the reverse)
            if (more) {
                __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
                conv_v<TX>(smem + (size_t)((cc + 1) & 1) * STG + xw_off + xcol, XW::ROWB, wt, lg,
                           min(CH, L - (cc + 1) * CH), vnext);
            }
        }
        if constexpr (NORM) {
            // this chunk's o to its LDS rows (read after the next chunk-top
            // barrier; the buffer is rewritten two chunks on, after every wave
            // has passed the barrier in between); the previous chunk's y out
            float *ob = reinterpret_cast<float *>(smem + OBASE + (size_t)(cc & 1) * NORM_BUF);
#pragma unroll
            for (int tau = 0; tau < 2; ++tau)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    ob[(16 * tau + 4 * lg + e) * NORM_ROW + irow] = OQ[tau][e] * inv_sqrt_d;
            if (cc > 0) store_y(tb - CH, CH, ypk);
        } else {
            const __amdgpu_buffer_rsrc_t orr = wave_rsrc(o + ((int64_t)tb * Hv + h) * D,
                                                         (uint32_t)((Lc - 1) * Hv + 1) * D * sizeof(TO));
#pragma unroll
            for (int tau = 0; tau < 2; ++tau)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = 16 * tau + 4 * lg + e;
                    store_o<TO>(orr, (uint32_t)(t * Hv * D + irow), OQ[tau][e] * inv_sqrt_d);
                }
        }
        // prefix-cache snapshot after this chunk (full chunks only)
        if (snap.slots != nullptr && (cc + 1) % snap.every == 0 && (cc + 1) * CH <= L &&
            (cc + 1) / snap.every <= snap.max) {
            TS *sp = state + ((int64_t)snap.slots[(int64_t)r * snap.max + (cc + 1) / snap.every - 1] * Hv + h) * D * D;
#pragma unroll
            for (int jt = 0; jt < 8; ++jt)
                st4(sp + (int64_t)irow * D + 16 * jt + 4 * lg, make_float4(ST[jt][0], ST[jt][1], ST[jt][2], ST[jt][3]));
        }
    }

#pragma unroll
    for (int jt = 0; jt < 8; ++jt)
        st4(sbase + (int64_t)irow * D + 16 * jt + 4 * lg, make_float4(ST[jt][0], ST[jt][1], ST[jt][2], ST[jt][3]));
    if constexpr (NORM) {
        // the last chunk's gated output: its z has landed and every wave's o
        // rows are in LDS
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        const int cl = nch - 1;
        store_y(tok0 + cl * CH, L - cl * CH, gated(cl, zc));
    }
    if constexpr (XCONV) {
        // new history (every reader of the old one is done: the prep kernel for
        // q / k, this block's prologue for its v channels): this lane's v
        // channel, and the key head's q / k channels from one block of the key
        // head's first value head
        if (lg == 0) chain_write_history<TX>(cv, cb + 16 * w + lr, slot, hi_init, tok0, L);
        if (h % group == 0 && rb == 0)
            for (int j = threadIdx.x; j < 2 * D; j += 64 * NW)
                chain_write_history<TX>(cv, (j < D ? 0 : cv.nq) + kh * D + (j & (D - 1)), slot, hi_init, tok0, L);
    }
}

// ---------------------------------------------------------------------------
// chain, paired variant for few (request, head) units, e.g. one long
// sequence, where each block's critical path per chunk sets the kernel's
// time.  Each 16-row tile of the per-head block gets two waves.  The state
// wave carries the recurrence: X = K S^T, E, Delta = T E and the state
// update.  The output wave keeps its own copy of the state, advanced by the
// same MFMAs on the same operands (so the two copies stay bit-identical), and
// forms the output one chunk behind: gamma Q S^T + P Delta, from the Delta
// splits the state wave leaves in LDS, and the o stores.  (Fused) two of the
// copy waves convolve the x rows of the tiles' v channels a chunk ahead and
// leave v in LDS.  The recurrence then waits on neither the output products,
// the stores nor the conv.  Waves 0-1: state waves of tiles 0-1; 2-3: their
// output waves; 4-7 copy the images, and 6-7 (on the output waves' SIMDs,
// which have more room) convolve for tiles 0-1.  Three image stages rotate:
// while the state waves work on chunk c, the output waves read chunk c - 1's
// images and chunk c + 1's land.
// ---------------------------------------------------------------------------
constexpr int PAIR_TILES = 2;  // 16-row tiles per block
constexpr int PAIR_NCW = 4;    // copy waves
constexpr int PAIR_WAVES = 2 * PAIR_TILES + PAIR_NCW;

// LDS of the paired chain: three image stages, the Delta splits of two chunks
// (4 fragments per tile) and (fused) the conv waves' x rows and the v they
// form (2 fragments of fp32 per tile), both for two chunks.
constexpr uint32_t PAIR_VTILE = 2 * chunk::FRAG;
template <bool XCONV, typename TX>
constexpr size_t pair_smem_bytes() {
    return 3 * (chunk::KIMG + chunk::TIMG) + 2 * (size_t)PAIR_TILES * 4 * chunk::FRAG +
           (XCONV ? 2 * (size_t)PAIR_TILES * (XWave<TX, 1>::BYTES + PAIR_VTILE) : 0);
}

template <typename TA, typename TO, bool XCONV, typename TX, typename TS>
__global__ __launch_bounds__(64 * PAIR_WAVES) void prefill_chain_pair_kernel(
    const TA *__restrict__ v, TS *__restrict__ state, const int32_t *__restrict__ qsl,
    const int32_t *__restrict__ slots, const uint8_t *__restrict__ has_init,
    const int32_t *__restrict__ chunk_off, const int32_t *__restrict__ order,
    const uint8_t *__restrict__ kimg, const uint8_t *__restrict__ timg, int32_t nreq, int32_t Hk,
    int32_t Hv, TO *__restrict__ o, ChainConvIn cv, ChainSnap snap) {
    using namespace chunk;
    constexpr int IB = 16 * PAIR_TILES;  // state rows per block
    constexpr int NRB = D / IB;          // blocks per (request, head)
    using XW = XWave<TX, 1>;
    constexpr uint32_t STG = (uint32_t)(KIMG + TIMG);  // one image stage
    constexpr uint32_t DTILE = 4 * FRAG;               // dbh, dbl, tbh, tbl of one tile
    constexpr uint32_t DBASE = 3 * STG;                // Delta [chunk parity][tile]
    constexpr uint32_t XBASE = DBASE + 2 * PAIR_TILES * DTILE;  // (fused) x rows [parity][tile]
    constexpr uint32_t VBASE = XBASE + 2 * PAIR_TILES * XW::BYTES;  // (fused) v [parity][tile]
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t lds0 = lds_addr(smem);
    const int lr = lane & 15, lg = lane >> 4;

    const int group = Hv / Hk;
    const int per_group = group * NRB;
    const int xcd = blockIdx.x & 7;
    const int qd = blockIdx.x >> 3;
    const int gi = 8 * (qd / per_group) + xcd;  // (request rank, key head) group
    const int jj = qd % per_group;
    if (gi >= nreq * Hk) return;
    int c_first;
    const int r = order != nullptr ? order[gi / Hk] : wave_plan_rank(wave_plan(qsl, nreq, lane), nreq, lane, gi / Hk, c_first);
    if (order != nullptr) c_first = chunk_off[r];
    const int kh = gi % Hk;
    const int h = kh * group + jj / NRB;
    const int rb = jj % NRB;
    const int tok0 = qsl[r];
    const int L = qsl[r + 1] - tok0;
    if (L <= 0) return;  // empty request: slot untouched
    const int nch = (L + CH - 1) / CH;
    const bool hi_init = has_init == nullptr || has_init[r] != 0;
    const uint8_t *kim0 = kimg + ((size_t)c_first * Hk + kh) * KIMG;
    const uint8_t *tim0 = timg + ((size_t)c_first * Hv + h) * TIMG;
    const size_t kstep = (size_t)Hk * KIMG, tstep = (size_t)Hv * TIMG;
    const int tok_last = tok0 + L - 1;
    const int cb = 2 * cv.nq + h * D + IB * rb;  // the block's first v channel (fused)
    const int slot = slots[r];

    // Every wave passes nch + 1 barriers: barrier i opens iteration i, in which
    // the state waves take chunk i (i < nch) and the output waves chunk i - 1
    // (i > 0).
    if (w >= 2 * PAIR_TILES) {
        // copy wave: chunk i + 1's images go into stage (i + 1) % 3, last read by
        // the output waves in iteration i - 1.  A conv wave also forms chunk
        // i + 1's v in iteration i, from x rows it copied in iteration i - 1,
        // into the v buffer the state wave read in iteration i - 1.
        const int cw = w - 2 * PAIR_TILES;
        const int ctile = cw - (PAIR_NCW - PAIR_TILES);
        const bool conv_wave = XCONV && ctile >= 0;
        const int xcol = lr * (int)sizeof(TX);
        const uint32_t xw_off = XBASE + (uint32_t)(ctile * XW::BYTES);  // + parity * XPAR
        constexpr uint32_t XPAR = (uint32_t)(PAIR_TILES * XW::BYTES);
        const uint32_t vw_off = VBASE + (uint32_t)ctile * PAIR_VTILE + 16u * (uint32_t)lane;  // + parity, + tau
        constexpr uint32_t VPAR = PAIR_TILES * PAIR_VTILE;
        float wt[4] = {0.f, 0.f, 0.f, 0.f};
        XCopyPlan<TX, 1> xp;
        auto conv_to_lds = [&](int cn) {
            float vc[2][4];
            conv_v<TX>(smem + xw_off + (uint32_t)(cn & 1) * XPAR + xcol, XW::ROWB, wt, lg, min(CH, L - cn * CH), vc);
#pragma unroll
            for (int tau = 0; tau < 2; ++tau)
                *reinterpret_cast<float4 *>(smem + vw_off + (uint32_t)(cn & 1) * VPAR + (uint32_t)tau * FRAG) =
                    make_float4(vc[tau][0], vc[tau][1], vc[tau][2], vc[tau][3]);
        };
        if (conv_wave) {
            load_taps(cv, cb + 16 * ctile + lr, wt);
            xp.init(cb + 16 * ctile, 1, lane);
            if (lg == 0) stage_history<TX>(smem + xw_off + xcol, XW::ROWB, cv, cb + 16 * ctile + lr, slot, hi_init);
            xp.issue(lds0 + xw_off, cv, tok0, tok_last, true);
            if (nch > 1) xp.issue(lds0 + xw_off + XPAR, cv, tok0 + CH, tok_last, false);
        }
#pragma unroll
        for (int part = 0; part < NPART; ++part) issue_images<PAIR_NCW>(lds0, kim0, tim0, cw, lane, part);
        if (conv_wave) {
            __builtin_amdgcn_s_waitcnt(0);
            conv_to_lds(0);
        }
        for (int it = 0; it <= nch; ++it) {
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (it + 1 < nch) {
                const uint32_t nstg = lds0 + (uint32_t)((it + 1) % 3) * STG;
#pragma unroll
                for (int part = 0; part < NPART; ++part)
                    issue_images<PAIR_NCW>(nstg, kim0 + (it + 1) * kstep, tim0 + (it + 1) * tstep, cw, lane, part);
                if (conv_wave) {
                    // chunk it + 2's rows go into the buffer chunk it's conv read
                    // in iteration it - 1
                    if (it + 2 < nch)
                        xp.issue(lds0 + xw_off + (uint32_t)(it & 1) * XPAR, cv, tok0 + (it + 2) * CH, tok_last, false);
                    conv_to_lds(it + 1);
                }
            }
        }
        // new history of this conv wave's v channels (their old history was
        // read in its prologue)
        if (conv_wave && lg == 0) chain_write_history<TX>(cv, cb + 16 * ctile + lr, slot, hi_init, tok0, L);
        return;
    }
    const bool state_wave = w < PAIR_TILES;
    const int tile = state_wave ? w : w - PAIR_TILES;
    const int irow = IB * rb + 16 * tile + lr;  // this lane's state row (value channel)
    TS *sbase = state + ((int64_t)slot * Hv + h) * D * D;

    // state rows of this lane, transposed accumulator layout:
    // ST[jt][e] = S[irow][16 jt + 4 lg + e]
    floatx4_t ST[8];
#pragma unroll
    for (int jt = 0; jt < 8; ++jt) {
        ST[jt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
        if (hi_init) {
            const float4 s4 = ld4(sbase + (int64_t)irow * D + 16 * jt + 4 * lg);
            ST[jt] = floatx4_t{s4.x, s4.y, s4.z, s4.w};
        }
    }
    const uint32_t kt_off = kt_lane_off(lr, lg);
    const uint32_t dt_off = DBASE + (uint32_t)tile * DTILE + 16u * (uint32_t)lane;  // + parity, + plane
    // (fused) this lane's v of its 8 tokens: [parity][tile][tau][lane] float4
    const uint32_t vt_off = VBASE + (uint32_t)tile * PAIR_VTILE + 16u * (uint32_t)lane;  // + parity, + tau
    constexpr uint32_t VPAR = PAIR_TILES * PAIR_VTILE;
    (void)vt_off;

    // the state update of one chunk on this wave's copy: S = gC S + (K^T)(tDelta)
    auto state_update = [&](const uint8_t *stg, float gC, const bf16x8_t &tbh, const bf16x8_t &tbl) {
        bf16x8_t kth[8], ktlo[8];
        const uint8_t *ktl = stg + kt_off;
#pragma unroll
        for (int jt = 0; jt < 8; ++jt) {
            kth[jt] = kt_frag(ktl, 0, jt);
            ktlo[jt] = kt_frag(ktl, 1, jt);
        }
#pragma unroll
        for (int jt = 0; jt < 8; ++jt) {
            ST[jt] *= gC;
            mma3(ST[jt], kth[jt], ktlo[jt], tbh, tbl);
        }
    };
    // A S^T for the 32 x 128 operand A of K-image plane pair f0 (hi: f0, lo:
    // f0 + 8), all four k-steps.  While k-step ks's six MFMAs run, the wave
    // reads k-step ks + 1's fragments and splits its slice of the state
    // (scheduling groups interleave the split's VALU work between the MFMAs
    // and keep the compiler from sinking the reads to their uses).
    auto contract_state = [&](const uint8_t *kst, int f0, floatx4_t (&acc)[2]) {
#pragma unroll
        for (int tau = 0; tau < 2; ++tau) acc[tau] = floatx4_t{0.f, 0.f, 0.f, 0.f};
        bf16x8_t fr[2][4];  // [k-step parity][2 tau + plane]
        bf16x8_t sbh[2], sbl[2];
        auto read = [&](int ks, bf16x8_t (&f)[4]) {
#pragma unroll
            for (int tau = 0; tau < 2; ++tau) {
                f[2 * tau + 0] = frag(kst + (f0 + (0 + tau) * 4 + ks) * FRAG);
                f[2 * tau + 1] = frag(kst + (f0 + (2 + tau) * 4 + ks) * FRAG);
            }
        };
        auto split_state = [&](int ks) {
            float sv[8];
#pragma unroll
            for (int p = 0; p < 8; ++p) sv[p] = ST[2 * ks + (p >> 2)][p & 3];
            split_vals(sv, sbh[ks & 1], sbl[ks & 1]);
        };
        read(0, fr[0]);
        split_state(0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            if (ks + 1 < 4) {
                read(ks + 1, fr[(ks + 1) & 1]);
                split_state(ks + 1);
            }
#pragma unroll
            for (int tau = 0; tau < 2; ++tau)
                mma3(acc[tau], fr[ks & 1][2 * tau + 0], fr[ks & 1][2 * tau + 1], sbh[ks & 1], sbl[ks & 1]);
            if (ks + 1 < 4) {
                __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // the four reads first
#pragma unroll
                for (int m = 0; m < 6; ++m) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // four VALU of the split
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    if (state_wave) {
        ChainVLoads<1, TA> vr;
        const int irows[1] = {irow};
        auto load_v = [&](int cc) { vr.load(v, irows, h, Hv, tok0 + cc * CH, min(CH, L - cc * CH), lane); };
        if constexpr (!XCONV) load_v(0);
        __builtin_amdgcn_s_waitcnt(0);
        for (int cc = 0; cc <= nch; ++cc) {
            __syncthreads();
            if (cc == nch) break;
            const uint8_t *stg = smem + (size_t)(cc % 3) * STG;
            const bool more = cc + 1 < nch;
            float vcur[2][4];
            if constexpr (XCONV) {
                // v of chunk cc, formed by a conv wave in iteration cc - 1
#pragma unroll
                for (int tau = 0; tau < 2; ++tau) {
                    const float4 f = *reinterpret_cast<const float4 *>(
                        smem + vt_off + (uint32_t)(cc & 1) * VPAR + (uint32_t)tau * FRAG);
                    vcur[tau][0] = f.x;
                    vcur[tau][1] = f.y;
                    vcur[tau][2] = f.z;
                    vcur[tau][3] = f.w;
                }
            } else {
                float vcur1[1][2][4];
                vr.get(vcur1);
#pragma unroll
                for (int tau = 0; tau < 2; ++tau)
#pragma unroll
                    for (int e = 0; e < 4; ++e) vcur[tau][e] = vcur1[0][tau][e];
            }
            // X = K S^T (tokens x this tile's rows)
            floatx4_t X[2];
            contract_state(stg + 16 * lane, FK, X);
            if (!XCONV && more) load_v(cc + 1);
            const uint8_t *tvec = stg + KIMG;
            const uint8_t *tst = stg + KIMG + 16 * lane;
            float4 gam[2], rev[2], bet[2];
#pragma unroll
            for (int tau = 0; tau < 2; ++tau) {
                const int t0 = 16 * tau + 4 * lg;
                gam[tau] = *reinterpret_cast<const float4 *>(tvec + T_GAM + 4 * t0);
                rev[tau] = *reinterpret_cast<const float4 *>(tvec + T_REV + 4 * t0);
                bet[tau] = *reinterpret_cast<const float4 *>(tvec + T_BETA + 4 * t0);
            }
            const float gC = *reinterpret_cast<const float *>(tvec + T_GAM + 4 * (CH - 1));
            // E = beta (V - gamma X), then Delta = T E
            bf16x8_t ebh, ebl;
            {
                float ev[8];
#pragma unroll
                for (int p = 0; p < 8; ++p) {
                    const int tau = p >> 2, e = p & 3;
                    const float g = e == 0 ? gam[tau].x : e == 1 ? gam[tau].y : e == 2 ? gam[tau].z : gam[tau].w;
                    const float b = e == 0 ? bet[tau].x : e == 1 ? bet[tau].y : e == 2 ? bet[tau].z : bet[tau].w;
                    ev[p] = b * (vcur[tau][e] - g * X[tau][e]);
                }
                split_vals(ev, ebh, ebl);
            }
            floatx4_t Dl[2];
#pragma unroll
            for (int tau = 0; tau < 2; ++tau) {
                Dl[tau] = floatx4_t{0.f, 0.f, 0.f, 0.f};
                mma3(Dl[tau], frag(tst + (FT + tau) * FRAG), frag(tst + (FT + 2 + tau) * FRAG), ebh, ebl);
            }
            bf16x8_t dbh, dbl, tbh, tbl;
            {
                const float r8[8] = {rev[0].x, rev[0].y, rev[0].z, rev[0].w,
                                     rev[1].x, rev[1].y, rev[1].z, rev[1].w};
                float dv[8], dtv[8];
#pragma unroll
                for (int p = 0; p < 8; ++p) {
                    dv[p] = Dl[p >> 2][p & 3];
                    dtv[p] = dv[p] * r8[p];
                }
                split_vals(dv, dbh, dbl);
                split_vals(dtv, tbh, tbl);
            }
            // Delta's splits for the output wave (read after the next barrier)
            {
                uint8_t *dp = smem + dt_off + (uint32_t)(cc & 1) * (PAIR_TILES * DTILE);
                *reinterpret_cast<bf16x8_t *>(dp + 0 * FRAG) = dbh;
                *reinterpret_cast<bf16x8_t *>(dp + 1 * FRAG) = dbl;
                *reinterpret_cast<bf16x8_t *>(dp + 2 * FRAG) = tbh;
                *reinterpret_cast<bf16x8_t *>(dp + 3 * FRAG) = tbl;
            }
            state_update(stg, gC, tbh, tbl);
            // prefix-cache snapshot after this chunk (full chunks only)
            if (snap.slots != nullptr && (cc + 1) % snap.every == 0 && (cc + 1) * CH <= L &&
                (cc + 1) / snap.every <= snap.max) {
                TS *sp = state + ((int64_t)snap.slots[(int64_t)r * snap.max + (cc + 1) / snap.every - 1] * Hv + h) * D * D;
#pragma unroll
                for (int jt = 0; jt < 8; ++jt)
                    st4(sp + (int64_t)irow * D + 16 * jt + 4 * lg, make_float4(ST[jt][0], ST[jt][1], ST[jt][2], ST[jt][3]));
            }
        }
#pragma unroll
        for (int jt = 0; jt < 8; ++jt)
            st4(sbase + (int64_t)irow * D + 16 * jt + 4 * lg, make_float4(ST[jt][0], ST[jt][1], ST[jt][2], ST[jt][3]));
        if constexpr (XCONV) {
            // new history of the key head's q / k channels (their old history
            // was read by the prep kernel), from one block of the key head's
            // first value head
            if (h % group == 0 && rb == 0)
                for (int j = threadIdx.x; j < 2 * D; j += 64 * PAIR_TILES)
                    chain_write_history<TX>(cv, (j < D ? 0 : cv.nq) + kh * D + (j & (D - 1)), slot, hi_init, tok0, L);
        }
    } else {
        // output wave: chunk cc - 1's output in iteration cc
        const float inv_sqrt_d = 1.0f / sqrtf((float)D);
        __builtin_amdgcn_s_waitcnt(0);
        for (int cc = 0; cc <= nch; ++cc) {
            __syncthreads();
            if (cc == 0) continue;
            const int c = cc - 1;
            const int tb = tok0 + c * CH;
            const int Lc = min(CH, L - c * CH);
            const uint8_t *stg = smem + (size_t)(c % 3) * STG;
            const uint8_t *tst = stg + KIMG + 16 * lane;
            // OQ = gamma Q S^T + P Delta
            floatx4_t OQ[2];
            contract_state(stg + 16 * lane, FQ, OQ);
            const uint8_t *tvec = stg + KIMG;
            const uint8_t *dp = smem + dt_off + (uint32_t)(c & 1) * (PAIR_TILES * DTILE);
            const bf16x8_t dbh = frag(dp + 0 * FRAG), dbl = frag(dp + 1 * FRAG);
            const bf16x8_t tbh = frag(dp + 2 * FRAG), tbl = frag(dp + 3 * FRAG);
            const float gC = *reinterpret_cast<const float *>(tvec + T_GAM + 4 * (CH - 1));
#pragma unroll
            for (int tau = 0; tau < 2; ++tau) {
                const float4 g = *reinterpret_cast<const float4 *>(tvec + T_GAM + 4 * (16 * tau + 4 * lg));
                OQ[tau][0] *= g.x;
                OQ[tau][1] *= g.y;
                OQ[tau][2] *= g.z;
                OQ[tau][3] *= g.w;
                mma3(OQ[tau], frag(tst + (FP + tau) * FRAG), frag(tst + (FP + 2 + tau) * FRAG), dbh, dbl);
            }
            {
                const __amdgpu_buffer_rsrc_t orr = wave_rsrc(o + ((int64_t)tb * Hv + h) * D,
                                                             (uint32_t)((Lc - 1) * Hv + 1) * D * sizeof(TO));
#pragma unroll
                for (int tau = 0; tau < 2; ++tau)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int t = 16 * tau + 4 * lg + e;
                        store_o<TO>(orr, (uint32_t)(t * Hv * D + irow), OQ[tau][e] * inv_sqrt_d);
                    }
            }
            if (cc < nch) state_update(stg, gC, tbh, tbl);  // the state chunk cc's output starts from
        }
    }
}

// ---------------------------------------------------------------------------
// chain, group variant for large batches: one block per (request, key head,
// block of 64 state rows) covering the 3 value heads that read the key head,
// so the chunk's K image is staged once for them.  The 12 row tiles of 16 rows
// go to 8 waves: four waves hold two tiles of one head (every K / Q / K^T
// operand read feeds both) and four hold one, so that with waves dealt to the
// 4 SIMDs in turn each SIMD carries one of each, 3 tiles (6 waves of two
// tiles left two SIMDs with twice the work of the others, and the block waited
// for them at every chunk).  Same per-row algebra and operand layout as above.
// ---------------------------------------------------------------------------
constexpr int GRP_ROWS = 64;          // state rows per head per block
constexpr int GRP_RPW = 2;            // 16-row tiles per wave, at most
constexpr int GRP_NW = 8;             // waves per block

// LDS of one stage of the group chain: the chunk's K image, its G T images and
// (fused) the waves' staged x rows: waves 0-3 hold two row tiles, 4-7 one.
template <int G, bool XCONV, typename TX>
constexpr size_t group_stage_bytes() {
    return chunk::KIMG + G * chunk::TIMG +
           (XCONV ? 4 * (size_t)(XWave<TX, 2>::BYTES + XWave<TX, 1>::BYTES) : 0);
}

template <int G, typename TA, typename TO, bool XCONV, typename TX, typename TS>
__global__ __launch_bounds__(64 * GRP_NW) void prefill_chain_group_kernel(
    const TA *__restrict__ v, TS *__restrict__ state, const int32_t *__restrict__ qsl,
    const int32_t *__restrict__ slots, const uint8_t *__restrict__ has_init,
    const int32_t *__restrict__ chunk_off, const int32_t *__restrict__ order,
    const uint8_t *__restrict__ kimg, const uint8_t *__restrict__ timg, int32_t nreq, int32_t Hk,
    int32_t Hv, TO *__restrict__ o, ChainConvIn cv, ChainSnap snap) {
    using namespace chunk;
    static_assert(G == 3 && GRP_ROWS == 64 && GRP_RPW == 2, "tile map below is for 3 heads x 4 tiles");
    constexpr int NW = GRP_NW;
    constexpr int NRB = D / GRP_ROWS;               // row blocks per head
    constexpr int NFRAG = KIMG_FRAGS + G * TIMG_FRAGS;
    constexpr uint32_t XOFF = (uint32_t)(KIMG + G * TIMG);
    constexpr uint32_t GSTG = (uint32_t)group_stage_bytes<G, XCONV, TX>();
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t lds0 = lds_addr(smem);
    const int lr = lane & 15, lg = lane >> 4;

    // blocks of one (request, key head) group run on one XCD; longest requests first
    const int xcd = blockIdx.x & 7;
    const int qd = blockIdx.x >> 3;
    const int gi = 8 * (qd / NRB) + xcd;
    const int rb = qd % NRB;
    if (gi >= nreq * Hk) return;
    int c_first;
    const int r = order != nullptr ? order[gi / Hk] : wave_plan_rank(wave_plan(qsl, nreq, lane), nreq, lane, gi / Hk, c_first);
    if (order != nullptr) c_first = chunk_off[r];
    const int kh = gi % Hk;
    // this wave's head within the group, first tile and tile count: waves 0-2
    // tiles 0-1 of heads 0-2, wave 3 tiles 2-3 of head 0, waves 4-7 tile 2 or 3
    // of heads 1, 2
    const int hh = w < 4 ? (w < 3 ? w : 0) : 1 + ((w - 4) >> 1);
    const int tile0 = w < 4 ? (w < 3 ? 0 : 2) : 2 + ((w - 4) & 1);
    const int nt = w < 4 ? 2 : 1;
    const int h = kh * G + hh;
    const int tok0 = qsl[r];
    const int L = qsl[r + 1] - tok0;
    if (L <= 0) return;
    const int nch = (L + CH - 1) / CH;
    const bool hi_init = has_init == nullptr || has_init[r] != 0;
    const int tok_last = tok0 + L - 1;
    // a one-tile wave's second tile repeats its first: loads stay in bounds and
    // every store of it is dropped or skipped
    int irow[GRP_RPW], ci[GRP_RPW];
#pragma unroll
    for (int rt = 0; rt < GRP_RPW; ++rt) {
        ci[rt] = 16 * (tile0 + (rt < nt ? rt : 0)) + lr;  // row within the block's 64 of head hh
        irow[rt] = GRP_ROWS * rb + ci[rt];
    }
    const int slot = slots[r];
    TS *sbase = state + ((int64_t)slot * Hv + h) * D * D;
    // fused: the group's v channels of this row block, head hd at cb + hd D; this
    // wave's staged x rows (its nt tiles' channels) and their row stride
    const int cb = 2 * cv.nq + kh * G * D + GRP_ROWS * rb;
    const uint32_t xw_off = XOFF + (uint32_t)(w < 4 ? w * XWave<TX, 2>::BYTES
                                                    : 4 * XWave<TX, 2>::BYTES + (w - 4) * XWave<TX, 1>::BYTES);
    const int xrowb = nt == 2 ? XWave<TX, 2>::ROWB : XWave<TX, 1>::ROWB;

    floatx4_t ST[GRP_RPW][8];
#pragma unroll
    for (int rt = 0; rt < GRP_RPW; ++rt)
#pragma unroll
        for (int jt = 0; jt < 8; ++jt) {
            ST[rt][jt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
            if (hi_init) {
                const float4 s4 = ld4(sbase + (int64_t)irow[rt] * D + 16 * jt + 4 * lg);
                ST[rt][jt] = floatx4_t{s4.x, s4.y, s4.z, s4.w};
            }
        }
    const float inv_sqrt_d = 1.0f / sqrtf((float)D);
    const uint32_t kt_off = kt_lane_off(lr, lg);

    const uint8_t *kim0 = kimg + ((size_t)c_first * Hk + kh) * KIMG;
    const uint8_t *tim0 = timg + ((size_t)c_first * Hv + kh * G) * TIMG;  // the group's G heads are adjacent
    const size_t kstep = (size_t)Hk * KIMG, tstep = (size_t)Hv * TIMG;

    XCopyPlan<TX, 2> xp;
    if constexpr (XCONV) xp.init(cb + hh * D + 16 * tile0, nt, lane);
    // this wave's copies of chunk cc's images, in NPART slices so that they can
    // be spread over the previous chunk's MFMA phases instead of stalling the
    // wave on a full memory queue in one burst
    constexpr int PER_WAVE = (NFRAG + NW - 1) / NW;
    auto issue = [&](uint32_t stage, int cc, int part) {
        const uint8_t *kim = kim0 + cc * kstep;
        const uint8_t *tim = tim0 + cc * tstep;
#pragma unroll
        for (int m = part * PER_WAVE / NPART; m < (part + 1) * PER_WAVE / NPART; ++m) {
            const int f = w + NW * m;
            if (f < NFRAG) {
                const uint8_t *src = f < KIMG_FRAGS ? kim + (size_t)f * FRAG : tim + (size_t)(f - KIMG_FRAGS) * FRAG;
                copy_frag(src, stage + (uint32_t)f * FRAG, 16u * lane);
            }
        }
    };
    float wt[GRP_RPW][4];
    ChainVLoads<GRP_RPW, TA> vr;
    auto load_v = [&](int cc) { vr.load(v, irow, h, Hv, tok0 + cc * CH, min(CH, L - cc * CH), lane); };
    // (fused) v of the next chunk, formed at the end of the current one from this
    // wave's own rows; a one-tile wave's second tile repeats its first
    float vnext[GRP_RPW][2][4];
    auto conv_next = [&](int cn) {
        const uint8_t *xs = smem + (size_t)(cn & 1) * GSTG + xw_off;
        const int Lc = min(CH, L - cn * CH);
        conv_v<TX>(xs + lr * (int)sizeof(TX), xrowb, wt[0], lg, Lc, vnext[0]);
        if (nt > 1) conv_v<TX>(xs + (16 + lr) * (int)sizeof(TX), xrowb, wt[1], lg, Lc, vnext[1]);
        else {
#pragma unroll
            for (int tau = 0; tau < 2; ++tau)
#pragma unroll
                for (int e = 0; e < 4; ++e) vnext[1][tau][e] = vnext[0][tau][e];
        }
    };

    if constexpr (XCONV) {
#pragma unroll
        for (int rt = 0; rt < GRP_RPW; ++rt) {
            load_taps(cv, cb + hh * D + ci[rt], wt[rt]);
            if (lg == 0 && rt < nt)
                stage_history<TX>(smem + xw_off + (16 * rt + lr) * (int)sizeof(TX), xrowb, cv, cb + hh * D + ci[rt],
                                  slot, hi_init);
        }
        xp.issue(lds0 + xw_off, cv, tok0, tok_last, true);
    }
#pragma unroll
    for (int part = 0; part < NPART; ++part) issue(lds0, 0, part);
    if constexpr (!XCONV) load_v(0);
    // everything above (state rows, chunk 0's copies and v) lands before the
    // loop, so that no wait for the state rows' loads is left inside it
    __builtin_amdgcn_s_waitcnt(0);
    if constexpr (XCONV) conv_next(0);
    for (int cc = 0; cc < nch; ++cc) {
        const int tb = tok0 + cc * CH;
        const int Lc = min(CH, L - cc * CH);
        const uint8_t *stg = smem + (size_t)(cc & 1) * GSTG;
        const uint32_t nstg = lds0 + (uint32_t)((cc + 1) & 1) * GSTG;
        const bool prefetch = cc + 1 < nch;
        // as in the per-head chain: the previous chunk's o stores stay in flight
        if (cc > 0) __builtin_amdgcn_s_waitcnt(waitcnt_vm(8 * GRP_RPW));
        else __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        float vcur[GRP_RPW][2][4];
        if constexpr (XCONV) {
#pragma unroll
            for (int rt = 0; rt < GRP_RPW; ++rt)
#pragma unroll
                for (int tau = 0; tau < 2; ++tau)
#pragma unroll
                    for (int e = 0; e < 4; ++e) vcur[rt][tau][e] = vnext[rt][tau][e];
            if (prefetch) xp.issue(nstg + xw_off, cv, tb + CH, tok_last, false);
        } else {
            vr.get(vcur);
        }
        if (prefetch) issue(nstg, cc + 1, 0);
        const uint8_t *kst = stg + 16 * lane;
        const uint8_t *tst = stg + KIMG + (size_t)hh * TIMG + 16 * lane;
        const uint8_t *tvec = stg + KIMG + (size_t)hh * TIMG;

        // X = K S0^T, OQ = Q S0^T for both row tiles
        floatx4_t X[GRP_RPW][2], OQ[GRP_RPW][2];
#pragma unroll
        for (int rt = 0; rt < GRP_RPW; ++rt)
#pragma unroll
            for (int tau = 0; tau < 2; ++tau) {
                X[rt][tau] = floatx4_t{0.f, 0.f, 0.f, 0.f};
                OQ[rt][tau] = X[rt][tau];
            }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            if (prefetch && ks > 0) issue(nstg, cc + 1, ks);
            bf16x8_t sbh[GRP_RPW], sbl[GRP_RPW];
#pragma unroll
            for (int rt = 0; rt < GRP_RPW; ++rt) {
                float sv[8];
#pragma unroll
                for (int p = 0; p < 8; ++p) sv[p] = ST[rt][2 * ks + (p >> 2)][p & 3];
                split_vals(sv, sbh[rt], sbl[rt]);
            }
#pragma unroll
            for (int tau = 0; tau < 2; ++tau) {
                const bf16x8_t kh_ = frag(kst + (FK + (0 + tau) * 4 + ks) * FRAG);
                const bf16x8_t kl_ = frag(kst + (FK + (2 + tau) * 4 + ks) * FRAG);
                const bf16x8_t qh_ = frag(kst + (FQ + (0 + tau) * 4 + ks) * FRAG);
                const bf16x8_t ql_ = frag(kst + (FQ + (2 + tau) * 4 + ks) * FRAG);
#pragma unroll
                for (int rt = 0; rt < GRP_RPW; ++rt) {
                    if (rt < nt) {
                        mma3(X[rt][tau], kh_, kl_, sbh[rt], sbl[rt]);
                        mma3(OQ[rt][tau], qh_, ql_, sbh[rt], sbl[rt]);
                    }
                }
            }
        }
        if (!XCONV && prefetch) load_v(cc + 1);
        float4 gam[2], rev[2], bet[2];
#pragma unroll
        for (int tau = 0; tau < 2; ++tau) {
            const int t0 = 16 * tau + 4 * lg;
            gam[tau] = *reinterpret_cast<const float4 *>(tvec + T_GAM + 4 * t0);
            rev[tau] = *reinterpret_cast<const float4 *>(tvec + T_REV + 4 * t0);
            bet[tau] = *reinterpret_cast<const float4 *>(tvec + T_BETA + 4 * t0);
        }
        const float gC = *reinterpret_cast<const float *>(tvec + T_GAM + 4 * (CH - 1));
#pragma unroll
        for (int tau = 0; tau < 2; ++tau) {
            const float g4[4] = {gam[tau].x, gam[tau].y, gam[tau].z, gam[tau].w};
            const float b4[4] = {bet[tau].x, bet[tau].y, bet[tau].z, bet[tau].w};
#pragma unroll
            for (int rt = 0; rt < GRP_RPW; ++rt)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    X[rt][tau][e] = b4[e] * (vcur[rt][tau][e] - g4[e] * X[rt][tau][e]);
                    OQ[rt][tau][e] *= g4[e];
                }
        }
        // Delta = T (beta E)
        const bf16x8_t th0 = frag(tst + (FT + 0) * FRAG), th1 = frag(tst + (FT + 1) * FRAG);
        const bf16x8_t tl0 = frag(tst + (FT + 2) * FRAG), tl1 = frag(tst + (FT + 3) * FRAG);
        floatx4_t Dl[GRP_RPW][2];
#pragma unroll
        for (int rt = 0; rt < GRP_RPW; ++rt) {
            bf16x8_t ebh, ebl;
            float ev[8];
#pragma unroll
            for (int p = 0; p < 8; ++p) ev[p] = X[rt][p >> 2][p & 3];
            split_vals(ev, ebh, ebl);
            Dl[rt][0] = floatx4_t{0.f, 0.f, 0.f, 0.f};
            Dl[rt][1] = Dl[rt][0];
            if (rt < nt) {
                mma3(Dl[rt][0], th0, tl0, ebh, ebl);
                mma3(Dl[rt][1], th1, tl1, ebh, ebl);
            }
        }
        // O = OQ + P Delta and S^T = gamma_C S^T + K^T Delta~
        const float r8[8] = {rev[0].x, rev[0].y, rev[0].z, rev[0].w, rev[1].x, rev[1].y, rev[1].z, rev[1].w};
        const bf16x8_t ph0 = frag(tst + (FP + 0) * FRAG), ph1 = frag(tst + (FP + 1) * FRAG);
        const bf16x8_t pl0 = frag(tst + (FP + 2) * FRAG), pl1 = frag(tst + (FP + 3) * FRAG);
        bf16x8_t tbh[GRP_RPW], tbl[GRP_RPW];
#pragma unroll
        for (int rt = 0; rt < GRP_RPW; ++rt) {
            float dv[8], dtv[8];
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                dv[p] = Dl[rt][p >> 2][p & 3];
                dtv[p] = dv[p] * r8[p];
            }
            bf16x8_t dbh, dbl;
            split_vals(dv, dbh, dbl);
            split_vals(dtv, tbh[rt], tbl[rt]);
            if (rt < nt) {
                mma3(OQ[rt][0], ph0, pl0, dbh, dbl);
                mma3(OQ[rt][1], ph1, pl1, dbh, dbl);
            }
        }
        const uint8_t *ktl = stg + kt_off;
#pragma unroll
        for (int jt = 0; jt < 8; ++jt) {
            const bf16x8_t kth = kt_frag(ktl, 0, jt);
            const bf16x8_t ktlo = kt_frag(ktl, 1, jt);
#pragma unroll
            for (int rt = 0; rt < GRP_RPW; ++rt) {
                if (rt < nt) {
                    ST[rt][jt] *= gC;
                    mma3(ST[rt][jt], kth, ktlo, tbh[rt], tbl[rt]);
                }
            }
        }
        {
            const __amdgpu_buffer_rsrc_t orr = wave_rsrc(o + ((int64_t)tb * Hv + h) * D,
                                                         (uint32_t)((Lc - 1) * Hv + 1) * D * sizeof(TO));
#pragma unroll
            for (int rt = 0; rt < GRP_RPW; ++rt)
#pragma unroll
                for (int tau = 0; tau < 2; ++tau)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int t = 16 * tau + 4 * lg + e;
                        // every wave issues the same number of stores (the chunk-top
                        // wait counts them); a one-tile wave's second tile falls
                        // outside the resource and is dropped
                        const uint32_t off = rt < nt ? (uint32_t)(t * Hv * D + irow[rt]) : 0x3FFFFFFFu;
                        store_o<TO>(orr, off, OQ[rt][tau][e] * inv_sqrt_d);
                    }
        }
        // prefix-cache snapshot after this chunk (full chunks only)
        if (snap.slots != nullptr && (cc + 1) % snap.every == 0 && (cc + 1) * CH <= L &&
            (cc + 1) / snap.every <= snap.max) {
            TS *sp = state + ((int64_t)snap.slots[(int64_t)r * snap.max + (cc + 1) / snap.every - 1] * Hv + h) * D * D;
#pragma unroll
            for (int rt = 0; rt < GRP_RPW; ++rt)
                if (rt < nt)
#pragma unroll
                    for (int jt = 0; jt < 8; ++jt)
                        st4(sp + (int64_t)irow[rt] * D + 16 * jt + 4 * lg,
                            make_float4(ST[rt][jt][0], ST[rt][jt][1], ST[rt][jt][2], ST[rt][jt][3]));
        }
        if constexpr (XCONV) {
            // v of the next chunk, from this wave's own copies of its rows: they
            // have landed once no more than this chunk's o stores are in flight
            if (prefetch) {
                __builtin_amdgcn_s_waitcnt(waitcnt_vm(8 * GRP_RPW));
                conv_next(cc + 1);
            }
        }
    }
#pragma unroll
    for (int rt = 0; rt < GRP_RPW; ++rt)
        if (rt < nt)
#pragma unroll
            for (int jt = 0; jt < 8; ++jt)
                st4(sbase + (int64_t)irow[rt] * D + 16 * jt + 4 * lg,
                    make_float4(ST[rt][jt][0], ST[rt][jt][1], ST[rt][jt][2], ST[rt][jt][3]));
    if constexpr (XCONV) {
        // new history (every reader of the old one is done): this lane's v
        // channels, and the key head's q / k channels from the first row block
        if (lg == 0)
#pragma unroll
            for (int rt = 0; rt < GRP_RPW; ++rt)
                if (rt < nt) chain_write_history<TX>(cv, cb + hh * D + ci[rt], slot, hi_init, tok0, L);
        if (rb == 0)
            for (int j = threadIdx.x; j < 2 * D; j += 64 * NW)
                chain_write_history<TX>(cv, (j < D ? 0 : cv.nq) + kh * D + (j & (D - 1)), slot, hi_init, tok0, L);
    }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// chunk offsets and request order, then the images of every possible chunk
// (a request of L tokens has ceil(L / 32) <= L / 32 + 1 chunks)
struct ChunkWorkspace {
    size_t meta, kimg, timg, total;
    ChunkWorkspace(int32_t Hk, int32_t Hv, int32_t T, int32_t nreq) {
        const size_t max_chunks = (size_t)T / chunk::CH + (size_t)nreq;
        meta = align256((size_t)(2 * nreq + 1) * 4);
        kimg = max_chunks * (size_t)Hk * chunk::KIMG;
        timg = max_chunks * (size_t)Hv * chunk::TIMG;
        total = meta + kimg + timg;
    }
};

size_t prefill_chunk_workspace_bytes(int32_t Hk, int32_t Hv, int32_t T, int32_t nreq) {
    return ChunkWorkspace(Hk, Hv, T, nreq).total;
}

// TA: the type of v (the unfused prefill); XCONV: the fused prefill, where the
// chain forms v from x (of type TX) and writes the new conv history.
template <int NW, typename TA, typename TO, bool XCONV, typename TX, typename TS, bool NORM = false>
static hipError_t launch_chain(const PrefillArgs &a, hipStream_t s, const int32_t *chunk_off,
                               const int32_t *order, const uint8_t *kimg, const uint8_t *timg,
                               const ChainConvIn &cv, const ChainSnap &sn, const ChainNorm &nm = ChainNorm{}) {
    using namespace chunk;
    static std::atomic<uint64_t> set{0};
    constexpr size_t smem = chain_smem_bytes<NW, XCONV, TX, NORM>();
    static_assert(smem <= 160 * 1024, "the chain's stages (and staged o) must fit in LDS");
    hipError_t e = set_smem_once(&prefill_chain_kernel<NW, TA, TO, XCONV, TX, TS, NORM>, smem, set);
    if (e != hipSuccess) return e;
    const int64_t per_group = (int64_t)(a.Hv / a.Hk) * (D / (16 * NW));
    const int64_t groups = (int64_t)a.nreq * a.Hk;
    const int64_t blocks = 8 * per_group * ((groups + 7) / 8);
    hipLaunchKernelGGL((prefill_chain_kernel<NW, TA, TO, XCONV, TX, TS, NORM>), dim3((unsigned)blocks),
                       dim3(64 * NW), smem, s, (const TA *)a.v, (TS *)a.state, a.qsl, a.slots,
                       a.has_init, chunk_off, order, kimg, timg, a.nreq, a.Hk, a.Hv, (TO *)a.o, cv, sn, nm);
    return hipGetLastError();
}

template <int G, typename TA, typename TO, bool XCONV, typename TX, typename TS>
static hipError_t launch_chain_group(const PrefillArgs &a, hipStream_t s, const int32_t *chunk_off,
                                     const int32_t *order, const uint8_t *kimg, const uint8_t *timg,
                                     const ChainConvIn &cv, const ChainSnap &sn) {
    using namespace chunk;
    constexpr int NW = GRP_NW;
    static std::atomic<uint64_t> set{0};
    constexpr size_t smem = 2 * group_stage_bytes<G, XCONV, TX>();
    static_assert(smem <= 160 * 1024, "two chain stages must fit in LDS");
    hipError_t e = set_smem_once(&prefill_chain_group_kernel<G, TA, TO, XCONV, TX, TS>, smem, set);
    if (e != hipSuccess) return e;
    const int64_t groups = (int64_t)a.nreq * a.Hk;
    const int64_t blocks = 8 * (int64_t)(D / GRP_ROWS) * ((groups + 7) / 8);
    hipLaunchKernelGGL((prefill_chain_group_kernel<G, TA, TO, XCONV, TX, TS>), dim3((unsigned)blocks),
                       dim3(64 * NW), smem, s, (const TA *)a.v, (TS *)a.state, a.qsl, a.slots,
                       a.has_init, chunk_off, order, kimg, timg, a.nreq, a.Hk, a.Hv, (TO *)a.o, cv, sn);
    return hipGetLastError();
}

// Block shape: large batches take key-head group blocks (the K image staged
// once for the group's 3 value heads; in the fused prefill only with bf16 x,
// whose staged rows leave two stages within LDS); else per-head blocks, a
// whole head (8 waves) when there are enough (request, head) units to fill the
// chip, else 32 rows.
template <typename TA, typename TO, bool XCONV, typename TX, typename TS>
static hipError_t launch_chain_pair(const PrefillArgs &a, hipStream_t s, const int32_t *chunk_off,
                                    const int32_t *order, const uint8_t *kimg, const uint8_t *timg,
                                    const ChainConvIn &cv, const ChainSnap &sn) {
    using namespace chunk;
    static std::atomic<uint64_t> set{0};
    constexpr size_t smem = pair_smem_bytes<XCONV, TX>();
    static_assert(smem <= 160 * 1024, "the paired chain's stages must fit in LDS");
    hipError_t e = set_smem_once(&prefill_chain_pair_kernel<TA, TO, XCONV, TX, TS>, smem, set);
    if (e != hipSuccess) return e;
    const int64_t per_group = (int64_t)(a.Hv / a.Hk) * (D / (16 * PAIR_TILES));
    const int64_t groups = (int64_t)a.nreq * a.Hk;
    const int64_t blocks = 8 * per_group * ((groups + 7) / 8);
    hipLaunchKernelGGL((prefill_chain_pair_kernel<TA, TO, XCONV, TX, TS>), dim3((unsigned)blocks),
                       dim3(64 * PAIR_WAVES), smem, s, (const TA *)a.v, (TS *)a.state, a.qsl, a.slots,
                       a.has_init, chunk_off, order, kimg, timg, a.nreq, a.Hk, a.Hv, (TO *)a.o, cv, sn);
    return hipGetLastError();
}

template <typename TA, typename TO, bool XCONV, typename TX, typename TS>
static hipError_t launch_chain_any(const PrefillArgs &a, hipStream_t s, const int32_t *chunk_off,
                                   const int32_t *order, const uint8_t *kimg, const uint8_t *timg,
                                   const ChainConvIn &cv, const ChainSnap &sn, bool *normed) {
    const int64_t units = (int64_t)a.nreq * a.Hv;
    *normed = false;
    if constexpr (XCONV && std::is_same<TX, bf16>::value) {
        // enough units for whole-head blocks and a bf16 gated output in 16-byte
        // pieces: the chain forms y itself (no o round trip, no norm pass)
        auto al16 = [](const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
        if (units >= 256 && a.y != nullptr && a.y_bf16 && a.z_bf16 && a.z_ld % 8 == 0 && al16(a.z) &&
            al16(a.y) && al16(a.gamma)) {
            *normed = true;
            const ChainNorm nm{static_cast<const bf16 *>(a.z), a.z_ld, a.gamma, a.gamma_bf16, a.norm_eps,
                               static_cast<bf16 *>(a.y)};
            return launch_chain<8, TA, TO, XCONV, TX, TS, true>(a, s, chunk_off, order, kimg, timg, cv, sn, nm);
        }
    }
    if constexpr (!XCONV || std::is_same<TX, bf16>::value) {
        if (units >= 256 && a.Hv == 3 * a.Hk)
            return launch_chain_group<3, TA, TO, XCONV, TX, TS>(a, s, chunk_off, order, kimg, timg, cv, sn);
    }
    return units >= 256 ? launch_chain<8, TA, TO, XCONV, TX, TS>(a, s, chunk_off, order, kimg, timg, cv, sn)
                        : launch_chain_pair<TA, TO, XCONV, TX, TS>(a, s, chunk_off, order, kimg, timg, cv, sn);
}

template <typename TA, typename TG, typename TX, typename TW, bool CONV>
static hipError_t launch_prep(const PrefillArgs &a, hipStream_t s, const int32_t *chunk_off,
                              uint8_t *kimg, uint8_t *timg, const PrepConvIn &cv) {
    using namespace chunk;
    static std::atomic<uint64_t> set{0};
    hipError_t e = set_smem_once(&prefill_prep_kernel<TA, TG, TX, TW, CONV>, sizeof(PrepSmem), set);
    if (e != hipSuccess) return e;
    const int64_t max_chunks = (int64_t)a.T / CH + a.nreq;
    hipLaunchKernelGGL((prefill_prep_kernel<TA, TG, TX, TW, CONV>), dim3((unsigned)(max_chunks * a.Hk)),
                       dim3(256), sizeof(PrepSmem), s, (const TA *)a.q, (const TA *)a.k,
                       (const TG *)a.a, (const TG *)a.b, a.gate_ld, a.qsl, chunk_off, a.nreq, a.Hk,
                       a.Hv, kimg, timg, cv);
    return hipGetLastError();
}

template <typename TA, typename TG, typename TO>
static hipError_t launch_chunk_t(const PrefillArgs &a, hipStream_t s) {
    using namespace chunk;
    const ChunkWorkspace wl(a.Hk, a.Hv, a.T, a.nreq);
    uint8_t *base = static_cast<uint8_t *>(a.ws);
    int32_t *chunk_off = reinterpret_cast<int32_t *>(base);
    int32_t *order = chunk_off + (a.nreq + 1);
    uint8_t *kimg = base + wl.meta;
    uint8_t *timg = kimg + wl.kimg;

    hipError_t e = hipSuccess;
    if (a.nreq <= PLAN_WAVE_MAX) {
        // few requests: the prep and chain waves work the plan out themselves
        chunk_off = nullptr;
        order = nullptr;
    } else {
        hipLaunchKernelGGL(prefill_plan_kernel, dim3(1), dim3(1024), 0, s, a.qsl, a.nreq, chunk_off, order);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }

    const PrepConvIn cv{a.x, a.x_ld, a.conv_w, a.pool, a.slots, a.has_init,
                        2 * a.Hk * D + a.Hv * D, a.l2_eps};
    const ChainSnap sn{a.max_snaps > 0 ? a.snap_slots : nullptr, a.max_snaps > 0 ? a.snap_interval / CH : 1,
                       a.max_snaps};
    bool normed = false;  // the chain formed the gated output itself
    if (a.x) {
        // conv mode: the prep kernel forms q and k (into the K images) from x;
        // the chain forms v from x itself and writes the new history of every
        // channel; o is fp32 scratch in this mode
        e = a.x_bf16 ? (a.w_bf16 ? launch_prep<TA, TG, bf16, bf16, true>(a, s, chunk_off, kimg, timg, cv)
                                 : launch_prep<TA, TG, bf16, float, true>(a, s, chunk_off, kimg, timg, cv))
                     : (a.w_bf16 ? launch_prep<TA, TG, float, bf16, true>(a, s, chunk_off, kimg, timg, cv)
                                 : launch_prep<TA, TG, float, float, true>(a, s, chunk_off, kimg, timg, cv));
        if (e != hipSuccess) return e;
        const ChainConvIn ci{a.x, a.x_ld, a.conv_w, a.w_bf16, a.pool, 2 * a.Hk * D + a.Hv * D, a.Hk * D};
        if constexpr (std::is_same<TO, float>::value) {
            if (a.state_bf16)
                e = a.x_bf16 ? launch_chain_any<float, float, true, bf16, bf16>(a, s, chunk_off, order, kimg, timg, ci, sn, &normed)
                             : launch_chain_any<float, float, true, float, bf16>(a, s, chunk_off, order, kimg, timg, ci, sn, &normed);
            else
                e = a.x_bf16 ? launch_chain_any<float, float, true, bf16, float>(a, s, chunk_off, order, kimg, timg, ci, sn, &normed)
                             : launch_chain_any<float, float, true, float, float>(a, s, chunk_off, order, kimg, timg, ci, sn, &normed);
        } else {
            return hipErrorInvalidValue;
        }
    } else {
        e = launch_prep<TA, TG, float, float, false>(a, s, chunk_off, kimg, timg, cv);
        if (e != hipSuccess) return e;
        if (a.state_bf16) return hipErrorInvalidValue;  // the unfused prefill keeps an fp32 state
        e = launch_chain_any<TA, TO, false, float, float>(a, s, chunk_off, order, kimg, timg, ChainConvIn{}, sn, &normed);
    }
    if (e != hipSuccess || !a.y || normed) return e;
    // gated output of the other block shapes (whose blocks hold part of a
    // head): a separate HBM-streaming pass over o
    GatedNormArgs g{D, a.o, a.o_bf16, a.z, a.z_ld, a.z_bf16, a.gamma, a.gamma_bf16, a.norm_eps,
                    a.T, a.Hv, a.y, a.y_bf16};
    return launch_gated_norm(g, s);
}
template <typename TA, typename TG>
static hipError_t launch_chunk_o(const PrefillArgs &a, hipStream_t s) {
    return a.o_bf16 ? launch_chunk_t<TA, TG, bf16>(a, s) : launch_chunk_t<TA, TG, float>(a, s);
}
template <typename TA>
static hipError_t launch_chunk_g(const PrefillArgs &a, hipStream_t s) {
    return a.gate_bf16 ? launch_chunk_o<TA, bf16>(a, s) : launch_chunk_o<TA, float>(a, s);
}

hipError_t launch_prefill_chunk(const PrefillArgs &a, hipStream_t s) {
    if (a.D != chunk::D) return hipErrorInvalidValue;
    return a.act_bf16 ? launch_chunk_g<bf16>(a, s) : launch_chunk_g<float>(a, s);
}

}  // namespace gdn
