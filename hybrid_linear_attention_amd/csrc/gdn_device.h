// Internal device helpers shared by the gfx950 kernels of libgdn.
// (Not part of the ABI; include/gdn.h is the public interface.)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// Native 4-float vector (usable with the nontemporal builtins, unlike float4).
typedef float f32x4 __attribute__((ext_vector_type(4)));

// bf16 is carried as its raw 16-bit pattern; conversions are explicit.
struct bf16 {
    uint16_t bits;
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return __uint_as_float(uint32_t(x.bits) << 16); }

// fp32 -> bf16, round to nearest even (NaN kept quiet).
__device__ __forceinline__ bf16 to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return bf16{uint16_t((u >> 16) | 0x40u)};
    u += 0x7fffu + ((u >> 16) & 1u);
    return bf16{uint16_t(u >> 16)};
}

template <typename T> __device__ __forceinline__ T from_f32(float f);
template <> __device__ __forceinline__ float from_f32<float>(float f) { return f; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float f) { return to_bf16(f); }

template <typename T> __device__ __forceinline__ float ld(const T *p) { return to_f32(*p); }
template <typename T> __device__ __forceinline__ void st(T *p, float f) { *p = from_f32<T>(f); }

// Two consecutive elements (p must be aligned to two elements).
__device__ __forceinline__ float2 ld2(const float *p) { return *reinterpret_cast<const float2 *>(p); }
__device__ __forceinline__ float2 ld2(const bf16 *p) {
    uint32_t u = *reinterpret_cast<const uint32_t *>(p);
    return make_float2(__uint_as_float(u << 16), __uint_as_float(u & 0xffff0000u));
}
__device__ __forceinline__ void st2(float *p, float a, float b) {
    *reinterpret_cast<float2 *>(p) = make_float2(a, b);
}
__device__ __forceinline__ void st2(bf16 *p, float a, float b) {
    uint32_t u = uint32_t(to_bf16(a).bits) | (uint32_t(to_bf16(b).bits) << 16);
    *reinterpret_cast<uint32_t *>(p) = u;
}

// Four consecutive elements (p aligned to four elements).
__device__ __forceinline__ float4 ld4(const float *p) { return *reinterpret_cast<const float4 *>(p); }
__device__ __forceinline__ float4 ld4(const bf16 *p) {
    uint2 u = *reinterpret_cast<const uint2 *>(p);
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                       __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
}

// Store four consecutive elements (p aligned to four elements); bf16 rounds
// once (RNE).
__device__ __forceinline__ void st4(float *p, float4 v) { *reinterpret_cast<float4 *>(p) = v; }
__device__ __forceinline__ void st4(bf16 *p, float4 v) {
    const uint32_t a = uint32_t(to_bf16(v.x).bits) | (uint32_t(to_bf16(v.y).bits) << 16);
    const uint32_t b = uint32_t(to_bf16(v.z).bits) | (uint32_t(to_bf16(v.w).bits) << 16);
    *reinterpret_cast<uint2 *>(p) = make_uint2(a, b);
}

// Eight consecutive elements (p aligned to 16 bytes), kept in their storage
// format until converted, so that issuing a load never waits for its data.
template <typename T> struct Raw8;
template <> struct Raw8<bf16> {
    uint4 u;
    __device__ __forceinline__ void load(const bf16 *p) { u = *reinterpret_cast<const uint4 *>(p); }
    __device__ __forceinline__ void zero() { u = make_uint4(0, 0, 0, 0); }
    __device__ __forceinline__ void get(float (&f)[8]) const {
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(w[i] << 16);
            f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
};
template <> struct Raw8<float> {
    float4 a, b;
    __device__ __forceinline__ void load(const float *p) {
        a = reinterpret_cast<const float4 *>(p)[0];
        b = reinterpret_cast<const float4 *>(p)[1];
    }
    __device__ __forceinline__ void zero() { a = b = make_float4(0.f, 0.f, 0.f, 0.f); }
    __device__ __forceinline__ void get(float (&f)[8]) const {
        f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
        f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
    }
};

// Store eight consecutive elements (p aligned to 16 bytes); bf16 rounds once (RNE).
__device__ __forceinline__ void store8(float *p, const float (&f)[8]) {
    reinterpret_cast<float4 *>(p)[0] = make_float4(f[0], f[1], f[2], f[3]);
    reinterpret_cast<float4 *>(p)[1] = make_float4(f[4], f[5], f[6], f[7]);
}
__device__ __forceinline__ void store8(bf16 *p, const float (&f)[8]) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        w[i] = uint32_t(to_bf16(f[2 * i]).bits) | (uint32_t(to_bf16(f[2 * i + 1]).bits) << 16);
    *reinterpret_cast<uint4 *>(p) = make_uint4(w[0], w[1], w[2], w[3]);
}

// State rows streamed through range-checked buffer loads and stores: a row of D
// elements is held by D / 8 lanes, 8 elements (two float4) per lane.  fp32 rows:
// lane l holds columns 4 l .. 4 l + 3 and 4 l + D / 2 .. + 3 (two 16-byte
// accesses, each covering half the row across the lanes); bf16 rows: columns
// 8 l .. 8 l + 7 (one 16-byte access), widened exactly on load and rounded to
// nearest-even on store.  `off` is the byte offset of the row in the resource;
// AUX the cache policy of the accesses.
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
template <typename TS, int LPR> struct StateRow;
template <int LPR> struct StateRow<float, LPR> {
    __device__ static __forceinline__ int col(int l, int m) { return 4 * l + 4 * LPR * m; }
    template <int AUX>
    __device__ static __forceinline__ void load(f32x4 (&dst)[2], __amdgpu_buffer_rsrc_t r, uint32_t off, int l) {
#pragma unroll
        for (int m = 0; m < 2; ++m)
            dst[m] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off + 16 * l + 16 * LPR * m, 0, AUX));
    }
    template <int AUX>
    __device__ static __forceinline__ void store(const f32x4 &a, const f32x4 &b, __amdgpu_buffer_rsrc_t r,
                                                 uint32_t off, int l) {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, a), r, off + 16 * l, 0, AUX);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, b), r, off + 16 * l + 16 * LPR, 0, AUX);
    }
};
template <int LPR> struct StateRow<bf16, LPR> {
    __device__ static __forceinline__ int col(int l, int m) { return 8 * l + 4 * m; }
    template <int AUX>
    __device__ static __forceinline__ void load(f32x4 (&dst)[2], __amdgpu_buffer_rsrc_t r, uint32_t off, int l) {
        const u32x4_t u = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off + 16 * l, 0, AUX));
        dst[0] = f32x4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                       __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u)};
        dst[1] = f32x4{__uint_as_float(u.z << 16), __uint_as_float(u.z & 0xffff0000u),
                       __uint_as_float(u.w << 16), __uint_as_float(u.w & 0xffff0000u)};
    }
    __device__ static __forceinline__ uint32_t pack(float lo, float hi) {
        return uint32_t(to_bf16(lo).bits) | (uint32_t(to_bf16(hi).bits) << 16);
    }
    template <int AUX>
    __device__ static __forceinline__ void store(const f32x4 &a, const f32x4 &b, __amdgpu_buffer_rsrc_t r,
                                                 uint32_t off, int l) {
        const u32x4_t u = u32x4_t{pack(a.x, a.y), pack(a.z, a.w), pack(b.x, b.y), pack(b.z, b.w)};
        __builtin_amdgcn_raw_buffer_store_b128(u, r, off + 16 * l, 0, AUX);
    }
};

// Lane permutations inside rows of 16 lanes (DPP): xor 1 and xor 2 inside a
// quad, then the mirror of an 8-lane half and of the 16-lane row.
__device__ __forceinline__ float dpp_f(float v, int ctrl_sel) {
    int r;
    switch (ctrl_sel) {
        case 0: r = __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true); break;   // quad_perm 1,0,3,2
        case 1: r = __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true); break;   // quad_perm 2,3,0,1
        case 2: r = __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xF, 0xF, true); break;  // row_half_mirror
        default: r = __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x140, 0xF, 0xF, true); break; // row_mirror
    }
    return __builtin_bit_cast(float, r);
}

// Butterfly sum over aligned groups of `width` lanes (width a power of two <=
// 64); every lane of a group ends with the group's sum.  Up to 16 lanes the
// partner values move by DPP (no LDS round trip): once the 4 (8) lanes below
// hold equal partial sums, the mirrored lane holds the same partial sum as the
// xor-4 (xor-8) partner, so the additions are those of the xor butterfly.
template <int WIDTH> __device__ __forceinline__ float group_sum(float v) {
    if constexpr (WIDTH >= 2) v += dpp_f(v, 0);
    if constexpr (WIDTH >= 4) v += dpp_f(v, 1);
    if constexpr (WIDTH >= 8) v += dpp_f(v, 2);
    if constexpr (WIDTH >= 16) v += dpp_f(v, 3);
#pragma unroll
    for (int m = 16; m < WIDTH; m <<= 1) v += __shfl_xor(v, m, 64);
    return v;
}

__device__ __forceinline__ float silu_f(float y) { return y / (1.0f + __expf(-y)); }
// SiLU with the hardware reciprocal (about 1 ulp of fp32 more error than silu_f)
__device__ __forceinline__ float silu_fast(float y) {
    return y * __builtin_amdgcn_rcpf(1.0f + __expf(-y));
}

// alpha = exp(-softplus(a)) = 1 / (1 + e^a); beta = sigmoid(b) = 1 / (1 + e^-b).
// Written in the forms that stay finite for any |a|, |b|.
__device__ __forceinline__ float gate_alpha(float a) {
    float sp = fmaxf(a, 0.0f) + log1pf(expf(-fabsf(a)));
    return expf(-sp);
}
__device__ __forceinline__ float gate_log_alpha(float a) {
    return -(fmaxf(a, 0.0f) + log1pf(expf(-fabsf(a))));
}
__device__ __forceinline__ float gate_beta(float b) { return 1.0f / (1.0f + expf(-b)); }

// First index r in [0, n) with qsl[r] <= t < qsl[r + 1] (qsl non-decreasing,
// qsl[0] = 0 <= t < qsl[n]); empty requests are skipped.
__device__ __forceinline__ int find_request(const int32_t *__restrict__ qsl, int n, int t) {
    int lo = 0, hi = n;  // invariant: qsl[lo] <= t < qsl[hi]
    while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (qsl[mid] <= t) lo = mid; else hi = mid;
    }
    return lo;
}

}  // namespace gdn
