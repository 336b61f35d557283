// Device-side helpers for the gfx950 (CDNA4) attention kernels: 16-bit element
// traits, the MFMA wrappers, conversions that round to nearest-even, and
// cross-lane moves.  Internal to libsdpa.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdpa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// Element traits for the two 16-bit input formats.  Data moves as raw 16-bit
// words (uint16_t / uint4) and is reinterpreted only at the MFMA.
struct BF16 {
    typedef bf16x8_t vec8;
    static __device__ __forceinline__ f32x16_t mfma32(vec8 a, vec8 b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4_t mfma16(vec8 a, vec8 b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    // round-to-nearest-even float -> bf16 bits
    static __device__ __forceinline__ uint16_t from_f32(float x) {
        __bf16 h = (__bf16)x;
        return __builtin_bit_cast(uint16_t, h);
    }
    static __device__ __forceinline__ float to_f32(uint16_t b) {
        return __uint_as_float(((uint32_t)b) << 16);
    }
    // two floats -> packed pair (low half = a), nearest-even
    static __device__ __forceinline__ uint32_t pack2(float a, float b) {
        typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
        bf16x2_t v = {(__bf16)a, (__bf16)b};
        return __builtin_bit_cast(uint32_t, v);
    }
    // acc + both halves of a packed pair, in fp32 (v_dot2c against (1, 1))
    static __device__ __forceinline__ float sum2(uint32_t pair, float acc) {
        typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pair),
                                               __builtin_bit_cast(bf16x2_t, 0x3f803f80u), acc, false);
    }
};

struct F16 {
    typedef f16x8_t vec8;
    static __device__ __forceinline__ f32x16_t mfma32(vec8 a, vec8 b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4_t mfma16(vec8 a, vec8 b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ uint16_t from_f32(float x) {
        _Float16 h = (_Float16)x;
        return __builtin_bit_cast(uint16_t, h);
    }
    static __device__ __forceinline__ float to_f32(uint16_t b) {
        return (float)__builtin_bit_cast(_Float16, b);
    }
    static __device__ __forceinline__ uint32_t pack2(float a, float b) {
        typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
        f16x2_t v = {(_Float16)a, (_Float16)b};
        return __builtin_bit_cast(uint32_t, v);
    }
    static __device__ __forceinline__ float sum2(uint32_t pair, float acc) {
        typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, pair), __builtin_bit_cast(f16x2_t, 0x3c003c00u),
                                      acc, false);
    }
};

template <typename Tr>
__device__ __forceinline__ typename Tr::vec8 as_vec8(uint4 u) {
    return __builtin_bit_cast(typename Tr::vec8, u);
}

// 2^x on the transcendental unit (v_exp_f32); exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
// log2(x) on the transcendental unit (v_log_f32); log2(0) = -inf.
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Value of lane (lane ^ mask) for mask in {1..32} (ds_bpermute based).
__device__ __forceinline__ float xor_lane(float x, int mask) { return __shfl_xor(x, mask, 64); }

// max / sum of x over the lane pair (l, l ^ 32), on the VALU (v_permlane32_swap).
// The swap hands each lane its partner's value in one of the two results and
// keeps its own in the other, so max and sum of the pair are symmetric.
__device__ __forceinline__ float pair32_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair32_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Wait until every vector-memory load issued so far has returned (s_waitcnt
// vmcnt(0); expcnt and lgkmcnt left at their maxima, gfx9 encoding).  Used once
// before a loop whose first use of those registers would otherwise carry the
// wait into every iteration, where it would also wait for prefetches.
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Flip the sign bit of eight 16-bit values (exact negation, NaN kept).
__device__ __forceinline__ uint4 negate8(uint4 u) {
    u.x ^= 0x80008000u; u.y ^= 0x80008000u; u.z ^= 0x80008000u; u.w ^= 0x80008000u;
    return u;
}

__device__ __forceinline__ uint4 zero4() { return make_uint4(0, 0, 0, 0); }

// Raw buffer access (gfx9 buffer resource, stride 0).  The hardware checks each
// access against the resource's byte size: loads past it return 0 and stores
// past it are dropped, so tile edges need no branches and offsets stay 32-bit.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
constexpr int kRawBufferWord3 = 0x00020000;  // 32-bit data format, no swizzle, no stride

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes < 0 ? 0 : bytes,
                                             kRawBufferWord3);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, int off) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 buf_load8(__amdgpu_buffer_rsrc_t r, int off) {
    const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint32_t buf_load4(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t buf_load1(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
}
__device__ __forceinline__ void buf_store8(uint2 v, __amdgpu_buffer_rsrc_t r, int off) {
    const u32x2_t w = {v.x, v.y};
    __builtin_amdgcn_raw_buffer_store_b64(w, r, off, 0, 0);
}
__device__ __forceinline__ void buf_store4(float v, __amdgpu_buffer_rsrc_t r, int off) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, 0);
}
__device__ __forceinline__ void buf_store16(uint4 v, __amdgpu_buffer_rsrc_t r, int off) {
    const u32x4_t w = {v.x, v.y, v.z, v.w};
    __builtin_amdgcn_raw_buffer_store_b128(w, r, off, 0, 0);
}
// Streaming variants for data written once and read once much later (the
// non-temporal cache policy, bit 1 of the policy operand): such lines are the
// first the caches give up, so they do not push out data that is reused.
constexpr int kCachePolicyNT = 2;
__device__ __forceinline__ uint4 buf_load16_nt(__amdgpu_buffer_rsrc_t r, int off) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCachePolicyNT);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void buf_store16_nt(uint4 v, __amdgpu_buffer_rsrc_t r, int off) {
    const u32x4_t w = {v.x, v.y, v.z, v.w};
    __builtin_amdgcn_raw_buffer_store_b128(w, r, off, 0, kCachePolicyNT);
}

}  // namespace sdpa
