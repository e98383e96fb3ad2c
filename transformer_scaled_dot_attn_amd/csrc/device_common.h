// Device-side helpers shared by the gfx950 attention kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tsda {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

#define TSDA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;

// Valid length of sequence b clamped to [0, Skv]; Skv when no lengths are given.
__device__ __forceinline__ int valid_length(const int32_t* kv_lens, int b, int Skv) {
    if (kv_lens == nullptr) return Skv;
    int L = kv_lens[b];
    return L < 0 ? 0 : (L > Skv ? Skv : L);
}

// Reinterpret a 32-bit word as a bfloat16 pair.  Takes the word by value:
// applying __builtin_bit_cast to a vector element in place reads element 0.
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t w) { return __builtin_bit_cast(bf16x2, w); }

// bfloat16 pair in a 32-bit word -> two floats (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats -> bfloat16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    f32x2 f = {lo, hi};
    bf16x2 h = __builtin_convertvector(f, bf16x2);
    return __builtin_bit_cast(uint32_t, h);
}

// One float -> bfloat16 bits, round to nearest even.
__device__ __forceinline__ uint16_t to_bf16(float x) {
    return static_cast<uint16_t>(pack_bf16(x, 0.0f) & 0xffffu);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Value of x held by lane (lane ^ 32) of the wavefront.
__device__ __forceinline__ float other_half(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return (threadIdx.x & 32) ? __uint_as_float(r[0]) : __uint_as_float(r[1]);
}

// max / sum of x over lanes l and l^32 (result in both).
__device__ __forceinline__ float halves_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// Sum over each aligned group of G lanes (G = 8 or 16); every lane gets it.
template <int G>
__device__ __forceinline__ float group_sum(float x) {
    x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
    x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
    if constexpr (G == 16) {
        x += dpp<0x124>(x);  // row_ror:4
        x += dpp<0x128>(x);  // row_ror:8
    } else {
        static_assert(G == 8, "group of 8 or 16 lanes");
        x += dpp<0x141>(x);  // row_half_mirror
    }
    return x;
}

__device__ __forceinline__ u32x4 ldg16(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

// 16-byte load marked non-temporal: for data streamed once, it keeps the
// caches for data that is reused and sustains more HBM bandwidth.
__device__ __forceinline__ u32x4 ldg16_stream(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// One 4-byte word of an allowed-mask row: keys j .. j+3, one byte each.
__device__ __forceinline__ uint32_t ldg_word(const uint8_t* p) {
    return *reinterpret_cast<const uint32_t*>(p);
}

// Nonzero iff some byte of w is zero, i.e. one of its four keys is hidden
// (exact as a yes/no test: a borrow can only run past a zero byte).
__device__ __forceinline__ uint32_t has_zero_byte(uint32_t w) {
    return (w - 0x01010101u) & ~w & 0x80808080u;
}

// Byte e (0..3) of mask word w is nonzero: key j+e is allowed.
__device__ __forceinline__ bool byte_set(uint32_t w, int e) { return ((w >> (8 * e)) & 0xffu) != 0; }

}  // namespace tsda
