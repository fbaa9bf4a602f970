// pkv_mfma.h - device helpers shared by the attention kernels (gfx950):
// LDS ordering, compile-time loops, matrix-core wrappers, the transposing LDS
// read, 16-bit pair packing and FP8 pair decoding.
#pragma once

#include <type_traits>
#include <utility>

#include "pkv_common.h"

namespace pkv {

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Orders LDS writes of some lanes before LDS reads of other lanes of the same
// wave (and reads before later overwrites).  Without it the exchange is a data
// race in the language model, and the compiler may move a lane's read under
// another lane's write predicate.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Workgroup barrier that orders LDS accesses only.  __syncthreads() also
// waits for every outstanding global store of the workgroup, which costs a
// full memory round trip; none of the exchanges below needs that.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Calls f(integral_constant<int, i>) for i = 0 .. N-1 in order.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <typename T> struct Mfma;
template <> struct Mfma<BF16> {
  __device__ static __forceinline__ f32x4_t run(const uint4& a, const uint4& b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
};
template <> struct Mfma<F16> {
  __device__ static __forceinline__ f32x4_t run(const uint4& a, const uint4& b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
};

// 16x16x16 products for P.V (k = the 16 tokens of a tile): four elements of
// A and of B per lane, as two dwords.
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
template <typename T> struct Mfma16;
template <> struct Mfma16<BF16> {
  __device__ static __forceinline__ f32x4_t run(s16x4_t a, const uint2& b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, __builtin_bit_cast(s16x4_t, b), c, 0, 0,
                                                     0);
  }
};
template <> struct Mfma16<F16> {
  __device__ static __forceinline__ f32x4_t run(s16x4_t a, const uint2& b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a),
                                                 __builtin_bit_cast(f16x4_t, b), c, 0, 0, 0);
  }
};

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane i receives element i % 4 of the 8-byte chunks addressed by lanes
// i / 4, 4 + i / 4, 8 + i / 4 and 12 + i / 4 of the same group, in that order.
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
__device__ __forceinline__ s16x4_t lds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4_t*)(__attribute__((address_space(3))) char*)(p));
}

// Two floats packed to the element type (round to nearest even), and the
// two halves of such a pair back as floats.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
template <typename T> struct Pair;
template <> struct Pair<BF16> {
  __device__ static __forceinline__ uint32_t pack(float a, float b) {
    const bf16x2_t v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
  }
  __device__ static __forceinline__ float lo(uint32_t w) { return bf16_lo(w); }
  __device__ static __forceinline__ float hi(uint32_t w) { return bf16_hi(w); }
};
template <> struct Pair<F16> {
  __device__ static __forceinline__ uint32_t pack(float a, float b) {
    const f16x2_t v = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, v);
  }
  __device__ static __forceinline__ float lo(uint32_t w) { return f16_lo(w); }
  __device__ static __forceinline__ float hi(uint32_t w) { return f16_hi(w); }
};

// Cross-row exchanges without LDS (gfx950 v_permlane16_swap /
// v_permlane32_swap): swapping a register with itself leaves, in every lane l,
// the values of lanes l and l ^ 16 (l ^ 32) in the two results, in some
// order (checked on the GPU).  Max and sum are symmetric, so each lane gets
// the combination of its pair.
__device__ __forceinline__ float max_xor16(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Two E4M3FN codes (bytes 2*hi, 2*hi + 1 of w) decoded straight to a pair of
// the element type: every E4M3FN value is exact in bf16 and f16, and a unit
// scale leaves it unchanged.
template <typename T> struct Fp8Pair;
template <> struct Fp8Pair<BF16> {
  template <bool kHi>
  __device__ static __forceinline__ uint32_t decode(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, kHi));
  }
};
template <> struct Fp8Pair<F16> {
  template <bool kHi>
  __device__ static __forceinline__ uint32_t decode(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, kHi));
  }
};

}  // namespace pkv
