// pkv_common.h - device helpers shared by the libpagedkv kernels (gfx950 only).
//
// Sources cited by tag and section:
//   [arch] "PagedAttention: Virtual-Memory KV Cache Management, Continuous
//          Batching, and PyTorch Architecture"
//   [note] "PagedAttention: Manage the Cache Without Moving the Sequence"
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pagedkv.h"

namespace pkv {

// 16-bit element types are carried as raw bits; the tag selects conversions.
struct F32 { using storage = float;    static constexpr int bytes = 4; static constexpr int code = PKV_F32; };
struct F16 { using storage = uint16_t; static constexpr int bytes = 2; static constexpr int code = PKV_F16; };
struct BF16 { using storage = uint16_t; static constexpr int bytes = 2; static constexpr int code = PKV_BF16; };

inline int dtype_bytes(int dtype) {
  switch (dtype) {
    case PKV_F32: return 4;
    case PKV_F16: return 2;
    case PKV_BF16: return 2;
    case PKV_FP8_E4M3: return 1;
    default: return 0;
  }
}

// ---------------------------------------------------------------------------
// Block-table resolution.  Token t of a sequence lives in physical block
// table[t / B] at offset t % B ([arch] "1. Paged Virtual Memory Mapping";
// [note] "Map a ten-token sequence into pages").  The page's address formula
// omits the head term and mixes bytes with elements; in the
// [num_blocks, B, H_kv, D] pool the element (head h, channel 0) of that row is
// at ((block * B + t % B) * H_kv + h) * D.  B is a power of two, passed as
// its log2.  Every kernel that touches the pool goes through this function.
// ---------------------------------------------------------------------------
__device__ __forceinline__ size_t row_offset(int block, int token, int log2_b, int num_kv_heads,
                                             int kv_head, int head_dim) {
  const int offset = token & ((1 << log2_b) - 1);
  return ((((size_t)block << log2_b) + offset) * (size_t)num_kv_heads + kv_head) * (size_t)head_dim;
}

// Logical block index of token t.
__device__ __forceinline__ int logical_block(int token, int log2_b) { return token >> log2_b; }

// True when a table entry names a block of the pool.
__device__ __forceinline__ bool valid_block(int id, int num_blocks) {
  return id >= 0 && id < num_blocks;
}

// A per-head FP8 scale is usable when it is finite and positive; with any
// other scale the appends store NaN codes in that head of that pool, and
// attention gives the head's rows NaN.
__device__ __forceinline__ bool scale_ok(float s) { return s > 0.f && s < INFINITY; }

// ---------------------------------------------------------------------------
// Conversions.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// fp32 -> bf16 bits, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// fp32 -> fp16 bits with the hardware conversion (round to nearest even).
__device__ __forceinline__ uint16_t f32_to_f16_rne(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// store4 writes four consecutive elements with one store (dst aligned to
// four elements).
template <typename T> struct Cvt;
template <> struct Cvt<F32> {
  // Unpack the 4 floats of a 16-byte chunk.
  __device__ static __forceinline__ void unpack(const uint4& c, float* out) {
    out[0] = __uint_as_float(c.x); out[1] = __uint_as_float(c.y);
    out[2] = __uint_as_float(c.z); out[3] = __uint_as_float(c.w);
  }
  __device__ static __forceinline__ void store(float* dst, float v) { *dst = v; }
  __device__ static __forceinline__ void store4(float* dst, float a, float b, float c, float d) {
    *reinterpret_cast<float4*>(dst) = make_float4(a, b, c, d);
  }
};
template <> struct Cvt<BF16> {
  __device__ static __forceinline__ void unpack(const uint4& c, float* out) {
    out[0] = bf16_lo(c.x); out[1] = bf16_hi(c.x); out[2] = bf16_lo(c.y); out[3] = bf16_hi(c.y);
    out[4] = bf16_lo(c.z); out[5] = bf16_hi(c.z); out[6] = bf16_lo(c.w); out[7] = bf16_hi(c.w);
  }
  __device__ static __forceinline__ void store(uint16_t* dst, float v) { *dst = f32_to_bf16_rne(v); }
  __device__ static __forceinline__ void store4(uint16_t* dst, float a, float b, float c, float d) {
    *reinterpret_cast<uint2*>(dst) =
        make_uint2(f32_to_bf16_rne(a) | ((uint32_t)f32_to_bf16_rne(b) << 16),
                   f32_to_bf16_rne(c) | ((uint32_t)f32_to_bf16_rne(d) << 16));
  }
};
template <> struct Cvt<F16> {
  __device__ static __forceinline__ void unpack(const uint4& c, float* out) {
    out[0] = f16_lo(c.x); out[1] = f16_hi(c.x); out[2] = f16_lo(c.y); out[3] = f16_hi(c.y);
    out[4] = f16_lo(c.z); out[5] = f16_hi(c.z); out[6] = f16_lo(c.w); out[7] = f16_hi(c.w);
  }
  __device__ static __forceinline__ void store(uint16_t* dst, float v) { *dst = f32_to_f16_rne(v); }
  __device__ static __forceinline__ void store4(uint16_t* dst, float a, float b, float c, float d) {
    *reinterpret_cast<uint2*>(dst) =
        make_uint2(f32_to_f16_rne(a) | ((uint32_t)f32_to_f16_rne(b) << 16),
                   f32_to_f16_rne(c) | ((uint32_t)f32_to_f16_rne(d) << 16));
  }
};

__device__ __forceinline__ uint4 load16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
// Streaming load (non-temporal hint): for data read once per call, such as
// the K/V cache in decode attention; it keeps the caches for reused data and
// lets the memory system run closer to peak.
__device__ __forceinline__ uint4 load16_stream(const void* p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 load8(const void* p) { return *reinterpret_cast<const uint2*>(p); }
__device__ __forceinline__ uint2 load8_stream(const void* p) {
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return make_uint2(v.x, v.y);
}

// ---------------------------------------------------------------------------
// FP8 cache codes: E4M3FN of the OCP 8-bit floating point format (bias 7,
// 3 mantissa bits, no infinities, S.1111.111 = NaN, largest finite 448).
// gfx950's v_cvt_pk_f32_fp8 decodes this format exactly; its encoder rounds
// to nearest even but turns magnitudes past the largest rounding boundary
// into NaN, so the encoder below saturates first and keeps NaN explicitly.
// ---------------------------------------------------------------------------
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Four codes (one 32-bit word, code i in byte i) -> four floats.
__device__ __forceinline__ void e4m3_decode4(uint32_t w, float* out) {
  const f32x2_t a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  const f32x2_t b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  out[0] = a.x; out[1] = a.y; out[2] = b.x; out[3] = b.y;
}

// Four floats -> four codes: nearest, ties to even, |v| >= 448 -> +-448,
// NaN -> 0x7F or 0xFF by the sign bit.
__device__ __forceinline__ uint32_t e4m3_encode4(float v0, float v1, float v2, float v3) {
  auto sat = [](float v) { return fminf(fmaxf(v, -448.f), 448.f); };   // NaN: fixed below
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(sat(v0), sat(v1), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(sat(v2), sat(v3), w, true);
  uint32_t u = (uint32_t)w;
  const float v[4] = {v0, v1, v2, v3};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (v[i] != v[i]) {
      const uint32_t nan_code = (__float_as_uint(v[i]) >> 31) ? 0xFFu : 0x7Fu;
      u = (u & ~(0xFFu << (8 * i))) | (nan_code << (8 * i));
    }
  }
  return u;
}
__device__ __forceinline__ void store16(void* p, const uint4& v) { *reinterpret_cast<uint4*>(p) = v; }

inline int log2_exact(int x) {
  if (x <= 0 || (x & (x - 1)) != 0) return -1;
  int r = 0;
  while ((1 << r) < x) ++r;
  return r;
}

}  // namespace pkv
