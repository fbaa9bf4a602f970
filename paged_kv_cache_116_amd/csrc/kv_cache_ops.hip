// kv_cache_ops.hip - cache append, whole-block copy and debug gather (gfx950).
//
// Sources cited by tag and section:
//   [pofe] "PagedAttention: paging the KV cache"
//   [arch] "PagedAttention: Virtual-Memory KV Cache Management, Continuous
//          Batching, and PyTorch Architecture"
//
// All three are byte moves of whole 16-byte chunks: a token's row in the pool
// (all KV heads, all channels) is contiguous, Hkv * D * sizeof(T) bytes, and a
// multiple of 16 for every supported head size.  Each kernel resolves block
// ids through pkv::row_offset, the same function the attention kernels use.
#include "pkv_common.h"
#include "pkv_host.h"

namespace pkv {
namespace {

constexpr int kThreads = 256;

// One workgroup per sequence: copy the new token's row into slot len % B of
// block table[len / B] ([pofe] "How it works", decode-step write).
__global__ __launch_bounds__(kThreads) void append_kernel(
    char* __restrict__ k_pool, char* __restrict__ v_pool, const char* __restrict__ k_new,
    const char* __restrict__ v_new, const int32_t* __restrict__ tables, int max_blocks,
    const int32_t* __restrict__ lens_pre, int num_blocks, int log2_b, int num_kv_heads,
    int head_dim, int elem_bytes) {
  const int s = blockIdx.x;
  const int len = lens_pre[s];
  if (len < 0) return;                                   // padding row
  const int lb = logical_block(len, log2_b);
  if (lb >= max_blocks) return;                          // table row too short: skip
  const int blk = tables[(size_t)s * max_blocks + lb];
  if (!valid_block(blk, num_blocks)) return;             // id outside the pool: skip
  const size_t row_bytes = (size_t)num_kv_heads * head_dim * elem_bytes;
  const size_t dst = row_offset(blk, len, log2_b, num_kv_heads, 0, head_dim) * elem_bytes;
  const size_t src = (size_t)s * row_bytes;
  const int chunks = (int)(row_bytes / 16);
  for (int c = threadIdx.x; c < chunks; c += kThreads) {
    store16(k_pool + dst + 16 * (size_t)c, load16(k_new + src + 16 * (size_t)c));
    store16(v_pool + dst + 16 * (size_t)c, load16(v_new + src + 16 * (size_t)c));
  }
}

// FP8 pools: one workgroup per sequence; each thread quantises 8 elements of
// the new token's row, code = e4m3(fp32(x) / fp32(scale)), and stores them
// as 8 bytes.  T is the element type of k_new / v_new.  k_scales / v_scales
// (per-head scales, [num_kv_heads]) replace k_scale / v_scale when not null.
template <typename T>
__global__ __launch_bounds__(kThreads) void append_fp8_kernel(
    uint8_t* __restrict__ k_pool, uint8_t* __restrict__ v_pool, const char* __restrict__ k_new,
    const char* __restrict__ v_new, const int32_t* __restrict__ tables, int max_blocks,
    const int32_t* __restrict__ lens_pre, int num_blocks, int log2_b, int num_kv_heads,
    int head_dim, float k_scale, float v_scale, const float* __restrict__ k_scales,
    const float* __restrict__ v_scales) {
  const int s = blockIdx.x;
  const int len = lens_pre[s];
  if (len < 0) return;
  const int lb = logical_block(len, log2_b);
  if (lb >= max_blocks) return;
  const int blk = tables[(size_t)s * max_blocks + lb];
  if (!valid_block(blk, num_blocks)) return;
  const int row = num_kv_heads * head_dim;          // elements, a multiple of 16
  const size_t dst = row_offset(blk, len, log2_b, num_kv_heads, 0, head_dim);
  for (int c = threadIdx.x; c < row / 8; c += kThreads) {
    float kf[8], vf[8];
    const size_t src = ((size_t)s * row + 8 * c) * T::bytes;
    if constexpr (T::bytes == 4) {
      Cvt<T>::unpack(load16(k_new + src), kf);
      Cvt<T>::unpack(load16(k_new + src + 16), kf + 4);
      Cvt<T>::unpack(load16(v_new + src), vf);
      Cvt<T>::unpack(load16(v_new + src + 16), vf + 4);
    } else {
      Cvt<T>::unpack(load16(k_new + src), kf);
      Cvt<T>::unpack(load16(v_new + src), vf);
    }
    float ks = k_scale, vs = v_scale;
    if (k_scales) {   // the chunk's KV head (head_dim is a multiple of 16)
      ks = k_scales[8 * c / head_dim];
      vs = v_scales[8 * c / head_dim];
    }
    const bool k_ok = scale_ok(ks), v_ok = scale_ok(vs);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      kf[e] = k_ok ? kf[e] / ks : __builtin_nanf("");
      vf[e] = v_ok ? vf[e] / vs : __builtin_nanf("");
    }
    const uint2 kc = make_uint2(e4m3_encode4(kf[0], kf[1], kf[2], kf[3]),
                                e4m3_encode4(kf[4], kf[5], kf[6], kf[7]));
    const uint2 vc = make_uint2(e4m3_encode4(vf[0], vf[1], vf[2], vf[3]),
                                e4m3_encode4(vf[4], vf[5], vf[6], vf[7]));
    *reinterpret_cast<uint2*>(k_pool + dst + 8 * c) = kc;
    *reinterpret_cast<uint2*>(v_pool + dst + 8 * c) = vc;
  }
}

// Several new tokens per sequence (prefill chunks): thread i copies 16-byte
// chunk i % row_chunks of packed token i / row_chunks.  The token's sequence
// is the s with cu[s] <= token < cu[s + 1] (binary search; cu is
// non-decreasing), its position lens_pre[s] + token - cu[s] ([pofe] "How it
// works": prefill writes the prompt into its blocks).
__global__ __launch_bounds__(kThreads) void append_tokens_kernel(
    char* __restrict__ k_pool, char* __restrict__ v_pool, const char* __restrict__ k_new,
    const char* __restrict__ v_new, const int32_t* __restrict__ cu, int num_tokens,
    const int32_t* __restrict__ tables, int max_blocks, const int32_t* __restrict__ lens_pre,
    int num_seqs, int num_blocks, int log2_b, int num_kv_heads, int head_dim, int elem_bytes) {
  const size_t row_bytes = (size_t)num_kv_heads * head_dim * elem_bytes;
  const int row_chunks = (int)(row_bytes / 16);
  const long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (i >= (long long)num_tokens * row_chunks) return;
  const int tok = (int)(i / row_chunks);
  const int c = (int)(i - (long long)tok * row_chunks);
  if (tok < cu[0] || tok >= cu[num_seqs]) return;           // not in any chunk
  int lo = 0, hi = num_seqs - 1;                            // last s with cu[s] <= tok
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= tok) lo = mid;
    else hi = mid - 1;
  }
  const int s = lo;
  const int start = lens_pre[s];
  if (start < 0) return;                                    // padding row
  const int pos = start + (tok - cu[s]);
  const int lb = logical_block(pos, log2_b);
  if (pos < 0 || lb >= max_blocks) return;                  // past the table row: skip
  const int blk = tables[(size_t)s * max_blocks + lb];
  if (!valid_block(blk, num_blocks)) return;                // id outside the pool: skip
  const size_t dst = row_offset(blk, pos, log2_b, num_kv_heads, 0, head_dim) * elem_bytes;
  const size_t src = (size_t)tok * row_bytes;
  store16(k_pool + dst + 16 * (size_t)c, load16(k_new + src + 16 * (size_t)c));
  store16(v_pool + dst + 16 * (size_t)c, load16(v_new + src + 16 * (size_t)c));
}

// Several new tokens per sequence into FP8 pools: thread i quantises 8
// elements (chunk i % row_chunks) of packed token i / row_chunks, as
// append_fp8_kernel does for one token, at the position append_tokens_kernel
// gives it.  T is the element type of k_new / v_new.
template <typename T>
__global__ __launch_bounds__(kThreads) void append_tokens_fp8_kernel(
    uint8_t* __restrict__ k_pool, uint8_t* __restrict__ v_pool, const char* __restrict__ k_new,
    const char* __restrict__ v_new, const int32_t* __restrict__ cu, int num_tokens,
    const int32_t* __restrict__ tables, int max_blocks, const int32_t* __restrict__ lens_pre,
    int num_seqs, int num_blocks, int log2_b, int num_kv_heads, int head_dim, float k_scale,
    float v_scale) {
  const int row = num_kv_heads * head_dim;           // elements, a multiple of 16
  const int row_chunks = row / 8;
  const long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (i >= (long long)num_tokens * row_chunks) return;
  const int tok = (int)(i / row_chunks);
  const int c = (int)(i - (long long)tok * row_chunks);
  if (tok < cu[0] || tok >= cu[num_seqs]) return;           // not in any chunk
  int lo = 0, hi = num_seqs - 1;                            // last s with cu[s] <= tok
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= tok) lo = mid;
    else hi = mid - 1;
  }
  const int s = lo;
  const int start = lens_pre[s];
  if (start < 0) return;                                    // padding row
  const int pos = start + (tok - cu[s]);
  const int lb = logical_block(pos, log2_b);
  if (pos < 0 || lb >= max_blocks) return;                  // past the table row: skip
  const int blk = tables[(size_t)s * max_blocks + lb];
  if (!valid_block(blk, num_blocks)) return;                // id outside the pool: skip
  const size_t dst = row_offset(blk, pos, log2_b, num_kv_heads, 0, head_dim) + 8 * (size_t)c;
  const size_t src = ((size_t)tok * row + 8 * (size_t)c) * T::bytes;
  float kf[8], vf[8];
  if constexpr (T::bytes == 4) {
    Cvt<T>::unpack(load16(k_new + src), kf);
    Cvt<T>::unpack(load16(k_new + src + 16), kf + 4);
    Cvt<T>::unpack(load16(v_new + src), vf);
    Cvt<T>::unpack(load16(v_new + src + 16), vf + 4);
  } else {
    Cvt<T>::unpack(load16(k_new + src), kf);
    Cvt<T>::unpack(load16(v_new + src), vf);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    kf[e] = kf[e] / k_scale;
    vf[e] = vf[e] / v_scale;
  }
  *reinterpret_cast<uint2*>(k_pool + dst) = make_uint2(e4m3_encode4(kf[0], kf[1], kf[2], kf[3]),
                                                       e4m3_encode4(kf[4], kf[5], kf[6], kf[7]));
  *reinterpret_cast<uint2*>(v_pool + dst) = make_uint2(e4m3_encode4(vf[0], vf[1], vf[2], vf[3]),
                                                       e4m3_encode4(vf[4], vf[5], vf[6], vf[7]));
}

// blockIdx.x = pair, blockIdx.y = slice of the block's chunks.
__global__ __launch_bounds__(kThreads) void copy_blocks_kernel(
    char* __restrict__ k_pool, char* __restrict__ v_pool, const int32_t* __restrict__ src,
    const int32_t* __restrict__ dst, int num_blocks, size_t block_bytes) {
  const int a = src[blockIdx.x];
  const int b = dst[blockIdx.x];
  if (!valid_block(a, num_blocks) || !valid_block(b, num_blocks)) return;
  const size_t chunks = block_bytes / 16;
  const size_t sa = (size_t)a * block_bytes, sb = (size_t)b * block_bytes;
  for (size_t c = (size_t)blockIdx.y * kThreads + threadIdx.x; c < chunks;
       c += (size_t)gridDim.y * kThreads) {
    store16(k_pool + sb + 16 * c, load16(k_pool + sa + 16 * c));
    store16(v_pool + sb + 16 * c, load16(v_pool + sa + 16 * c));
  }
}

// Swap ([pofe] "When memory runs out": a preempted sequence's blocks are
// copied to CPU memory and back; [lesson] "Preemption": pinned host memory).
// blockIdx.x = list entry i, blockIdx.y = slice of the block's chunks.  The
// host buffers are pinned, device-mapped memory: the kernel reads or writes
// them directly over the host link, one 16-byte chunk per thread, so one
// launch moves any set of scattered blocks.
template <bool kToHost>
__global__ __launch_bounds__(kThreads) void swap_kernel(
    char* __restrict__ k_pool, char* __restrict__ v_pool, char* __restrict__ host_k,
    char* __restrict__ host_v, const int32_t* __restrict__ ids, int num_blocks,
    size_t block_bytes) {
  const int b = ids[blockIdx.x];
  if (!valid_block(b, num_blocks)) return;
  const size_t chunks = block_bytes / 16;
  const size_t pb = (size_t)b * block_bytes, hb = (size_t)blockIdx.x * block_bytes;
  for (size_t c = (size_t)blockIdx.y * kThreads + threadIdx.x; c < chunks;
       c += (size_t)gridDim.y * kThreads) {
    if constexpr (kToHost) {
      store16(host_k + hb + 16 * c, load16(k_pool + pb + 16 * c));
      store16(host_v + hb + 16 * c, load16(v_pool + pb + 16 * c));
    } else {
      store16(k_pool + pb + 16 * c, load16(host_k + hb + 16 * c));
      store16(v_pool + pb + 16 * c, load16(host_v + hb + 16 * c));
    }
  }
}

constexpr int kGatherTokens = 16;

// blockIdx.y = sequence, blockIdx.x = group of kGatherTokens tokens.
__global__ __launch_bounds__(kThreads) void gather_kernel(
    char* __restrict__ k_out, char* __restrict__ v_out, const char* __restrict__ k_pool,
    const char* __restrict__ v_pool, const int32_t* __restrict__ tables, int max_blocks,
    const int32_t* __restrict__ lens, int num_blocks, int log2_b, int num_kv_heads, int head_dim,
    int elem_bytes, int max_len_out) {
  const int s = blockIdx.y;
  const int len = min(lens[s], max_len_out);
  const int t0 = blockIdx.x * kGatherTokens;
  if (t0 >= len) return;
  const size_t row_bytes = (size_t)num_kv_heads * head_dim * elem_bytes;
  const int row_chunks = (int)(row_bytes / 16);
  for (int i = threadIdx.x; i < kGatherTokens * row_chunks; i += kThreads) {
    const int t = t0 + i / row_chunks;
    const int c = i % row_chunks;
    if (t >= len) continue;
    const int lb = logical_block(t, log2_b);
    if (lb >= max_blocks) continue;
    const int blk = tables[(size_t)s * max_blocks + lb];
    if (!valid_block(blk, num_blocks)) continue;
    const size_t from = row_offset(blk, t, log2_b, num_kv_heads, 0, head_dim) * elem_bytes + 16 * (size_t)c;
    const size_t to = ((size_t)s * max_len_out + t) * row_bytes + 16 * (size_t)c;
    store16(k_out + to, load16(k_pool + from));
    store16(v_out + to, load16(v_pool + from));
  }
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" int paged_kv_append(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                               const int32_t* block_tables, int max_blocks_per_seq,
                               const int32_t* context_lens_pre, int num_seqs, int num_blocks,
                               int block_size, int num_kv_heads, int head_dim, int dtype,
                               void* stream) {
  int st = check_pool_shape(num_blocks, block_size, num_kv_heads, head_dim, dtype);
  if (st != PKV_OK) return st;
  if (num_seqs < 0 || max_blocks_per_seq < 1) return PKV_ERR_INVALID_ARG;
  if (num_seqs == 0) return PKV_OK;
  if (!k_pool || !v_pool || !k_new || !v_new || !block_tables || !context_lens_pre)
    return PKV_ERR_INVALID_ARG;
  hipLaunchKernelGGL(append_kernel, dim3(num_seqs), dim3(kThreads), 0, (hipStream_t)stream,
                     (char*)k_pool, (char*)v_pool, (const char*)k_new, (const char*)v_new,
                     block_tables, max_blocks_per_seq, context_lens_pre, num_blocks,
                     log2_exact(block_size), num_kv_heads, head_dim, dtype_bytes(dtype));
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

extern "C" int paged_kv_append_tokens(void* k_pool, void* v_pool, const void* k_new,
                                      const void* v_new, const int32_t* cu_seqlens,
                                      int num_tokens, const int32_t* block_tables,
                                      int max_blocks_per_seq, const int32_t* context_lens_pre,
                                      int num_seqs, int num_blocks, int block_size,
                                      int num_kv_heads, int head_dim, int dtype, void* stream) {
  int st = check_pool_shape(num_blocks, block_size, num_kv_heads, head_dim, dtype);
  if (st != PKV_OK) return st;
  if (num_seqs < 0 || num_tokens < 0 || max_blocks_per_seq < 1) return PKV_ERR_INVALID_ARG;
  if (num_seqs == 0 || num_tokens == 0) return PKV_OK;
  if (!k_pool || !v_pool || !k_new || !v_new || !cu_seqlens || !block_tables ||
      !context_lens_pre)
    return PKV_ERR_INVALID_ARG;
  const long long row_chunks = (long long)num_kv_heads * head_dim * dtype_bytes(dtype) / 16;
  const long long blocks = (num_tokens * row_chunks + kThreads - 1) / kThreads;
  if (blocks > 0x7fffffffLL) return PKV_ERR_INVALID_ARG;
  hipLaunchKernelGGL(append_tokens_kernel, dim3((unsigned)blocks), dim3(kThreads), 0,
                     (hipStream_t)stream, (char*)k_pool, (char*)v_pool, (const char*)k_new,
                     (const char*)v_new, cu_seqlens, num_tokens, block_tables,
                     max_blocks_per_seq, context_lens_pre, num_seqs, num_blocks,
                     log2_exact(block_size), num_kv_heads, head_dim, dtype_bytes(dtype));
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

namespace {

// paged_kv_append_fp8 with per-pool scales (k_scales == v_scales == null) or
// per-head ones.
int append_fp8_impl(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                    const int32_t* block_tables, int max_blocks_per_seq,
                    const int32_t* context_lens_pre, int num_seqs, int num_blocks, int block_size,
                    int num_kv_heads, int head_dim, int new_dtype, float k_scale, float v_scale,
                    const float* k_scales, const float* v_scales, void* stream) {
  int st = check_pool_shape(num_blocks, block_size, num_kv_heads, head_dim, PKV_FP8_E4M3);
  if (st != PKV_OK) return st;
  if (!supported_dtype(new_dtype)) return PKV_ERR_UNSUPPORTED;
  if (!(k_scale > 0.f) || !(v_scale > 0.f) || k_scale == INFINITY || v_scale == INFINITY)
    return PKV_ERR_INVALID_ARG;
  if (num_seqs < 0 || max_blocks_per_seq < 1) return PKV_ERR_INVALID_ARG;
  if (num_seqs == 0) return PKV_OK;
  if (!k_pool || !v_pool || !k_new || !v_new || !block_tables || !context_lens_pre)
    return PKV_ERR_INVALID_ARG;
  const int log2_b = log2_exact(block_size);
  auto launch = [&](auto tag) {
    using T = decltype(tag);
    hipLaunchKernelGGL(append_fp8_kernel<T>, dim3(num_seqs), dim3(kThreads), 0,
                       (hipStream_t)stream, (uint8_t*)k_pool, (uint8_t*)v_pool,
                       (const char*)k_new, (const char*)v_new, block_tables, max_blocks_per_seq,
                       context_lens_pre, num_blocks, log2_b, num_kv_heads, head_dim, k_scale,
                       v_scale, k_scales, v_scales);
  };
  if (new_dtype == PKV_F32) launch(F32{});
  else if (new_dtype == PKV_F16) launch(F16{});
  else launch(BF16{});
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

}  // namespace

extern "C" int paged_kv_append_fp8(void* k_pool, void* v_pool, const void* k_new,
                                   const void* v_new, const int32_t* block_tables,
                                   int max_blocks_per_seq, const int32_t* context_lens_pre,
                                   int num_seqs, int num_blocks, int block_size, int num_kv_heads,
                                   int head_dim, int new_dtype, float k_scale, float v_scale,
                                   void* stream) {
  return append_fp8_impl(k_pool, v_pool, k_new, v_new, block_tables, max_blocks_per_seq,
                         context_lens_pre, num_seqs, num_blocks, block_size, num_kv_heads,
                         head_dim, new_dtype, k_scale, v_scale, nullptr, nullptr, stream);
}

extern "C" int paged_kv_append_fp8_per_head(void* k_pool, void* v_pool, const void* k_new,
                                            const void* v_new, const int32_t* block_tables,
                                            int max_blocks_per_seq,
                                            const int32_t* context_lens_pre, int num_seqs,
                                            int num_blocks, int block_size, int num_kv_heads,
                                            int head_dim, int new_dtype, const float* k_scales,
                                            const float* v_scales, void* stream) {
  if (num_seqs > 0 && (!k_scales || !v_scales)) return PKV_ERR_INVALID_ARG;
  return append_fp8_impl(k_pool, v_pool, k_new, v_new, block_tables, max_blocks_per_seq,
                         context_lens_pre, num_seqs, num_blocks, block_size, num_kv_heads,
                         head_dim, new_dtype, 1.f, 1.f, k_scales, v_scales, stream);
}

extern "C" int paged_kv_append_tokens_fp8(void* k_pool, void* v_pool, const void* k_new,
                                          const void* v_new, const int32_t* cu_seqlens,
                                          int num_tokens, const int32_t* block_tables,
                                          int max_blocks_per_seq,
                                          const int32_t* context_lens_pre, int num_seqs,
                                          int num_blocks, int block_size, int num_kv_heads,
                                          int head_dim, int new_dtype, float k_scale,
                                          float v_scale, void* stream) {
  int st = check_pool_shape(num_blocks, block_size, num_kv_heads, head_dim, PKV_FP8_E4M3);
  if (st != PKV_OK) return st;
  if (!supported_dtype(new_dtype)) return PKV_ERR_UNSUPPORTED;
  if (!(k_scale > 0.f) || !(v_scale > 0.f) || k_scale == INFINITY || v_scale == INFINITY)
    return PKV_ERR_INVALID_ARG;
  if (num_seqs < 0 || num_tokens < 0 || max_blocks_per_seq < 1) return PKV_ERR_INVALID_ARG;
  if (num_seqs == 0 || num_tokens == 0) return PKV_OK;
  if (!k_pool || !v_pool || !k_new || !v_new || !cu_seqlens || !block_tables ||
      !context_lens_pre)
    return PKV_ERR_INVALID_ARG;
  const long long row_chunks = (long long)num_kv_heads * head_dim / 8;
  const long long blocks = (num_tokens * row_chunks + kThreads - 1) / kThreads;
  if (blocks > 0x7fffffffLL) return PKV_ERR_INVALID_ARG;
  const int log2_b = log2_exact(block_size);
  auto launch = [&](auto tag) {
    using T = decltype(tag);
    hipLaunchKernelGGL(append_tokens_fp8_kernel<T>, dim3((unsigned)blocks), dim3(kThreads), 0,
                       (hipStream_t)stream, (uint8_t*)k_pool, (uint8_t*)v_pool,
                       (const char*)k_new, (const char*)v_new, cu_seqlens, num_tokens,
                       block_tables, max_blocks_per_seq, context_lens_pre, num_seqs, num_blocks,
                       log2_b, num_kv_heads, head_dim, k_scale, v_scale);
  };
  if (new_dtype == PKV_F32) launch(F32{});
  else if (new_dtype == PKV_F16) launch(F16{});
  else launch(BF16{});
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

extern "C" int paged_kv_copy_blocks(void* k_pool, void* v_pool, const int32_t* src,
                                    const int32_t* dst, int num_pairs, int num_blocks,
                                    int block_size, int num_kv_heads, int head_dim, int dtype,
                                    void* stream) {
  int st = check_pool_shape(num_blocks, block_size, num_kv_heads, head_dim, dtype);
  if (st != PKV_OK) return st;
  if (num_pairs < 0) return PKV_ERR_INVALID_ARG;
  if (num_pairs == 0) return PKV_OK;
  if (!k_pool || !v_pool || !src || !dst) return PKV_ERR_INVALID_ARG;
  const size_t block_bytes = (size_t)block_size * num_kv_heads * head_dim * dtype_bytes(dtype);
  const size_t chunks = block_bytes / 16;
  const int slices = (int)std::min<size_t>(16, (chunks + kThreads - 1) / kThreads);
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(num_pairs, slices), dim3(kThreads), 0,
                     (hipStream_t)stream, (char*)k_pool, (char*)v_pool, src, dst, num_blocks,
                     block_bytes);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

static int swap_blocks(bool to_host, void* k_pool, void* v_pool, void* host_k, void* host_v,
                       const int32_t* block_ids, int num, int num_blocks, int block_size,
                       int num_kv_heads, int head_dim, int dtype, void* stream) {
  int st = check_pool_shape(num_blocks, block_size, num_kv_heads, head_dim, dtype);
  if (st != PKV_OK) return st;
  if (num < 0 || num > 0x7fffffff / 2) return PKV_ERR_INVALID_ARG;
  if (num == 0) return PKV_OK;
  if (!k_pool || !v_pool || !host_k || !host_v || !block_ids) return PKV_ERR_INVALID_ARG;
  const size_t block_bytes = (size_t)block_size * num_kv_heads * head_dim * dtype_bytes(dtype);
  const size_t chunks = block_bytes / 16;
  const int slices = (int)std::min<size_t>(16, (chunks + kThreads - 1) / kThreads);
  if (to_host)
    hipLaunchKernelGGL(swap_kernel<true>, dim3(num, slices), dim3(kThreads), 0,
                       (hipStream_t)stream, (char*)k_pool, (char*)v_pool, (char*)host_k,
                       (char*)host_v, block_ids, num_blocks, block_bytes);
  else
    hipLaunchKernelGGL(swap_kernel<false>, dim3(num, slices), dim3(kThreads), 0,
                       (hipStream_t)stream, (char*)k_pool, (char*)v_pool, (char*)host_k,
                       (char*)host_v, block_ids, num_blocks, block_bytes);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

extern "C" int paged_kv_swap_out(const void* k_pool, const void* v_pool,
                                 const int32_t* block_ids, int num, void* host_k, void* host_v,
                                 int num_blocks, int block_size, int num_kv_heads, int head_dim,
                                 int dtype, void* stream) {
  return swap_blocks(true, (void*)k_pool, (void*)v_pool, host_k, host_v, block_ids, num,
                     num_blocks, block_size, num_kv_heads, head_dim, dtype, stream);
}

extern "C" int paged_kv_swap_in(void* k_pool, void* v_pool, const int32_t* block_ids, int num,
                                const void* host_k, const void* host_v, int num_blocks,
                                int block_size, int num_kv_heads, int head_dim, int dtype,
                                void* stream) {
  return swap_blocks(false, k_pool, v_pool, (void*)host_k, (void*)host_v, block_ids, num,
                     num_blocks, block_size, num_kv_heads, head_dim, dtype, stream);
}

extern "C" int paged_kv_gather(void* k_out, void* v_out, const void* k_pool, const void* v_pool,
                               const int32_t* block_tables, int max_blocks_per_seq,
                               const int32_t* context_lens, int num_seqs, int num_blocks,
                               int block_size, int num_kv_heads, int head_dim, int max_len_out,
                               int dtype, void* stream) {
  int st = check_pool_shape(num_blocks, block_size, num_kv_heads, head_dim, dtype);
  if (st != PKV_OK) return st;
  if (num_seqs < 0 || num_seqs > 65535 || max_blocks_per_seq < 1 || max_len_out < 0)
    return PKV_ERR_INVALID_ARG;
  if (num_seqs == 0 || max_len_out == 0) return PKV_OK;
  if (!k_out || !v_out || !k_pool || !v_pool || !block_tables || !context_lens)
    return PKV_ERR_INVALID_ARG;
  const int groups = (max_len_out + kGatherTokens - 1) / kGatherTokens;
  hipLaunchKernelGGL(gather_kernel, dim3(groups, num_seqs), dim3(kThreads), 0,
                     (hipStream_t)stream, (char*)k_out, (char*)v_out, (const char*)k_pool,
                     (const char*)v_pool, block_tables, max_blocks_per_seq, context_lens,
                     num_blocks, log2_exact(block_size), num_kv_heads, head_dim,
                     dtype_bytes(dtype), max_len_out);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}
