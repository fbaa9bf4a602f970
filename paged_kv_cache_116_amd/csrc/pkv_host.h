// pkv_host.h - host-side argument checks shared by the libpagedkv entry points.
#pragma once

#include <algorithm>
#include <stddef.h>
#include <stdint.h>

#include "../../include/pagedkv.h"

namespace pkv {

inline bool supported_block_size(int b) {
  return b == 1 || b == 2 || b == 4 || b == 8 || b == 16 || b == 32 || b == 64 || b == 128;
}

inline bool supported_head_dim(int d) {
  return d == 16 || d == 32 || d == 64 || d == 128 || d == 256;
}

inline bool supported_dtype(int dt) { return dt == PKV_F32 || dt == PKV_F16 || dt == PKV_BF16; }
// Pools may also hold FP8 codes (byte moves and the FP8 entry points).
inline bool supported_pool_dtype(int dt) { return supported_dtype(dt) || dt == PKV_FP8_E4M3; }

// Shape checks every pool operation shares.  Sizes must be positive; block
// size, head size and dtype must be in the supported lists.
inline int check_pool_shape(int num_blocks, int block_size, int num_kv_heads, int head_dim,
                            int dtype) {
  if (num_blocks < 1 || num_kv_heads < 1 || block_size < 1 || head_dim < 1)
    return PKV_ERR_INVALID_ARG;
  if (!supported_block_size(block_size) || !supported_head_dim(head_dim) ||
      !supported_pool_dtype(dtype))
    return PKV_ERR_UNSUPPORTED;
  return PKV_OK;
}

// Defined in prefill_attention.hip; used by the cascade decode.
int launch_prefix_states(const void* q, const void* k_pool, const void* v_pool,
                         const int32_t* tables, const int32_t* lens, int max_blocks,
                         int num_seqs, int num_blocks, int block_size, int num_q_heads,
                         int num_kv_heads, int head_dim, float scale, const int32_t* offsets,
                         const int32_t* members, int num_members,
                         const int32_t* prefix_blocks, int num_groups, int max_group_size,
                         int splits, float* o_states, float* lse, int32_t* suf_tables,
                         int32_t* suf_lens, const int32_t* owners, int dtype, void* stream,
                         bool kv_fp8, float k_scale, float v_scale);

// Defined in decode_attention.hip; used by the cascade decode.  The first
// validates a decode call without launching anything (PKV_OK or an error),
// the second runs one with log normalisers (paged_decode_attention_lse with
// balanced claims); both over 16-bit or FP8 pools.
int decode_attention_check(int kernel, void* out, const void* q, const void* k_pool,
                           const void* v_pool, const int32_t* block_tables,
                           int max_blocks_per_seq, const int32_t* context_lens, int num_seqs,
                           int num_blocks, int block_size, int num_q_heads, int num_kv_heads,
                           int head_dim, float scale, void* workspace, size_t workspace_bytes,
                           int dtype, bool kv_fp8, float k_scale, float v_scale);
int decode_attention_with_lse(int kernel, void* out, float* lse, const void* q,
                              const void* k_pool, const void* v_pool,
                              const int32_t* block_tables, int max_blocks_per_seq,
                              const int32_t* context_lens, int num_seqs, int num_blocks,
                              int block_size, int num_q_heads, int num_kv_heads, int head_dim,
                              float scale, void* workspace, size_t workspace_bytes, int dtype,
                              void* stream, bool kv_fp8, float k_scale, float v_scale);

}  // namespace pkv
