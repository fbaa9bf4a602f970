// cascade.hip - decode attention over groups of sequences that share a
// prompt prefix (gfx950).
//
// Sources cited by tag and section:
//   [lesson] "PagedAttention" lesson in "How Text Is Generated"
//   [arch]   "PagedAttention: Virtual-Memory KV Cache Management, Continuous
//            Batching, and PyTorch Architecture"
//
// Sequences with a common prompt prefix share its blocks ([lesson] "Sharing,
// and the reference counting it needs").  Plain decode attention reads those
// blocks once per sequence; here each group's prefix is read once for all of
// its members, and the per-part results are merged the way [arch] "3.
// Non-Contiguous Online Softmax Attention Kernel" merges partial states, with
// each part already normalised and carrying its log normaliser.
#include <math.h>

#include <algorithm>

#include "pkv_common.h"
#include "pkv_host.h"

namespace pkv {
namespace {

constexpr int kThreads = 256;
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// ---------------------------------------------------------------------------
// Cascade decode over shared prefixes ([lesson] "Sharing, and the reference
// counting it needs": sequences with a common prompt prefix share its
// blocks).  Each group's shared prefix is read once for all its members
// (attn_prefill_mfma in prefix mode, its tiles split into key ranges), each
// sequence's private suffix by the decode path above, and the normalised
// results are combined with their log normalisers:
//     O = sum_r e^(a_r - M) O_r / sum_r e^(a_r - M),
// over the prefix ranges and the suffix, a_r their natural log normalisers
// and M = max_r a_r.
// ---------------------------------------------------------------------------

// Key ranges a prefix may be split into: at most one per 128 table tokens
// and at most kMaxPrefixSplits (the workspace holds that many states).
constexpr int kMaxPrefixSplits = 8;
int prefix_split_cap(int max_blocks, int block_size) {
  const long long tokens = (long long)max_blocks * block_size;
  return (int)std::max<long long>(1, std::min<long long>(kMaxPrefixSplits, (tokens + 127) / 128));
}

// Suffix tables start as copies of the tables (sequences outside every group
// keep their whole history); the prefix kernel then rewrites the members'.
// The membership counts start at zero.
__global__ __launch_bounds__(kThreads) void cascade_tables(const int32_t* __restrict__ tables,
                                                           const int32_t* __restrict__ lens,
                                                           int mb, int32_t* __restrict__ suf_tables,
                                                           int32_t* __restrict__ suf_lens,
                                                           int32_t* __restrict__ owners) {
  const size_t row = (size_t)blockIdx.x * mb;
  for (int j = threadIdx.x; j < mb; j += kThreads) suf_tables[row + j] = tables[row + j];
  if (threadIdx.x == 0) {
    suf_lens[blockIdx.x] = lens[blockIdx.x];
    owners[blockIdx.x] = 0;
  }
}

// Workgroup z counts the groups each member of group z belongs to.  Only a
// group whose offsets lie in [0, num_members] and do not decrease counts, and
// only its member ids in [0, num_seqs); the prefix kernel skips the rest.
__global__ __launch_bounds__(kThreads) void cascade_count(const int32_t* __restrict__ offsets,
                                                          const int32_t* __restrict__ members,
                                                          int num_members, int num_seqs,
                                                          int32_t* __restrict__ owners) {
  const int lo = offsets[blockIdx.x];
  const int hi = offsets[blockIdx.x + 1];
  if (lo < 0 || hi < lo || hi > num_members) return;
  for (int m = lo + (int)threadIdx.x; m < hi; m += kThreads) {
    const int s = members[m];
    if (s >= 0 && s < num_seqs) atomicAdd(&owners[s], 1);
  }
}

// out[s] = combination of the prefix states of `splits` key ranges (o_pre,
// lse_pre, range r at offset r * state_stride rows) and the suffix output
// already in out[s] (lse_suf), for every member s; workgroup (z, y) takes
// the members offsets[z] + y, + gridDim.y, ...; 8 channels per thread.  An
// empty part (log normaliser -inf) weighs 0; NaN propagates.
template <typename T>
__global__ __launch_bounds__(kThreads) void cascade_combine(
    void* __restrict__ out, const float* __restrict__ o_pre, const float* __restrict__ lse_pre,
    const float* __restrict__ lse_suf, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ members, int num_members, int num_seqs, int num_q_heads,
    int head_dim, int splits, size_t state_stride) {
  using S = typename T::storage;
  const int z = blockIdx.x;
  const int row = num_q_heads * head_dim;
  // The group and member checks of cascade_count: a group outside
  // [0, num_members] and member ids outside [0, num_seqs) are skipped.
  const int lo = offsets[z];
  const int hi = offsets[z + 1];
  if (lo < 0 || hi < lo || hi > num_members) return;
  for (int m = lo + (int)blockIdx.y; m < hi; m += gridDim.y) {
    const int s = members[m];
    if (s < 0 || s >= num_seqs) continue;
    S* o = (S*)out + (size_t)s * row;
    for (int c = threadIdx.x; c < row / 8; c += kThreads) {
      const int h = (8 * c) / head_dim;
      const size_t sh = (size_t)s * num_q_heads + h;
      // Every load first (they are independent), then the weights: a range
      // with log normaliser -inf (empty) holds zeros and weighs 0.
      float a[kMaxPrefixSplits];
      float4 x0[kMaxPrefixSplits], x1[kMaxPrefixSplits];
      const size_t d0 = (size_t)(8 * c) % head_dim;
#pragma unroll
      for (int r = 0; r < kMaxPrefixSplits; ++r) {
        const bool use = r < splits;
        const float* pre = o_pre + (r * state_stride + sh) * head_dim + d0;
        a[r] = use ? lse_pre[r * state_stride + sh] : -INFINITY;
        x0[r] = use ? *reinterpret_cast<const float4*>(pre) : make_float4(0.f, 0.f, 0.f, 0.f);
        x1[r] = use ? *reinterpret_cast<const float4*>(pre + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
      }
      const float b = lse_suf[sh];
      float suf[8];
      Cvt<T>::unpack(load16(o + 8 * c), suf);
      bool nan_in = b != b;
      float mx = b;
#pragma unroll
      for (int r = 0; r < kMaxPrefixSplits; ++r) {
        nan_in |= a[r] != a[r];
        mx = fmaxf(mx, a[r]);
      }
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = 0.f;
      float den = 0.f;
      if (mx != -INFINITY) {
        // A part with weight 0 adds nothing (not 0 * its value, which could be NaN).
#pragma unroll
        for (int r = 0; r < kMaxPrefixSplits; ++r) {
          const float wa = a[r] == -INFINITY ? 0.f : expf(a[r] - mx);
          if (wa > 0.f) {
            v[0] += wa * x0[r].x; v[1] += wa * x0[r].y; v[2] += wa * x0[r].z; v[3] += wa * x0[r].w;
            v[4] += wa * x1[r].x; v[5] += wa * x1[r].y; v[6] += wa * x1[r].z; v[7] += wa * x1[r].w;
          }
          den += wa;
        }
        if (b != -INFINITY) {
          const float wb = expf(b - mx);
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] += wb * suf[e];
          den += wb;
        }
      }
      const float inv = den > 0.f ? 1.f / den : 0.f;
      const float nan = __builtin_nanf("");
#pragma unroll
      for (int e = 0; e < 8; e += 4)
        Cvt<T>::store4(o + 8 * c + e, nan_in ? nan : v[e] * inv, nan_in ? nan : v[e + 1] * inv,
                       nan_in ? nan : v[e + 2] * inv, nan_in ? nan : v[e + 3] * inv);
    }
  }
}

// Workspace of the cascade: suffix tables and lengths, membership counts,
// prefix states of up to prefix_split_cap key ranges, the two log-normaliser
// arrays, then the decode workspace.
struct CascadeWs {
  size_t tables, lens, owners, o_pre, lse_pre, lse_suf, decode, total;
};
CascadeWs cascade_layout(int num_seqs, int num_q_heads, int head_dim, int max_blocks,
                         int block_size) {
  CascadeWs w;
  const size_t S = (size_t)num_seqs;
  const size_t R = (size_t)prefix_split_cap(max_blocks, block_size);
  w.tables = 0;
  w.lens = w.tables + align256(S * max_blocks * 4);
  w.owners = w.lens + align256(S * 4);
  w.o_pre = w.owners + align256(S * 4);
  w.lse_pre = w.o_pre + align256(R * S * num_q_heads * head_dim * 4);
  w.lse_suf = w.lse_pre + align256(R * S * num_q_heads * 4);
  w.decode = w.lse_suf + align256(S * num_q_heads * 4);
  w.total = w.decode + align256(paged_decode_workspace_bytes(
                           num_seqs, num_q_heads, head_dim,
                           (int)std::min<long long>((long long)max_blocks * block_size, 1 << 30),
                           0));
  return w;
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" size_t paged_decode_cascade_workspace_bytes(int num_seqs, int num_q_heads,
                                                       int head_dim, int max_blocks_per_seq,
                                                       int block_size) {
  if (num_seqs < 0 || num_q_heads < 1 || head_dim < 1 || max_blocks_per_seq < 1 ||
      block_size < 1)
    return 0;
  return pkv::cascade_layout(num_seqs, num_q_heads, head_dim, max_blocks_per_seq, block_size)
      .total;
}

namespace pkv {
namespace {

// The cascade over 16-bit pools (kv_fp8 = false) or FP8 pools.
int cascade_impl(int kernel, void* out, const void* q, const void* k_pool, const void* v_pool,
                 const int32_t* block_tables, int max_blocks_per_seq,
                 const int32_t* context_lens, int num_seqs, const int32_t* group_offsets,
                 const int32_t* group_members, int num_members,
                 const int32_t* group_prefix_blocks, int num_groups, int max_group_size,
                 int num_blocks, int block_size,
                 int num_q_heads, int num_kv_heads, int head_dim, float scale, void* workspace,
                 size_t workspace_bytes, int dtype, void* stream, bool kv_fp8, float k_scale,
                 float v_scale) {
  if (dtype != PKV_F16 && dtype != PKV_BF16) return PKV_ERR_UNSUPPORTED;
  if (head_dim % 32 != 0 || !supported_head_dim(head_dim)) return PKV_ERR_UNSUPPORTED;
  if (num_groups < 0 || num_groups > 65535 || max_group_size < 0 || num_seqs < 0 ||
      num_members < 0)
    return PKV_ERR_INVALID_ARG;
  if (num_groups > 0 &&
      (!group_offsets || !group_prefix_blocks || (num_members > 0 && !group_members)))
    return PKV_ERR_INVALID_ARG;
  if (num_seqs == 0) return PKV_OK;
  if (max_blocks_per_seq < 1 || num_q_heads < 1 || num_kv_heads < 1 ||
      num_q_heads % num_kv_heads != 0 || num_kv_heads > 65535)
    return PKV_ERR_INVALID_ARG;
  const CascadeWs w =
      cascade_layout(num_seqs, num_q_heads, head_dim, max_blocks_per_seq, block_size);
  if (!workspace || workspace_bytes < w.total || ((uintptr_t)workspace & 255) != 0)
    return PKV_ERR_WORKSPACE;
  char* ws = (char*)workspace;
  int32_t* suf_tables = (int32_t*)(ws + w.tables);
  int32_t* suf_lens = (int32_t*)(ws + w.lens);
  int32_t* owners = (int32_t*)(ws + w.owners);
  float* o_pre = (float*)(ws + w.o_pre);
  float* lse_pre = (float*)(ws + w.lse_pre);
  float* lse_suf = (float*)(ws + w.lse_suf);
  // Validate the decode call on the suffix tables before launching anything.
  {
    const int st = decode_attention_check(kernel, out, q, k_pool, v_pool, suf_tables,
                                          max_blocks_per_seq, suf_lens, num_seqs, num_blocks,
                                          block_size, num_q_heads, num_kv_heads, head_dim, scale,
                                          ws + w.decode, workspace_bytes - w.decode, dtype,
                                          kv_fp8, k_scale, v_scale);
    if (st != PKV_OK) return st;
  }
  // No group (the export policy found none that pays): plain decode over the
  // tables as given, the same launches as paged_decode_attention_with.
  if (num_groups == 0)
    return decode_attention_with_lse(kernel, out, nullptr, q, k_pool, v_pool, block_tables,
                                     max_blocks_per_seq, context_lens, num_seqs, num_blocks,
                                     block_size, num_q_heads, num_kv_heads, head_dim, scale,
                                     ws + w.decode, workspace_bytes - w.decode, dtype, stream,
                                     kv_fp8, k_scale, v_scale);
  hipStream_t hs = (hipStream_t)stream;
  hipLaunchKernelGGL(cascade_tables, dim3(num_seqs), dim3(kThreads), 0, hs, block_tables,
                     context_lens, max_blocks_per_seq, suf_tables, suf_lens, owners);
  if (num_groups > 0)
    hipLaunchKernelGGL(cascade_count, dim3(num_groups), dim3(kThreads), 0, hs, group_offsets,
                       group_members, num_members, num_seqs, owners);
  // Key ranges per prefix: enough workgroups for about four per compute unit
  // (64-row blocks x KV heads x groups x ranges), within the workspace's cap.
  const long long base = std::max<long long>(
      1, ((long long)max_group_size * (num_q_heads / num_kv_heads) + 63) / 64 * num_kv_heads *
             num_groups);
  const int splits = (int)std::max<long long>(
      1, std::min<long long>(prefix_split_cap(max_blocks_per_seq, block_size),
                             (1024 + base - 1) / base));
  if (num_groups > 0) {
    const int st = launch_prefix_states(
        q, k_pool, v_pool, block_tables, context_lens, max_blocks_per_seq, num_seqs, num_blocks,
        block_size, num_q_heads, num_kv_heads, head_dim, scale, group_offsets, group_members,
        num_members, group_prefix_blocks, num_groups, max_group_size, splits, o_pre, lse_pre,
        suf_tables, suf_lens, owners, dtype, stream, kv_fp8, k_scale, v_scale);
    if (st != PKV_OK) return st;
  }
  int st = decode_attention_with_lse(kernel, out, lse_suf, q, k_pool, v_pool, suf_tables,
                                     max_blocks_per_seq, suf_lens, num_seqs, num_blocks,
                                     block_size, num_q_heads, num_kv_heads, head_dim, scale,
                                     ws + w.decode, workspace_bytes - w.decode, dtype, stream,
                                     kv_fp8, k_scale, v_scale);
  if (st != PKV_OK) return st;
  if (num_groups > 0) {
    // Any grid height covers every member (workgroups stride over them).
    const dim3 grid(num_groups, std::max(1, std::min(max_group_size, 65535)));
    const size_t stride = (size_t)num_seqs * num_q_heads;
    if (dtype == PKV_F16)
      hipLaunchKernelGGL(cascade_combine<F16>, grid, dim3(kThreads), 0, hs, out, o_pre, lse_pre,
                         lse_suf, group_offsets, group_members, num_members, num_seqs,
                         num_q_heads, head_dim, splits, stride);
    else
      hipLaunchKernelGGL(cascade_combine<BF16>, grid, dim3(kThreads), 0, hs, out, o_pre, lse_pre,
                         lse_suf, group_offsets, group_members, num_members, num_seqs,
                         num_q_heads, head_dim, splits, stride);
  }
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

}  // namespace
}  // namespace pkv

extern "C" int paged_decode_attention_cascade(
    int kernel, void* out, const void* q, const void* k_pool, const void* v_pool,
    const int32_t* block_tables, int max_blocks_per_seq, const int32_t* context_lens,
    int num_seqs, const int32_t* group_offsets, const int32_t* group_members, int num_members,
    const int32_t* group_prefix_blocks, int num_groups, int max_group_size, int num_blocks,
    int block_size, int num_q_heads, int num_kv_heads, int head_dim, float scale,
    void* workspace, size_t workspace_bytes, int dtype, void* stream) {
  return pkv::cascade_impl(kernel, out, q, k_pool, v_pool, block_tables, max_blocks_per_seq,
                           context_lens, num_seqs, group_offsets, group_members, num_members,
                           group_prefix_blocks, num_groups, max_group_size, num_blocks,
                           block_size, num_q_heads, num_kv_heads, head_dim, scale, workspace,
                           workspace_bytes, dtype, stream, false, 1.f, 1.f);
}

extern "C" int paged_decode_attention_cascade_fp8(
    int kernel, void* out, const void* q, const void* k_pool, const void* v_pool,
    const int32_t* block_tables, int max_blocks_per_seq, const int32_t* context_lens,
    int num_seqs, const int32_t* group_offsets, const int32_t* group_members, int num_members,
    const int32_t* group_prefix_blocks, int num_groups, int max_group_size, int num_blocks,
    int block_size, int num_q_heads, int num_kv_heads, int head_dim, float scale, float k_scale,
    float v_scale, void* workspace, size_t workspace_bytes, int dtype, void* stream) {
  return pkv::cascade_impl(kernel, out, q, k_pool, v_pool, block_tables, max_blocks_per_seq,
                           context_lens, num_seqs, group_offsets, group_members, num_members,
                           group_prefix_blocks, num_groups, max_group_size, num_blocks,
                           block_size, num_q_heads, num_kv_heads, head_dim, scale, workspace,
                           workspace_bytes, dtype, stream, true, k_scale, v_scale);
}
