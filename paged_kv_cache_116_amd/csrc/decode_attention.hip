// decode_attention.hip - paged decode attention for gfx950 (MI355X).
//
// Sources cited by tag and section:
//   [pofe] "PagedAttention: paging the KV cache"
//   [arch] "PagedAttention: Virtual-Memory KV Cache Management, Continuous
//          Batching, and PyTorch Architecture"
//
// What is computed ([pofe] "How it works": ordinary attention regrouped by
// block, addresses indirect; [arch] "3. Non-Contiguous Online Softmax Attention
// Kernel"): for sequence s, query head h, KV head h / g,
//     out[s,h] = sum_{t<L} softmax_t(scale * q . K[t]) V[t]
// with K[t], V[t] fetched through the block table, and a running maximum m,
// normaliser l and unnormalised accumulator o updated tile by tile.
//
// Work decomposition: three launches.
//   attn_plan (16 workgroups): counts each live sequence's 16-token tiles,
//     prefix-sums them, and cuts the flattened space
//         (quad of kw KV-head groups, sequence, tile)
//     into claims: stage 0 gives each resident workgroup one claim of half
//     its share, each later stage halves the claim size down to a few tiles
//     per wave.  It writes a descriptor per claim (where it starts, its
//     size, the first sequence's tile count and length, its successor and
//     the claim count), the lists of split sequences for the merge, and
//     fills the rows of empty sequences.
//   attn_partition_* (persistent workgroups, 4 waves each): workgroup b takes
//     claim b of stage 0 and claim b of stage 1, then the next unclaimed one
//     from an atomic counter, so compute units that stream faster take more
//     of the small late claims and all of them finish together.  Each
//     stretch of one sequence inside a claim is a segment.  With kw = 1 the
//     four waves take the segment's tiles in turn and combine their
//     online-softmax states in LDS at its end; with kw = 4
//     each wave serves its own KV-head group over the same tiles.  A segment
//     that is the whole sequence writes the final output; otherwise it writes
//     a partial state (m, l, o) in a slot named by (claim + sequence slot).
//   attn_merge: combines the partial states of each split sequence with the
//     log-sum-exp rule
//         O = sum_p e^(m_p - M) o_p / sum_p e^(m_p - M) l_p.
//   The pages stop at the per-block recurrence; the split, the claims and
//   the merge are this library's addition, to keep all 256 compute units
//   busy to the end whatever the length mix.
//
// Cache policy: by default every block is read once per call, and K/V are
// streamed with non-temporal loads (kw = 1).  When the caller says blocks
// are shared between sequences (PKV_ATTN_CACHE_KV) the loads keep K/V in
// cache and kw = 4 makes a workgroup's rows adjacent.
//
// Two partition kernels:
//   attn_partition_mfma  (fp16 / bf16, D >= 32): the grouped score tile
//     S^T[16 tokens x 16 heads] = K_tile . Q^T is one chain of D/32
//     v_mfma_f32_16x16x32 ops.  K and V rows are loaded whole (every load
//     instruction covers complete rows); K goes through a per-wave swizzled
//     LDS tile to reach the MFMA operand layout (lane: row l % 16, channels
//     8 * (l / 16) .. +7 of each 32-channel chunk).  P.V is O^T = V^T . P^T,
//     D/16 v_mfma_f32_16x16x16 ops per tile: a lane's four probabilities
//     (four tokens of one head, straight from the score tile) are its B
//     operand, and V goes through a per-wave LDS tile read back with
//     transposing reads (ds_read_b64_tr_b16) as the A operand.  Each lane
//     then holds channels of its own head, so the rescale is lane-local.
//     Block ids come through scalar loads, one tile at a time.
//   attn_partition_valu  (any dtype incl. fp32): one token row per group of
//     D*sizeof/16 lanes, dot products reduced across the group with shuffles,
//     a separate online-softmax stream per lane group, merged at the end.
//
// Lazy rescale: a wave keeps its running maximum m until a tile's maximum
// exceeds m by more than kRescaleThreshold (log2 units), so probabilities are
// at most 2^8 and the accumulator is rescaled only when the maximum really
// moves.  Numerator and denominator share m, so the result is the same
// softmax; only the rescale count changes.
#include <math.h>

#include <mutex>
#include <type_traits>
#include <utility>
#include <unordered_map>

#include "pkv_common.h"
#include "pkv_host.h"
#include "pkv_mfma.h"

namespace pkv {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 16;
constexpr float kRescaleThreshold = 8.0f;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kMaxGD = 1024;    // G * D bound: the cross-wave LDS buffer is 16 KiB
constexpr int kMaxGroup = 8;    // query heads per workgroup (larger groups are split)
constexpr int kMaxWgPerCu = 8;  // 2048 threads per CU / 256
constexpr int kClaimsPerCu = 16;    // claim descriptors per compute unit
constexpr int kMinClaimWaveTiles = 6;  // smallest claim: tiles per wave
constexpr int kMaxStages = 16;      // claim-size stages (sizes halve stage to stage)
constexpr int kMergeBlock = 8;      // partial states one merge item combines
constexpr int kMergeWaves = 8;      // waves per merge workgroup
constexpr int kMergeThreads = 64 * kMergeWaves;
constexpr int kPlanThreads = 1024;
constexpr int kPlanLdsCum = 8192;   // prefix sums kept in LDS up to this many sequences
constexpr int kDescWords = 8;       // words per claim descriptor
// The claim walk reads descriptor blockIdx.x before it knows the claim count:
// the partition grid (at most kMaxWgPerCu per CU) never exceeds the
// descriptor slots (at least kClaimsPerCu per CU).
static_assert(kMaxWgPerCu <= kClaimsPerCu, "first descriptor inside the descriptor area");

// Plan area (int32 words): header | cum[S + 1] | desc[range_cap][8] |
// short tasks[kvq * S][4] | long tasks[kvq * S][4]; plan workgroup b writes
// its tasks from entry b * task_seg of each list.
// Header: the claim counter and each plan workgroup's task counts; the claim
// schedule itself lives in the descriptors.
constexpr int kPlanGroups = 16;     // workgroups of the plan launch that plan
constexpr int kAppendGroups = 16;   // further workgroups that do the decode-step append
constexpr int kHdrWords = 128;
enum Hdr {
  kHdrNext = 4,     // claim counter
  kHdrShort = 64,   // per plan workgroup: split pairs of at most kMergeBlock partials
  kHdrLong = 64 + kPlanGroups,   // per plan workgroup: split pairs of more partials
};
static_assert(kHdrLong + kPlanGroups <= kHdrWords, "header");

typedef const __attribute__((address_space(4))) int32_t cint;   // read with scalar loads

struct AttnParams {
  void* out;
  const void* q;
  const char* k_pool;
  const char* v_pool;
  const int32_t* tables;
  const int32_t* lens;
  const char* k_new;  // decode step: token L-1 of each sequence, written by the plan
  const char* v_new;  // (null: attention only)
  int32_t* plan;     // header, cum, desc, task
  float* ws_m;       // [pairs][G]
  float* ws_l;       // [pairs][G]
  float* ws_acc;     // [pairs][G][D]
  int num_seqs;
  int max_blocks;
  int num_blocks;
  int log2_b;
  int num_q_heads;
  int num_kv_heads;
  int head_dim;
  int group;        // g = Hq / Hkv
  int gsize;        // G: query heads per KV-head group
  int head_groups;  // ceil(g / G)
  int kvg_count;    // Hkv * head_groups: KV-head groups of G query heads
  int kw;           // KV-head groups a workgroup takes together (1, 2 or 4)
  int wpk;          // waves per KV-head group: kWaves / kw
  int kvq_count;    // ceil(kvg_count / kw): "quads" of kw groups
  int cap_tiles;    // 0 = no cap, else at most this many tiles per claim
  int grid;         // workgroups of the partition and merge launches
  int range_cap;    // claim descriptor slots
  int off_desc;     // plan-area word offsets of the claim descriptors
  int off_short;    // and of the merge task lists
  int off_long;
  int task_seg;     // task-list entries per plan workgroup
  float scale_log2;  // scale * log2(e) (* k_scale for FP8 pools): scores in log2 units
  int kv_fp8;        // pools hold E4M3FN codes
  float k_scale;     // FP8 pools: value = code * scale (the decode-step append divides)
  float v_scale;     // multiplies the weighted V sum (1 unless FP8)
  // FP8 pools with one scale per KV head: [num_kv_heads] each (device), in
  // place of k_scale / v_scale (both 1 then); nullptr for per-pool scales.
  const float* k_scales;
  const float* v_scales;
  float* lse;        // optional [S, Hq]: natural log of each head's softmax normaliser
};

// A sequence is live when 0 < L <= max_blocks * B; it then has ceil(L/16) tiles.
__device__ __forceinline__ int live_tiles(int L, int max_len) {
  return (L > 0 && L <= max_len) ? (L + kTile - 1) / kTile : 0;
}

// ---------------------------------------------------------------------------
// Plan: kPlanGroups workgroups.  Each one prefix-sums the tile counts and
// builds the claim schedule for itself (a few microseconds of LDS work), then
// writes its share of the claim descriptors, merge tasks and empty-row fills.
// A decode step adds kAppendGroups workgroups that write the new tokens.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kPlanThreads) void attn_plan(const AttnParams p) {
  using S = typename T::storage;
  __shared__ int carry_lds;
  __shared__ int dead_count;
  __shared__ int dead_list[kPlanThreads];
  __shared__ int wave_sum[kPlanThreads / 64];
  __shared__ int cum_lds[kPlanLdsCum + 1];
  __shared__ int st_x[kMaxStages + 1], st_c[kMaxStages + 1], st_z[kMaxStages + 1];
  __shared__ int n_stages, n_claims, n_short, n_long;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int b = blockIdx.x;
  const int S_ = p.num_seqs;
  const int max_len = p.max_blocks << p.log2_b;
  const size_t row_elems = (size_t)p.num_q_heads * p.head_dim;
  // Past kPlanLdsCum sequences the prefix sums live in memory only (every
  // workgroup writes the same values and reads back its own).
  const bool in_lds = S_ <= kPlanLdsCum;
  int32_t* cum = p.plan + kHdrWords;

  // Decode step: append token L-1 of every sequence with 0 < L <= max_len
  // (the cache append of [pofe] "How it works"), one 16-byte chunk per
  // thread, spread over kAppendGroups workgroups of their own, so that it
  // runs beside the planning rather than ahead of it.  The partition launch
  // that follows on the stream reads it from the pool.
  if (b >= kPlanGroups) {
    const int ab = b - kPlanGroups;
    // One 16-byte chunk of the new row (16 / sizeof(T) elements) per thread;
    // FP8 pools get its codes, encode(x / scale), as in paged_kv_append_fp8.
    constexpr int E = 16 / T::bytes;
    const int row_chunks = p.num_kv_heads * p.head_dim / E;
    for (long long i = (long long)ab * kPlanThreads + tid; i < (long long)S_ * row_chunks;
         i += kAppendGroups * kPlanThreads) {
      const int s = (int)(i / row_chunks);
      const int ch = (int)(i - (long long)s * row_chunks);
      const int L = p.lens[s];
      if (L <= 0 || L > max_len) continue;
      const int blk = p.tables[(size_t)s * p.max_blocks + ((L - 1) >> p.log2_b)];
      if (!valid_block(blk, p.num_blocks)) continue;
      const size_t elem = row_offset(blk, L - 1, p.log2_b, p.num_kv_heads, 0, p.head_dim) +
                          (size_t)E * ch;
      const size_t src = ((size_t)s * row_chunks + ch) * 16;
      if (p.kv_fp8) {
        if constexpr (E == 8) {
          float kf[8], vf[8];
          Cvt<T>::unpack(load16(p.k_new + src), kf);
          Cvt<T>::unpack(load16(p.v_new + src), vf);
          float ks = p.k_scale, vs = p.v_scale;
          if (p.k_scales) {   // the chunk's KV head (chunks never straddle heads)
            const int hh = E * ch / p.head_dim;
            ks = p.k_scales[hh];
            vs = p.v_scales[hh];
          }
          const bool k_ok = scale_ok(ks), v_ok = scale_ok(vs);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            kf[e] = k_ok ? kf[e] / ks : __builtin_nanf("");
            vf[e] = v_ok ? vf[e] / vs : __builtin_nanf("");
          }
          *reinterpret_cast<uint2*>((char*)p.k_pool + elem) =
              make_uint2(e4m3_encode4(kf[0], kf[1], kf[2], kf[3]),
                         e4m3_encode4(kf[4], kf[5], kf[6], kf[7]));
          *reinterpret_cast<uint2*>((char*)p.v_pool + elem) =
              make_uint2(e4m3_encode4(vf[0], vf[1], vf[2], vf[3]),
                         e4m3_encode4(vf[4], vf[5], vf[6], vf[7]));
        }
      } else {
        store16((char*)p.k_pool + elem * T::bytes, load16(p.k_new + src));
        store16((char*)p.v_pool + elem * T::bytes, load16(p.v_new + src));
      }
    }
    return;
  }

  // Exclusive prefix sum of tile counts, kPlanThreads sequences per pass.
  // Sequences with nothing to attend get their rows filled on the way, each
  // by workgroup s % kPlanGroups: zeros for L <= 0, NaN for a length the
  // table row cannot hold.
  if (tid == 0) carry_lds = 0;
  for (int base = 0; base < S_; base += kPlanThreads) {
    if (tid == 0) dead_count = 0;
    lds_barrier();
    const int s = base + tid;
    const int L = s < S_ ? p.lens[s] : 1;
    const int nt = s < S_ ? live_tiles(L, max_len) : 0;
    if (s < S_ && nt == 0 && s % kPlanGroups == b) dead_list[atomicAdd(&dead_count, 1)] = s;
    int incl = nt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o);
      if (lane >= o) incl += v;
    }
    if (lane == 63) wave_sum[wv] = incl;
    lds_barrier();
    int before = carry_lds;
    for (int i = 0; i < wv; ++i) before += wave_sum[i];
    const int excl = before + incl - nt;
    if (s < S_) {
      if (in_lds) cum_lds[s] = excl;
      else cum[s] = excl;
      if (in_lds && b == 0) cum[s] = excl;
    }
    const int ndead = dead_count;
    for (int k = 0; k < ndead; ++k) {
      const int sd = dead_list[k];
      const float fill = p.lens[sd] <= 0 ? 0.f : __builtin_nanf("");
      S* row = (S*)p.out + (size_t)sd * row_elems;
      for (size_t i = tid; i < row_elems; i += kPlanThreads) Cvt<T>::store(row + i, fill);
      if (p.lse) {   // nothing to attend: log 0; an over-long length: NaN
        const float lfill = p.lens[sd] <= 0 ? -INFINITY : __builtin_nanf("");
        for (int h = tid; h < p.num_q_heads; h += kPlanThreads)
          p.lse[(size_t)sd * p.num_q_heads + h] = lfill;
      }
    }
    lds_barrier();
    if (tid == kPlanThreads - 1) carry_lds = excl + nt;
    lds_barrier();
  }
  const int tot = carry_lds;
  if (tid == 0) {
    if (in_lds) cum_lds[S_] = tot;
    if (!in_lds || b == 0) cum[S_] = tot;
  }
  if (in_lds) lds_barrier(); else __syncthreads();
  auto cum_at = [&](int i) { return in_lds ? cum_lds[i] : cum[i]; };

  // Claim schedule.  Stage 0 hands every workgroup one claim of half its
  // share (5/8 of it for FP8 pools with grouped query heads, whose segments
  // carry half the bytes of 16-bit ones for the same fixed costs: measured
  // 2 % faster on the 70B-shaped batch and 7 % on the long-context one,
  // while the 16-bit and ungrouped FP8 workloads were slower with it); each
  // later stage halves the claim size, down to kMinClaimWaveTiles tiles per
  // wave; the final stage takes what is left.
  // A workgroup claims its next piece when it finishes one, so faster units
  // take more pieces and the last ones are short.  The descriptor budget
  // range_cap always leaves room for the rest at the cap size (when capped).
  // All counts stay below 2^31 (the host checks the tile total).
  const int total = tot * p.kvq_count;
  if (tid == 0) {
    const unsigned g = (unsigned)p.grid;
    const unsigned zmin = kMinClaimWaveTiles * p.wpk;
    const unsigned cap = (unsigned)p.cap_tiles;
    const unsigned budget_all = (unsigned)p.range_cap;
    const unsigned long long num = (p.kv_fp8 && p.gsize >= 2) ? 5 : 4;
    unsigned x = 0, c = 0,
             z = (unsigned)(((unsigned long long)total * num + 8ull * g - 1) / (8ull * g));
    int ns = 0;
    while (x < (unsigned)total) {
      const unsigned rem = (unsigned)total - x;
      unsigned zz = z > zmin ? z : zmin;
      if (cap > 0 && zz > cap) zz = cap;
      const unsigned count_all = rem / zz + (rem % zz != 0);
      bool final_stage = count_all <= g || zz <= zmin || ns == kMaxStages - 1;
      if (!final_stage) {
        const unsigned rest = rem - g * zz;
        const unsigned need_after = cap > 0 ? rest / cap + (rest % cap != 0) : 1;
        if (c + g + need_after > budget_all) final_stage = true;
      }
      unsigned count;
      if (final_stage) {
        const unsigned budget = budget_all - c;   // >= 1 by construction
        if (count_all > budget) zz = rem / budget + (rem % budget != 0);
        count = rem / zz + (rem % zz != 0);
      } else {
        count = g;
      }
      st_x[ns] = (int)x;
      st_c[ns] = (int)c;
      st_z[ns] = (int)zz;
      ++ns;
      c += count;
      x = final_stage ? (unsigned)total : x + g * zz;
      z = (z + 1) / 2;
    }
    st_x[ns] = total;
    st_c[ns] = (int)c;
    st_z[ns] = 0;
    n_stages = ns;
    n_claims = (int)c;
    n_short = 0;
    n_long = 0;
  }
  lds_barrier();
  const int ns = n_stages;
  const int C = n_claims;
  auto stage_of_claim = [&](int c) {
    int k = 0;
    while (k + 1 < ns && st_c[k + 1] <= c) ++k;
    return k;
  };
  auto claim_at = [&](int x) {
    int k = 0;
    while (k + 1 < ns && st_x[k + 1] <= x) ++k;
    return st_c[k] + (x - st_x[k]) / st_z[k];
  };

  // Claim descriptors, this workgroup's share: qd, sequence, first tile,
  // tiles; the first sequence's tile count and length; the successor; the
  // claim count.  With all a claim needs in one 32-byte load, a workgroup
  // reaches its first tiles after the descriptor and the block ids alone.
  // Stages 0 and 1 have one claim per workgroup, handed out by index
  // (successor c + grid); the counter serves stage 2 on, or the final stage
  // when there are fewer stages (successor -1 - c_dyn: ask the counter,
  // which numbers claims from c_dyn).
  const int c_dyn = max(ns > 2 ? st_c[2] : ns > 0 ? st_c[ns - 1] : 0, p.grid);
  auto successor = [&](int c) { return c + p.grid < c_dyn ? c + p.grid : -1 - c_dyn; };
  int32_t* desc = p.plan + p.off_desc;
  for (int c = b * kPlanThreads + tid; c < C; c += kPlanGroups * kPlanThreads) {
    const int k = stage_of_claim(c);
    const int x = st_x[k] + (c - st_c[k]) * st_z[k];
    const int size = min(st_z[k], st_x[k + 1] - x);
    const int qd = x / tot;
    const int rem = x - qd * tot;
    // Last sequence whose first tile is at or before rem (skips empty ones).
    int lo = 0, hi = S_;   // cum[lo] <= rem < cum[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (cum_at(mid) <= rem) lo = mid; else hi = mid;
    }
    *reinterpret_cast<int4*>(desc + kDescWords * c) = make_int4(qd, lo, rem - cum_at(lo), size);
    *reinterpret_cast<int4*>(desc + kDescWords * c + 4) =
        make_int4(cum_at(lo + 1) - cum_at(lo), p.lens[lo], successor(c), C);
  }
  // Workgroups past the last claim read an empty descriptor (no tiles, the
  // claim count as successor) and stop.
  for (int c = C + b * kPlanThreads + tid; c < p.grid; c += kPlanGroups * kPlanThreads) {
    *reinterpret_cast<int4*>(desc + kDescWords * c) = make_int4(0, 0, 0, 0);
    *reinterpret_cast<int4*>(desc + kDescWords * c + 4) = make_int4(0, 0, C, C);
  }

  // Merge tasks.  A (quad, sequence) pair whose tiles span claims c0 .. c1
  // with c0 < c1 is a task: its partial states sit in pairs c0 + t .. c1 + t
  // (t = quad * S + sequence).  Tasks of at most kMergeBlock partials go to
  // the short list (one wave each), longer ones to the long list (one
  // workgroup each).  This workgroup takes pairs [t_begin, t_end) and writes
  // its own segment of each list.
  const int pairs = p.kvq_count * S_;
  const int t_begin = b * p.task_seg;
  const int t_end = min(pairs, t_begin + p.task_seg);
  int32_t* short_list = p.plan + p.off_short + 4 * t_begin;
  int32_t* long_list = p.plan + p.off_long + 4 * t_begin;
  for (int t = t_begin + tid; t < t_end; t += kPlanThreads) {
    const int qd = t / S_;
    const int sq = t - qd * S_;
    const int c_a = cum_at(sq);
    const int c_b = cum_at(sq + 1);
    if (c_b == c_a) continue;   // empty: its rows were filled above
    const int c0 = claim_at(qd * tot + c_a);
    const int c1 = claim_at(qd * tot + c_b - 1);
    if (c0 == c1) continue;
    const int n = c1 - c0 + 1;
    const bool is_short = n <= kMergeBlock;
    const int ti = atomicAdd(is_short ? &n_short : &n_long, 1);
    *reinterpret_cast<int4*>((is_short ? short_list : long_list) + 4 * ti) =
        make_int4(t, c0, n, 0);
  }
  lds_barrier();
  if (tid == 0) {
    p.plan[kHdrShort + b] = n_short;
    p.plan[kHdrLong + b] = n_long;
  }
  if (b == 0 && tid == 0) p.plan[kHdrNext] = 0;
}

// Natural log of a softmax normaliser kept as (m, l) in log2 units:
// ln(l * 2^m) = (m + log2 l) * ln 2.
__device__ __forceinline__ float lse_of(float m, float l) {
  return (m + log2f(l)) * 0.69314718055994531f;
}

// ---------------------------------------------------------------------------
// Claim walk shared by both partition kernels.
// ---------------------------------------------------------------------------
struct Segment {
  int qd, s, L, t0, take;   // tiles [t0, t0 + take) of sequence s, KV-head quad qd
  bool final;               // the segment is the whole sequence
  int pair;                 // partial-state slot when not final
};

// Runs `process` on every segment of every claim this workgroup takes.  The
// first two stages, when neither is the final one, have one claim per
// workgroup each: workgroup b takes claim b of stage 0 and claim b of stage
// 1 (= b + gridDim.x).  The claims of the later stages come from the
// counter, one at a time (taken at the start of a claim, published through
// LDS at its end), so that faster workgroups take more of them.  (With the
// counter from stage 1 on, every workgroup asks for its second claim
// within a few microseconds of the others as stage 0 ends; handing stage 1
// out statically measured 1-3 % faster on every workload, and stages past
// the second are better balanced by the counter.)
template <typename Fn>
__device__ __forceinline__ void walk_claims(const AttnParams& p, Fn&& process) {
  cint* cum = (cint*)(p.plan + kHdrWords);
  cint* desc = (cint*)(p.plan + p.off_desc);
  // Every load before a claim's first tiles is a dependent round trip, and
  // at the start of the launch all workgroups wait on them together, so a
  // claim's descriptor carries all the walk needs.  Descriptor blockIdx.x
  // exists whatever the claim count (gridDim.x <= range_cap; the plan
  // writes empty ones past the last claim).
  auto load_desc = [&](int c, int (&d)[kDescWords]) {
#pragma unroll
    for (int i = 0; i < kDescWords; ++i) d[i] = desc[kDescWords * c + i];
  };
  int d[kDescWords];
  load_desc(blockIdx.x, d);
  __shared__ int next_lds[2];
  int parity = 0;
  for (int c = blockIdx.x;;) {
    const int succ = d[6];
    const int C = d[7];
    int next = 0;
    if (threadIdx.x == 0)
      next = succ >= 0 ? succ : (-1 - succ) + atomicAdd(p.plan + kHdrNext, 1);
    int qd = d[0];
    int s = d[1];
    int t0 = d[2];
    int remaining = d[3];
    // The first sequence's tile count and length come with the descriptor.
    int nt = d[4];
    int L = d[5];
    // The claim holds `remaining` tiles of the flattened space; the walk can
    // never pass the last quad, which bounds the loop for any input.
    bool first = true;
    while (remaining > 0 && qd < p.kvq_count) {
      if (!first) {
        nt = cum[s + 1] - cum[s];
        L = ((cint*)p.lens)[s];
      }
      first = false;
      const int take = min(nt - t0, remaining);
      if (take > 0) {
        Segment sg;
        sg.qd = qd;
        sg.s = s;
        sg.L = L;
        sg.t0 = t0;
        sg.take = take;
        sg.final = (t0 == 0 && take == nt);
        // Unique: along the walk both c and qd * S + s never decrease and
        // one of them grows from one segment to the next.
        sg.pair = c + qd * p.num_seqs + s;
        process(sg);
        remaining -= take;
      }
      t0 = 0;
      if (++s == p.num_seqs) {
        s = 0;
        ++qd;
      }
    }
    if (threadIdx.x == 0) next_lds[parity] = next;
    // One barrier suffices: a slot is written again two claims later, after
    // every thread has passed the barrier that follows its read.
    lds_barrier();
    c = __builtin_amdgcn_readfirstlane(next_lds[parity]);
    parity ^= 1;
    if (c >= C) break;
    load_desc(c, d);
  }
}

// The KV-head group a wave serves in a segment: quad qd, member kw.
struct WaveKv {
  bool live;   // kvg < kvg_count (the last quad may be short)
  int kvg, kvh, h0, nh;
};
__device__ __forceinline__ WaveKv wave_kv(const AttnParams& p, int qd, int kw) {
  WaveKv r;
  r.kvg = qd * p.kw + kw;
  r.live = r.kvg < p.kvg_count;
  r.kvh = r.kvg / p.head_groups;
  const int hg = r.kvg - r.kvh * p.head_groups;
  r.h0 = r.kvh * p.group + hg * p.gsize;
  r.nh = r.live ? min(p.gsize, p.group - hg * p.gsize) : 0;
  return r;
}

// One output item: channels d .. d+3 of head h of KV-head group kw, from the
// (m, l, o) states of waves w0 .. w0+n-1 held in LDS.  Writes the final
// output when the segment is the whole sequence, else the partial state
// (M, weighted l, weighted o) of slot (pair, kw, h).
template <typename T, int D, int G, bool kScaleV>
__device__ __forceinline__ void emit_item(const AttnParams& p, const Segment& sg, const WaveKv& kv,
                                          int kw, int w0, int n, int h, int d, int bad,
                                          const float (*red_m)[G], const float (*red_l)[G],
                                          const float (*red_acc)[G][D]) {
  using S = typename T::storage;
  float big_m = -INFINITY;
  for (int j = 0; j < n; ++j) big_m = fmaxf(big_m, red_m[w0 + j][h]);
  float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
  float den = 0.f;
  for (int j = 0; j < n; ++j) {
    const float mw = red_m[w0 + j][h];
    const float wgt = mw == -INFINITY ? 0.f : fast_exp2(mw - big_m);
    const float4 a = *reinterpret_cast<const float4*>(&red_acc[w0 + j][h][d]);
    num.x += wgt * a.x;
    num.y += wgt * a.y;
    num.z += wgt * a.z;
    num.w += wgt * a.w;
    den += wgt * red_l[w0 + j][h];
  }
  const float nan = __builtin_nanf("");
  if constexpr (kScaleV) {   // FP8 pools: the V codes' scale
    float vs = p.v_scale;
    if (p.v_scales) {
      vs = p.v_scales[kv.kvh];
      if (!scale_ok(vs) || !scale_ok(p.k_scales[kv.kvh])) bad = 1;
    }
    num.x *= vs;
    num.y *= vs;
    num.z *= vs;
    num.w *= vs;
  }
  if (sg.final) {
    S* o = (S*)p.out + ((size_t)sg.s * p.num_q_heads + kv.h0 + h) * D + d;
    const float inv = 1.f / den;
    Cvt<T>::store4(o, bad ? nan : num.x * inv, bad ? nan : num.y * inv, bad ? nan : num.z * inv,
                   bad ? nan : num.w * inv);
    if (p.lse && d == 0)
      p.lse[(size_t)sg.s * p.num_q_heads + kv.h0 + h] = bad ? nan : lse_of(big_m, den);
  } else {
    const size_t slot = ((size_t)sg.pair * p.kw + kw) * G + h;
    *reinterpret_cast<float4*>(p.ws_acc + slot * D + d) =
        bad ? make_float4(nan, nan, nan, nan) : num;
    if (d == 0) {
      p.ws_m[slot] = bad ? 0.f : big_m;
      p.ws_l[slot] = bad ? nan : den;
    }
  }
}

// End of a segment, after each wave has put its (m, l, o) in LDS slot w.
// One wave per KV-head group: the wave writes its own results, no barrier.
// Several waves per group: the workgroup combines them after a barrier.
template <typename T, int D, int G, bool kScaleV = false>
__device__ __forceinline__ void finish_segment(const AttnParams& p, const Segment& sg, int w,
                                               int bad, const float (*red_m)[G],
                                               const float (*red_l)[G],
                                               const float (*red_acc)[G][D]) {
  constexpr int D4 = D / 4;
  if (p.wpk == 1) {
    wave_lds_sync();
    const WaveKv kv = wave_kv(p, sg.qd, w);
    const int any_bad = __any(bad) ? 1 : 0;
    if (kv.live) {
      for (int it = threadIdx.x & 63; it < kv.nh * D4; it += 64) {
        const int h = it / D4;
        emit_item<T, D, G, kScaleV>(p, sg, kv, w, w, 1, h, (it - h * D4) * 4, any_bad, red_m,
                                    red_l, red_acc);
      }
    }
    wave_lds_sync();   // the wave's LDS slot is rewritten by its next segment
  } else {
    __shared__ int bad_lds[kWaves];
    if ((threadIdx.x & 63) == 0) bad_lds[w] = 0;
    wave_lds_sync();
    if (bad) bad_lds[w] = 1;
    lds_barrier();
    int any_bad = 0;
#pragma unroll
    for (int j = 0; j < kWaves; ++j) any_bad |= bad_lds[j];
    for (int it = threadIdx.x; it < p.kw * G * D4; it += kThreads) {
      const int kw = it / (G * D4);
      const int r = it - kw * G * D4;
      const int h = r / D4;
      const WaveKv kv = wave_kv(p, sg.qd, kw);
      if (h < kv.nh)
        emit_item<T, D, G, kScaleV>(p, sg, kv, kw, kw * p.wpk, p.wpk, h, (r - h * D4) * 4,
                                    any_bad, red_m, red_l, red_acc);
    }
    lds_barrier();   // the LDS buffers (and bad_lds) are reused by the next segment
  }
}

// Block ids of the 16-token tile starting at token tb (a multiple of 16):
// lane j of the result holds the id of logical block (tb >> log2_b) + j, for
// each block the tile's valid tokens touch.  Scalar loads; an id outside the
// pool sets `bad` and reads block 0 instead.
__device__ __forceinline__ int tile_block_ids(const AttnParams& p, cint* trow, int tb, int L,
                                              int& first, int& nid, int& bad) {
  first = tb >> p.log2_b;
  nid = ((min(tb + kTile, L) - 1) >> p.log2_b) - first + 1;
  int v = 0;
  for (int j = 0; j < nid; ++j) {
    int id = trow[first + j];
    if (!valid_block(id, p.num_blocks)) {
      bad = 1;
      id = 0;
    }
    v = (int)(threadIdx.x & 63) == j ? id : v;
  }
  return v;
}

// K/V cache load: streamed (non-temporal) when every block is read once per
// call, cache-retaining when blocks are shared between sequences.
template <bool kStream>
__device__ __forceinline__ uint4 load_kv(const char* p) {
  if constexpr (kStream) return load16_stream(p);
  else return load16(p);
}
template <bool kStream>
__device__ __forceinline__ uint2 load_kv8(const char* p) {
  if constexpr (kStream) return load8_stream(p);
  else return load8(p);
}

// 8 pool elements as 8 elements of T: the identity for 16-bit pools; for FP8
// pools the exact decode of 8 codes, each value representable in T.
template <typename T>
__device__ __forceinline__ uint4 expand8(const uint4& v) { return v; }
template <typename T>
__device__ __forceinline__ uint4 expand8(const uint2& c) {
  return make_uint4(Fp8Pair<T>::template decode<false>(c.x),
                    Fp8Pair<T>::template decode<true>(c.x),
                    Fp8Pair<T>::template decode<false>(c.y),
                    Fp8Pair<T>::template decode<true>(c.y));
}

// ---------------------------------------------------------------------------
// MFMA partition kernel (fp16 / bf16).
// ---------------------------------------------------------------------------
template <typename T, int D, int G, bool kStream, bool kF8>
__global__ __launch_bounds__(kThreads, 2) void attn_partition_mfma(const AttnParams p) {
  using S = typename T::storage;
  // A lane loads 16 bytes of a K or V row at a time: 8 elements of a 16-bit
  // pool, 16 codes of an FP8 pool (decoded to T on use), so that every load
  // instruction moves 1 KiB whatever the pool type.  FP8 rows of 32 channels
  // (D = 32) take 8 codes per lane, which keeps a whole row group per tile.
  constexpr bool kWide = kF8 && D >= 64;
  constexpr int EPL = kWide ? 16 : 8;   // elements per lane load
  using KvReg = typename std::conditional<kF8 && !kWide, uint2, uint4>::type;
  constexpr int KVB = kF8 ? 1 : T::bytes;   // bytes per pool element
  constexpr int KCH = D / 32;        // MFMA k-chunks of 32 channels
  constexpr int CPR = D / 8;         // 8-element chunks per K/V row in LDS
  constexpr int LPR = D / EPL;       // lanes per K/V row
  constexpr int RPL = 64 / LPR;      // rows per load instruction
  constexpr int TPR = kTile / RPL;   // tokens per row group per tile
  // Tiles in flight per wave: three when the accumulator is large (G >= 4:
  // occupancy is register bound at two waves per SIMD anyway) and a slot
  // costs <= 32 registers; otherwise two, which keeps small groups at a
  // higher occupancy.
  // FP8 slots cost half the registers and carry half the bytes, so the FP8
  // kernel keeps more tiles in flight for the same bytes in flight.
  constexpr int kSlotRegs = 2 * TPR * (int)(sizeof(KvReg) / 4);
  constexpr int kSlots = (kF8 && G >= 4 && kSlotRegs <= 16) ? 5
                       : (kSlotRegs <= 32 && G >= 4) ? 3 : 2;
  static_assert(D % 32 == 0 && TPR >= 1 && G <= kMaxGroup && G * D <= kMaxGD, "shape");

  __shared__ float red_m[kWaves][G];
  __shared__ float red_l[kWaves][G];
  __shared__ __align__(16) float red_acc[kWaves][G][D];
  // K tile of each wave, 16 rows of CPR 16-byte chunks; chunk c of row r
  // sits at position c ^ kswz(r), which keeps both the row-wise writes and
  // the operand-wise reads free of bank conflicts.
  __shared__ __align__(16) uint4 k_lds[kWaves][kTile * CPR];
  // V tile of each wave, token-major, rows padded by 32 bytes: the four rows
  // one 16-lane group reads at a time (a 32-byte piece of each) then land in
  // distinct banks, and so do the two groups of a half-wave.
  constexpr int VP = D + 16;
  __shared__ __align__(16) uint16_t v_lds[kWaves][kTile * VP];
  auto kswz = [](int r) {
    if constexpr (CPR >= 16) return r & 15;          // rows of >= 256 bytes
    else if constexpr (CPR == 8) return (r >> 1) & 7; // 128-byte rows: two per 256 bytes
    else return (r >> 2) & 3;                         // 64-byte rows: four per 256 bytes
  };

  const int lane = threadIdx.x & 63;
  // The wave index is uniform across the wave; saying so lets the tile loop
  // run on scalar branches and the block ids come through scalar loads.
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15;     // A row (token of tile) / B and C column (head)
  const int kgrp = lane >> 4;    // k group of A and B; C rows 4*kgrp .. 4*kgrp+3
  const int vc = lane % LPR;     // K/V: EPL-element piece within the row
  const int vr = lane / LPR;     // K/V: row group, tokens TPR*vr .. TPR*vr+TPR-1
  const size_t bytes = KVB;
  // KV-head group kw of the quad; with several waves per group, sub-wave sw
  // takes every wpk-th tile.
  const int kw = w / p.wpk;
  const int sw = w - kw * p.wpk;

  walk_claims(p, [&](const Segment& sg) {
    cint* trow = (cint*)(p.tables + (size_t)sg.s * p.max_blocks);
    const int L = sg.L;
    const int last = L - 1;
    const WaveKv kv = wave_kv(p, sg.qd, kw);
    // Score scale in log2 units.  FP8 pools with per-head scales fold in the
    // KV head's key scale here (an unusable one leaves the factor 1, and the
    // head's rows come out NaN at the end of the segment).
    float sl2 = p.scale_log2;
    if constexpr (kF8) {
      if (p.k_scales && kv.live) {
        const float ks = p.k_scales[kv.kvh];
        if (scale_ok(ks)) sl2 *= ks;
      }
    }

    // B operand: query head `col` of this group, channels 32j + 8*kgrp .. +7.
    uint4 qop[KCH];
    {
      const S* qrow = (const S*)p.q + ((size_t)sg.s * p.num_q_heads + kv.h0 + col) * D + kgrp * 8;
#pragma unroll
      for (int j = 0; j < KCH; ++j)
        qop[j] = col < kv.nh ? load16(qrow + 32 * j) : make_uint4(0, 0, 0, 0);
    }

    int bad = 0;
    const int tile_end = sg.t0 + sg.take;
    // Register ring: while one tile is consumed the next kSlots - 1 are in
    // flight.
    KvReg kb[kSlots][TPR], vb[kSlots][TPR];
    auto ld = [&](const char* a) {
      if constexpr (kF8 && !kWide) return load_kv8<kStream>(a);
      else return load_kv<kStream>(a);
    };
    auto issue = [&](auto slot, int tile) {
      constexpr int SL = decltype(slot)::value;
      // Past the segment's last tile the slot is never consumed: load nothing.
      if (tile >= tile_end) return;
      const int tb = tile * kTile;
      int first, nid;
      const int ids = tile_block_ids(p, trow, tb, L, first, nid, bad);
      const int id0 = __builtin_amdgcn_readfirstlane(ids);
      if (nid == 1) {
        // The whole tile lies in one block: one scalar base per pool, and
        // per-lane 32-bit offsets of rows (clamped to the last valid token).
        const int rlim = last - tb;
        const size_t base = row_offset(id0, tb, p.log2_b, p.num_kv_heads, kv.kvh, D) * bytes;
        const char* kbase = p.k_pool + base;
        const char* vbase = p.v_pool + base;
        const uint32_t rstride = (uint32_t)(p.num_kv_heads * D * bytes);
        // K and V alike: lane (vr, vc) reads chunk vc of rows TPR*vr + i, so
        // every load instruction covers whole rows.
#pragma unroll
        for (int i = 0; i < TPR; ++i) {
          const uint32_t o = (uint32_t)min(TPR * vr + i, rlim) * rstride + vc * EPL * bytes;
          kb[SL][i] = ld(kbase + o);
          vb[SL][i] = ld(vbase + o);
        }
      } else {
        auto row = [&](int t, int ch) -> size_t {
          const int tt = min(t, last);
          const int blk = __shfl(ids, (tt >> p.log2_b) - first);
          return (row_offset(blk, tt, p.log2_b, p.num_kv_heads, kv.kvh, D) + ch) * bytes;
        };
#pragma unroll
        for (int i = 0; i < TPR; ++i) {
          const size_t o = row(tb + TPR * vr + i, vc * EPL);
          kb[SL][i] = ld(p.k_pool + o);
          vb[SL][i] = ld(p.v_pool + o);
        }
      }
    };

    float m_run = -INFINITY;  // running maximum of head `col` (log2 units)
    float l_run = 0.f;        // normaliser partial: tokens of C row group kgrp
    // O^T accumulator: block j holds channels 16j + 4*kgrp .. +3 of head col.
    f32x4_t acc[D / 16];
#pragma unroll
    for (int j = 0; j < D / 16; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // This lane's piece of the transposed V reads: row 4*kgrp + col / 4,
    // channels 4 * (col % 4) .. +3 of each 16-channel block.
    const uint16_t* vt = &v_lds[w][(4 * kgrp + (col >> 2)) * VP + 4 * (col & 3)];

    auto consume = [&](auto slot, int tile) {
      constexpr int SL = decltype(slot)::value;
      // K and V rows to LDS.  K: each lane then takes its operand, row `col`,
      // channels 32j + 8*kgrp .. +7 = chunk 4j + kgrp.  (The previous tile's
      // reads are ordered before these writes by the sync ending it.)
#pragma unroll
      for (int i = 0; i < TPR; ++i) {
        const int r = TPR * vr + i;
        if constexpr (kWide) {
          // 16 codes: chunks 2vc and 2vc + 1 of the row.
          k_lds[w][r * CPR + ((2 * vc) ^ kswz(r))] =
              expand8<T>(make_uint2(kb[SL][i].x, kb[SL][i].y));
          k_lds[w][r * CPR + ((2 * vc + 1) ^ kswz(r))] =
              expand8<T>(make_uint2(kb[SL][i].z, kb[SL][i].w));
          *reinterpret_cast<uint4*>(&v_lds[w][r * VP + vc * 16]) =
              expand8<T>(make_uint2(vb[SL][i].x, vb[SL][i].y));
          *reinterpret_cast<uint4*>(&v_lds[w][r * VP + vc * 16 + 8]) =
              expand8<T>(make_uint2(vb[SL][i].z, vb[SL][i].w));
        } else {
          k_lds[w][r * CPR + (vc ^ kswz(r))] = expand8<T>(kb[SL][i]);
          *reinterpret_cast<uint4*>(&v_lds[w][r * VP + vc * 8]) = expand8<T>(vb[SL][i]);
        }
      }
      wave_lds_sync();
      f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < KCH; ++j)
        sc = Mfma<T>::run(k_lds[w][col * CPR + ((4 * j + kgrp) ^ kswz(col))], qop[j], sc);
      const int tb = tile * kTile;
      float sv[4];
      float mt = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sv[i] = (tb + 4 * kgrp + i < L) ? sc[i] * sl2 : -INFINITY;
        mt = fmaxf(mt, sv[i]);
      }
      mt = max_xor32(max_xor16(mt));

      // Every lane holds its own head's maximum, so the rescale is lane-local.
      if (__any(mt > m_run + kRescaleThreshold)) {
        const float mn = fmaxf(m_run, mt);
        const float alpha = fast_exp2(m_run - mn);   // 0 on the first tile
        m_run = mn;
        l_run *= alpha;
#pragma unroll
        for (int j = 0; j < D / 16; ++j) acc[j] *= alpha;
      }

      float pv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pv[i] = fast_exp2(sv[i] - m_run);   // masked: exp2(-inf) = 0
      // P rounded to the element type for the product; the normaliser sums
      // the same rounded values, so the weights still sum to one.  The lane's
      // four probabilities (tokens 4*kgrp + i, head col) are exactly its B
      // operand of O^T = V^T . P^T.
      const uint32_t q01 = Pair<T>::pack(pv[0], pv[1]);
      const uint32_t q23 = Pair<T>::pack(pv[2], pv[3]);
      l_run += (Pair<T>::lo(q01) + Pair<T>::hi(q01)) + (Pair<T>::lo(q23) + Pair<T>::hi(q23));
      const uint2 pop = make_uint2(q01, q23);
      // A operand of block j: V[4*kgrp + i][16j + col], i = 0..3, one
      // transposed read.
#pragma unroll
      for (int j = 0; j < D / 16; ++j) acc[j] = Mfma16<T>::run(lds_read_tr16(vt + 16 * j), pop, acc[j]);
      wave_lds_sync();
    };

    // The ring: slots 0 .. kSlots-2 are filled first; then each step issues
    // the tile kSlots-1 steps ahead into the slot freed last and consumes the
    // oldest one (slot indices are compile-time constants).
    const int step = p.wpk;
    int tile = sg.t0 + sw;
    if (kv.live && tile < tile_end) {
      static_for<kSlots - 1>([&](auto k) { issue(k, tile + decltype(k)::value * step); });
      bool done = false;
      while (!done) {
        static_for<kSlots>([&](auto k) {
          constexpr int K = decltype(k)::value;
          if (!done) {
            issue(std::integral_constant<int, (K + kSlots - 1) % kSlots>{},
                  tile + (kSlots - 1) * step);
            consume(k, tile);
            tile += step;
            done = tile >= tile_end;
          }
        });
      }
    }

    // Wave totals: l over the four C row groups; o is complete per lane.
    l_run = sum_xor32(sum_xor16(l_run));
    if (col < G) {
#pragma unroll
      for (int j = 0; j < D / 16; ++j)
        *reinterpret_cast<float4*>(&red_acc[w][col][16 * j + 4 * kgrp]) =
            make_float4(acc[j][0], acc[j][1], acc[j][2], acc[j][3]);
      if (kgrp == 0) {
        red_m[w][col] = m_run;
        red_l[w][col] = l_run;
      }
    }
    finish_segment<T, D, G, kF8>(p, sg, w, bad, red_m, red_l, red_acc);
  });
}

// ---------------------------------------------------------------------------
// Vector-ALU partition kernel (any dtype).
// ---------------------------------------------------------------------------
template <typename T, int D, int G, bool kStream>
__global__ __launch_bounds__(kThreads, 2) void attn_partition_valu(const AttnParams p) {
  using S = typename T::storage;
  constexpr int E = 16 / T::bytes;   // elements per 16-byte chunk
  constexpr int LPR = D / E;         // lanes per token row
  constexpr int RPL = 64 / LPR;      // tokens per wave step
  static_assert(LPR >= 1 && LPR <= 64 && G <= kMaxGroup && G * D <= kMaxGD, "shape");

  __shared__ float red_m[kWaves][G];
  __shared__ float red_l[kWaves][G];
  __shared__ __align__(16) float red_acc[kWaves][G][D];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane % LPR;   // chunk of the row
  const int r = lane / LPR;   // token slot within the wave step
  const size_t bytes = T::bytes;
  const int kw = w / p.wpk;
  const int sw = w - kw * p.wpk;

  walk_claims(p, [&](const Segment& sg) {
    const int32_t* trow = p.tables + (size_t)sg.s * p.max_blocks;
    const WaveKv kv = wave_kv(p, sg.qd, kw);
    float qf[G][E];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if (h < kv.nh) {
        const S* qrow = (const S*)p.q + ((size_t)sg.s * p.num_q_heads + kv.h0 + h) * D + c * E;
        Cvt<T>::unpack(load16(qrow), qf[h]);
#pragma unroll
        for (int e = 0; e < E; ++e) qf[h][e] *= p.scale_log2;
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) qf[h][e] = 0.f;
      }
    }

    float m[G], l[G], acc[G][E];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m[h] = -INFINITY;
      l[h] = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[h][e] = 0.f;
    }

    int bad = 0;
    const int tok0 = sg.t0 * kTile;
    const int tok_end = kv.live ? min(sg.L, (sg.t0 + sg.take) * kTile) : tok0;
    for (int base = tok0 + sw * RPL; base < tok_end; base += RPL * p.wpk) {
      const int t = base + r;
      const bool valid = t < tok_end;
      const int tt = valid ? t : tok_end - 1;
      int blk = trow[tt >> p.log2_b];
      if (!valid_block(blk, p.num_blocks)) {
        bad = 1;
        blk = 0;
      }
      const size_t off = (row_offset(blk, tt, p.log2_b, p.num_kv_heads, kv.kvh, D) + c * E) * bytes;
      float kf[E], vf[E];
      Cvt<T>::unpack(load_kv<kStream>(p.k_pool + off), kf);
      Cvt<T>::unpack(load_kv<kStream>(p.v_pool + off), vf);
      float sh[G];
      bool grow = false;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) part = fmaf(qf[h][e], kf[e], part);
#pragma unroll
        for (int o = 1; o < LPR; o <<= 1) part += __shfl_xor(part, o);
        sh[h] = part;
        grow |= valid && part > m[h] + kRescaleThreshold;
      }
      if (__any(grow)) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float mn = valid ? fmaxf(m[h], sh[h]) : m[h];
          const float a = mn == -INFINITY ? 1.f : fast_exp2(m[h] - mn);
          m[h] = mn;
          l[h] *= a;
#pragma unroll
          for (int e = 0; e < E; ++e) acc[h][e] *= a;
        }
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float ph = valid ? fast_exp2(sh[h] - m[h]) : 0.f;
        l[h] += ph;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[h][e] = fmaf(ph, vf[e], acc[h][e]);
      }
    }

    // Merge the RPL streams of the wave (lanes r and r ^ k hold the same chunk).
#pragma unroll
    for (int o = LPR; o < 64; o <<= 1) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float mo = __shfl_xor(m[h], o);
        const float lo = __shfl_xor(l[h], o);
        const float big = fmaxf(m[h], mo);
        const float wa = m[h] == -INFINITY ? 0.f : fast_exp2(m[h] - big);
        const float wb = mo == -INFINITY ? 0.f : fast_exp2(mo - big);
        l[h] = l[h] * wa + lo * wb;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[h][e] = acc[h][e] * wa + __shfl_xor(acc[h][e], o) * wb;
        m[h] = big;
      }
    }
    if (r == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < E; ++e) red_acc[w][h][c * E + e] = acc[h][e];
    }
    if (lane == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        red_m[w][h] = m[h];
        red_l[w][h] = l[h];
      }
    }
    finish_segment<T, D, G>(p, sg, w, bad, red_m, red_l, red_acc);
  });
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of the partial states of split sequences,
//     M = max_i m_i,  l = sum_i e^(m_i - M) l_i,  o = sum_i e^(m_i - M) o_i,
// out = o / l, for each (task, KV-head group of the quad).  Short tasks (at
// most kMergeBlock partials) take one wave with all of its loads in flight
// together; long tasks take a workgroup whose waves combine chunks of
// kMergeBlock in turn and then merge their four states through LDS.
// ---------------------------------------------------------------------------
struct MergeState {
  float run_m;              // running maximum of head lh (per lane)
  float den;                // weighted l of partial (li, lh); summed over li by the caller
  float4 acc[kMaxGD / 256]; // weighted o, channels 4 * lane + 256 * j
};

__device__ __forceinline__ void merge_init(MergeState& st) {
  st.run_m = -INFINITY;
  st.den = 0.f;
#pragma unroll
  for (int j = 0; j < kMaxGD / 256; ++j) st.acc[j] = make_float4(0.f, 0.f, 0.f, 0.f);
}

// Adds the states of pairs first .. first + count - 1 (count <= kMergeBlock)
// of KV-head group kw_i to st.  Slot of pair q, head h: (q * kw + kw_i) * G + h.
__device__ __forceinline__ void merge_block(const AttnParams& p, size_t first, int count,
                                            int kw_i, int nh, MergeState& st) {
  constexpr int kF4 = kMaxGD / 256;
  const int G = p.gsize, D = p.head_dim, KW = p.kw;
  const int lane = threadIdx.x & 63;
  const int lh = lane & (G - 1);
  const int li = lane / G;
  const int nf = nh * D;
  const bool ok = li < count && lh < nh;
  const size_t slot = ((first + li) * KW + kw_i) * G + lh;
  const float mi = ok ? p.ws_m[slot] : -INFINITY;
  const float lv = ok ? p.ws_l[slot] : 0.f;
  float4 x[kMergeBlock][kF4];
#pragma unroll
  for (int i = 0; i < kMergeBlock; ++i)
#pragma unroll
    for (int j = 0; j < kF4; ++j) {
      const int f = 4 * lane + 256 * j;
      x[i][j] = (i < count && f < nf)
                    ? *reinterpret_cast<const float4*>(p.ws_acc + ((first + i) * KW + kw_i) * G * D + f)
                    : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  float cm = mi;
  for (int o = G; o < 64; o <<= 1) cm = fmaxf(cm, __shfl_xor(cm, o));
  const float mn = fmaxf(st.run_m, cm);
  const float so = st.run_m == -INFINITY ? 0.f : fast_exp2(st.run_m - mn);
  st.run_m = mn;
  const float wi = mi == -INFINITY ? 0.f : fast_exp2(mi - mn);
  st.den = st.den * so + wi * lv;
#pragma unroll
  for (int j = 0; j < kF4; ++j) {
    const int f = 4 * lane + 256 * j;
    const int h = min(f / D, G - 1);
    const float sj = __shfl(so, h);
    float4 a = st.acc[j];
    a.x *= sj; a.y *= sj; a.z *= sj; a.w *= sj;
#pragma unroll
    for (int i = 0; i < kMergeBlock; ++i) {
      const float wj = __shfl(wi, i * G + h);
      a.x += wj * x[i][j].x;
      a.y += wj * x[i][j].y;
      a.z += wj * x[i][j].z;
      a.w += wj * x[i][j].w;
    }
    st.acc[j] = a;
  }
}

// Sum of den over the partials of each head (lanes with the same lh).
__device__ __forceinline__ float head_den(const MergeState& st, int G) {
  float d = st.den;
  for (int o = G; o < 64; o <<= 1) d += __shfl_xor(d, o);
  return d;
}

template <typename T>
__device__ __forceinline__ void store4(const AttnParams& p, int s, int head, int d, float4 v) {
  using S = typename T::storage;
  S* o = (S*)p.out + ((size_t)s * p.num_q_heads + head) * p.head_dim + d;
  Cvt<T>::store4(o, v.x, v.y, v.z, v.w);
}

template <typename T>
__global__ __launch_bounds__(kMergeThreads) void attn_merge(const AttnParams p) {
  constexpr int kF4 = kMaxGD / 256;
  __shared__ float m_lds[kMergeWaves][kMaxGroup];
  __shared__ float l_lds[kMergeWaves][kMaxGroup];
  __shared__ __align__(16) float acc_lds[kMergeWaves][kMaxGD];
  const int G = p.gsize, D = p.head_dim, KW = p.kw;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // The task lists come in kPlanGroups segments.  Lanes 0..15 hold the
  // inclusive prefix of the short-list counts, lanes 16..31 that of the
  // long-list counts; entry i of a list is then found with one ballot.
  static_assert(kPlanGroups == 16, "two 16-lane prefix groups");
  int pre = lane < 2 * kPlanGroups ? p.plan[kHdrShort + lane] : 0;   // kHdrLong = kHdrShort + 16
#pragma unroll
  for (int o = 1; o < kPlanGroups; o <<= 1) {
    const int v = __shfl_up(pre, o);
    if ((lane & (kPlanGroups - 1)) >= o) pre += v;
  }
  auto entry = [&](int list_off, int group0, int i) {
    const unsigned long long below = __ballot(lane >= group0 && lane < group0 + kPlanGroups && pre <= i);
    const int seg = __builtin_amdgcn_readfirstlane(__popcll(below));
    const int start =
        seg > 0 ? __builtin_amdgcn_readfirstlane(__shfl(pre, group0 + seg - 1)) : 0;
    // Uniform address: the entry comes through scalar loads.
    cint* e = (cint*)(p.plan + list_off) + 4 * ((size_t)seg * p.task_seg + (i - start));
    return make_int4(e[0], e[1], e[2], 0);
  };

  // Long tasks: one workgroup per (task, KV-head group).
  const int n_long = __builtin_amdgcn_readfirstlane(__shfl(pre, 2 * kPlanGroups - 1)) * KW;
  for (int u = blockIdx.x; u < n_long; u += gridDim.x) {
    const int ti = u / KW;
    const int kw_i = u - ti * KW;
    const int4 e = entry(p.off_long, kPlanGroups, ti);
    const int t = e.x, c0 = e.y, n = e.z;
    const int qd = t / p.num_seqs;
    const int s = t - qd * p.num_seqs;
    const WaveKv kv = wave_kv(p, qd, kw_i);
    if (!kv.live) continue;   // uniform over the workgroup
    const size_t pair0 = (size_t)c0 + t;
    MergeState st;
    merge_init(st);
    for (int i0 = wv * kMergeBlock; i0 < n; i0 += kMergeWaves * kMergeBlock)
      merge_block(p, pair0 + i0, min(kMergeBlock, n - i0), kw_i, kv.nh, st);
    const float den = head_den(st, G);
    if (lane < kv.nh) {
      m_lds[wv][lane] = st.run_m;
      l_lds[wv][lane] = den;
    }
#pragma unroll
    for (int j = 0; j < kF4; ++j) {
      const int f = 4 * lane + 256 * j;
      if (f < kv.nh * D) *reinterpret_cast<float4*>(&acc_lds[wv][f]) = st.acc[j];
    }
    lds_barrier();
    for (int f = 4 * threadIdx.x; f < kv.nh * D; f += 4 * kMergeThreads) {
      const int h = f / D;
      float big = -INFINITY;
#pragma unroll
      for (int w = 0; w < kMergeWaves; ++w) big = fmaxf(big, m_lds[w][h]);
      float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
      float dsum = 0.f;
#pragma unroll
      for (int w = 0; w < kMergeWaves; ++w) {
        const float mw = m_lds[w][h];
        const float wt = mw == -INFINITY ? 0.f : fast_exp2(mw - big);
        const float4 a = *reinterpret_cast<const float4*>(&acc_lds[w][f]);
        num.x += wt * a.x;
        num.y += wt * a.y;
        num.z += wt * a.z;
        num.w += wt * a.w;
        dsum += wt * l_lds[w][h];
      }
      const float inv = 1.f / dsum;
      store4<T>(p, s, kv.h0 + h, f - h * D,
                make_float4(num.x * inv, num.y * inv, num.z * inv, num.w * inv));
      if (p.lse && f == h * D) p.lse[(size_t)s * p.num_q_heads + kv.h0 + h] = lse_of(big, dsum);
    }
    lds_barrier();   // the LDS buffers are reused by the next task
  }

  // Short tasks: one wave per (task, KV-head group), counted from the last
  // workgroup down so that they land on workgroups without a long task
  // whenever the grid has room for both.
  const int n_short = __builtin_amdgcn_readfirstlane(__shfl(pre, kPlanGroups - 1)) * KW;
  for (int it = (gridDim.x - 1 - blockIdx.x) * kMergeWaves + wv; it < n_short;
       it += gridDim.x * kMergeWaves) {
    const int ti = it / KW;
    const int kw_i = it - ti * KW;
    const int4 e = entry(p.off_short, 0, ti);
    const int t = e.x, c0 = e.y, n = e.z;
    const int qd = t / p.num_seqs;
    const int s = t - qd * p.num_seqs;
    const WaveKv kv = wave_kv(p, qd, kw_i);
    if (!kv.live) continue;
    MergeState st;
    merge_init(st);
    merge_block(p, (size_t)c0 + t, n, kw_i, kv.nh, st);
    const float den = head_den(st, G);
#pragma unroll
    for (int j = 0; j < kF4; ++j) {
      const int f = 4 * lane + 256 * j;
      const int h = min(f / D, G - 1);
      const float dh = __shfl(den, h);
      const float mh = __shfl(st.run_m, h);
      const float inv = 1.f / dh;
      if (f < kv.nh * D)
        store4<T>(p, s, kv.h0 + h, f - h * D,
                  make_float4(st.acc[j].x * inv, st.acc[j].y * inv, st.acc[j].z * inv,
                              st.acc[j].w * inv));
      if (p.lse && f < kv.nh * D && f == h * D)
        p.lse[(size_t)s * p.num_q_heads + kv.h0 + h] = lse_of(mh, dh);
    }
  }
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct WsLayout {
  size_t off_desc, off_short, off_long, task_seg, plan_words;   // plan-area words
  size_t m_off, l_off, acc_off, total;         // bytes
};

// Workspace of a call: the plan words, then the partial states.  Pair slots:
// one per (claim, quad-sequence) along the monotone walk, at most
// range_cap + kvq_count * S of them, kw * G heads each.  The two merge task
// lists hold at most kvq_count * S entries each (16-byte aligned).
inline WsLayout ws_layout(int num_seqs, int kvq_count, int pair_heads, int head_dim,
                          int range_cap) {
  WsLayout w;
  const size_t pairs_q = (size_t)kvq_count * num_seqs;
  w.task_seg = (pairs_q + kPlanGroups - 1) / kPlanGroups;
  w.off_desc = (kHdrWords + (size_t)num_seqs + 1 + 3) & ~(size_t)3;
  w.off_short = w.off_desc + kDescWords * (size_t)range_cap;
  w.off_long = w.off_short + 4 * w.task_seg * kPlanGroups;
  const size_t plan_words = w.off_long + 4 * w.task_seg * kPlanGroups;
  w.plan_words = plan_words;
  const size_t heads = ((size_t)range_cap + pairs_q) * pair_heads;
  w.m_off = align256(plan_words * 4);
  w.l_off = w.m_off + align256(heads * 4);
  w.acc_off = w.l_off + align256(heads * 4);
  w.total = w.acc_off + align256(heads * head_dim * 4);
  return w;
}

inline int device_cu_count() {
  static std::mutex mu;
  static std::unordered_map<int, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(dev);
  if (it != cache.end()) return it->second;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  cache[dev] = n;
  return n;
}

// Resident workgroups per CU of a kernel (256 threads), cached per function.
inline int resident_per_cu(const void* fn) {
  static std::mutex mu;
  static std::unordered_map<const void*, int> cache;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(fn);
  if (it != cache.end()) return it->second;
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, kThreads, 0) != hipSuccess || n <= 0) n = 1;
  if (n > kMaxWgPerCu) n = kMaxWgPerCu;
  cache[fn] = n;
  return n;
}

enum Family { kFamilyValu = 1, kFamilyMfma = 2 };

// Largest head group one workgroup takes: bounded by the cross-wave LDS
// buffer (G * D <= kMaxGD) and by registers (a 16-head group spills, and so
// does the vector-ALU kernel's 8-head group with 8 elements per lane).
inline int max_group(int head_dim, int family, int dtype) {
  int g = kMaxGD / head_dim;
  if (g > kMaxGroup) g = kMaxGroup;
  if (family == kFamilyValu && dtype != PKV_F32 && g > 4) g = 4;
  if (family == kFamilyMfma && head_dim >= 256 && g > 2) g = 2;
  return g;
}

inline int pow2_at_least(int x) {
  int r = 1;
  while (r < x) r <<= 1;
  return r;
}

template <typename T, int D, int G, bool kStream, bool kF8>
const void* partition_fn(int family) {
  if (family == kFamilyMfma) {
    if constexpr (!std::is_same<T, F32>::value && D >= 32 && G * D <= kMaxGD && (D < 256 || G <= 2))
      return reinterpret_cast<const void*>(&attn_partition_mfma<T, D, G, kStream, kF8>);
  } else if constexpr (!kF8) {
    if constexpr (G * D <= kMaxGD && (std::is_same<T, F32>::value || G <= 4))
      return reinterpret_cast<const void*>(&attn_partition_valu<T, D, G, kStream>);
  }
  return nullptr;
}

template <typename T, int D, bool kStream, bool kF8>
const void* partition_fn_g(int family, int G) {
  switch (G) {
    case 1: return partition_fn<T, D, 1, kStream, kF8>(family);
    case 2: return partition_fn<T, D, 2, kStream, kF8>(family);
    case 4: return partition_fn<T, D, 4, kStream, kF8>(family);
    default: return partition_fn<T, D, 8, kStream, kF8>(family);
  }
}

template <typename T, bool kStream, bool kF8>
const void* partition_fn_d(int family, int D, int G) {
  switch (D) {
    case 16: return partition_fn_g<T, 16, kStream, kF8>(family, G);
    case 32: return partition_fn_g<T, 32, kStream, kF8>(family, G);
    case 64: return partition_fn_g<T, 64, kStream, kF8>(family, G);
    case 128: return partition_fn_g<T, 128, kStream, kF8>(family, G);
    default: return partition_fn_g<T, 256, kStream, kF8>(family, G);
  }
}

template <bool kStream, bool kF8>
const void* pick_partition_s(int family, int dtype, int D, int G) {
  switch (dtype) {
    case PKV_F32: return kF8 ? nullptr : partition_fn_d<F32, kStream, false>(family, D, G);
    case PKV_F16: return partition_fn_d<F16, kStream, kF8>(family, D, G);
    default: return partition_fn_d<BF16, kStream, kF8>(family, D, G);
  }
}

// The partition kernel for a call: family, q/out dtype, head size, group,
// streamed or cached loads, 16-bit or FP8 pools; nullptr if none exists.
inline const void* pick_partition(int family, int dtype, int D, int G, bool stream, bool fp8) {
  if (fp8)
    return stream ? pick_partition_s<true, true>(family, dtype, D, G)
                  : pick_partition_s<false, true>(family, dtype, D, G);
  return stream ? pick_partition_s<true, false>(family, dtype, D, G)
                : pick_partition_s<false, false>(family, dtype, D, G);
}

enum Phase { kPhasePlan = 1, kPhasePartitions = 2, kPhaseMerge = 4, kPhaseAll = 7 };

// What a plan was made for: the arguments that shape its schedule, its
// empty-row fills and the workspace layout.  The later phases of the same
// step must agree on all of them.
struct PlanKey {
  int kernel, dtype, kv_fp8, num_seqs, num_blocks, block_size, max_blocks_per_seq;
  int num_q_heads, num_kv_heads, head_dim, partition_tokens;
  const void* out;
  const void* context_lens;
  const void* block_tables;
  size_t workspace_bytes;
  bool operator==(const PlanKey& o) const {
    return kernel == o.kernel && dtype == o.dtype && kv_fp8 == o.kv_fp8 &&
           num_seqs == o.num_seqs && num_blocks == o.num_blocks &&
           block_size == o.block_size && max_blocks_per_seq == o.max_blocks_per_seq &&
           num_q_heads == o.num_q_heads && num_kv_heads == o.num_kv_heads &&
           head_dim == o.head_dim && partition_tokens == o.partition_tokens && out == o.out &&
           context_lens == o.context_lens && block_tables == o.block_tables &&
           workspace_bytes == o.workspace_bytes;
  }
};

// The plan resets the claim counter and writes the schedule that exactly one
// partitions launch consumes, and the merge reads what that launch left, so
// the phase entry points hold each workspace to plan -> partitions -> merge
// with one PlanKey.  The host records, per workspace address, the phase the
// last call left it ready for; a whole call (all three phases) leaves it
// ready for a plan.  Returns PKV_OK and advances the record, or
// PKV_ERR_ORDER and leaves it as it was.
int advance_phase(void* workspace, int phase, const PlanKey& key) {
  struct Expect {
    int next;   // kPhasePartitions or kPhaseMerge
    PlanKey key;
  };
  static std::mutex mu;
  static std::unordered_map<const void*, Expect> state;
  std::lock_guard<std::mutex> lock(mu);
  auto it = state.find(workspace);
  switch (phase) {
    case kPhaseAll:
      if (it != state.end()) state.erase(it);
      return PKV_OK;
    case kPhasePlan:   // a new plan replaces one that was never used
      state[workspace] = Expect{kPhasePartitions, key};
      return PKV_OK;
    default:
      if (it == state.end() || it->second.next != phase || !(it->second.key == key))
        return PKV_ERR_ORDER;
      if (phase == kPhasePartitions)
        it->second.next = kPhaseMerge;
      else
        state.erase(it);
      return PKV_OK;
  }
}

struct Launch {
  AttnParams p;
  const void* part_fn;
};

// Validates a call and fills the launch description; PKV_OK or an error.
int prepare(int kernel, void* out, const void* q, const void* k_pool, const void* v_pool,
            const int32_t* block_tables, int max_blocks_per_seq, const int32_t* context_lens,
            int num_seqs, int num_blocks, int block_size, int num_q_heads, int num_kv_heads,
            int head_dim, float scale, int partition_tokens, void* workspace,
            size_t workspace_bytes, int dtype, Launch* L, bool kv_fp8 = false,
            float k_scale = 1.f, float v_scale = 1.f, const float* k_scales = nullptr,
            const float* v_scales = nullptr) {
  int st = check_pool_shape(num_blocks, block_size, num_kv_heads, head_dim, dtype);
  if (st != PKV_OK) return st;
  if (!supported_dtype(dtype)) return PKV_ERR_UNSUPPORTED;   // q / out element type
  if (kv_fp8 && (!(k_scale > 0.f) || !(v_scale > 0.f) || k_scale == INFINITY ||
                 v_scale == INFINITY))
    return PKV_ERR_INVALID_ARG;
  if (num_seqs < 0 || max_blocks_per_seq < 1 || num_q_heads < 1 ||
      num_q_heads % num_kv_heads != 0 || !(scale == scale) || scale == INFINITY ||
      scale == -INFINITY)
    return PKV_ERR_INVALID_ARG;
  if ((kernel & ~(PKV_ATTN_KERNEL_MASK | PKV_ATTN_CACHE_KV)) != 0) return PKV_ERR_INVALID_ARG;
  const bool cache_kv = (kernel & PKV_ATTN_CACHE_KV) != 0;
  kernel &= PKV_ATTN_KERNEL_MASK;
  if (kernel > PKV_ATTN_MFMA) return PKV_ERR_INVALID_ARG;
  if (partition_tokens < 0 || (partition_tokens > 0 && partition_tokens % kTile != 0))
    return PKV_ERR_INVALID_ARG;
  const long long max_len = (long long)max_blocks_per_seq * block_size;
  if (max_len > (1LL << 30)) return PKV_ERR_INVALID_ARG;
  int family;
  if (kernel == PKV_ATTN_AUTO)
    family = (dtype != PKV_F32 && head_dim >= 32) ? kFamilyMfma : kFamilyValu;
  else
    family = kernel == PKV_ATTN_MFMA ? kFamilyMfma : kFamilyValu;
  if (family == kFamilyMfma && (dtype == PKV_F32 || head_dim < 32)) return PKV_ERR_UNSUPPORTED;
  // FP8 pools: the matrix-core kernel only (it decodes codes into its
  // 16-bit operands).
  if (kv_fp8 && family != kFamilyMfma) {
    if (kernel != PKV_ATTN_AUTO || dtype == PKV_F32 || head_dim < 32) return PKV_ERR_UNSUPPORTED;
    family = kFamilyMfma;
  }

  const int g = num_q_heads / num_kv_heads;
  const int gmax = max_group(head_dim, family, dtype);
  const int G = pow2_at_least(g < gmax ? g : gmax);
  const int head_groups = (g + G - 1) / G;
  const long long kvg = (long long)num_kv_heads * head_groups;
  // Tile counts are 32-bit on the device.
  if ((long long)num_seqs * ((max_len + kTile - 1) / kTile) * kvg >= (1LL << 31))
    return PKV_ERR_INVALID_ARG;
  if ((k_scales == nullptr) != (v_scales == nullptr) || (k_scales && !kv_fp8))
    return PKV_ERR_INVALID_ARG;
  if (num_seqs == 0) return PKV_OK;
  if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens)
    return PKV_ERR_INVALID_ARG;

  const void* fn = pick_partition(family, dtype, head_dim, G, !cache_kv, kv_fp8);
  if (!fn) return PKV_ERR_UNSUPPORTED;
  const int grid = device_cu_count() * resident_per_cu(fn);
  // Streamed K/V: the four waves of a workgroup take turns on the tiles of
  // one KV-head group.  Shared (cached) K/V: they serve four KV-head groups
  // of the same tokens when there are that many, so the rows a workgroup
  // reads are adjacent and a block read by several sequences stays hot.
  const int kw = !cache_kv ? 1 : kvg >= kWaves ? kWaves : (kvg >= 2 ? 2 : 1);
  const long long kvq = (kvg + kw - 1) / kw;
  const int cap_tiles = partition_tokens / kTile;
  long long range_cap = (long long)device_cu_count() * kClaimsPerCu;
  if (cap_tiles > 0)
    range_cap += kvq * num_seqs * ((max_len + partition_tokens - 1) / partition_tokens);
  if (range_cap >= (1LL << 30)) return PKV_ERR_INVALID_ARG;
  const WsLayout ws = ws_layout(num_seqs, (int)kvq, kw * G, head_dim, (int)range_cap);
  if (ws.plan_words >= (1ULL << 31)) return PKV_ERR_INVALID_ARG;   // 32-bit word offsets
  if (!workspace || workspace_bytes < ws.total || ((uintptr_t)workspace & 255) != 0)
    return PKV_ERR_WORKSPACE;

  AttnParams& p = L->p;
  p.out = out;
  p.q = q;
  p.k_pool = (const char*)k_pool;
  p.v_pool = (const char*)v_pool;
  p.tables = block_tables;
  p.lens = context_lens;
  char* wsb = (char*)workspace;
  p.plan = (int32_t*)wsb;
  p.ws_m = (float*)(wsb + ws.m_off);
  p.ws_l = (float*)(wsb + ws.l_off);
  p.ws_acc = (float*)(wsb + ws.acc_off);
  p.num_seqs = num_seqs;
  p.max_blocks = max_blocks_per_seq;
  p.num_blocks = num_blocks;
  p.log2_b = log2_exact(block_size);
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.head_dim = head_dim;
  p.group = g;
  p.gsize = G;
  p.head_groups = head_groups;
  p.kvg_count = (int)kvg;
  p.kw = kw;
  p.wpk = kWaves / kw;
  p.kvq_count = (int)kvq;
  p.cap_tiles = cap_tiles;
  p.grid = grid;
  p.range_cap = (int)range_cap;
  p.off_desc = (int)ws.off_desc;
  p.off_short = (int)ws.off_short;
  p.off_long = (int)ws.off_long;
  p.task_seg = (int)ws.task_seg;
  p.scale_log2 = scale * kLog2e * (kv_fp8 ? k_scale : 1.f);
  p.kv_fp8 = kv_fp8 ? 1 : 0;
  p.k_scale = kv_fp8 ? k_scale : 1.f;
  p.v_scale = kv_fp8 ? v_scale : 1.f;
  p.k_scales = k_scales;
  p.v_scales = v_scales;
  p.lse = nullptr;
  L->part_fn = fn;
  return PKV_OK;
}

template <typename T>
hipError_t launch_plan(const AttnParams& p, hipStream_t st) {
  // The append workgroups only when there is a token to append.
  const int groups = kPlanGroups + (p.k_new ? kAppendGroups : 0);
  hipLaunchKernelGGL(attn_plan<T>, dim3(groups), dim3(kPlanThreads), 0, st, p);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_merge(const AttnParams& p, hipStream_t st) {
  hipLaunchKernelGGL(attn_merge<T>, dim3(p.grid), dim3(kMergeThreads), 0, st, p);
  return hipGetLastError();
}

int decode_attention_impl(int phase, int kernel, void* out, const void* q, const void* k_pool,
                          const void* v_pool, const int32_t* block_tables, int max_blocks_per_seq,
                          const int32_t* context_lens, int num_seqs, int num_blocks,
                          int block_size, int num_q_heads, int num_kv_heads, int head_dim,
                          float scale, int partition_tokens, void* workspace,
                          size_t workspace_bytes, int dtype, void* stream,
                          const void* k_new = nullptr, const void* v_new = nullptr,
                          bool kv_fp8 = false, float k_scale = 1.f, float v_scale = 1.f,
                          float* lse = nullptr, const float* k_scales = nullptr,
                          const float* v_scales = nullptr) {
  Launch L;
  const int st = prepare(kernel, out, q, k_pool, v_pool, block_tables, max_blocks_per_seq,
                         context_lens, num_seqs, num_blocks, block_size, num_q_heads,
                         num_kv_heads, head_dim, scale, partition_tokens, workspace,
                         workspace_bytes, dtype, &L, kv_fp8, k_scale, v_scale, k_scales,
                         v_scales);
  if (st != PKV_OK || num_seqs == 0) return st;
  const PlanKey key{kernel,       dtype,           kv_fp8 ? 1 : 0, num_seqs,
                    num_blocks,   block_size,      max_blocks_per_seq,
                    num_q_heads,  num_kv_heads,    head_dim,
                    partition_tokens, out,         context_lens,
                    block_tables, workspace_bytes};
  const int order = advance_phase(workspace, phase, key);
  if (order != PKV_OK) return order;
  L.p.k_new = (const char*)k_new;
  L.p.lse = lse;
  L.p.v_new = (const char*)v_new;
  hipStream_t hs = (hipStream_t)stream;
  if (phase & kPhasePlan) {
    hipError_t e = dtype == PKV_F32 ? launch_plan<F32>(L.p, hs)
                 : dtype == PKV_F16 ? launch_plan<F16>(L.p, hs) : launch_plan<BF16>(L.p, hs);
    if (e != hipSuccess) return PKV_ERR_HIP;
  }
  if (phase & kPhasePartitions) {
    void* args[] = {(void*)&L.p};
    if (hipLaunchKernel(L.part_fn, dim3(L.p.grid), dim3(kThreads), args, 0, hs) != hipSuccess)
      return PKV_ERR_HIP;
  }
  if (phase & kPhaseMerge) {
    hipError_t e = dtype == PKV_F32 ? launch_merge<F32>(L.p, hs)
                 : dtype == PKV_F16 ? launch_merge<F16>(L.p, hs) : launch_merge<BF16>(L.p, hs);
    if (e != hipSuccess) return PKV_ERR_HIP;
  }
  return PKV_OK;
}

}  // namespace

// For the cascade decode (cascade.hip): validate a decode call without
// launching anything, and run one with log normalisers.
int decode_attention_check(int kernel, void* out, const void* q, const void* k_pool,
                           const void* v_pool, const int32_t* block_tables,
                           int max_blocks_per_seq, const int32_t* context_lens, int num_seqs,
                           int num_blocks, int block_size, int num_q_heads, int num_kv_heads,
                           int head_dim, float scale, void* workspace, size_t workspace_bytes,
                           int dtype, bool kv_fp8, float k_scale, float v_scale) {
  Launch L;
  return prepare(kernel, out, q, k_pool, v_pool, block_tables, max_blocks_per_seq, context_lens,
                 num_seqs, num_blocks, block_size, num_q_heads, num_kv_heads, head_dim, scale,
                 0, workspace, workspace_bytes, dtype, &L, kv_fp8, k_scale, v_scale);
}

int decode_attention_with_lse(int kernel, void* out, float* lse, const void* q,
                              const void* k_pool, const void* v_pool,
                              const int32_t* block_tables, int max_blocks_per_seq,
                              const int32_t* context_lens, int num_seqs, int num_blocks,
                              int block_size, int num_q_heads, int num_kv_heads, int head_dim,
                              float scale, void* workspace, size_t workspace_bytes, int dtype,
                              void* stream, bool kv_fp8, float k_scale, float v_scale) {
  return decode_attention_impl(kPhaseAll, kernel, out, q, k_pool, v_pool, block_tables,
                               max_blocks_per_seq, context_lens, num_seqs, num_blocks,
                               block_size, num_q_heads, num_kv_heads, head_dim, scale, 0,
                               workspace, workspace_bytes, dtype, stream, nullptr, nullptr, kv_fp8,
                               k_scale, v_scale, lse);
}

// Workspace of paged_decode_step_noalloc: one copy per GPU, in the code
// object's zero-filled data, so it exists from when the library loads on a
// GPU until the process ends.  Host code never passes this name to a
// kernel (on the host it is only a stand-in): the device address comes from
// hipGetSymbolAddress, once per GPU.
static __device__ __align__(256) unsigned char scratch[PKV_NOALLOC_SCRATCH_BYTES];

namespace {

// Device address of `scratch` on the current GPU, looked up on the first
// call there; PKV_OK or PKV_ERR_HIP.
int noalloc_scratch(void** out) {
  static std::mutex mu;
  static std::unordered_map<int, void*> ptrs;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return PKV_ERR_HIP;
  std::lock_guard<std::mutex> lock(mu);
  auto it = ptrs.find(dev);
  if (it == ptrs.end()) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return PKV_ERR_HIP;
    it = ptrs.emplace(dev, p).first;
  }
  *out = it->second;
  return PKV_OK;
}

}  // namespace

}  // namespace pkv

extern "C" size_t paged_decode_workspace_bytes(int num_seqs, int num_q_heads, int head_dim,
                                               int max_context_len, int partition_tokens) {
  if (num_seqs < 0 || num_q_heads < 1 || head_dim < 1 || max_context_len < 0 ||
      partition_tokens < 0)
    return 0;
  // Bounds that hold for every KV head count: kvq_count <= kvg_count <= Hq,
  // kw * G <= 4 * 8 and kvq_count * kw * G <= (kvg_count + 3) * G <= 2 * Hq + 24.
  const long long parts = partition_tokens > 0
      ? ((long long)max_context_len + partition_tokens - 1) / partition_tokens : 0;
  const long long range_cap = (long long)pkv::device_cu_count() * pkv::kClaimsPerCu +
                              (long long)num_q_heads * num_seqs * parts;
  if (range_cap >= (1LL << 30)) return 0;
  // Plan words: header, cum, descriptors, then the two merge task lists of
  // at most kvq_count * S <= Hq * S entries each (rounded up per plan
  // workgroup).
  const size_t plan_words = pkv::kHdrWords + (size_t)num_seqs + 4 +
                            pkv::kDescWords * (size_t)range_cap +
                            8 * ((size_t)num_q_heads * num_seqs + pkv::kPlanGroups);
  const size_t heads = (size_t)pkv::device_cu_count() * pkv::kClaimsPerCu * pkv::kWaves *
                           pkv::kMaxGroup +
                       (size_t)(2LL * num_q_heads + 24) * num_seqs * (size_t)(1 + parts);
  return pkv::align256(plan_words * 4) + 2 * pkv::align256(heads * 4) +
         pkv::align256(heads * head_dim * 4);
}

#define PKV_ATTN_ARGS                                                                      \
  void *out, const void *q, const void *k_pool, const void *v_pool,                        \
      const int32_t *block_tables, int max_blocks_per_seq, const int32_t *context_lens,    \
      int num_seqs, int num_blocks, int block_size, int num_q_heads, int num_kv_heads,     \
      int head_dim, float scale, int partition_tokens, void *workspace,                    \
      size_t workspace_bytes, int dtype, void *stream
#define PKV_ATTN_PASS                                                                      \
  out, q, k_pool, v_pool, block_tables, max_blocks_per_seq, context_lens, num_seqs,       \
      num_blocks, block_size, num_q_heads, num_kv_heads, head_dim, scale, partition_tokens, \
      workspace, workspace_bytes, dtype, stream

extern "C" int paged_decode_attention(PKV_ATTN_ARGS) {
  return pkv::decode_attention_impl(pkv::kPhaseAll, PKV_ATTN_AUTO, PKV_ATTN_PASS);
}

extern "C" int paged_decode_attention_with(int kernel, PKV_ATTN_ARGS) {
  return pkv::decode_attention_impl(pkv::kPhaseAll, kernel, PKV_ATTN_PASS);
}

extern "C" int paged_decode_attention_plan(int kernel, PKV_ATTN_ARGS) {
  return pkv::decode_attention_impl(pkv::kPhasePlan, kernel, PKV_ATTN_PASS);
}

extern "C" int paged_decode_attention_partitions(int kernel, PKV_ATTN_ARGS) {
  return pkv::decode_attention_impl(pkv::kPhasePartitions, kernel, PKV_ATTN_PASS);
}

extern "C" int paged_decode_attention_merge(int kernel, PKV_ATTN_ARGS) {
  return pkv::decode_attention_impl(pkv::kPhaseMerge, kernel, PKV_ATTN_PASS);
}

extern "C" int paged_decode_step(int kernel, void* out, const void* q, void* k_pool, void* v_pool,
                                 const void* k_new, const void* v_new,
                                 const int32_t* block_tables, int max_blocks_per_seq,
                                 const int32_t* context_lens, int num_seqs, int num_blocks,
                                 int block_size, int num_q_heads, int num_kv_heads, int head_dim,
                                 float scale, int partition_tokens, void* workspace,
                                 size_t workspace_bytes, int dtype, void* stream) {
  if (num_seqs > 0 && (!k_new || !v_new)) return PKV_ERR_INVALID_ARG;
  return pkv::decode_attention_impl(pkv::kPhaseAll, kernel, out, q, k_pool, v_pool, block_tables,
                                    max_blocks_per_seq, context_lens, num_seqs, num_blocks,
                                    block_size, num_q_heads, num_kv_heads, head_dim, scale,
                                    partition_tokens, workspace, workspace_bytes, dtype, stream,
                                    k_new, v_new);
}

extern "C" int paged_decode_attention_fp8(int kernel, void* out, const void* q,
                                          const void* k_pool, const void* v_pool,
                                          const int32_t* block_tables, int max_blocks_per_seq,
                                          const int32_t* context_lens, int num_seqs,
                                          int num_blocks, int block_size, int num_q_heads,
                                          int num_kv_heads, int head_dim, float scale,
                                          float k_scale, float v_scale, int partition_tokens,
                                          void* workspace, size_t workspace_bytes, int dtype,
                                          void* stream) {
  return pkv::decode_attention_impl(pkv::kPhaseAll, kernel, out, q, k_pool, v_pool, block_tables,
                                    max_blocks_per_seq, context_lens, num_seqs, num_blocks,
                                    block_size, num_q_heads, num_kv_heads, head_dim, scale,
                                    partition_tokens, workspace, workspace_bytes, dtype, stream,
                                    nullptr, nullptr, true, k_scale, v_scale);
}

extern "C" int paged_decode_step_fp8(int kernel, void* out, const void* q, void* k_pool,
                                     void* v_pool, const void* k_new, const void* v_new,
                                     const int32_t* block_tables, int max_blocks_per_seq,
                                     const int32_t* context_lens, int num_seqs, int num_blocks,
                                     int block_size, int num_q_heads, int num_kv_heads,
                                     int head_dim, float scale, float k_scale, float v_scale,
                                     int partition_tokens, void* workspace,
                                     size_t workspace_bytes, int dtype, void* stream) {
  if (num_seqs > 0 && (!k_new || !v_new)) return PKV_ERR_INVALID_ARG;
  return pkv::decode_attention_impl(pkv::kPhaseAll, kernel, out, q, k_pool, v_pool, block_tables,
                                    max_blocks_per_seq, context_lens, num_seqs, num_blocks,
                                    block_size, num_q_heads, num_kv_heads, head_dim, scale,
                                    partition_tokens, workspace, workspace_bytes, dtype, stream,
                                    k_new, v_new, true, k_scale, v_scale);
}

extern "C" int paged_decode_attention_fp8_per_head(
    int kernel, void* out, const void* q, const void* k_pool, const void* v_pool,
    const int32_t* block_tables, int max_blocks_per_seq, const int32_t* context_lens,
    int num_seqs, int num_blocks, int block_size, int num_q_heads, int num_kv_heads,
    int head_dim, float scale, const float* k_scales, const float* v_scales,
    int partition_tokens, void* workspace, size_t workspace_bytes, int dtype, void* stream) {
  if (num_seqs > 0 && (!k_scales || !v_scales)) return PKV_ERR_INVALID_ARG;
  return pkv::decode_attention_impl(pkv::kPhaseAll, kernel, out, q, k_pool, v_pool, block_tables,
                                    max_blocks_per_seq, context_lens, num_seqs, num_blocks,
                                    block_size, num_q_heads, num_kv_heads, head_dim, scale,
                                    partition_tokens, workspace, workspace_bytes, dtype, stream,
                                    nullptr, nullptr, true, 1.f, 1.f, nullptr, k_scales,
                                    v_scales);
}

extern "C" int paged_decode_step_fp8_per_head(
    int kernel, void* out, const void* q, void* k_pool, void* v_pool, const void* k_new,
    const void* v_new, const int32_t* block_tables, int max_blocks_per_seq,
    const int32_t* context_lens, int num_seqs, int num_blocks, int block_size, int num_q_heads,
    int num_kv_heads, int head_dim, float scale, const float* k_scales, const float* v_scales,
    int partition_tokens, void* workspace, size_t workspace_bytes, int dtype, void* stream) {
  if (num_seqs > 0 && (!k_new || !v_new || !k_scales || !v_scales)) return PKV_ERR_INVALID_ARG;
  return pkv::decode_attention_impl(pkv::kPhaseAll, kernel, out, q, k_pool, v_pool, block_tables,
                                    max_blocks_per_seq, context_lens, num_seqs, num_blocks,
                                    block_size, num_q_heads, num_kv_heads, head_dim, scale,
                                    partition_tokens, workspace, workspace_bytes, dtype, stream,
                                    k_new, v_new, true, 1.f, 1.f, nullptr, k_scales, v_scales);
}

extern "C" int paged_decode_attention_lse(int kernel, float* lse, PKV_ATTN_ARGS) {
  if (num_seqs > 0 && !lse) return PKV_ERR_INVALID_ARG;
  return pkv::decode_attention_impl(pkv::kPhaseAll, kernel, PKV_ATTN_PASS, nullptr, nullptr,
                                    false, 1.f, 1.f, lse);
}

extern "C" int paged_decode_step_noalloc(int kernel, void* out, const void* q, void* k_pool,
                                         void* v_pool, const void* k_new, const void* v_new,
                                         const int32_t* block_tables, int max_blocks_per_seq,
                                         const int32_t* context_lens, int num_seqs,
                                         int num_blocks, int block_size, int num_q_heads,
                                         int num_kv_heads, int head_dim, float scale,
                                         int partition_tokens, int dtype, void* stream) {
  if (num_seqs > 0 && (!k_new || !v_new)) return PKV_ERR_INVALID_ARG;
  // Validation first: given no workspace, a valid call stops at the
  // workspace check and launches nothing.
  int st = pkv::decode_attention_impl(pkv::kPhaseAll, kernel, out, q, k_pool, v_pool,
                                      block_tables, max_blocks_per_seq, context_lens, num_seqs,
                                      num_blocks, block_size, num_q_heads, num_kv_heads,
                                      head_dim, scale, partition_tokens, nullptr, 0, dtype,
                                      stream, k_new, v_new);
  if (st != PKV_ERR_WORKSPACE) return st;
  void* ws = nullptr;
  st = pkv::noalloc_scratch(&ws);
  if (st != PKV_OK) return st;
  return pkv::decode_attention_impl(pkv::kPhaseAll, kernel, out, q, k_pool, v_pool, block_tables,
                                    max_blocks_per_seq, context_lens, num_seqs, num_blocks,
                                    block_size, num_q_heads, num_kv_heads, head_dim, scale,
                                    partition_tokens, ws, PKV_NOALLOC_SCRATCH_BYTES, dtype,
                                    stream, k_new, v_new);
}
