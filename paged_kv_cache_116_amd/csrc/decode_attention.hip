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
//   attn_plan (1 workgroup): counts each live sequence's 16-token tiles,
//     prefix-sums them, and cuts the flattened space
//         (KV-head group, sequence, tile)
//     into R equal ranges of T tiles, one per resident workgroup of the next
//     launch (T can be capped by the caller's partition size).  It writes a
//     start descriptor per range and fills the rows of empty sequences.
//   attn_partition_* (persistent workgroups, 4 waves each): a workgroup walks
//     its ranges; each stretch of one sequence inside a range is a segment.
//     The four waves take the segment's tiles in turn, each with its own
//     online-softmax state, combined in LDS at the segment's end.  A segment
//     that is the whole sequence writes the final output; otherwise it writes
//     a partial state (m, l, o) in a slot named by (range + sequence slot).
//   attn_merge: the range where a split sequence starts combines the partial
//     states of every range it covers with the log-sum-exp rule
//         O = sum_p e^(m_p - M) o_p / sum_p e^(m_p - M) l_p.
//   The pages stop at the per-block recurrence; the balanced split and the
//   merge are this library's addition, to keep all 256 compute units busy
//   whatever the length mix, without launching idle workgroups.
//
// Two partition kernels:
//   attn_partition_mfma  (fp16 / bf16, D >= 32): the grouped score tile
//     S^T[16 tokens x 16 heads] = K_tile . Q^T is one chain of D/32
//     v_mfma_f32_16x16x32 ops whose A operand is loaded straight from the pool
//     (each lane's 8 elements are 16 contiguous bytes of one K row).  P.V is
//     fp32 FMA on the vector ALU: each lane owns 8 channels of one V row group
//     and reads the probabilities of its tokens from a per-wave LDS tile.
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
#include <unordered_map>

#include "pkv_common.h"
#include "pkv_host.h"

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
constexpr int kPlanThreads = 1024;
constexpr int kPlanLdsCum = 8192;   // prefix sums kept in LDS up to this many sequences

// Plan area (int32 words): header | cum[S + 1] | desc[range_cap * 4] | task[range_cap]
constexpr int kHdrWords = 16;
enum Hdr { kHdrTot = 0, kHdrRanges = 1, kHdrTiles = 2, kHdrTotal = 3 };

typedef const __attribute__((address_space(4))) int32_t cint;   // read with scalar loads

struct AttnParams {
  void* out;
  const void* q;
  const char* k_pool;
  const char* v_pool;
  const int32_t* tables;
  const int32_t* lens;
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
  int gsize;        // G: query heads per workgroup slot
  int head_groups;  // ceil(g / G)
  int kvg_count;    // Hkv * head_groups
  int cap_tiles;    // 0 = balanced ranges, else at most this many tiles per range
  int grid;         // workgroups of the partition and merge launches
  int range_cap;    // descriptor slots
  float scale_log2;  // scale * log2(e): scores live in log2 units
};

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

// Pairs of 16-bit values for the P.V product: probabilities of two tokens
// packed to the element type (round to nearest even) and multiplied with the
// same channel of the two tokens' V rows, accumulated in fp32.
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
  __device__ static __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
  }
};
template <> struct Pair<F16> {
  __device__ static __forceinline__ uint32_t pack(float a, float b) {
    const f16x2_t v = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, v);
  }
  __device__ static __forceinline__ float lo(uint32_t w) { return f16_lo(w); }
  __device__ static __forceinline__ float hi(uint32_t w) { return f16_hi(w); }
  __device__ static __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b), c,
                                  false);
  }
};

// (v0, v1) -> low halves and high halves of two dwords, paired per channel.
__device__ __forceinline__ uint32_t pair_lo(uint32_t t0, uint32_t t1) {
  return __builtin_amdgcn_perm(t1, t0, 0x05040100u);
}
__device__ __forceinline__ uint32_t pair_hi(uint32_t t0, uint32_t t1) {
  return __builtin_amdgcn_perm(t1, t0, 0x07060302u);
}

// A sequence is live when 0 < L <= max_blocks * B; it then has ceil(L/16) tiles.
__device__ __forceinline__ int live_tiles(int L, int max_len) {
  return (L > 0 && L <= max_len) ? (L + kTile - 1) / kTile : 0;
}

// ---------------------------------------------------------------------------
// Plan: one workgroup.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kPlanThreads) void attn_plan(const AttnParams p) {
  using S = typename T::storage;
  __shared__ int carry_lds;
  __shared__ int dead_count;
  __shared__ int dead_list[kPlanThreads];
  __shared__ int wave_sum[kPlanThreads / 64];
  __shared__ int cum_lds[kPlanLdsCum + 1];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int S_ = p.num_seqs;
  const int max_len = p.max_blocks << p.log2_b;
  const size_t row_elems = (size_t)p.num_q_heads * p.head_dim;
  int32_t* cum = p.plan + kHdrWords;

  // Exclusive prefix sum of tile counts, kPlanThreads sequences per pass.
  // Sequences with nothing to attend get their rows filled on the way:
  // zeros for L <= 0, NaN for a length the table row cannot hold.
  if (tid == 0) carry_lds = 0;
  for (int base = 0; base < S_; base += kPlanThreads) {
    if (tid == 0) dead_count = 0;
    __syncthreads();
    const int s = base + tid;
    const int L = s < S_ ? p.lens[s] : 1;
    const int nt = s < S_ ? live_tiles(L, max_len) : 0;
    if (s < S_ && nt == 0) dead_list[atomicAdd(&dead_count, 1)] = s;
    int incl = nt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o);
      if (lane >= o) incl += v;
    }
    if (lane == 63) wave_sum[wv] = incl;
    __syncthreads();
    int before = carry_lds;
    for (int i = 0; i < wv; ++i) before += wave_sum[i];
    const int excl = before + incl - nt;
    if (s < S_) {
      cum[s] = excl;
      if (s < kPlanLdsCum) cum_lds[s] = excl;
    }
    const int ndead = dead_count;
    for (int k = 0; k < ndead; ++k) {
      const int sd = dead_list[k];
      const int Ld = p.lens[sd];
      const float fill = Ld <= 0 ? 0.f : __builtin_nanf("");
      S* row = (S*)p.out + (size_t)sd * row_elems;
      for (size_t i = tid; i < row_elems; i += kPlanThreads) Cvt<T>::store(row + i, fill);
    }
    __syncthreads();
    if (tid == kPlanThreads - 1) carry_lds = excl + nt;
    __syncthreads();
  }
  const int tot = carry_lds;
  if (tid == 0) {
    cum[S_] = tot;
    if (S_ <= kPlanLdsCum) cum_lds[S_] = tot;
  }
  __syncthreads();

  const int total = tot * p.kvg_count;
  int T_ = total > 0 ? (total + p.grid - 1) / p.grid : 1;
  if (p.cap_tiles > 0 && T_ > p.cap_tiles) T_ = p.cap_tiles;
  const int R = total > 0 ? (total + T_ - 1) / T_ : 0;
  int32_t* desc = p.plan + kHdrWords + S_ + 1;
  int32_t* task = desc + 4 * p.range_cap;
  for (int r = tid; r < R; r += kPlanThreads) {
    const int x = r * T_;
    const int kvg = x / tot;
    const int rem = x - kvg * tot;
    // Last sequence whose first tile is at or before rem (skips empty ones).
    int lo = 0, hi = S_;   // cum[lo] <= rem < cum[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      const int c = S_ <= kPlanLdsCum ? cum_lds[mid] : cum[mid];
      if (c <= rem) lo = mid; else hi = mid;
    }
    const int c_lo = S_ <= kPlanLdsCum ? cum_lds[lo] : cum[lo];
    desc[4 * r + 0] = kvg;
    desc[4 * r + 1] = lo;
    desc[4 * r + 2] = rem - c_lo;
    desc[4 * r + 3] = 0;
    task[r] = -1;
  }
  if (tid == 0) {
    p.plan[kHdrTot] = tot;
    p.plan[kHdrRanges] = R;
    p.plan[kHdrTiles] = T_;
    p.plan[kHdrTotal] = total;
  }
}

// ---------------------------------------------------------------------------
// Range walk shared by both partition kernels.
// ---------------------------------------------------------------------------
struct Segment {
  int kvg, kvh, h0, nh, s, L, t0, take;   // tiles [t0, t0 + take) of sequence s
  bool final;                             // the segment is the whole sequence
  int pair;                               // partial-state slot when not final
};

template <int G, typename Fn>
__device__ __forceinline__ void walk_ranges(const AttnParams& p, Fn&& process) {
  cint* hdr = (cint*)p.plan;
  cint* cum = (cint*)(p.plan + kHdrWords);
  cint* desc = (cint*)(p.plan + kHdrWords + p.num_seqs + 1);
  int32_t* task_out = p.plan + kHdrWords + p.num_seqs + 1 + 4 * p.range_cap;
  const int R = hdr[kHdrRanges];
  const int T_ = hdr[kHdrTiles];
  const int total = hdr[kHdrTotal];
  for (int r = blockIdx.x; r < R; r += gridDim.x) {
    int kvg = desc[4 * r + 0];
    int s = desc[4 * r + 1];
    int t0 = desc[4 * r + 2];
    int remaining = min(T_, total - r * T_);
    int task = -1;
    // The range holds `remaining` tiles of the flattened space; the walk can
    // never pass the last KV-head group, which bounds the loop for any input.
    while (remaining > 0 && kvg < p.kvg_count) {
      const int nt = cum[s + 1] - cum[s];
      const int take = min(nt - t0, remaining);
      if (take > 0) {
        Segment sg;
        sg.kvg = kvg;
        sg.kvh = kvg / p.head_groups;
        const int hg = kvg - sg.kvh * p.head_groups;
        sg.h0 = sg.kvh * p.group + hg * G;
        sg.nh = min(G, p.group - hg * G);
        sg.s = s;
        sg.L = ((cint*)p.lens)[s];
        sg.t0 = t0;
        sg.take = take;
        sg.final = (t0 == 0 && take == nt);
        sg.pair = r + kvg * p.num_seqs + s;
        if (t0 == 0 && !sg.final) task = kvg * p.num_seqs + s;
        process(sg);
        remaining -= take;
      }
      t0 = 0;
      if (++s == p.num_seqs) {
        s = 0;
        ++kvg;
      }
    }
    if (threadIdx.x == 0) task_out[r] = task;
  }
}

// Combine the per-wave (m, l, o) states held in LDS and store the result:
// the final output when the segment is the whole sequence, else its partial
// state (M, weighted l, weighted o) in slot sg.pair.
template <typename T, int D, int G>
__device__ void combine_waves(const AttnParams& p, const Segment& sg, int bad,
                              const float (*red_m)[G], const float (*red_l)[G],
                              const float (*red_acc)[G][D]) {
  using S = typename T::storage;
  for (int idx = threadIdx.x; idx < sg.nh * D; idx += kThreads) {
    const int h = idx / D, d = idx % D;
    float big_m = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) big_m = fmaxf(big_m, red_m[w][h]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = red_m[w][h];
      const float wgt = mw == -INFINITY ? 0.f : fast_exp2(mw - big_m);
      num += wgt * red_acc[w][h][d];
      den += wgt * red_l[w][h];
    }
    if (sg.final) {
      const size_t row = (size_t)sg.s * p.num_q_heads + sg.h0 + h;
      Cvt<T>::store((S*)p.out + row * D + d, bad ? __builtin_nanf("") : num / den);
    } else {
      const size_t slot = (size_t)sg.pair * G + h;
      p.ws_acc[slot * D + d] = bad ? __builtin_nanf("") : num;
      if (d == 0) {
        p.ws_m[slot] = bad ? 0.f : big_m;
        p.ws_l[slot] = bad ? __builtin_nanf("") : den;
      }
    }
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

// ---------------------------------------------------------------------------
// MFMA partition kernel (fp16 / bf16).
// ---------------------------------------------------------------------------
template <typename T, int D, int G>
__global__ __launch_bounds__(kThreads, 2) void attn_partition_mfma(const AttnParams p) {
  using S = typename T::storage;
  constexpr int KCH = D / 32;        // MFMA k-chunks of 32 channels
  constexpr int LPR = D / 8;         // lanes per V row (16 bytes each)
  constexpr int RPL = 64 / LPR;      // V rows per load instruction
  constexpr int TPR = kTile / RPL;   // tokens per V row group per tile
  // Tiles in flight per wave: three when the accumulator is large (G >= 4:
  // occupancy is register bound at two waves per SIMD anyway) and a slot
  // costs <= 32 registers; otherwise two, which keeps small groups at a
  // higher occupancy.
  constexpr int kSlots = ((KCH + TPR) * 4 <= 32 && G >= 4) ? 3 : 2;
  static_assert(D % 32 == 0 && TPR >= 1 && G <= kMaxGroup && G * D <= kMaxGD, "shape");

  // Probabilities of the current tile per head: fp32 for the FMA form,
  // pairs of 16-bit values (tokens 2j, 2j+1) for the dot2 form.
  constexpr bool kDot2 = TPR >= 2;
  __shared__ __align__(16) float p_lds[kWaves][G][kTile];
  __shared__ __align__(16) float alpha_lds[kWaves][G];
  __shared__ float red_m[kWaves][G];
  __shared__ float red_l[kWaves][G];
  __shared__ __align__(16) float red_acc[kWaves][G][D];
  uint32_t (*p2_lds)[G][kTile / 2] = reinterpret_cast<uint32_t (*)[G][kTile / 2]>(p_lds);

  const int lane = threadIdx.x & 63;
  // The wave index is uniform across the wave; saying so lets the tile loop
  // run on scalar branches and the block ids come through scalar loads.
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15;     // A row (token of tile) / B and C column (head)
  const int kgrp = lane >> 4;    // k group of A and B; C rows 4*kgrp .. 4*kgrp+3
  const int vc = lane % LPR;     // V: 16-byte chunk within the row
  const int vr = lane / LPR;     // V: row group, tokens TPR*vr .. TPR*vr+TPR-1
  const size_t bytes = T::bytes;

  walk_ranges<G>(p, [&](const Segment& sg) {
    cint* trow = (cint*)(p.tables + (size_t)sg.s * p.max_blocks);
    const int L = sg.L;
    const int last = L - 1;

    // B operand: query head `col` of this group, channels 32j + 8*kgrp .. +7.
    uint4 qop[KCH];
    {
      const S* qrow = (const S*)p.q + ((size_t)sg.s * p.num_q_heads + sg.h0 + col) * D + kgrp * 8;
#pragma unroll
      for (int j = 0; j < KCH; ++j)
        qop[j] = col < sg.nh ? load16(qrow + 32 * j) : make_uint4(0, 0, 0, 0);
    }

    int bad = 0;
    const int tile_end = sg.t0 + sg.take;
    // Register ring: while one tile is consumed the next kSlots - 1 are in
    // flight.  Loads past the segment's last tile repeat that tile.
    uint4 kb[kSlots][KCH], vb[kSlots][TPR];
    auto issue = [&](auto slot, int tile) {
      constexpr int SL = decltype(slot)::value;
      const int tc = min(tile, tile_end - 1);
      const int tb = tc * kTile;
      int first, nid;
      const int ids = tile_block_ids(p, trow, tb, L, first, nid, bad);
      const int id0 = __builtin_amdgcn_readfirstlane(ids);
      if (nid == 1) {
        // The whole tile lies in one block: one scalar base per pool, and
        // per-lane 32-bit offsets of rows (clamped to the last valid token).
        const int rlim = last - tb;
        const size_t base = row_offset(id0, tb, p.log2_b, p.num_kv_heads, sg.kvh, D) * bytes;
        const char* kbase = p.k_pool + base;
        const char* vbase = p.v_pool + base;
        const uint32_t rstride = (uint32_t)(p.num_kv_heads * D * bytes);
        const uint32_t ko = (uint32_t)min(col, rlim) * rstride + kgrp * 8 * bytes;
#pragma unroll
        for (int j = 0; j < KCH; ++j) kb[SL][j] = load16(kbase + ko + 32 * j * bytes);
#pragma unroll
        for (int i = 0; i < TPR; ++i)
          vb[SL][i] = load16(vbase + (uint32_t)min(TPR * vr + i, rlim) * rstride + vc * 8 * bytes);
      } else {
        auto row = [&](int t, int ch) -> size_t {
          const int tt = min(t, last);
          const int blk = __shfl(ids, (tt >> p.log2_b) - first);
          return (row_offset(blk, tt, p.log2_b, p.num_kv_heads, sg.kvh, D) + ch) * bytes;
        };
        const size_t ko = row(tb + col, kgrp * 8);
#pragma unroll
        for (int j = 0; j < KCH; ++j) kb[SL][j] = load16(p.k_pool + ko + 32 * j * bytes);
#pragma unroll
        for (int i = 0; i < TPR; ++i) vb[SL][i] = load16(p.v_pool + row(tb + TPR * vr + i, vc * 8));
      }
    };

    float m_run = -INFINITY;  // running maximum of head `col` (log2 units)
    float l_run = 0.f;        // normaliser partial: tokens of C row group kgrp
    float acc[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;

    auto consume = [&](auto slot, int tile) {
      constexpr int SL = decltype(slot)::value;
      f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < KCH; ++j) sc = Mfma<T>::run(kb[SL][j], qop[j], sc);
      const int tb = tile * kTile;
      float sv[4];
      float mt = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sv[i] = (tb + 4 * kgrp + i < L) ? sc[i] * p.scale_log2 : -INFINITY;
        mt = fmaxf(mt, sv[i]);
      }
      mt = fmaxf(mt, __shfl_xor(mt, 16));
      mt = fmaxf(mt, __shfl_xor(mt, 32));

      // The previous tile's reads of alpha_lds / p_lds come before this
      // tile's writes.
      wave_lds_sync();
      if (__any(mt > m_run + kRescaleThreshold)) {
        const float mn = fmaxf(m_run, mt);
        const float alpha = fast_exp2(m_run - mn);   // 0 on the first tile
        m_run = mn;
        l_run *= alpha;
        if (kgrp == 0 && col < G) alpha_lds[w][col] = alpha;
        wave_lds_sync();
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float a = alpha_lds[w][h];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[h][e] *= a;
        }
      }

      float pv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pv[i] = fast_exp2(sv[i] - m_run);   // masked: exp2(-inf) = 0
      if constexpr (kDot2) {
        // P rounded to the element type for the dot2 product; the normaliser
        // sums the same rounded values, so the weights still sum to one.
        const uint32_t q01 = Pair<T>::pack(pv[0], pv[1]);
        const uint32_t q23 = Pair<T>::pack(pv[2], pv[3]);
        l_run += (Pair<T>::lo(q01) + Pair<T>::hi(q01)) + (Pair<T>::lo(q23) + Pair<T>::hi(q23));
        if (col < G) *reinterpret_cast<uint2*>(&p2_lds[w][col][2 * kgrp]) = make_uint2(q01, q23);
      } else {
        l_run += (pv[0] + pv[1]) + (pv[2] + pv[3]);
        if (col < G)
          *reinterpret_cast<float4*>(&p_lds[w][col][4 * kgrp]) = make_float4(pv[0], pv[1], pv[2], pv[3]);
      }
      wave_lds_sync();

      // P.V on the vector ALU: lane (vr, vc) owns channels 8vc..8vc+7 of the
      // tile's tokens TPR*vr + i.
      if constexpr (kDot2) {
        constexpr int NP = TPR / 2;   // token pairs per lane
        uint32_t vp[NP][8];           // channel e of tokens (2k, 2k+1)
#pragma unroll
        for (int k = 0; k < NP; ++k) {
          const uint4 a = vb[SL][2 * k], b = vb[SL][2 * k + 1];
          vp[k][0] = pair_lo(a.x, b.x); vp[k][1] = pair_hi(a.x, b.x);
          vp[k][2] = pair_lo(a.y, b.y); vp[k][3] = pair_hi(a.y, b.y);
          vp[k][4] = pair_lo(a.z, b.z); vp[k][5] = pair_hi(a.z, b.z);
          vp[k][6] = pair_lo(a.w, b.w); vp[k][7] = pair_hi(a.w, b.w);
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
          uint32_t pp[NP];
#pragma unroll
          for (int k = 0; k < NP; ++k) pp[k] = p2_lds[w][h][NP * vr + k];
#pragma unroll
          for (int k = 0; k < NP; ++k)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] = Pair<T>::dot2(pp[k], vp[k][e], acc[h][e]);
        }
      } else {
        float vf[TPR][8];
#pragma unroll
        for (int i = 0; i < TPR; ++i) Cvt<T>::unpack(vb[SL][i], vf[i]);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float ph[TPR];
#pragma unroll
          for (int i = 0; i < TPR; ++i) ph[i] = p_lds[w][h][TPR * vr + i];
#pragma unroll
          for (int i = 0; i < TPR; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(ph[i], vf[i][e], acc[h][e]);
        }
      }
    };

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    int tile = sg.t0 + w;
    if (tile < tile_end) {
      if constexpr (kSlots == 3) {
        issue(I0{}, tile);
        issue(I1{}, tile + kWaves);
        while (true) {
          issue(I2{}, tile + 2 * kWaves);
          consume(I0{}, tile);
          tile += kWaves;
          if (tile >= tile_end) break;
          issue(I0{}, tile + 2 * kWaves);
          consume(I1{}, tile);
          tile += kWaves;
          if (tile >= tile_end) break;
          issue(I1{}, tile + 2 * kWaves);
          consume(I2{}, tile);
          tile += kWaves;
          if (tile >= tile_end) break;
        }
      } else {
        issue(I0{}, tile);
        while (true) {
          issue(I1{}, tile + kWaves);
          consume(I0{}, tile);
          tile += kWaves;
          if (tile >= tile_end) break;
          issue(I0{}, tile + kWaves);
          consume(I1{}, tile);
          tile += kWaves;
          if (tile >= tile_end) break;
        }
      }
    }

    // Wave totals: l over the four C row groups, o over the V row groups.
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1)
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] += __shfl_xor(acc[h][e], off);
    if (vr == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        *reinterpret_cast<float4*>(&red_acc[w][h][vc * 8]) =
            make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
        *reinterpret_cast<float4*>(&red_acc[w][h][vc * 8 + 4]) =
            make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
      }
    }
    if (kgrp == 0 && col < G) {
      red_m[w][col] = m_run;
      red_l[w][col] = l_run;
    }
    const int any_bad = __syncthreads_or(bad);
    combine_waves<T, D, G>(p, sg, any_bad, red_m, red_l, red_acc);
    __syncthreads();   // the LDS buffers are reused by the next segment
  });
}

// ---------------------------------------------------------------------------
// Vector-ALU partition kernel (any dtype).
// ---------------------------------------------------------------------------
template <typename T, int D, int G>
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

  walk_ranges<G>(p, [&](const Segment& sg) {
    const int32_t* trow = p.tables + (size_t)sg.s * p.max_blocks;
    float qf[G][E];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if (h < sg.nh) {
        const S* qrow = (const S*)p.q + ((size_t)sg.s * p.num_q_heads + sg.h0 + h) * D + c * E;
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
    const int tok_end = min(sg.L, (sg.t0 + sg.take) * kTile);
    for (int base = tok0 + w * RPL; base < tok_end; base += RPL * kWaves) {
      const int t = base + r;
      const bool valid = t < tok_end;
      const int tt = valid ? t : tok_end - 1;
      int blk = trow[tt >> p.log2_b];
      if (!valid_block(blk, p.num_blocks)) {
        bad = 1;
        blk = 0;
      }
      const size_t off = (row_offset(blk, tt, p.log2_b, p.num_kv_heads, sg.kvh, D) + c * E) * bytes;
      float kf[E], vf[E];
      Cvt<T>::unpack(load16(p.k_pool + off), kf);
      Cvt<T>::unpack(load16(p.v_pool + off), vf);
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
    const int any_bad = __syncthreads_or(bad);
    combine_waves<T, D, G>(p, sg, any_bad, red_m, red_l, red_acc);
    __syncthreads();
  });
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge: the range where a split sequence starts combines the
// partial states of all ranges the sequence covers.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kThreads) void attn_merge(const AttnParams p) {
  using S = typename T::storage;
  constexpr int kChunk = 64;                    // partial states staged per pass
  constexpr int kItems = kMaxGD / kThreads;     // (head, channel) outputs per thread
  __shared__ float w_lds[kChunk][kMaxGroup];    // m of each partial, then its weight
  __shared__ float l_lds[kChunk][kMaxGroup];
  __shared__ float run_m[kMaxGroup], run_den[kMaxGroup], rescale[kMaxGroup];
  cint* hdr = (cint*)p.plan;
  cint* cum = (cint*)(p.plan + kHdrWords);
  cint* task_in = (cint*)(p.plan + kHdrWords + p.num_seqs + 1 + 4 * p.range_cap);
  const int tot = hdr[kHdrTot];
  const int R = hdr[kHdrRanges];
  const int T_ = hdr[kHdrTiles];
  const int G = p.gsize, D = p.head_dim;
  const int tid = threadIdx.x;
  for (int r = blockIdx.x; r < R; r += gridDim.x) {
    const int task = task_in[r];
    if (task < 0) continue;
    const int kvg = task / p.num_seqs;
    const int s = task - kvg * p.num_seqs;
    const int n = (kvg * tot + cum[s + 1] - 1) / T_ - r + 1;   // ranges covered
    const int kvh = kvg / p.head_groups;
    const int hg = kvg - kvh * p.head_groups;
    const int h0 = kvh * p.group + hg * G;
    const int nh = min(G, p.group - hg * G);
    const size_t first_slot = (size_t)(r + task) * G;          // slot of (range r, head 0)
    float num[kItems];
#pragma unroll
    for (int k = 0; k < kItems; ++k) num[k] = 0.f;
    if (tid < nh) {
      run_m[tid] = -INFINITY;
      run_den[tid] = 0.f;
    }
    for (int c0 = 0; c0 < n; c0 += kChunk) {
      const int cn = min(kChunk, n - c0);
      __syncthreads();
      for (int t = tid; t < cn * nh; t += kThreads) {
        const int i = t / nh, h = t - i * nh;
        const size_t slot = first_slot + (size_t)(c0 + i) * G + h;
        w_lds[i][h] = p.ws_m[slot];
        l_lds[i][h] = p.ws_l[slot];
      }
      __syncthreads();
      if (tid < nh) {
        const int h = tid;
        float cm = -INFINITY;
        for (int i = 0; i < cn; ++i) cm = fmaxf(cm, w_lds[i][h]);
        const float mn = fmaxf(run_m[h], cm);
        const float so = run_m[h] == -INFINITY ? 0.f : fast_exp2(run_m[h] - mn);
        float den = run_den[h] * so;
        for (int i = 0; i < cn; ++i) {
          const float wt = fast_exp2(w_lds[i][h] - mn);
          w_lds[i][h] = wt;
          den += wt * l_lds[i][h];
        }
        run_m[h] = mn;
        run_den[h] = den;
        rescale[h] = so;
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < kItems; ++k) {
        const int idx = tid + k * kThreads;
        if (idx < nh * D) {
          const int h = idx / D, d = idx - (idx / D) * D;
          const float* src = p.ws_acc + (first_slot + (size_t)c0 * G + h) * D + d;
          float a = num[k] * rescale[h];
          int i = 0;
          for (; i + 4 <= cn; i += 4) {
            const float x0 = src[(size_t)(i + 0) * G * D], x1 = src[(size_t)(i + 1) * G * D];
            const float x2 = src[(size_t)(i + 2) * G * D], x3 = src[(size_t)(i + 3) * G * D];
            a += w_lds[i][h] * x0 + w_lds[i + 1][h] * x1 + w_lds[i + 2][h] * x2 + w_lds[i + 3][h] * x3;
          }
          for (; i < cn; ++i) a += w_lds[i][h] * src[(size_t)i * G * D];
          num[k] = a;
        }
      }
    }
#pragma unroll
    for (int k = 0; k < kItems; ++k) {
      const int idx = tid + k * kThreads;
      if (idx < nh * D) {
        const int h = idx / D, d = idx - (idx / D) * D;
        Cvt<T>::store((S*)p.out + ((size_t)s * p.num_q_heads + h0 + h) * D + d, num[k] / run_den[h]);
      }
    }
    __syncthreads();   // LDS is reused by the next task
  }
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct WsLayout {
  size_t m_off, l_off, acc_off, total;
};

// Workspace of a call: the plan words, then the partial states.  Pair slots:
// one per (range, sequence slot) along the monotone walk, at most
// range_cap + kvg_count * S of them, G heads each.
inline WsLayout ws_layout(int num_seqs, int kvg_count, int gsize, int head_dim, int range_cap) {
  WsLayout w;
  const size_t plan_words = kHdrWords + (size_t)num_seqs + 1 + 5 * (size_t)range_cap;
  const size_t pairs = (size_t)range_cap + (size_t)kvg_count * num_seqs;
  w.m_off = align256(plan_words * 4);
  w.l_off = w.m_off + align256(pairs * gsize * 4);
  w.acc_off = w.l_off + align256(pairs * gsize * 4);
  w.total = w.acc_off + align256(pairs * gsize * head_dim * 4);
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

template <typename T, int D, int G>
const void* partition_fn(int family) {
  if (family == kFamilyMfma) {
    if constexpr (!std::is_same<T, F32>::value && D >= 32 && G * D <= kMaxGD && (D < 256 || G <= 2))
      return reinterpret_cast<const void*>(&attn_partition_mfma<T, D, G>);
  } else {
    if constexpr (G * D <= kMaxGD && (std::is_same<T, F32>::value || G <= 4))
      return reinterpret_cast<const void*>(&attn_partition_valu<T, D, G>);
  }
  return nullptr;
}

template <typename T, int D>
const void* partition_fn_g(int family, int G) {
  switch (G) {
    case 1: return partition_fn<T, D, 1>(family);
    case 2: return partition_fn<T, D, 2>(family);
    case 4: return partition_fn<T, D, 4>(family);
    default: return partition_fn<T, D, 8>(family);
  }
}

template <typename T>
const void* partition_fn_d(int family, int D, int G) {
  switch (D) {
    case 16: return partition_fn_g<T, 16>(family, G);
    case 32: return partition_fn_g<T, 32>(family, G);
    case 64: return partition_fn_g<T, 64>(family, G);
    case 128: return partition_fn_g<T, 128>(family, G);
    default: return partition_fn_g<T, 256>(family, G);
  }
}

inline const void* pick_partition(int family, int dtype, int D, int G) {
  switch (dtype) {
    case PKV_F32: return partition_fn_d<F32>(family, D, G);
    case PKV_F16: return partition_fn_d<F16>(family, D, G);
    default: return partition_fn_d<BF16>(family, D, G);
  }
}

enum Phase { kPhasePlan = 1, kPhasePartitions = 2, kPhaseMerge = 4, kPhaseAll = 7 };

struct Launch {
  AttnParams p;
  const void* part_fn;
};

// Validates a call and fills the launch description; PKV_OK or an error.
int prepare(int kernel, void* out, const void* q, const void* k_pool, const void* v_pool,
            const int32_t* block_tables, int max_blocks_per_seq, const int32_t* context_lens,
            int num_seqs, int num_blocks, int block_size, int num_q_heads, int num_kv_heads,
            int head_dim, float scale, int partition_tokens, void* workspace,
            size_t workspace_bytes, int dtype, Launch* L) {
  int st = check_pool_shape(num_blocks, block_size, num_kv_heads, head_dim, dtype);
  if (st != PKV_OK) return st;
  if (num_seqs < 0 || max_blocks_per_seq < 1 || num_q_heads < 1 ||
      num_q_heads % num_kv_heads != 0 || !(scale == scale) || scale == INFINITY ||
      scale == -INFINITY)
    return PKV_ERR_INVALID_ARG;
  if (kernel < PKV_ATTN_AUTO || kernel > PKV_ATTN_MFMA) return PKV_ERR_INVALID_ARG;
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

  const int g = num_q_heads / num_kv_heads;
  const int gmax = max_group(head_dim, family, dtype);
  const int G = pow2_at_least(g < gmax ? g : gmax);
  const int head_groups = (g + G - 1) / G;
  const long long kvg = (long long)num_kv_heads * head_groups;
  // Tile counts are 32-bit on the device.
  if ((long long)num_seqs * ((max_len + kTile - 1) / kTile) * kvg >= (1LL << 31))
    return PKV_ERR_INVALID_ARG;
  if (num_seqs == 0) return PKV_OK;
  if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens)
    return PKV_ERR_INVALID_ARG;

  const void* fn = pick_partition(family, dtype, head_dim, G);
  if (!fn) return PKV_ERR_UNSUPPORTED;
  // The merge and plan must size the same layout whichever kernel runs, so
  // the grid is the largest one the device holds of any partition kernel.
  const int grid = device_cu_count() * resident_per_cu(fn);
  const int cap_tiles = partition_tokens / kTile;
  long long range_cap = (long long)device_cu_count() * kMaxWgPerCu;
  if (cap_tiles > 0)
    range_cap += kvg * num_seqs * ((max_len + partition_tokens - 1) / partition_tokens);
  if (range_cap >= (1LL << 30)) return PKV_ERR_INVALID_ARG;
  const WsLayout ws = ws_layout(num_seqs, (int)kvg, G, head_dim, (int)range_cap);
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
  p.cap_tiles = cap_tiles;
  p.grid = grid;
  p.range_cap = (int)range_cap;
  p.scale_log2 = scale * kLog2e;
  L->part_fn = fn;
  return PKV_OK;
}

template <typename T>
hipError_t launch_plan(const AttnParams& p, hipStream_t st) {
  hipLaunchKernelGGL(attn_plan<T>, dim3(1), dim3(kPlanThreads), 0, st, p);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_merge(const AttnParams& p, hipStream_t st) {
  hipLaunchKernelGGL(attn_merge<T>, dim3(p.grid), dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

int decode_attention_impl(int phase, int kernel, void* out, const void* q, const void* k_pool,
                          const void* v_pool, const int32_t* block_tables, int max_blocks_per_seq,
                          const int32_t* context_lens, int num_seqs, int num_blocks,
                          int block_size, int num_q_heads, int num_kv_heads, int head_dim,
                          float scale, int partition_tokens, void* workspace,
                          size_t workspace_bytes, int dtype, void* stream) {
  Launch L;
  const int st = prepare(kernel, out, q, k_pool, v_pool, block_tables, max_blocks_per_seq,
                         context_lens, num_seqs, num_blocks, block_size, num_q_heads,
                         num_kv_heads, head_dim, scale, partition_tokens, workspace,
                         workspace_bytes, dtype, &L);
  if (st != PKV_OK || num_seqs == 0) return st;
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
}  // namespace pkv

extern "C" size_t paged_decode_workspace_bytes(int num_seqs, int num_q_heads, int head_dim,
                                               int max_context_len, int partition_tokens) {
  if (num_seqs < 0 || num_q_heads < 1 || head_dim < 1 || max_context_len < 0 ||
      partition_tokens < 0)
    return 0;
  // Bounds that hold for every KV head count: G <= 8 and kvg_count * G <= 2 * Hq.
  long long range_cap = (long long)pkv::device_cu_count() * pkv::kMaxWgPerCu;
  const long long kvg_bound = 2LL * num_q_heads;
  if (partition_tokens > 0)
    range_cap += kvg_bound * num_seqs *
                 (((long long)max_context_len + partition_tokens - 1) / partition_tokens);
  if (range_cap >= (1LL << 30)) return 0;
  const size_t plan_words = pkv::kHdrWords + (size_t)num_seqs + 1 + 5 * (size_t)range_cap;
  const size_t pair_heads = (size_t)range_cap * pkv::kMaxGroup + (size_t)kvg_bound * num_seqs;
  return pkv::align256(plan_words * 4) + 2 * pkv::align256(pair_heads * 4) +
         pkv::align256(pair_heads * head_dim * 4);
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

extern "C" int paged_decode_attention_plan(PKV_ATTN_ARGS) {
  return pkv::decode_attention_impl(pkv::kPhasePlan, PKV_ATTN_AUTO, PKV_ATTN_PASS);
}

extern "C" int paged_decode_attention_partitions(int kernel, PKV_ATTN_ARGS) {
  return pkv::decode_attention_impl(pkv::kPhasePartitions, kernel, PKV_ATTN_PASS);
}

extern "C" int paged_decode_attention_merge(PKV_ATTN_ARGS) {
  return pkv::decode_attention_impl(pkv::kPhaseMerge, PKV_ATTN_AUTO, PKV_ATTN_PASS);
}
