// decode_attention.hip - paged decode attention for gfx950 (MI355X).
//
// Sources cited by tag and section:
//   [pofe] "PagedAttention: paging the KV cache"
//   [arch] "PagedAttention: Virtual-Memory KV Cache Management, Continuous
//          Batching, and PyTorch Architecture"
//   [lesson] "PagedAttention" lesson in "How Text Is Generated"
//
// What is computed ([pofe] "How it works": ordinary attention regrouped by
// block, addresses indirect; [arch] "3. Non-Contiguous Online Softmax Attention
// Kernel"): for sequence s, query head h, KV head h / g,
//     out[s,h] = sum_{t<L} softmax_t(scale * q . K[t]) V[t]
// with K[t], V[t] fetched through the block table, and a running maximum m,
// normaliser l and unnormalised accumulator o updated block by block.
//
// Work decomposition (one launch + a merge launch):
//   grid = (partition, KV head x head group, sequence), 256 threads = 4 waves.
//   A partition is `part_tokens` consecutive tokens (a multiple of B and 16).
//   Each wave walks 16-token tiles of the partition (tile w, w+4, ...) with its
//   own (m, l, o) state; the four wave states are combined in LDS and written
//   either as the final output (single-partition sequences) or as a partial
//   state that attn_merge combines with the log-sum-exp rule
//   O = sum_p e^(m_p - M) o_p / sum_p e^(m_p - M) l_p.  The pages stop at the
//   per-block recurrence; splitting one sequence over workgroups with this
//   merge is this library's addition, needed to spread long contexts over the
//   256 compute units.
//
// Two partition kernels:
//   attn_partition_mfma  (fp16 / bf16, D >= 32): the grouped score tile
//     S^T[16 tokens x 16 heads] = K_tile . Q^T is one chain of D/32
//     v_mfma_f32_16x16x32 ops whose A operand is loaded straight from the pool
//     (each lane's 8 elements are 16 contiguous bytes of one K row).  P.V is
//     fp32 FMA on the vector ALU: each lane owns 8 channels of one V row group
//     and reads the probabilities of its tokens from a per-wave LDS tile.
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

#include <type_traits>

#include "pkv_common.h"
#include "pkv_host.h"

namespace pkv {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 16;
constexpr float kRescaleThreshold = 8.0f;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kMaxPartTokens = 4096;
constexpr int kMaxGD = 1024;   // G * D bound: the cross-wave LDS buffer is 16 KiB
constexpr int kMaxGroup = 8;   // query heads per workgroup (larger groups are split)

struct AttnParams {
  void* out;
  const void* q;
  const char* k_pool;
  const char* v_pool;
  const int32_t* tables;
  const int32_t* lens;
  float* ws_acc;   // [S, Hq, max_parts, D]
  float* ws_m;     // [S, Hq, max_parts]
  float* ws_l;     // [S, Hq, max_parts]
  int max_blocks;
  int num_blocks;
  int log2_b;
  int num_q_heads;
  int num_kv_heads;
  int group;        // g = Hq / Hkv
  int head_groups;  // ceil(g / G)
  int part_tokens;
  int max_parts;
  float scale_log2;  // scale * log2(e): scores live in log2 units
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

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

// Work item of one workgroup; `live` false means nothing to do.
struct Item {
  int s, kvh, h0, nh, L, nparts, part, p0, pend, lb0, nblk;
  bool live;
};

template <int G>
__device__ __forceinline__ Item make_item(const AttnParams& p) {
  Item it;
  it.part = blockIdx.x;
  it.kvh = blockIdx.y / p.head_groups;
  const int hg = blockIdx.y % p.head_groups;
  it.s = blockIdx.z;
  it.h0 = it.kvh * p.group + hg * G;
  it.nh = min(G, p.group - hg * G);
  it.L = p.lens[it.s];
  it.live = false;
  const int max_len = p.max_blocks << p.log2_b;
  // Empty sequence (zeros) or a length its table row cannot hold (NaN):
  // handled by handle_dead.
  if (it.L <= 0 || it.L > max_len) return it;
  it.nparts = (it.L + p.part_tokens - 1) / p.part_tokens;
  if (it.part >= it.nparts) return it;
  it.p0 = it.part * p.part_tokens;
  it.pend = min(it.L, it.p0 + p.part_tokens);
  it.lb0 = it.p0 >> p.log2_b;
  it.nblk = ((it.pend - 1) >> p.log2_b) - it.lb0 + 1;
  it.live = true;
  return it;
}

// Partition 0 of a sequence with no valid history writes its rows directly.
template <typename T, int D>
__device__ void fill_rows(const AttnParams& p, const Item& it, float value) {
  using S = typename T::storage;
  S* out = (S*)p.out;
  for (int i = threadIdx.x; i < it.nh * D; i += kThreads) {
    const size_t o = ((size_t)it.s * p.num_q_heads + it.h0 + i / D) * D + (i % D);
    Cvt<T>::store(out + o, value);
  }
}

template <typename T, int D>
__device__ __forceinline__ bool handle_dead(const AttnParams& p, const Item& it) {
  if (it.live) return false;
  if (it.part == 0 && (it.L <= 0 || it.L > (p.max_blocks << p.log2_b)))
    fill_rows<T, D>(p, it, it.L <= 0 ? 0.f : __builtin_nanf(""));
  return true;
}

// Stage this partition's block ids in LDS; returns nonzero (for every thread)
// when an id lies outside the pool.
__device__ __forceinline__ int stage_table(const AttnParams& p, const Item& it, int* tbl) {
  int bad = 0;
  for (int i = threadIdx.x; i < it.nblk; i += kThreads) {
    int id = p.tables[(size_t)it.s * p.max_blocks + it.lb0 + i];
    if (!valid_block(id, p.num_blocks)) {
      bad = 1;
      id = 0;
    }
    tbl[i] = id;
  }
  return __syncthreads_or(bad);
}

// Combine the per-wave (m, l, o) states held in LDS and store the result:
// the final output when the sequence has one partition, else the partial
// state (M, sum of weighted l, sum of weighted o) for attn_merge.
template <typename T, int D, int G>
__device__ void combine_waves(const AttnParams& p, const Item& it, int bad,
                              const float (*red_m)[G], const float (*red_l)[G],
                              const float (*red_acc)[G][D]) {
  using S = typename T::storage;
  for (int idx = threadIdx.x; idx < it.nh * D; idx += kThreads) {
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
    const size_t row = (size_t)it.s * p.num_q_heads + it.h0 + h;
    if (it.nparts == 1) {
      const float o = bad ? __builtin_nanf("") : num / den;
      Cvt<T>::store((S*)p.out + row * D + d, o);
    } else {
      const size_t wi = row * p.max_parts + it.part;
      p.ws_acc[wi * D + d] = bad ? __builtin_nanf("") : num;
      if (d == 0) {
        p.ws_m[wi] = bad ? 0.f : big_m;
        p.ws_l[wi] = bad ? __builtin_nanf("") : den;
      }
    }
  }
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
  static_assert(D % 32 == 0 && TPR >= 1 && G <= kMaxGroup && G * D <= kMaxGD, "shape");

  extern __shared__ int tbl[];
  __shared__ __align__(16) float p_lds[kWaves][G][kTile];
  __shared__ __align__(16) float alpha_lds[kWaves][G];
  __shared__ float red_m[kWaves][G];
  __shared__ float red_l[kWaves][G];
  __shared__ __align__(16) float red_acc[kWaves][G][D];

  const Item it = make_item<G>(p);
  if (handle_dead<T, D>(p, it)) return;
  const int bad = stage_table(p, it, tbl);

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int col = lane & 15;     // A row (token of tile) / B and C column (head)
  const int kgrp = lane >> 4;    // k group of A and B; C rows 4*kgrp .. 4*kgrp+3
  const int vc = lane % LPR;     // V: 16-byte chunk within the row
  const int vr = lane / LPR;     // V: row group, tokens TPR*vr .. TPR*vr+TPR-1

  // B operand: query head `col` of this group, channels 32j + 8*kgrp .. +7.
  uint4 qop[KCH];
  {
    const S* qrow = (const S*)p.q + ((size_t)it.s * p.num_q_heads + it.h0 + col) * D + kgrp * 8;
#pragma unroll
    for (int j = 0; j < KCH; ++j)
      qop[j] = col < it.nh ? load16(qrow + 32 * j) : make_uint4(0, 0, 0, 0);
  }

  const int ntok = it.pend - it.p0;
  const int ntiles = (ntok + kTile - 1) / kTile;
  const int last = it.pend - 1;
  const size_t bytes = T::bytes;

  // Byte offset of channel `ch` of token t's row for this KV head; tokens past
  // the partition are clamped to its last token (never used: masked below).
  auto row_bytes = [&](int t, int ch) -> size_t {
    const int tt = min(t, last);
    const int blk = tbl[(tt >> p.log2_b) - it.lb0];
    return (row_offset(blk, tt, p.log2_b, p.num_kv_heads, it.kvh, D) + ch) * bytes;
  };

  uint4 kbuf[KCH], vbuf[TPR];
  auto load_tile = [&](int tile) {
    const int t0 = it.p0 + tile * kTile;
    const size_t ko = row_bytes(t0 + col, kgrp * 8);
#pragma unroll
    for (int j = 0; j < KCH; ++j) kbuf[j] = load16(p.k_pool + ko + 32 * j * bytes);
#pragma unroll
    for (int i = 0; i < TPR; ++i) vbuf[i] = load16(p.v_pool + row_bytes(t0 + TPR * vr + i, vc * 8));
  };

  float m_run = -INFINITY;  // running maximum of head `col` (log2 units)
  float l_run = 0.f;        // normaliser partial: tokens of C row group kgrp
  float acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;

  int tile = w;
  if (tile < ntiles) load_tile(tile);
  for (; tile < ntiles; tile += kWaves) {
    uint4 kcur[KCH], vcur[TPR];
#pragma unroll
    for (int j = 0; j < KCH; ++j) kcur[j] = kbuf[j];
#pragma unroll
    for (int i = 0; i < TPR; ++i) vcur[i] = vbuf[i];
    if (tile + kWaves < ntiles) load_tile(tile + kWaves);

    // Scores S^T[token 4*kgrp+i][head col] for this tile.
    f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < KCH; ++j) sc = Mfma<T>::run(kcur[j], qop[j], sc);
    const int t0 = it.p0 + tile * kTile;
    float sv[4];
    float mt = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[i] = (t0 + 4 * kgrp + i < it.pend) ? sc[i] * p.scale_log2 : -INFINITY;
      mt = fmaxf(mt, sv[i]);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));

    if (__any(mt > m_run + kRescaleThreshold)) {
      const float mn = fmaxf(m_run, mt);
      const float alpha = fast_exp2(m_run - mn);   // 0 on the first tile
      m_run = mn;
      l_run *= alpha;
      if (kgrp == 0 && col < G) alpha_lds[w][col] = alpha;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float a = alpha_lds[w][h];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] *= a;
      }
    }

    float pv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pv[i] = fast_exp2(sv[i] - m_run);   // masked tokens: exp2(-inf) = 0
      l_run += pv[i];
    }
    if (col < G)
      *reinterpret_cast<float4*>(&p_lds[w][col][4 * kgrp]) = make_float4(pv[0], pv[1], pv[2], pv[3]);

    // P.V on the vector ALU: lane (vr, vc) owns channels 8vc..8vc+7 of the
    // tile's tokens TPR*vr + i.
    float vf[TPR][8];
#pragma unroll
    for (int i = 0; i < TPR; ++i) Cvt<T>::unpack(vcur[i], vf[i]);
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
  __syncthreads();
  combine_waves<T, D, G>(p, it, bad, red_m, red_l, red_acc);
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

  extern __shared__ int tbl[];
  __shared__ float red_m[kWaves][G];
  __shared__ float red_l[kWaves][G];
  __shared__ __align__(16) float red_acc[kWaves][G][D];

  const Item it = make_item<G>(p);
  if (handle_dead<T, D>(p, it)) return;
  const int bad = stage_table(p, it, tbl);

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int c = lane % LPR;   // chunk of the row
  const int r = lane / LPR;   // token slot within the wave step
  const size_t bytes = T::bytes;

  float qf[G][E];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    if (h < it.nh) {
      const S* qrow = (const S*)p.q + ((size_t)it.s * p.num_q_heads + it.h0 + h) * D + c * E;
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

  const int last = it.pend - 1;
  for (int base = it.p0 + w * RPL; base < it.pend; base += RPL * kWaves) {
    const int t = base + r;
    const bool valid = t < it.pend;
    const int tt = valid ? t : last;
    const int blk = tbl[(tt >> p.log2_b) - it.lb0];
    const size_t off = (row_offset(blk, tt, p.log2_b, p.num_kv_heads, it.kvh, D) + c * E) * bytes;
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
  __syncthreads();
  combine_waves<T, D, G>(p, it, bad, red_m, red_l, red_acc);
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of partition states: one wave per (sequence, query head).
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(64) void attn_merge(const AttnParams p, int head_dim) {
  using S = typename T::storage;
  extern __shared__ float wts[];
  const int h = blockIdx.x, s = blockIdx.y;
  const int L = p.lens[s];
  if (L <= 0 || L > (p.max_blocks << p.log2_b)) return;   // written by partition 0
  const int nparts = (L + p.part_tokens - 1) / p.part_tokens;
  if (nparts <= 1) return;
  const int lane = threadIdx.x;
  const size_t base = ((size_t)s * p.num_q_heads + h) * p.max_parts;
  float big_m = -INFINITY;
  for (int i = lane; i < nparts; i += 64) big_m = fmaxf(big_m, p.ws_m[base + i]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) big_m = fmaxf(big_m, __shfl_xor(big_m, o));
  float den = 0.f;
  for (int i = lane; i < nparts; i += 64) {
    const float wgt = fast_exp2(p.ws_m[base + i] - big_m);
    wts[i] = wgt;
    den += wgt * p.ws_l[base + i];
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) den += __shfl_xor(den, o);
  __syncthreads();
  for (int d = lane; d < head_dim; d += 64) {
    float num = 0.f;
    for (int i = 0; i < nparts; ++i) num += wts[i] * p.ws_acc[(base + i) * head_dim + d];
    Cvt<T>::store((S*)p.out + ((size_t)s * p.num_q_heads + h) * head_dim + d, num / den);
  }
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
struct WsLayout {
  size_t acc_off, m_off, l_off, total;
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

inline WsLayout ws_layout(int num_seqs, int num_q_heads, int head_dim, int max_parts) {
  WsLayout w{0, 0, 0, 0};
  if (max_parts <= 1) return w;
  const size_t rows = (size_t)num_seqs * num_q_heads * max_parts;
  w.acc_off = 0;
  w.m_off = align256(rows * head_dim * sizeof(float));
  w.l_off = w.m_off + align256(rows * sizeof(float));
  w.total = w.l_off + align256(rows * sizeof(float));
  return w;
}

enum Family { kFamilyValu = 1, kFamilyMfma = 2 };

// Largest head group one workgroup takes: bounded by the cross-wave LDS
// buffer (G * D <= kMaxGD) and by registers (a 16-head group spills).
inline int max_group(int head_dim) {
  const int g = kMaxGD / head_dim;
  return g < kMaxGroup ? g : kMaxGroup;
}

inline int pow2_at_least(int x) {
  int r = 1;
  while (r < x) r <<= 1;
  return r;
}

template <typename T, int D, int G>
void launch_g(int family, const AttnParams& p, dim3 grid, size_t lds, hipStream_t st) {
  if (family == kFamilyMfma) {
    if constexpr (!std::is_same<T, F32>::value && D >= 32 && G * D <= kMaxGD)
      hipLaunchKernelGGL((attn_partition_mfma<T, D, G>), grid, dim3(kThreads), lds, st, p);
  } else {
    if constexpr (G * D <= kMaxGD)
      hipLaunchKernelGGL((attn_partition_valu<T, D, G>), grid, dim3(kThreads), lds, st, p);
  }
}

template <typename T, int D>
void launch_d(int family, int G, const AttnParams& p, dim3 grid, size_t lds, hipStream_t st) {
  switch (G) {
    case 1: launch_g<T, D, 1>(family, p, grid, lds, st); break;
    case 2: launch_g<T, D, 2>(family, p, grid, lds, st); break;
    case 4: launch_g<T, D, 4>(family, p, grid, lds, st); break;
    default: launch_g<T, D, 8>(family, p, grid, lds, st); break;
  }
}

template <typename T>
void launch_t(int family, int D, int G, const AttnParams& p, dim3 grid, size_t lds,
              hipStream_t st) {
  switch (D) {
    case 16: launch_d<T, 16>(family, G, p, grid, lds, st); break;
    case 32: launch_d<T, 32>(family, G, p, grid, lds, st); break;
    case 64: launch_d<T, 64>(family, G, p, grid, lds, st); break;
    case 128: launch_d<T, 128>(family, G, p, grid, lds, st); break;
    default: launch_d<T, 256>(family, G, p, grid, lds, st); break;
  }
}

enum Phase { kPhasePartitions = 1, kPhaseMerge = 2, kPhaseBoth = 3 };

int decode_attention_impl(int phase, int kernel, void* out, const void* q, const void* k_pool,
                          const void* v_pool, const int32_t* block_tables, int max_blocks_per_seq,
                          const int32_t* context_lens, int num_seqs, int num_blocks,
                          int block_size, int num_q_heads, int num_kv_heads, int head_dim,
                          float scale, int partition_tokens, void* workspace,
                          size_t workspace_bytes, int dtype, void* stream) {
  int st = check_pool_shape(num_blocks, block_size, num_kv_heads, head_dim, dtype);
  if (st != PKV_OK) return st;
  if (num_seqs < 0 || num_seqs > 65535 || max_blocks_per_seq < 1 || num_q_heads < 1 ||
      num_q_heads % num_kv_heads != 0 || !(scale == scale) || scale == INFINITY ||
      scale == -INFINITY)
    return PKV_ERR_INVALID_ARG;
  if (kernel < PKV_ATTN_AUTO || kernel > PKV_ATTN_MFMA) return PKV_ERR_INVALID_ARG;
  const int P = partition_tokens == 0 ? 512 : partition_tokens;
  if (P < kTile || P > kMaxPartTokens || P % kTile != 0 || P % block_size != 0)
    return PKV_ERR_INVALID_ARG;
  if (num_seqs == 0) return PKV_OK;
  if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens)
    return PKV_ERR_INVALID_ARG;
  if ((long long)max_blocks_per_seq * block_size > (1LL << 30)) return PKV_ERR_INVALID_ARG;

  int family;
  if (kernel == PKV_ATTN_AUTO)
    family = (dtype != PKV_F32 && head_dim >= 32) ? kFamilyMfma : kFamilyValu;
  else
    family = kernel == PKV_ATTN_MFMA ? kFamilyMfma : kFamilyValu;
  if (family == kFamilyMfma && (dtype == PKV_F32 || head_dim < 32)) return PKV_ERR_UNSUPPORTED;

  const int max_len = max_blocks_per_seq * block_size;
  const int max_parts = (max_len + P - 1) / P;
  const WsLayout ws = ws_layout(num_seqs, num_q_heads, head_dim, max_parts);
  if (ws.total > 0) {
    if (!workspace || workspace_bytes < ws.total || ((uintptr_t)workspace & 255) != 0)
      return PKV_ERR_WORKSPACE;
  }

  const int g = num_q_heads / num_kv_heads;
  const int gmax = max_group(head_dim);
  const int G = pow2_at_least(g < gmax ? g : gmax);
  const int head_groups = (g + G - 1) / G;

  AttnParams p;
  p.out = out;
  p.q = q;
  p.k_pool = (const char*)k_pool;
  p.v_pool = (const char*)v_pool;
  p.tables = block_tables;
  p.lens = context_lens;
  char* wsb = (char*)workspace;
  p.ws_acc = ws.total ? (float*)(wsb + ws.acc_off) : nullptr;
  p.ws_m = ws.total ? (float*)(wsb + ws.m_off) : nullptr;
  p.ws_l = ws.total ? (float*)(wsb + ws.l_off) : nullptr;
  p.max_blocks = max_blocks_per_seq;
  p.num_blocks = num_blocks;
  p.log2_b = log2_exact(block_size);
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.group = g;
  p.head_groups = head_groups;
  p.part_tokens = P;
  p.max_parts = max_parts;
  p.scale_log2 = scale * kLog2e;

  hipStream_t hs = (hipStream_t)stream;
  if (phase & kPhasePartitions) {
    const dim3 grid(max_parts, num_kv_heads * head_groups, num_seqs);
    const size_t tbl_lds = (size_t)(P / block_size) * sizeof(int);
    switch (dtype) {
      case PKV_F32: launch_t<F32>(family, head_dim, G, p, grid, tbl_lds, hs); break;
      case PKV_F16: launch_t<F16>(family, head_dim, G, p, grid, tbl_lds, hs); break;
      default: launch_t<BF16>(family, head_dim, G, p, grid, tbl_lds, hs); break;
    }
    if (hipGetLastError() != hipSuccess) return PKV_ERR_HIP;
  }
  if ((phase & kPhaseMerge) && max_parts > 1) {
    const dim3 mgrid(num_q_heads, num_seqs);
    const size_t mlds = (size_t)max_parts * sizeof(float);
    switch (dtype) {
      case PKV_F32: hipLaunchKernelGGL(attn_merge<F32>, mgrid, dim3(64), mlds, hs, p, head_dim); break;
      case PKV_F16: hipLaunchKernelGGL(attn_merge<F16>, mgrid, dim3(64), mlds, hs, p, head_dim); break;
      default: hipLaunchKernelGGL(attn_merge<BF16>, mgrid, dim3(64), mlds, hs, p, head_dim); break;
    }
    if (hipGetLastError() != hipSuccess) return PKV_ERR_HIP;
  }
  return PKV_OK;
}

}  // namespace
}  // namespace pkv

extern "C" size_t paged_decode_workspace_bytes(int num_seqs, int num_q_heads, int head_dim,
                                               int max_context_len, int partition_tokens) {
  if (num_seqs < 0 || num_q_heads < 1 || head_dim < 1 || max_context_len < 0) return 0;
  const int P = partition_tokens == 0 ? 512 : partition_tokens;
  if (P < 1) return 0;
  const int max_parts = (max_context_len + P - 1) / P;
  return pkv::ws_layout(num_seqs, num_q_heads, head_dim, max_parts).total;
}

extern "C" int paged_decode_attention(void* out, const void* q, const void* k_pool,
                                      const void* v_pool, const int32_t* block_tables,
                                      int max_blocks_per_seq, const int32_t* context_lens,
                                      int num_seqs, int num_blocks, int block_size,
                                      int num_q_heads, int num_kv_heads, int head_dim,
                                      float scale, int partition_tokens, void* workspace,
                                      size_t workspace_bytes, int dtype, void* stream) {
  return pkv::decode_attention_impl(pkv::kPhaseBoth, PKV_ATTN_AUTO, out, q, k_pool, v_pool, block_tables,
                                    max_blocks_per_seq, context_lens, num_seqs, num_blocks,
                                    block_size, num_q_heads, num_kv_heads, head_dim, scale,
                                    partition_tokens, workspace, workspace_bytes, dtype, stream);
}

extern "C" int paged_decode_attention_with(int kernel, void* out, const void* q,
                                           const void* k_pool, const void* v_pool,
                                           const int32_t* block_tables, int max_blocks_per_seq,
                                           const int32_t* context_lens, int num_seqs,
                                           int num_blocks, int block_size, int num_q_heads,
                                           int num_kv_heads, int head_dim, float scale,
                                           int partition_tokens, void* workspace,
                                           size_t workspace_bytes, int dtype, void* stream) {
  return pkv::decode_attention_impl(pkv::kPhaseBoth, kernel, out, q, k_pool, v_pool, block_tables,
                                    max_blocks_per_seq, context_lens, num_seqs, num_blocks,
                                    block_size, num_q_heads, num_kv_heads, head_dim, scale,
                                    partition_tokens, workspace, workspace_bytes, dtype, stream);
}

extern "C" int paged_decode_attention_partitions(
    int kernel, void* out, const void* q, const void* k_pool, const void* v_pool,
    const int32_t* block_tables, int max_blocks_per_seq, const int32_t* context_lens,
    int num_seqs, int num_blocks, int block_size, int num_q_heads, int num_kv_heads,
    int head_dim, float scale, int partition_tokens, void* workspace, size_t workspace_bytes,
    int dtype, void* stream) {
  return pkv::decode_attention_impl(pkv::kPhasePartitions, kernel, out, q, k_pool, v_pool,
                                    block_tables, max_blocks_per_seq, context_lens, num_seqs,
                                    num_blocks, block_size, num_q_heads, num_kv_heads, head_dim,
                                    scale, partition_tokens, workspace, workspace_bytes, dtype,
                                    stream);
}

extern "C" int paged_decode_attention_merge(
    void* out, const void* q, const void* k_pool, const void* v_pool,
    const int32_t* block_tables, int max_blocks_per_seq, const int32_t* context_lens,
    int num_seqs, int num_blocks, int block_size, int num_q_heads, int num_kv_heads,
    int head_dim, float scale, int partition_tokens, void* workspace, size_t workspace_bytes,
    int dtype, void* stream) {
  return pkv::decode_attention_impl(pkv::kPhaseMerge, PKV_ATTN_AUTO, out, q, k_pool, v_pool,
                                    block_tables, max_blocks_per_seq, context_lens, num_seqs,
                                    num_blocks, block_size, num_q_heads, num_kv_heads, head_dim,
                                    scale, partition_tokens, workspace, workspace_bytes, dtype,
                                    stream);
}
