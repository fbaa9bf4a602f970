// prefill_attention.hip - causal chunked prefill over the paged KV cache (gfx950).
//
// Sources cited by tag and section:
//   [pofe]   "PagedAttention: paging the KV cache"
//   [lesson] "PagedAttention" lesson in "How Text Is Generated"
//
// What is computed ([pofe] "How it works": at admission prefill writes the
// prompt into freshly allocated blocks, and attention over a block table is
// the ordinary attention sum, one row of weights per query, regrouped by
// block; [pofe] "When memory runs out" and [lesson] "Preemption": a
// recomputed sequence is prefilled again in one pass): sequence s holds L_s
// positions in the pool, its chunk of n_s query tokens is its last n_s
// positions, and query j (position p = L_s - n_s + j) attends positions
// 0 .. p, the decode rule applied to every token of the chunk:
//     out[j, h] = sum_{t <= p} softmax_t(scale * q[j, h] . K[t, h / g]) V[t, h / g]
//
// Work decomposition: one workgroup per (row block, KV head, sequence),
// where a row is a (chunk token, query head of the KV head's group) pair,
// token-major, so the g heads of a token sit in consecutive rows.  Each of
// the 4 waves owns two groups of 16 rows (one for D = 256 and in the
// shared-prefix mode), so a block holds 128 rows (64).  The workgroup
// streams 32-token K/V tiles from position 0 to the causal limit of its last
// row through two LDS buffers (loads of tile k+1 in flight while tile k is
// used); every wave reads the shared tiles.  Per wave and tile:
//   S^T[16 keys x 16 rows] = K . Q^T   for each 16-key half
//                                      (D/32 v_mfma_f32_16x16x32 each)
//   causal mask per row (on tiles that reach past a row's position), one
//   running max over the 32 keys with lazy rescale, exp2
//   O^T[D x 16 rows] += V^T . P^T      (D/16 v_mfma_f32_16x16x32 over all
//                                       32 keys; P stays in registers, V^T
//                                       comes from transposing LDS reads)
//   l[16 rows] += 1 . P^T               (one more MFMA: the row sums)
// Row blocks are taken from the last (heaviest) one down; workgroups loop
// over further row blocks with stride gridDim.x, so any grid width covers
// every chunk.
//
// Shared-prefix mode (for the cascade decode): the rows are (member, query
// head) pairs of a group whose members share their first blocks; every row
// sees the whole prefix, so only keys past its end are masked.  The prefix's tiles are split
// into `splits` contiguous key ranges, one per workgroup, each producing a
// normalised state and its log normaliser; the cascade's combine step merges
// them with the suffix result by the log-sum-exp rule.
#include <math.h>

#include <type_traits>

#include "pkv_common.h"
#include "pkv_host.h"
#include "pkv_mfma.h"

namespace pkv {
namespace {

typedef const __attribute__((address_space(4))) int32_t cint;   // read with scalar loads

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
// Keys per tile: two halves of 16, whose score products are separate
// 16-key MFMAs and whose P.V products run as one 32-deep MFMA.
constexpr int kTile = 32;
// Row groups of 16 per wave: two for prefill with D <= 128 (the groups share
// every K and V operand read and interleave two MFMA chains); one for
// D = 256, whose registers would not hold two accumulators, and for the
// shared-prefix states, whose short key ranges want more workgroups instead.
constexpr int row_groups(int d, bool prefix) { return (!prefix && d <= 128) ? 2 : 1; }
constexpr int rows_per_block(int d, bool prefix) { return 16 * kWaves * row_groups(d, prefix); }
constexpr float kRescaleThreshold = 8.0f;  // log2 units
constexpr float kLog2e = 1.4426950408889634f;

struct PrefillParams {
  void* out;
  const void* q;
  const char* k_pool;
  const char* v_pool;
  const int32_t* tables;
  const int32_t* lens;
  const int32_t* cu;
  int max_blocks;
  int num_blocks;
  int log2_b;
  int num_q_heads;
  int num_kv_heads;
  int group;          // g = Hq / Hkv
  float scale_log2;   // scale * log2(e) (* k_scale for FP8 pools)
  float v_scale;      // multiplies the weighted V sum (1 unless FP8)
  // Shared-prefix states (the kPrefix kernel): group z has members
  // members[offsets[z] .. offsets[z+1]) sharing their first prefix_blocks[z]
  // table entries; key range r of the prefix gives each member's rows the
  // normalised output over those positions (o_states + r * S * Hq * D, float
  // [S, Hq, D]) and its log normaliser (lse + r * S * Hq, [S, Hq]).  The
  // workgroups of range 0 and KV head 0 also write each member's suffix
  // table row (its entries past the prefix, then -1) and suffix length.
  // Offsets outside [0, num_members] or decreasing skip the group; member
  // ids outside [0, num_seqs) are skipped; a member whose first table
  // entries differ from the group's first member's, or that owners[] counts
  // in more than one group, gets an over-long suffix length (NaN rows).
  const int32_t* offsets;
  const int32_t* members;
  const int32_t* owners;
  int num_members;
  const int32_t* prefix_blocks;
  float* o_states;
  float* lse;
  int splits;          // key ranges per prefix (1 for prefill)
  int num_seqs;
  int32_t* suf_tables;
  int32_t* suf_lens;
};

// 8 pool elements as 8 elements of T: the identity for 16-bit pools, the
// exact decode of 8 E4M3FN codes for FP8 pools.
template <typename T>
__device__ __forceinline__ uint4 widen8_impl(const uint4& v) { return v; }
template <typename T>
__device__ __forceinline__ uint4 widen8_impl(const uint2& c) {
  return make_uint4(Fp8Pair<T>::template decode<false>(c.x), Fp8Pair<T>::template decode<true>(c.x),
                    Fp8Pair<T>::template decode<false>(c.y), Fp8Pair<T>::template decode<true>(c.y));
}

// kWB: blocks of at least 512 / D tokens, so that the rows a wave loads
// for one chunk of a tile lie in one block (see the tile loads).
// kPrefix = false: causal chunked prefill, blockIdx.z = sequence.
// kPrefix = true: attention of every member's query over its group's shared
// prefix (no causal mask; all prefix positions precede the query), blockIdx.z =
// group, blockIdx.x = row block * splits + key range; writes float states
// instead of the output.
template <typename T, int D, bool kPrefix, bool kF8, bool kWB>
// Two workgroups per compute unit (one for D = 256, whose accumulator would
// not fit): this also keeps the MFMA accumulators in ordinary vector
// registers (with a looser bound the compiler places them in the
// accumulation registers and copies all of them out and back every tile).
__global__ __launch_bounds__(kThreads, D <= 128 ? 2 : 1) void attn_prefill_mfma(
    const PrefillParams p) {
  using S = typename T::storage;
  constexpr int LPR = D / 8;                  // 16-byte chunks per K/V row
  constexpr int KCH = D / 32;                 // MFMA k-chunks of 32 channels
  constexpr int VP = D + 16;                  // V tile row pitch (elements)
  constexpr int NCH = kTile * LPR;            // chunks per tile and pool
  constexpr int CPT = (NCH + kThreads - 1) / kThreads;
  constexpr int kRG = row_groups(D, kPrefix);
  constexpr int kRows = rows_per_block(D, kPrefix);   // rows per workgroup
  static_assert(D % 32 == 0 && D <= 256, "head size");

  // K tiles: chunk c of row r at c ^ kswz(r), conflict-free for the row-wise
  // writes and the operand reads.  V tiles: rows padded by 32 bytes, so the
  // transposed reads of a 16-lane group hit distinct banks.
  __shared__ __align__(16) uint4 k_lds[2][kTile * LPR];
  __shared__ __align__(16) uint16_t v_lds[2][kTile * VP];
  __shared__ int bad_lds;
  __shared__ int mism_lds[kPrefix ? kRows : 1];   // prefix mode: per member of a row block
  auto kswz = [](int r) {
    if constexpr (LPR >= 16) return r & 15;
    else if constexpr (LPR == 8) return (r >> 1) & 7;
    else return (r >> 2) & 3;
  };

  // Prefix mode: key range `split` of the prefix's tiles, every workgroup
  // the same amount of work.  Prefill: a row block's work grows with its
  // index (its rows see more keys), so row blocks are dispatched from the
  // last one down.  The linear workgroup index i gives row block
  // gx - 1 - (8 * (i / 8 / P) + i % 8), (KV head, sequence) pair (i / 8) % P
  // (P pairs, gx a multiple of 8): heavy blocks start first and light ones
  // fill in at the end, and eight consecutive workgroups, which the
  // dispatcher places on the eight XCDs in turn, take eight row blocks of
  // one pair, so that the workgroups running on one XCD at a time belong to
  // many pairs.  (Giving all of a pair's row blocks to one XCD raised its L2
  // hit rate from 80 to 86 % and made the kernel 23 % slower: the
  // workgroups of a pair read the same tiles at the same time.)
  int z, kvh, rb_first;
  if constexpr (kPrefix) {
    z = blockIdx.z;
    kvh = blockIdx.y;
    rb_first = (int)(blockIdx.x / p.splits);
  } else {
    const uint64_t per = (uint64_t)gridDim.y * gridDim.z;
    const uint64_t lin =
        blockIdx.x + (uint64_t)gridDim.x * (blockIdx.y + (uint64_t)gridDim.y * blockIdx.z);
    const uint64_t slot = lin >> 3;
    const uint64_t rest = slot % per;
    rb_first = (int)(gridDim.x - 1 - ((slot / per) * 8 + (lin & 7)));
    z = (int)(rest / gridDim.y);
    kvh = (int)(rest % gridDim.y);
  }
  const int split = kPrefix ? (int)(blockIdx.x % p.splits) : 0;
  const int rb_stride = kPrefix ? (int)(gridDim.x / p.splits) : (int)gridDim.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15;    // score tile: key row / query row column
  const int kgrp = lane >> 4;
  const int g = p.group;
  const int max_len = p.max_blocks << p.log2_b;
  // Prefill: the chunk of sequence z is tokens cu0 .. cu0 + n - 1 of q, at
  // positions L - n .. L - 1.  Prefix: the n members of group z, every row
  // attending positions 0 .. L - 1 of the shared prefix (L = its tokens).
  int cu0, n, L;
  bool invalid;
  const int32_t* trow;
  if constexpr (kPrefix) {
    // Offsets outside [0, num_members], or decreasing, name no members: the
    // group is skipped (its sequences keep their whole tables).
    const int lo = p.offsets[z];
    const int hi = p.offsets[z + 1];
    const bool grp_ok = lo >= 0 && hi >= lo && hi <= p.num_members;
    cu0 = grp_ok ? lo : 0;
    n = grp_ok ? hi - lo : 0;
    L = p.prefix_blocks[z] << p.log2_b;
    // The prefix is read through the first member's table row.  A first
    // member outside the batch, or a prefix past the table row, has no
    // defined result: NaN rows.
    const int s0 = n > 0 ? p.members[cu0] : -1;
    const bool ref_ok = s0 >= 0 && s0 < p.num_seqs;
    invalid = !ref_ok || p.prefix_blocks[z] < 0 || p.prefix_blocks[z] > p.max_blocks;
    trow = p.tables + (size_t)(ref_ok ? s0 : 0) * p.max_blocks;
  } else {
    cu0 = p.cu[z];
    n = p.cu[z + 1] - cu0;
    L = p.lens[z];
    // A chunk longer than its history, or a history past the table, has no
    // defined result: its rows are NaN.
    invalid = n > L || L > max_len;
    trow = p.tables + (size_t)z * p.max_blocks;
  }
  const int rows = n * g;
  // Position of row i's query: keys 0 .. pos(i) are visible.
  auto pos_of = [&](int i) { return kPrefix ? L - 1 : L - n + i; };
  // Prefix mode: the sequence of member i, or -1 for an id outside the batch.
  auto member_of = [&](int i) {
    const int s = p.members[cu0 + i];
    return (s >= 0 && s < p.num_seqs) ? s : -1;
  };

  for (int rb = rb_first; rb * kRows < rows; rb += rb_stride) {
    if constexpr (kPrefix) {
      // Suffix tables of the members whose first row lies in this row block.
      if (split == 0 && kvh == 0) {
        const int pb = p.prefix_blocks[z];
        const int i0 = (rb * kRows + g - 1) / g;
        const int i1 = min(n, (rb * kRows + kRows + g - 1) / g);
        // At most kRows members; their (member, table entry) pairs are
        // spread over the workgroup: does the entry match the group's prefix
        // (j < pb), and the suffix table's entry j.
        const int nm = i1 - i0;
        const int mbk = p.max_blocks;
        if (tid < kRows) mism_lds[tid] = 0;
        lds_barrier();
        for (int e = tid; e < nm * mbk; e += kThreads) {
          const int i = e / mbk;
          const int j = e - i * mbk;
          const int s = member_of(i0 + i);
          if (s < 0) continue;
          const size_t row = (size_t)s * mbk;
          if (!invalid && j < pb && p.tables[row + j] != trow[j]) mism_lds[i] = 1;
          p.suf_tables[row + j] = (!invalid && j + pb < mbk) ? p.tables[row + j + pb] : -1;
        }
        lds_barrier();
        if (tid < nm) {
          // A member shorter than the prefix, a prefix past the table, a
          // member whose table does not start with the prefix or one listed
          // in several groups gets an over-long length, which the decode
          // path turns into NaN rows.
          const int s = member_of(i0 + tid);
          if (s >= 0) {
            const int Ls = p.lens[s];
            const bool bad = invalid || Ls < L || mism_lds[tid] != 0 || p.owners[s] != 1;
            p.suf_lens[s] = bad ? max_len + 1 : Ls - L;
          }
        }
      }
    }
    // This lane's rows: column `col` of each of the wave's kRG groups of 16.
    int pos[kRG];
    bool row_ok[kRG];
#pragma unroll
    for (int rg = 0; rg < kRG; ++rg) {
      const int r = rb * kRows + (w * kRG + rg) * 16 + col;
      row_ok[rg] = r < rows && (!kPrefix || member_of(r / g) >= 0);
      pos[rg] = pos_of(row_ok[rg] ? r / g : 0);   // the row's position; keys 0 .. pos
    }
    // Where this lane's row of group rg lives: its element offset in q and
    // in the output (packed token cu0 + i, or member i's sequence) and its
    // state index.  Recomputed where needed instead of held in registers
    // through the tile loop.
    struct RowAddr {
      size_t qoff, state;
    };
    auto row_addr = [&](int rg) {
      const int r = rb * kRows + (w * kRG + rg) * 16 + col;
      const bool ok = r < rows;
      const int i = ok ? r / g : 0;
      const int h = kvh * g + (ok ? r - i * g : 0);
      const size_t qi = kPrefix ? (size_t)(ok ? max(member_of(i), 0) : 0) : (size_t)(cu0 + i);
      return RowAddr{(qi * p.num_q_heads + h) * D,
                     (size_t)split * p.num_seqs * p.num_q_heads + qi * p.num_q_heads + h};
    };
    // Prefix mode: this workgroup's key range, tiles kt_lo .. kt_hi - 1.
    const int all_tiles = (L + kTile - 1) / kTile;
    const int span = kPrefix ? (all_tiles + p.splits - 1) / p.splits : all_tiles;
    const int kt_lo = kPrefix ? min(split * span, all_tiles) : 0;
    const int kt_hi = kPrefix ? min(kt_lo + span, all_tiles) : 0;

    if (invalid || (kPrefix && kt_lo == kt_hi)) {   // uniform across the workgroup
#pragma unroll
      for (int rg = 0; rg < kRG; ++rg) {
        if (!row_ok[rg]) continue;
        const RowAddr ra = row_addr(rg);
        // (Rolled loops: unrolled, their per-lane offsets would be hoisted
        // out of the row-block loop and held in registers throughout.)
        if constexpr (kPrefix) {   // NaN, or an empty key range: sum 0, log 0
          const float v = invalid ? __builtin_nanf("") : 0.f;
#pragma unroll 1
          for (int d = kgrp; d < D; d += 4) p.o_states[ra.state * D + d] = v;
          if (kgrp == 0) p.lse[ra.state] = invalid ? __builtin_nanf("") : -INFINITY;
        } else {
          S* orow = (S*)p.out + ra.qoff;
#pragma unroll 1
          for (int d = kgrp; d < D; d += 4) Cvt<T>::store(orow + d, __builtin_nanf(""));
        }
      }
      continue;
    }

    // Key limits: the workgroup reads keys up to its last row's position,
    // each wave computes up to its own last row's.
    const int last_row = min(rb * kRows + kRows, rows) - 1;
    const int tiles = kPrefix ? kt_hi : pos_of(last_row / g) / kTile + 1;
    const int w_first = rb * kRows + w * 16 * kRG;
    const int w_last = min(w_first + 16 * kRG, rows) - 1;
    const int w_tiles = w_first >= rows ? 0 : kPrefix ? kt_hi : pos_of(w_last / g) / kTile + 1;

    // B operands of the score products: row `col` of each group, channels
    // 32j + 8*kgrp .. +7.
    uint4 qop[kRG][KCH];
#pragma unroll
    for (int rg = 0; rg < kRG; ++rg) {
      const S* qrow = (const S*)p.q + row_addr(rg).qoff + kgrp * 8;
#pragma unroll
      for (int j = 0; j < KCH; ++j)
        qop[rg][j] = row_ok[rg] ? load16(qrow + 32 * j) : make_uint4(0, 0, 0, 0);
    }

    // Tile loads: thread tid takes chunks tid + 256u of the tile, the same
    // chunk of K and of V; rows past L - 1 read row L - 1 (masked anyway).
    // FP8 pools: a chunk is 8 codes (8 bytes), decoded to T when stored to
    // LDS, so the loads stay in flight until then.
    using KvReg = typename std::conditional<kF8, uint2, uint4>::type;
    constexpr int KVB = kF8 ? 1 : T::bytes;   // bytes per pool element
    // bad: a tile the workgroup used held an invalid block id; bad_ld: the
    // tile loaded last did.
    int bad = 0, bad_ld = 0;
    KvReg kreg[CPT], vreg[CPT];
    // Chunk u of a tile is row c / LPR, channels 8 * (c % LPR) .. +7, read
    // from position t = min(32 kt + row, L - 1) (rows past the history read
    // a written position, whose values the mask discards): in the pools at
    // byte blk * blk_bytes + (t mod B) * tok_bytes + lane_off.  A block's
    // bytes stay below 2^32 (at most 128 * 65535 * 256 * 2), so only the
    // block's own offset needs 64 bits.
    const uint64_t tok_bytes = (uint64_t)p.num_kv_heads * D * KVB;
    const uint64_t blk_bytes = tok_bytes << p.log2_b;
    const int bmask = (1 << p.log2_b) - 1;
    const uint32_t lane_off = (uint32_t)(kvh * D + 8 * (lane % LPR)) * KVB;
    // A wave's lanes cover 64 / LPR consecutive rows of each chunk, starting
    // at a multiple of 64 / LPR; with B >= 64 / LPR (kWB) they lie in one
    // block, whose id is then uniform over the wave: a scalar load, and loads
    // addressed as a scalar base plus a 32-bit lane offset.  Smaller blocks
    // take per-lane ids.
    static_assert(64 % LPR == 0, "lane layout");
    auto wave_row0 = [&](int u) { return (64 * w + kThreads * u) / LPR; };
    // Block ids of the tile loaded next, fetched one tile ahead of its data
    // so that the data loads never wait for them.
    int blk_nx[CPT];
    auto chunk_pos = [&](int kt, int c) { return min(kt * kTile + c / LPR, L - 1); };
    auto load_ids = [&](int kt) {
#pragma unroll
      for (int u = 0; u < CPT; ++u) {
        if (NCH % kThreads == 0 || 64 * w + kThreads * u < NCH) {
          if constexpr (kWB)
            blk_nx[u] = ((cint*)trow)[min(kt * kTile + wave_row0(u), L - 1) >> p.log2_b];
          else
            blk_nx[u] = trow[chunk_pos(kt, tid + kThreads * u) >> p.log2_b];
        }
      }
    };
    auto load_tile = [&](int kt) {
      bad_ld = 0;
#pragma unroll
      for (int u = 0; u < CPT; ++u) {
        const int c = tid + kThreads * u;
        if (NCH % kThreads == 0 || 64 * w + kThreads * u < NCH) {
          const uint32_t off =
              (uint32_t)(chunk_pos(kt, c) & bmask) * (uint32_t)tok_bytes + lane_off;
          int blk = blk_nx[u];
          if (!valid_block(blk, p.num_blocks)) {
            bad_ld = 1;
            blk = 0;
          }
          const uint64_t boff = (uint64_t)(uint32_t)blk * blk_bytes;
          if constexpr (kF8) {
            kreg[u] = *reinterpret_cast<const uint2*>(p.k_pool + boff + off);
            vreg[u] = *reinterpret_cast<const uint2*>(p.v_pool + boff + off);
          } else {
            kreg[u] = load16(p.k_pool + boff + off);
            vreg[u] = load16(p.v_pool + boff + off);
          }
        }
      }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
      for (int u = 0; u < CPT; ++u) {
        const int c = tid + kThreads * u;
        if (NCH % kThreads == 0 || c < NCH) {
          const int row = c / LPR;
          const int ch = c - row * LPR;
          k_lds[buf][row * LPR + (ch ^ kswz(row))] = widen8_impl<T>(kreg[u]);
          *reinterpret_cast<uint4*>(&v_lds[buf][row * VP + ch * 8]) = widen8_impl<T>(vreg[u]);
        }
      }
    };

    // Per group: running maximum of row `col` (scaled, log2 units); the
    // row's normaliser, accumulated by the matrix cores as the product of a
    // ones operand with P^T, so every entry holds the sum of the same
    // rounded weights the P.V product uses; O^T, block j holding channels
    // 16j + 4*kgrp .. +3.
    float m_run[kRG];
    f32x4_t l_acc[kRG];
    f32x4_t acc[kRG][D / 16];
#pragma unroll
    for (int rg = 0; rg < kRG; ++rg) {
      m_run[rg] = -INFINITY;
      l_acc[rg] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < D / 16; ++j) acc[rg][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    const uint32_t one2 = Pair<T>::pack(1.f, 1.f);
    const uint4 ones = make_uint4(one2, one2, one2, one2);
    // Tiles wholly at or before the position of the wave's first row need no
    // causal mask (rows past the chunk then compute values from zero queries
    // that are never written).
    const int w_pos0 = w_first >= rows ? -1 : pos_of(w_first / g);

    bool first_tile = true;   // uniform over the wave
    if (tid == 0) bad_lds = 0;
    load_ids(kt_lo);
    load_tile(kt_lo);
    load_ids(kt_lo + 1);
    for (int kt = kt_lo; kt < tiles; ++kt) {
      const int buf = (kt - kt_lo) & 1;
      store_tile(buf);
      bad |= bad_ld;
      // Tile kt visible to every wave; also, every wave is done with buffer
      // buf ^ 1 (read in iteration kt - 1) before it is written next.
      lds_barrier();
      // Loads of tile kt + 1 and the block ids of kt + 2, unconditional so
      // that the compiler's counted waits stay exact; past the last tile
      // they read clamped positions and are never stored.
      load_tile(kt + 1);
      load_ids(kt + 2);
      if (kt < w_tiles) {
        // Scores of the tile's two 16-key halves; the groups' products share
        // each K operand read.
        f32x4_t sc[2][kRG];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int kr = 16 * hf + col;
#pragma unroll
          for (int rg = 0; rg < kRG; ++rg) sc[hf][rg] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int j = 0; j < KCH; ++j) {
            const uint4 ka = k_lds[buf][kr * LPR + ((4 * j + kgrp) ^ kswz(kr))];
#pragma unroll
            for (int rg = 0; rg < kRG; ++rg) sc[hf][rg] = Mfma<T>::run(ka, qop[rg][j], sc[hf][rg]);
          }
        }
        // Lane (col, kgrp) holds keys 32kt + 16hf + 4*kgrp + e of each
        // group's row col.  Causal mask, where the tile reaches past the
        // position of the wave's first row: keys after a row's position, and
        // rows past the chunk, get -inf.
        if (kt * kTile + kTile - 1 > w_pos0) {
          const int t0 = kt * kTile + 4 * kgrp;
#pragma unroll
          for (int rg = 0; rg < kRG; ++rg) {
            const int lim = row_ok[rg] ? pos[rg] - t0 : -1;
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (16 * (e >> 2) + (e & 3) > lim) sc[e >> 2][rg][e & 3] = -INFINITY;
          }
        }
        // Row maxima of both groups first, then one wave-uniform rescale
        // branch for both: the exps and the P.V products after it form one
        // straight stretch in which one group's MFMAs can overlap the other
        // group's vector work.
        float mt[kRG];
        bool jump = false;
#pragma unroll
        for (int rg = 0; rg < kRG; ++rg) {
          float x = -INFINITY;
#pragma unroll
          for (int e = 0; e < 8; ++e) x = fmaxf(x, sc[e >> 2][rg][e & 3]);
          // The scale is positive, so the maximum of the raw scores scales.
          mt[rg] = max_xor32(max_xor16(x)) * p.scale_log2;
          jump |= mt[rg] > m_run[rg] + kRescaleThreshold;
        }
        // Every row's first tile holds a visible key, so m_run is finite from
        // then on (rows past the chunk stay at -inf and are never written).
        // On the first tile the accumulators are still zero: the maxima are
        // taken as they are, with nothing to rescale.
        if (first_tile) {
#pragma unroll
          for (int rg = 0; rg < kRG; ++rg) m_run[rg] = mt[rg];
          first_tile = false;
        } else if (__any(jump)) {
#pragma unroll
          for (int rg = 0; rg < kRG; ++rg) {
            const float mn = fmaxf(m_run[rg], mt[rg]);
            const float alpha = mn == -INFINITY ? 1.f : fast_exp2(m_run[rg] - mn);
            m_run[rg] = mn;
            l_acc[rg] *= alpha;
#pragma unroll
            for (int j = 0; j < D / 16; ++j) acc[rg][j] *= alpha;
          }
        }
        uint4 pop[kRG];
#pragma unroll
        for (int rg = 0; rg < kRG; ++rg) {
          // Weights exp2(scale * s - m), rounded to the element type (0 for
          // masked keys; a row with no visible key yet subtracts 0).  B
          // operand of the P.V product: k index 8*kgrp + e is key 4*kgrp + e
          // of the first half (e < 4), of the second (e >= 4).
          const float neg_m = m_run[rg] == -INFINITY ? 0.f : -m_run[rg];
          float pv[8];
#pragma unroll
          for (int e = 0; e < 8; ++e)
            pv[e] = fast_exp2(fmaf(sc[e >> 2][rg][e & 3], p.scale_log2, neg_m));
          pop[rg] = make_uint4(Pair<T>::pack(pv[0], pv[1]), Pair<T>::pack(pv[2], pv[3]),
                               Pair<T>::pack(pv[4], pv[5]), Pair<T>::pack(pv[6], pv[7]));
        }
        // Row sums of the rounded weights.
#pragma unroll
        for (int rg = 0; rg < kRG; ++rg) l_acc[rg] = Mfma<T>::run(ones, pop[rg], l_acc[rg]);
        // A operand of block j: V[4*kgrp + e][16j + col] and
        // V[16 + 4*kgrp + e][16j + col], two transposed reads shared by the
        // groups, the same key order as P's.
        const uint16_t* vt = &v_lds[buf][(4 * kgrp + (col >> 2)) * VP + 4 * (col & 3)];
#pragma unroll
        for (int j = 0; j < D / 16; ++j) {
          const uint2 v0 = __builtin_bit_cast(uint2, lds_read_tr16(vt + 16 * j));
          const uint2 v1 = __builtin_bit_cast(uint2, lds_read_tr16(vt + 16 * VP + 16 * j));
          const uint4 va = make_uint4(v0.x, v0.y, v1.x, v1.y);
#pragma unroll
          for (int rg = 0; rg < kRG; ++rg) acc[rg][j] = Mfma<T>::run(va, pop[rg], acc[rg][j]);
        }
      }
    }
    if (bad) bad_lds = 1;
    lds_barrier();
    const bool any_bad = bad_lds != 0;
#pragma unroll
    for (int rg = 0; rg < kRG; ++rg) {
      const float lsum = l_acc[rg][0];
      if (!row_ok[rg]) continue;
      const float inv = p.v_scale / lsum;
      const float nan = __builtin_nanf("");
      const RowAddr ra = row_addr(rg);
      if constexpr (kPrefix) {
        float* srow = p.o_states + ra.state * D;
#pragma unroll
        for (int j = 0; j < D / 16; ++j)
          *reinterpret_cast<float4*>(srow + 16 * j + 4 * kgrp) =
              any_bad ? make_float4(nan, nan, nan, nan)
                      : make_float4(acc[rg][j][0] * inv, acc[rg][j][1] * inv,
                                    acc[rg][j][2] * inv, acc[rg][j][3] * inv);
        if (kgrp == 0)   // ln(l * 2^m), m and l in log2 units
          p.lse[ra.state] = any_bad ? nan : (m_run[rg] + log2f(lsum)) * 0.69314718055994531f;
      } else {
        // Channels 16j + 4*kgrp .. +3 of the row: one 8-byte store each.
        const uint32_t nan2 = Pair<T>::pack(nan, nan);
#pragma unroll
        for (int j = 0; j < D / 16; ++j) {
          S* o = (S*)p.out + ra.qoff + 16 * j + 4 * kgrp;
          *reinterpret_cast<uint2*>(o) =
              any_bad ? make_uint2(nan2, nan2)
                      : make_uint2(Pair<T>::pack(acc[rg][j][0] * inv, acc[rg][j][1] * inv),
                                   Pair<T>::pack(acc[rg][j][2] * inv, acc[rg][j][3] * inv));
        }
      }
    }
    // LDS buffers and bad_lds are reused by the next row block.
    lds_barrier();
  }
}

template <typename T, int D, bool kPrefix, bool kF8>
void launch_prefill_d(const PrefillParams& p, dim3 grid, hipStream_t st) {
  // Blocks of at least 512 / D tokens: a wave's rows of a chunk share a block.
  if ((1 << p.log2_b) * D >= 512)
    hipLaunchKernelGGL((attn_prefill_mfma<T, D, kPrefix, kF8, true>), grid, dim3(kThreads), 0, st,
                       p);
  else
    hipLaunchKernelGGL((attn_prefill_mfma<T, D, kPrefix, kF8, false>), grid, dim3(kThreads), 0,
                       st, p);
}

template <typename T, bool kPrefix, bool kF8>
hipError_t launch_prefill(const PrefillParams& p, int head_dim, dim3 grid, hipStream_t st) {
  switch (head_dim) {
    case 32: launch_prefill_d<T, 32, kPrefix, kF8>(p, grid, st); break;
    case 64: launch_prefill_d<T, 64, kPrefix, kF8>(p, grid, st); break;
    case 128: launch_prefill_d<T, 128, kPrefix, kF8>(p, grid, st); break;
    default: launch_prefill_d<T, 256, kPrefix, kF8>(p, grid, st); break;
  }
  return hipGetLastError();
}

// Causal chunked prefill over 16-bit pools (kv_fp8 = false) or FP8 pools,
// whose K scale folds into the score scale and V scale into the output.
int prefill_attention_impl(void* out, const void* q, const void* k_pool, const void* v_pool,
                           const int32_t* cu_seqlens, const int32_t* block_tables,
                           int max_blocks_per_seq, const int32_t* context_lens, int num_seqs,
                           int max_chunk_tokens, int num_blocks, int block_size,
                           int num_q_heads, int num_kv_heads, int head_dim, float scale,
                           int dtype, void* stream, bool kv_fp8, float k_scale, float v_scale) {
  int st = check_pool_shape(num_blocks, block_size, num_kv_heads, head_dim,
                            kv_fp8 ? PKV_FP8_E4M3 : dtype);
  if (st != PKV_OK) return st;
  if (dtype != PKV_F16 && dtype != PKV_BF16) return PKV_ERR_UNSUPPORTED;
  if (head_dim % 32 != 0) return PKV_ERR_UNSUPPORTED;
  if (num_seqs < 0 || num_seqs > 65535 || max_chunk_tokens < 0 || max_blocks_per_seq < 1 ||
      num_q_heads < 1 || num_kv_heads > 65535 || num_q_heads % num_kv_heads != 0 ||
      !(scale > 0.f) || scale == INFINITY)
    return PKV_ERR_INVALID_ARG;
  if (kv_fp8 && (!(k_scale > 0.f) || !(v_scale > 0.f) || k_scale == INFINITY ||
                 v_scale == INFINITY))
    return PKV_ERR_INVALID_ARG;
  if (num_seqs == 0 || max_chunk_tokens == 0) return PKV_OK;
  if (!out || !q || !k_pool || !v_pool || !cu_seqlens || !block_tables || !context_lens)
    return PKV_ERR_INVALID_ARG;
  PrefillParams p{};
  p.out = out;
  p.q = q;
  p.k_pool = (const char*)k_pool;
  p.v_pool = (const char*)v_pool;
  p.tables = block_tables;
  p.lens = context_lens;
  p.cu = cu_seqlens;
  p.splits = 1;
  p.max_blocks = max_blocks_per_seq;
  p.num_blocks = num_blocks;
  p.log2_b = log2_exact(block_size);
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.group = num_q_heads / num_kv_heads;
  p.scale_log2 = scale * kLog2e * (kv_fp8 ? k_scale : 1.f);
  p.v_scale = kv_fp8 ? v_scale : 1.f;
  // The grid's width only sets the parallelism: workgroups loop over any
  // further row blocks of their (KV head, sequence).
  const int rpb = head_dim <= 128 ? rows_per_block(128, false) : rows_per_block(256, false);
  const long long row_blocks = ((long long)max_chunk_tokens * p.group + rpb - 1) / rpb;
  // A multiple of 8 row blocks, which the kernel's dispatch order needs.
  const dim3 grid((unsigned)std::min<long long>((row_blocks + 7) / 8 * 8, 65528), num_kv_heads,
                  num_seqs);
  hipStream_t hs = (hipStream_t)stream;
  hipError_t e;
  if (kv_fp8)
    e = dtype == PKV_F16 ? launch_prefill<F16, false, true>(p, head_dim, grid, hs)
                         : launch_prefill<BF16, false, true>(p, head_dim, grid, hs);
  else
    e = dtype == PKV_F16 ? launch_prefill<F16, false, false>(p, head_dim, grid, hs)
                         : launch_prefill<BF16, false, false>(p, head_dim, grid, hs);
  return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" int paged_prefill_attention(void* out, const void* q, const void* k_pool,
                                       const void* v_pool, const int32_t* cu_seqlens,
                                       const int32_t* block_tables, int max_blocks_per_seq,
                                       const int32_t* context_lens, int num_seqs,
                                       int max_chunk_tokens, int num_blocks, int block_size,
                                       int num_q_heads, int num_kv_heads, int head_dim,
                                       float scale, int dtype, void* stream) {
  return prefill_attention_impl(out, q, k_pool, v_pool, cu_seqlens, block_tables,
                                max_blocks_per_seq, context_lens, num_seqs, max_chunk_tokens,
                                num_blocks, block_size, num_q_heads, num_kv_heads, head_dim,
                                scale, dtype, stream, false, 1.f, 1.f);
}

extern "C" int paged_prefill_attention_fp8(void* out, const void* q, const void* k_pool,
                                           const void* v_pool, const int32_t* cu_seqlens,
                                           const int32_t* block_tables, int max_blocks_per_seq,
                                           const int32_t* context_lens, int num_seqs,
                                           int max_chunk_tokens, int num_blocks, int block_size,
                                           int num_q_heads, int num_kv_heads, int head_dim,
                                           float scale, float k_scale, float v_scale, int dtype,
                                           void* stream) {
  return prefill_attention_impl(out, q, k_pool, v_pool, cu_seqlens, block_tables,
                                max_blocks_per_seq, context_lens, num_seqs, max_chunk_tokens,
                                num_blocks, block_size, num_q_heads, num_kv_heads, head_dim,
                                scale, dtype, stream, true, k_scale, v_scale);
}

namespace pkv {

// Shared-prefix states for the cascade decode: for every member of every
// group and each of `splits` key ranges of the group's shared prefix, the
// normalised attention output over that range (float [splits, S, Hq, D]) and
// its natural log normaliser ([splits, S, Hq]); also the members' suffix
// tables and lengths.  FP8 pools: codes decoded, k_scale in the score scale,
// v_scale in the states.
int launch_prefix_states(const void* q, const void* k_pool, const void* v_pool,
                         const int32_t* tables, const int32_t* lens, int max_blocks,
                         int num_seqs, int num_blocks, int block_size, int num_q_heads,
                         int num_kv_heads, int head_dim, float scale, const int32_t* offsets,
                         const int32_t* members, int num_members,
                         const int32_t* prefix_blocks, int num_groups, int max_group_size,
                         int splits, float* o_states, float* lse, int32_t* suf_tables,
                         int32_t* suf_lens, const int32_t* owners, int dtype, void* stream,
                         bool kv_fp8, float k_scale, float v_scale) {
  PrefillParams p{};
  p.q = q;
  p.k_pool = (const char*)k_pool;
  p.v_pool = (const char*)v_pool;
  p.tables = tables;
  p.lens = lens;
  p.max_blocks = max_blocks;
  p.num_blocks = num_blocks;
  p.log2_b = log2_exact(block_size);
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.group = num_q_heads / num_kv_heads;
  p.scale_log2 = scale * kLog2e * (kv_fp8 ? k_scale : 1.f);
  p.v_scale = kv_fp8 ? v_scale : 1.f;
  p.splits = splits;
  p.num_seqs = num_seqs;
  p.suf_tables = suf_tables;
  p.suf_lens = suf_lens;
  p.offsets = offsets;
  p.members = members;
  p.num_members = num_members;
  p.owners = owners;
  p.prefix_blocks = prefix_blocks;
  p.o_states = o_states;
  p.lse = lse;
  if (splits < 1 || splits > 65535) return PKV_ERR_INVALID_ARG;
  // blockIdx.x = row block * splits + key range; workgroups loop over any
  // further row blocks.
  const int rpb = rows_per_block(head_dim, true);
  const long long row_blocks = ((long long)max_group_size * p.group + rpb - 1) / rpb;
  const long long rbx = std::max<long long>(1, std::min<long long>(row_blocks, 65535 / splits));
  const dim3 grid((unsigned)(rbx * splits), num_kv_heads, num_groups);
  hipStream_t hs = (hipStream_t)stream;
  hipError_t e;
  if (kv_fp8)
    e = dtype == PKV_F16 ? launch_prefill<F16, true, true>(p, head_dim, grid, hs)
                         : launch_prefill<BF16, true, true>(p, head_dim, grid, hs);
  else
    e = dtype == PKV_F16 ? launch_prefill<F16, true, false>(p, head_dim, grid, hs)
                         : launch_prefill<BF16, true, false>(p, head_dim, grid, hs);
  return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

}  // namespace pkv
