/*
 * pagedkv.h - C ABI of libpagedkv, paged KV cache decode for AMD MI355X (gfx950).
 *
 * Sources cited below by tag and section:
 *   [pofe]   "PagedAttention: paging the KV cache" (pofe.ai)
 *   [lesson] "PagedAttention" lesson in "How Text Is Generated" (learn.pranaymahendrakar.com)
 *   [note]   "PagedAttention: Manage the Cache Without Moving the Sequence" (neelmishra.github.io)
 *   [arch]   "PagedAttention: Virtual-Memory KV Cache Management, Continuous Batching,
 *            and PyTorch Architecture" (ailinkdeeptech.com)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every function returns an int status: PKV_OK (0) or a negative PKV_ERR_*.
 *   No C++ exception crosses this boundary.  pkv_status_string() names a code.
 * - Device pointers are owned by the caller and must stay valid until the work
 *   queued on `stream` has finished.  `stream` is a hipStream_t passed as void*
 *   (NULL = the null stream).  Device entry points only enqueue work; they do
 *   not synchronise and they allocate no memory.
 * - Arguments are validated on the host before anything is launched; an invalid
 *   call launches nothing and leaves every buffer untouched.
 * - Layouts are dense row-major; q, out, new tokens and pools start on 16-byte
 *   boundaries (any hipMalloc or torch allocation does).  KV pools are per layer:
 *       k_pool, v_pool : [num_blocks, block_size, num_kv_heads, head_dim]
 *   ([arch] "Production PyTorch Implementation", Step 2 cache tensors; one layer
 *   of the [pofe] "Minimal implementation" pool).  Token t of a sequence lives in
 *   physical block table[t / B] at offset t % B ([arch] "1. Paged Virtual Memory
 *   Mapping"; [note] "Map a ten-token sequence into pages"), so its element
 *   (head h, channel d) sits at ((block * B + t % B) * num_kv_heads + h) * head_dim + d.
 * - block_tables : int32 [num_seqs, max_blocks_per_seq], row s lists the physical
 *   block ids of sequence s in logical order.  Entries at or past ceil(L_s / B) are
 *   never read and may hold anything (for example -1).
 * - q, out : [num_seqs, num_q_heads, head_dim].  Query head h reads KV head
 *   h / (num_q_heads / num_kv_heads) ([pofe] "Minimal implementation" repeats each
 *   KV head over its group; [arch] Step 2 grouped-query ratio).
 * - dtype: q, pools, new tokens and out share one element type (pkv_dtype).
 *   Attention accumulates in fp32 and rounds the output to the element type
 *   with round-to-nearest-even.
 * - Supported shapes: block_size in {1, 2, 4, 8, 16, 32, 64, 128}; head_dim in
 *   {16, 32, 64, 128, 256}.  Other shapes return PKV_ERR_UNSUPPORTED; there is no
 *   slower fallback path.  Attention also needs
 *   num_seqs * ceil(max_blocks_per_seq * block_size / 16) * num_kv_heads * ceil(g / 8)
 *   below 2^31 (PKV_ERR_INVALID_ARG otherwise).
 * - Block ids are the caller's contract: entries a call reads must lie in
 *   [0, num_blocks).  Kernels never touch memory outside the pools for a bad id:
 *   append and copy skip the row, and attention writes NaN for every head of a
 *   sequence whose table names an id outside the pool.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* PKV_FP8_E4M3: pool element type only (the FP8 entry points below, and the
 * byte moves append / copy / gather): OCP E4M3FN codes, one byte each. */
typedef enum pkv_dtype { PKV_F32 = 0, PKV_F16 = 1, PKV_BF16 = 2, PKV_FP8_E4M3 = 3 } pkv_dtype;

enum pkv_status {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = -1,   /* null pointer, negative size, H_q % H_kv != 0, ...      */
  PKV_ERR_UNSUPPORTED = -2,   /* block size, head size or dtype outside the list above  */
  PKV_ERR_NO_FREE_BLOCK = -3, /* host block manager: free list empty ([pofe] "Minimal
                                 implementation" raises MemoryError for a preemption)   */
  PKV_ERR_WORKSPACE = -4,     /* workspace missing or smaller than required             */
  PKV_ERR_HIP = -5,           /* a HIP launch or runtime call failed                    */
  PKV_ERR_ORDER = -6          /* decode phase entry points called out of order for one
                                 workspace, or with arguments unlike its plan's         */
};

/* Name of a status code; never NULL, static storage. */
const char* pkv_status_string(int status);

/* Library version as 10000*major + 100*minor + patch. */
int pkv_version(void);

/* ------------------------------------------------------------------------- */
/* Device operations                                                         */
/* ------------------------------------------------------------------------- */

/*
 * paged_kv_append - write one new token per sequence into its cache slot.
 *
 * [pofe] "How it works", decode step: the new token's k and v go to slot
 * len % B of the block the table lists at index len / B (the last entry, once
 * the host has allocated it); [pofe] "Minimal implementation", Sequence.append.
 *
 *   k_new, v_new     : device, [num_seqs, num_kv_heads, head_dim], dtype
 *   context_lens_pre : device int32 [num_seqs], length BEFORE the append; a
 *                      negative value marks a padding row that writes nothing.
 *   block_tables     : device int32 [num_seqs, max_blocks_per_seq]
 * Writes exactly num_kv_heads*head_dim elements per sequence into each pool and
 * nothing else (bit copy).  Two sequences must not name the same slot.
 */
int paged_kv_append(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                    const int32_t* block_tables, int max_blocks_per_seq,
                    const int32_t* context_lens_pre, int num_seqs, int num_blocks,
                    int block_size, int num_kv_heads, int head_dim, int dtype, void* stream);

/*
 * paged_kv_copy_blocks - copy whole blocks src[i] -> dst[i] in both pools.
 *
 * The copy-on-write copy of [arch] "4. Automatic Prefix Caching (APC) and
 * Copy-on-Write (CoW)" step 2 (all B token slots, all KV heads) and of [pofe]
 * "Minimal implementation".  src, dst: device int32 [num_pairs].  The dst ids
 * must be distinct and must not appear in src (not checked on the device: the
 * ids live in device memory); bit copy.
 */
int paged_kv_copy_blocks(void* k_pool, void* v_pool, const int32_t* src, const int32_t* dst,
                         int num_pairs, int num_blocks, int block_size, int num_kv_heads,
                         int head_dim, int dtype, void* stream);

/*
 * paged_kv_gather - materialise contiguous K and V histories (test / debug).
 *
 * k_out, v_out : device [num_seqs, max_len_out, num_kv_heads, head_dim]; row t of
 * sequence s receives the pool row of token t for t < min(L_s, max_len_out);
 * rows at or past that are left untouched.  Uses the same device index function
 * as attention, so block-table resolution can be checked bit for bit against
 * an explicit gather ([pofe] "Minimal implementation", paged_attention's gather).
 */
int paged_kv_gather(void* k_out, void* v_out, const void* k_pool, const void* v_pool,
                    const int32_t* block_tables, int max_blocks_per_seq,
                    const int32_t* context_lens, int num_seqs, int num_blocks, int block_size,
                    int num_kv_heads, int head_dim, int max_len_out, int dtype, void* stream);

/*
 * paged_decode_workspace_bytes - scratch size paged_decode_attention needs on
 * the current device.
 *
 * The workspace holds the work plan (prefix sums of every sequence's 16-token
 * tiles and one start descriptor per range of work) and the partial softmax
 * states of sequences split across workgroups.  Its size depends on num_seqs,
 * num_q_heads, head_dim, the device's compute-unit count and, when
 * partition_tokens > 0, on max_context_len / partition_tokens.  Returns 0 for
 * invalid arguments.
 */
size_t paged_decode_workspace_bytes(int num_seqs, int num_q_heads, int head_dim,
                                    int max_context_len, int partition_tokens);

/*
 * paged_decode_attention - one decode query token per sequence over its paged
 * KV history.
 *
 * For each sequence s and query head h, with g = num_q_heads / num_kv_heads and
 * L = context_lens[s] (length AFTER this step's append):
 *     out[s,h] = sum_{t<L} softmax_t(scale * q[s,h] . K_s[t, h/g]) * V_s[t, h/g]
 * where K_s[t] is the pool row of token t resolved through block_tables[s].
 * This is the ordinary attention sum regrouped by block ([pofe] "How it works";
 * [arch] "3. Non-Contiguous Online Softmax Attention Kernel": running maximum,
 * normaliser and unnormalised accumulator, in fp32).  L <= 0 yields zeros; a
 * length above max_blocks_per_seq * block_size yields NaN.  Slots at or past L
 * are never read.
 *
 * Work split: the (KV head, sequence, 16-token tile) space is cut into equal
 * ranges, a few per resident workgroup, which the workgroups claim first come
 * first served, so every compute unit stays busy to the end whatever the
 * length mix and however unevenly the memory system serves the units.  Which
 * workgroup takes a range never changes a result.  A sequence cut across ranges is
 * finished by a log-sum-exp merge of the ranges' partial states,
 * O = sum_p e^(m_p-M) o_p / sum_p e^(m_p-M) l_p with M = max_p m_p.
 *   partition_tokens : 0 = balanced ranges (recommended); > 0 = in addition no
 *                      range longer than this many tokens (a multiple of 16),
 *                      i.e. classic fixed split-K partitions.
 *   scale            : usually 1/sqrt(head_dim) ([arch] section 3)
 *   workspace        : device scratch of at least
 *                      paged_decode_workspace_bytes(num_seqs, num_q_heads, head_dim,
 *                          max_blocks_per_seq*block_size, partition_tokens)
 *                      bytes, 256-byte aligned; contents on entry do not matter.
 *                      Calls that share a workspace must not overlap in time.
 */
int paged_decode_attention(void* out, const void* q, const void* k_pool, const void* v_pool,
                           const int32_t* block_tables, int max_blocks_per_seq,
                           const int32_t* context_lens, int num_seqs, int num_blocks,
                           int block_size, int num_q_heads, int num_kv_heads, int head_dim,
                           float scale, int partition_tokens, void* workspace,
                           size_t workspace_bytes, int dtype, void* stream);

/*
 * paged_decode_attention_with - paged_decode_attention with an explicit choice
 * of partition kernel (for measuring one design against the other) and of
 * the cache policy (PKV_ATTN_CACHE_KV below, OR-ed in):
 *   PKV_ATTN_AUTO  the default choice (MFMA for fp16/bf16 with head_dim >= 32,
 *                  vector ALU otherwise);
 *   PKV_ATTN_VALU  the vector-ALU kernel (every dtype and head size);
 *   PKV_ATTN_MFMA  the matrix-core kernel (fp16/bf16, head_dim >= 32 only,
 *                  else PKV_ERR_UNSUPPORTED).
 * Results agree to fp32 rounding; other arguments as paged_decode_attention,
 * which is paged_decode_attention_with(PKV_ATTN_AUTO, ...).  Other bits in
 * `kernel` give PKV_ERR_INVALID_ARG.
 */
enum pkv_attn_kernel {
  PKV_ATTN_AUTO = 0,
  PKV_ATTN_VALU = 1,
  PKV_ATTN_MFMA = 2,
  PKV_ATTN_KERNEL_MASK = 15,
  /* Flag, OR-ed into the kernel choice: blocks are shared between sequences
   * of the batch (a common prefix, forked sequences).  K/V are then read with
   * cache-retaining loads and the rows a workgroup reads are adjacent, so
   * the second and later readers of a block hit in cache.  Without it every
   * block is assumed to be read once per call and K/V are streamed past the
   * caches, which is faster for unshared caches. */
  PKV_ATTN_CACHE_KV = 16
};

int paged_decode_attention_with(int kernel, void* out, const void* q, const void* k_pool,
                                const void* v_pool, const int32_t* block_tables,
                                int max_blocks_per_seq, const int32_t* context_lens,
                                int num_seqs, int num_blocks, int block_size, int num_q_heads,
                                int num_kv_heads, int head_dim, float scale,
                                int partition_tokens, void* workspace, size_t workspace_bytes,
                                int dtype, void* stream);

/*
 * paged_decode_attention_plan / _partitions / _merge - the three launches
 * paged_decode_attention_with(kernel, ...) makes, exposed so a caller can time
 * or schedule them separately.  Same arguments, the same `kernel` in all three
 * (the kernel fixes how heads are grouped, and so the plan's layout); call
 * them in this order on one stream with one workspace.
 *  - plan: one workgroup prefix-sums the tile counts of all sequences, writes
 *    the start of every range of work and fills the rows of sequences with
 *    L <= 0 (zeros) or an over-long L (NaN);
 *  - partitions: persistent workgroups claim ranges from a counter the plan
 *    resets and walk them with the block recurrence of [arch] section 3; a
 *    sequence inside one range gets its final output, a split one leaves
 *    partial states (m, l, o).  Each plan serves one partitions launch: a
 *    second launch needs a new plan;
 *  - merge: the range where a split sequence starts combines its partial
 *    states with the rule above and writes the output.
 * The library holds each workspace (by address) to that order on the host:
 * partitions needs a plan that no partitions launch has used yet, merge needs
 * the partitions launch of that plan, and both need the plan's kernel, dtype,
 * out, block_tables, context_lens, sizes, partition_tokens and
 * workspace_bytes; otherwise PKV_ERR_ORDER and nothing is launched.  A new
 * plan replaces an unused one; any whole attention or decode-step call on the
 * workspace leaves it needing a plan.  The record follows the calls, not the
 * stream, so the three calls must also reach the stream in this order.
 */
int paged_decode_attention_plan(int kernel, void* out, const void* q, const void* k_pool,
                                const void* v_pool, const int32_t* block_tables,
                                int max_blocks_per_seq, const int32_t* context_lens,
                                int num_seqs, int num_blocks, int block_size, int num_q_heads,
                                int num_kv_heads, int head_dim, float scale,
                                int partition_tokens, void* workspace, size_t workspace_bytes,
                                int dtype, void* stream);
int paged_decode_attention_partitions(int kernel, void* out, const void* q, const void* k_pool,
                                      const void* v_pool, const int32_t* block_tables,
                                      int max_blocks_per_seq, const int32_t* context_lens,
                                      int num_seqs, int num_blocks, int block_size,
                                      int num_q_heads, int num_kv_heads, int head_dim,
                                      float scale, int partition_tokens, void* workspace,
                                      size_t workspace_bytes, int dtype, void* stream);
int paged_decode_attention_merge(int kernel, void* out, const void* q, const void* k_pool,
                                 const void* v_pool, const int32_t* block_tables,
                                 int max_blocks_per_seq, const int32_t* context_lens,
                                 int num_seqs, int num_blocks, int block_size, int num_q_heads,
                                 int num_kv_heads, int head_dim, float scale,
                                 int partition_tokens, void* workspace, size_t workspace_bytes,
                                 int dtype, void* stream);

/*
 * paged_decode_step - one decode step: cache append, then attention.
 *
 * [pofe] "How it works", decode step: the new token's k and v are written to
 * the cache (slot (L-1) % B of block table[(L-1) / B], as paged_kv_append
 * with context_lens_pre = L - 1), then attention runs over all L tokens, as
 * paged_decode_attention_with(kernel, ...).  The append rides in the plan
 * launch, so the step is three launches instead of four.
 *   k_pool, v_pool : device, writable (the append writes them)
 *   k_new, v_new   : device, [num_seqs, num_kv_heads, head_dim], dtype; must
 *                    not be NULL when num_seqs > 0 (else PKV_ERR_INVALID_ARG)
 *   context_lens   : device int32 [num_seqs], lengths AFTER the append; a
 *                    sequence with L <= 0 or L > max_blocks_per_seq *
 *                    block_size writes nothing (its output is as attention
 *                    defines: zeros, NaN), nor does one whose block id for
 *                    slot L-1 lies outside the pool (its output is NaN).
 * Other arguments, results and workspace as paged_decode_attention_with.
 * Equivalent bit for bit to paged_kv_append followed by
 * paged_decode_attention_with on the same stream.
 */
int paged_decode_step(int kernel, void* out, const void* q, void* k_pool, void* v_pool,
                      const void* k_new, const void* v_new, const int32_t* block_tables,
                      int max_blocks_per_seq, const int32_t* context_lens, int num_seqs,
                      int num_blocks, int block_size, int num_q_heads, int num_kv_heads,
                      int head_dim, float scale, int partition_tokens, void* workspace,
                      size_t workspace_bytes, int dtype, void* stream);

/*
 * paged_decode_step_noalloc - paged_decode_step with no workspace argument and
 * no allocation, for callers that cannot allocate device memory: work
 * recorded under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.
 *
 * The plan and the partial softmax states live in a library-owned device
 * array of PKV_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU, reserved when the
 * library's code is loaded on that GPU and held until the process ends; the
 * first call on a GPU looks up its address there (with that GPU current).
 * Arguments and results as paged_decode_step (bit for bit the same outputs
 * and pool writes) without workspace / workspace_bytes.  A call whose
 * workspace, as paged_decode_step would lay it out, exceeds the array returns
 * PKV_ERR_WORKSPACE and launches nothing (the five shapes of the benchmark
 * need at most 35 MiB without a partition cap).  The array keeps what the
 * last call left; nothing in it needs clearing, since the plan rewrites
 * every word a call reads.  Every call on one GPU shares that GPU's array:
 * calls that may overlap in time on one GPU (different streams, no ordering
 * between them) race and give wrong results; calls queued on one stream, or
 * otherwise ordered, are safe.
 */
#define PKV_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int paged_decode_step_noalloc(int kernel, void* out, const void* q, void* k_pool, void* v_pool,
                              const void* k_new, const void* v_new, const int32_t* block_tables,
                              int max_blocks_per_seq, const int32_t* context_lens, int num_seqs,
                              int num_blocks, int block_size, int num_q_heads, int num_kv_heads,
                              int head_dim, float scale, int partition_tokens, int dtype,
                              void* stream);

/* paged_decode_attention_lse - paged_decode_attention_with that also writes
 * the natural log of each head's softmax normaliser:
 *   lse : device float [num_seqs, num_q_heads],
 *         lse[s, h] = ln sum_{t < L_s} exp(scale * q[s, h] . K[t, kvh(h)]);
 * -inf for L_s <= 0, NaN where the output row is NaN.  Accurate to about
 * 2e-3 absolute on 16-bit pools (the normaliser sums probabilities rounded
 * to the element type, as the output's weights do).  Two normalised
 * results over disjoint key sets combine exactly with these weights (the
 * block-combining operator of [arch] "3. Non-Contiguous Online Softmax
 * Attention Kernel" applied to normalised parts). */
int paged_decode_attention_lse(int kernel, float* lse, void* out, const void* q,
                               const void* k_pool, const void* v_pool,
                               const int32_t* block_tables, int max_blocks_per_seq,
                               const int32_t* context_lens, int num_seqs, int num_blocks,
                               int block_size, int num_q_heads, int num_kv_heads, int head_dim,
                               float scale, int partition_tokens, void* workspace,
                               size_t workspace_bytes, int dtype, void* stream);

/*
 * paged_decode_attention_cascade - decode attention that reads each shared
 * prefix once per group of sequences ([lesson] "Sharing, and the reference
 * counting it needs": sequences with a common prompt prefix share its
 * blocks; [pofe] "Sharing and copy-on-write").  Group z has the members
 * group_members[group_offsets[z] .. group_offsets[z+1]) (device int32;
 * group_members holds num_members ids), which share their first
 * group_prefix_blocks[z] table entries; a sequence belongs to at most one
 * group; max_group_size bounds the member counts and only sizes the launch.
 * pkv_bm_export_cascade_groups produces such groups from the block manager
 * and pkv_validate_cascade_groups checks them on the host.  The kernels
 * check the contract too, and never read or write outside the buffers for
 * a broken one: a group whose offsets leave [0, num_members] or decrease is
 * skipped (its sequences get plain decode attention), member ids outside
 * [0, num_seqs) are skipped, and a member listed in two groups, whose table
 * does not start with the group's first member's prefix entries, or whose
 * group's first member id is outside the batch, gets NaN rows.  Result: the
 * same attention as paged_decode_attention_with, computed as
 *   - the group's queries against the prefix blocks, read once (matrix
 *     cores, states in float), the prefix split into up to 8 key ranges
 *     (one per 128 table tokens at most) so that the launch fills the GPU;
 *   - paged_decode_attention_lse over each sequence's remaining blocks;
 *   - per member, O = sum_r e^(a_r - M) O_r / sum_r e^(a_r - M) over the
 *     prefix ranges and the rest, a_r their log normalisers, M = max a_r.
 * Sequences outside every group get plain decode attention; with
 * num_groups = 0 the call is paged_decode_attention_with on the tables as
 * given (same launches, no extra work).  A member
 * shorter than its group's prefix, or a prefix longer than the table row,
 * gets NaN rows.  F16 / BF16 pools, head_dim % 32 == 0.  Workspace:
 * paged_decode_cascade_workspace_bytes (256-byte aligned). */
size_t paged_decode_cascade_workspace_bytes(int num_seqs, int num_q_heads, int head_dim,
                                            int max_blocks_per_seq, int block_size);
int paged_decode_attention_cascade(int kernel, void* out, const void* q, const void* k_pool,
                                   const void* v_pool, const int32_t* block_tables,
                                   int max_blocks_per_seq, const int32_t* context_lens,
                                   int num_seqs, const int32_t* group_offsets,
                                   const int32_t* group_members, int num_members,
                                   const int32_t* group_prefix_blocks, int num_groups,
                                   int max_group_size, int num_blocks, int block_size,
                                   int num_q_heads, int num_kv_heads, int head_dim, float scale,
                                   void* workspace, size_t workspace_bytes, int dtype,
                                   void* stream);

/* paged_decode_attention_cascade_fp8 - paged_decode_attention_cascade over
 * FP8 pools (the key of token t is decode(code) * k_scale, its value
 * decode(code) * v_scale, as for paged_decode_attention_fp8): the prefix
 * states and the suffix decode both decode the codes into 16-bit operands.
 * q and out have element type dtype (F16 or BF16); k_scale and v_scale
 * finite and > 0.  Workspace: paged_decode_cascade_workspace_bytes. */
int paged_decode_attention_cascade_fp8(int kernel, void* out, const void* q, const void* k_pool,
                                       const void* v_pool, const int32_t* block_tables,
                                       int max_blocks_per_seq, const int32_t* context_lens,
                                       int num_seqs, const int32_t* group_offsets,
                                       const int32_t* group_members, int num_members,
                                       const int32_t* group_prefix_blocks, int num_groups,
                                       int max_group_size, int num_blocks, int block_size,
                                       int num_q_heads, int num_kv_heads, int head_dim,
                                       float scale, float k_scale, float v_scale,
                                       void* workspace, size_t workspace_bytes, int dtype,
                                       void* stream);

/* ------------------------------------------------------------------------- */
/* FP8 cache blocks                                                           */
/* ------------------------------------------------------------------------- */

/*
 * [pofe] "Fine-tuned models and adapters": an FP8 cache halves the bytes per
 * block and nothing else about paging changes; [pofe] "Failure modes": once
 * the cache dominates step time, fewer bytes per token is the lever.  The
 * pages fix no format or scale; this library uses:
 *   - codes: OCP E4M3FN (bias 7, 3 mantissa bits, no infinities,
 *     S.1111.111 = NaN, largest finite 448), PKV_FP8_E4M3 pools;
 *   - one float32 scale per pool (k_scale for K, v_scale for V): a code c
 *     stands for decode(c) * scale, and a value x is stored as
 *     encode(fp32(x) / fp32(scale)), nearest with ties to even, magnitudes
 *     >= 448 saturating to +-448, NaN kept (0x7F, or 0xFF for a negative
 *     sign bit).
 * Scales must be finite and > 0 (else PKV_ERR_INVALID_ARG).  Pools are laid
 * out as the 16-bit pools, one byte per element; copy and gather move FP8
 * pools like any other (dtype PKV_FP8_E4M3).
 */

/* paged_kv_append_fp8 - paged_kv_append into FP8 pools: k_new, v_new
 * [num_seqs, num_kv_heads, head_dim] of new_dtype (F32, F16 or BF16) are
 * quantised as above.  Same slot rules and padding rows as paged_kv_append. */
int paged_kv_append_fp8(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                        const int32_t* block_tables, int max_blocks_per_seq,
                        const int32_t* context_lens_pre, int num_seqs, int num_blocks,
                        int block_size, int num_kv_heads, int head_dim, int new_dtype,
                        float k_scale, float v_scale, void* stream);

/* paged_decode_attention_fp8 - paged_decode_attention_with over FP8 pools:
 * the key of token t is decode(code) * k_scale, its value decode(code) *
 * v_scale.  q and out have element type dtype (F16 or BF16; F32 gives
 * PKV_ERR_UNSUPPORTED), head_dim >= 32, and the matrix-core kernel runs
 * (PKV_ATTN_VALU gives PKV_ERR_UNSUPPORTED).  Codes are decoded exactly into
 * the 16-bit operands; k_scale is folded into the softmax scale and v_scale
 * applied to the weighted sum, both in fp32.  Workspace as
 * paged_decode_workspace_bytes. */
int paged_decode_attention_fp8(int kernel, void* out, const void* q, const void* k_pool,
                               const void* v_pool, const int32_t* block_tables,
                               int max_blocks_per_seq, const int32_t* context_lens,
                               int num_seqs, int num_blocks, int block_size, int num_q_heads,
                               int num_kv_heads, int head_dim, float scale, float k_scale,
                               float v_scale, int partition_tokens, void* workspace,
                               size_t workspace_bytes, int dtype, void* stream);

/* paged_decode_step_fp8 - paged_decode_step over FP8 pools: token L-1 (k_new,
 * v_new in dtype) is quantised into its slot as paged_kv_append_fp8 does,
 * then paged_decode_attention_fp8 runs; equivalent bit for bit to the two
 * calls on one stream. */
int paged_decode_step_fp8(int kernel, void* out, const void* q, void* k_pool, void* v_pool,
                          const void* k_new, const void* v_new, const int32_t* block_tables,
                          int max_blocks_per_seq, const int32_t* context_lens, int num_seqs,
                          int num_blocks, int block_size, int num_q_heads, int num_kv_heads,
                          int head_dim, float scale, float k_scale, float v_scale,
                          int partition_tokens, void* workspace, size_t workspace_bytes,
                          int dtype, void* stream);

/*
 * Per-head FP8 scales: the three calls above with one float32 scale per KV
 * head and pool instead of one per pool.  The pages fix no scale convention
 * ([pofe] "Fine-tuned models and adapters" only says FP8 halves the bytes of
 * a block); per-tensor and per-head scales are the two usual choices, and
 * these calls take the second:
 *   k_scales, v_scales : device float32 [num_kv_heads], owned by the caller,
 *                        read by the kernels (not copied); head h's codes
 *                        follow the per-pool rule above with k_scales[h] /
 *                        v_scales[h].  NULL with num_seqs > 0 gives
 *                        PKV_ERR_INVALID_ARG.
 * The host cannot see device values, so an entry that is not finite and > 0
 * is handled on the device: the append stores the NaN code 0x7F in every
 * element of that head of that pool, and attention writes NaN to the rows of
 * that head's query heads (either of the head's two scales being unusable is
 * enough).  Everything
 * else as paged_kv_append_fp8, paged_decode_attention_fp8 and
 * paged_decode_step_fp8; with all entries equal to s the results are bit
 * for bit those of the per-pool calls at scale s.  Chunked prefill and the
 * cascade take per-pool scales only.
 */
int paged_kv_append_fp8_per_head(void* k_pool, void* v_pool, const void* k_new,
                                 const void* v_new, const int32_t* block_tables,
                                 int max_blocks_per_seq, const int32_t* context_lens_pre,
                                 int num_seqs, int num_blocks, int block_size, int num_kv_heads,
                                 int head_dim, int new_dtype, const float* k_scales,
                                 const float* v_scales, void* stream);
int paged_decode_attention_fp8_per_head(int kernel, void* out, const void* q,
                                        const void* k_pool, const void* v_pool,
                                        const int32_t* block_tables, int max_blocks_per_seq,
                                        const int32_t* context_lens, int num_seqs,
                                        int num_blocks, int block_size, int num_q_heads,
                                        int num_kv_heads, int head_dim, float scale,
                                        const float* k_scales, const float* v_scales,
                                        int partition_tokens, void* workspace,
                                        size_t workspace_bytes, int dtype, void* stream);
int paged_decode_step_fp8_per_head(int kernel, void* out, const void* q, void* k_pool,
                                   void* v_pool, const void* k_new, const void* v_new,
                                   const int32_t* block_tables, int max_blocks_per_seq,
                                   const int32_t* context_lens, int num_seqs, int num_blocks,
                                   int block_size, int num_q_heads, int num_kv_heads,
                                   int head_dim, float scale, const float* k_scales,
                                   const float* v_scales, int partition_tokens,
                                   void* workspace, size_t workspace_bytes, int dtype,
                                   void* stream);

/* ------------------------------------------------------------------------- */
/* Swap: preemption to host memory                                           */
/* ------------------------------------------------------------------------- */

/*
 * [pofe] "When memory runs out": a preempted sequence's blocks (all or none)
 * are copied to CPU memory and back later; [lesson] "Preemption": swap copies
 * blocks to pinned host memory and back, costing link bandwidth and no
 * compute.  One launch moves any list of scattered blocks:
 *   block_ids      : device int32 [num], block i of the list;
 *   host_k, host_v : pinned, device-mapped host memory (hipHostMalloc, or a
 *                    torch tensor made with pin_memory=True), each
 *                    [num, block_size, num_kv_heads, head_dim] of the pool
 *                    dtype (any pool dtype, FP8 included): slot i holds block
 *                    block_ids[i], bit for bit.
 * An id outside [0, num_blocks) is skipped (its slot or block is left
 * untouched).  Swap-in destinations must be distinct.  The host buffers must
 * stay allocated until the stream has finished the copy.  The block manager
 * (pkv_bm_seq_swap_out / _in) decides which blocks move.
 */
int paged_kv_swap_out(const void* k_pool, const void* v_pool, const int32_t* block_ids, int num,
                      void* host_k, void* host_v, int num_blocks, int block_size,
                      int num_kv_heads, int head_dim, int dtype, void* stream);
int paged_kv_swap_in(void* k_pool, void* v_pool, const int32_t* block_ids, int num,
                     const void* host_k, const void* host_v, int num_blocks, int block_size,
                     int num_kv_heads, int head_dim, int dtype, void* stream);

/* ------------------------------------------------------------------------- */
/* Chunked prefill                                                           */
/* ------------------------------------------------------------------------- */

/*
 * [pofe] "How it works": at admission the prompt's blocks are allocated and
 * prefill writes into them; [pofe] "When memory runs out" and [lesson]
 * "Preemption": a recomputed sequence is prefilled again, prompt and
 * generated tokens, in one pass.  A prefill batch is packed: sequence s
 * contributes the n_s = cu_seqlens[s+1] - cu_seqlens[s] tokens
 * cu_seqlens[s] .. cu_seqlens[s+1]-1 of the packed arrays.
 *   cu_seqlens : device int32 [num_seqs + 1], cu_seqlens[0] = 0, non-decreasing;
 *                tokens of the packed arrays outside [cu_seqlens[0],
 *                cu_seqlens[num_seqs]) belong to no sequence.
 */

/* paged_kv_append_tokens - write each sequence's run of new tokens into its
 * cache slots: packed token cu_seqlens[s] + j (k_new, v_new : device
 * [num_tokens, num_kv_heads, head_dim], dtype) goes to position
 * context_lens_pre[s] + j, i.e. slot (that position) % B of block
 * table[(that position) / B].  A negative context_lens_pre[s] marks a padding
 * row that writes nothing; positions past the table row or naming an id
 * outside the pool are skipped.  Bit copy; nothing else is written.  Two
 * tokens must not name the same slot. */
int paged_kv_append_tokens(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                           const int32_t* cu_seqlens, int num_tokens,
                           const int32_t* block_tables, int max_blocks_per_seq,
                           const int32_t* context_lens_pre, int num_seqs, int num_blocks,
                           int block_size, int num_kv_heads, int head_dim, int dtype,
                           void* stream);

/* paged_prefill_attention - causal attention of each sequence's chunk over
 * its paged history.  context_lens[s] = L_s counts every position in the
 * pool including the chunk's own (append them first); the chunk is the last
 * n_s positions, so packed query token cu_seqlens[s] + j sits at position
 * p = L_s - n_s + j and attends positions 0 .. p (the pages leave the mask
 * implicit; this is the decode rule applied to every chunk token):
 *     out[j, h] = sum_{t <= p} softmax_t(scale * q[j, h] . K[t, h / g]) V[t, h / g]
 *   q, out : device [num_tokens, num_q_heads, head_dim], dtype F16 or BF16
 *            (F32 gives PKV_ERR_UNSUPPORTED; FP8 pools take
 *            paged_prefill_attention_fp8), head_dim % 32 == 0.
 *   max_chunk_tokens : host upper bound on n_s used to size the launch; any
 *            value >= 1 computes every row (a smaller one only runs with
 *            less parallelism).
 * A sequence with n_s > L_s or L_s > max_blocks_per_seq * block_size gets NaN
 * rows; one whose table names an id outside the pool gets NaN rows for the
 * rows of every workgroup that read it.  Needs no workspace. */
int paged_prefill_attention(void* out, const void* q, const void* k_pool, const void* v_pool,
                            const int32_t* cu_seqlens, const int32_t* block_tables,
                            int max_blocks_per_seq, const int32_t* context_lens, int num_seqs,
                            int max_chunk_tokens, int num_blocks, int block_size,
                            int num_q_heads, int num_kv_heads, int head_dim, float scale,
                            int dtype, void* stream);

/* paged_kv_append_tokens_fp8 - paged_kv_append_tokens into FP8 pools: the
 * packed rows k_new, v_new [num_tokens, num_kv_heads, head_dim] of new_dtype
 * (F32, F16 or BF16) are quantised as paged_kv_append_fp8 does, code =
 * encode(fp32(x) / fp32(scale)).  Same positions, padding rows and skips as
 * paged_kv_append_tokens; k_scale, v_scale finite and > 0. */
int paged_kv_append_tokens_fp8(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                               const int32_t* cu_seqlens, int num_tokens,
                               const int32_t* block_tables, int max_blocks_per_seq,
                               const int32_t* context_lens_pre, int num_seqs, int num_blocks,
                               int block_size, int num_kv_heads, int head_dim, int new_dtype,
                               float k_scale, float v_scale, void* stream);

/* paged_prefill_attention_fp8 - paged_prefill_attention over FP8 pools: the
 * key of position t is decode(code) * k_scale, its value decode(code) *
 * v_scale ([pofe] "Fine-tuned models and adapters": an FP8 cache changes
 * nothing else about paging).  q and out have element type dtype (F16 or
 * BF16); codes are decoded exactly into the 16-bit operands, k_scale is
 * folded into the softmax scale and v_scale applied to the weighted sum,
 * both in fp32.  Other arguments, results and error rows as
 * paged_prefill_attention. */
int paged_prefill_attention_fp8(void* out, const void* q, const void* k_pool, const void* v_pool,
                                const int32_t* cu_seqlens, const int32_t* block_tables,
                                int max_blocks_per_seq, const int32_t* context_lens,
                                int num_seqs, int max_chunk_tokens, int num_blocks,
                                int block_size, int num_q_heads, int num_kv_heads, int head_dim,
                                float scale, float k_scale, float v_scale, int dtype,
                                void* stream);

/* ------------------------------------------------------------------------- */
/* Host block manager (CPU only; no device calls)                            */
/* ------------------------------------------------------------------------- */
/*
 * Free list, reference counts and per-sequence block tables with fork and
 * copy-on-write, as in [pofe] "Minimal implementation" (BlockPool, Sequence)
 * and the decode-step pseudocode of [pofe] "How it works":
 *  - the free list starts as 0..N-1 and hands out the id at its end (LIFO);
 *  - alloc sets a block's count to 1, share adds 1, release subtracts 1 and
 *    returns the block to the free list at 0 ([note] "Shared prefixes can share
 *    physical storage");
 *  - appending token `len`: if len % B == 0 a block is allocated and appended to
 *    the table; else if the last block's count is > 1 a block is allocated, the
 *    caller must copy old -> new (paged_kv_copy_blocks), the old block is
 *    released and the last entry remapped ([arch] section 4, steps 1-4).
 * Any call that returns PKV_ERR_NO_FREE_BLOCK leaves all state unchanged.
 * A manager is not thread safe; use one per thread or lock around it.
 */
typedef struct pkv_block_manager pkv_block_manager;

int pkv_bm_create(int num_blocks, int block_size, pkv_block_manager** out);
void pkv_bm_destroy(pkv_block_manager* bm);

int pkv_bm_num_free(const pkv_block_manager* bm);           /* >= 0, or error */
int pkv_bm_refcount(const pkv_block_manager* bm, int block); /* >= 0, or error */
int pkv_bm_alloc(pkv_block_manager* bm, int* block_out);
int pkv_bm_share(pkv_block_manager* bm, int block);          /* block must be allocated */
int pkv_bm_release(pkv_block_manager* bm, int block);        /* block must be allocated */

/* Sequences are named by small non-negative ids the manager hands out. */
int pkv_bm_seq_new(pkv_block_manager* bm, int* seq_out);
/* Admission / prefill: allocate the blocks n_tokens more prompt tokens need
 * ([pofe] "How it works", admit pseudocode).  The current last block must not
 * be a shared partial block. */
int pkv_bm_seq_extend(pkv_block_manager* bm, int seq, int n_tokens);
/* Start an empty sequence on the first n_blocks full blocks of src, shared
 * (a prefix hit: [arch] section 4). */
int pkv_bm_seq_adopt_prefix(pkv_block_manager* bm, int seq, int src, int n_blocks);
/* Parallel sampling: a new sequence sharing every block of parent ([pofe]
 * "Sharing and copy-on-write"). */
int pkv_bm_seq_fork(pkv_block_manager* bm, int parent, int* child_out);
/* Decide the slot of the next token; *cow_src_out is the block to copy from
 * (into *block_out) or -1 when no copy is needed.  len grows by one. */
int pkv_bm_seq_append_slot(pkv_block_manager* bm, int seq, int* block_out, int* slot_out,
                           int* cow_src_out);
/* One decode step for a batch: append_slot for seqs[0..n), all or nothing
 * (if the free list cannot cover every allocation nothing changes).
 * block_out, slot_out: [n]; cow_src_out, cow_dst_out: [n] (first *num_cow used). */
int pkv_bm_append_batch(pkv_block_manager* bm, const int* seqs, int n, int32_t* block_out,
                        int32_t* slot_out, int32_t* cow_src_out, int32_t* cow_dst_out,
                        int* num_cow_out);
int pkv_bm_seq_free(pkv_block_manager* bm, int seq);        /* release all blocks; id retired */
/* Preemption by swapping ([pofe] "When memory runs out": whole sequences).
 * swap_out writes seq's table (the blocks to copy out with paged_kv_swap_out;
 * host slot i = logical block i) to blocks_out[0..*n_out), releases every
 * block, shared ones included, and keeps the length; the sequence is then
 * swapped: append, extend, fork, adopt-prefix and export refuse it
 * (PKV_ERR_INVALID_ARG).  Enqueue the copy before any work that may write
 * the released blocks.  swap_in allocates ceil(len / B) fresh blocks, all or
 * none (PKV_ERR_NO_FREE_BLOCK changes nothing), and writes them in table
 * order for paged_kv_swap_in; sharing is not restored.  cap is the room in
 * blocks_out (too small: PKV_ERR_INVALID_ARG, nothing changes). */
int pkv_bm_seq_swap_out(pkv_block_manager* bm, int seq, int32_t* blocks_out, int cap,
                        int* n_out);
int pkv_bm_seq_swap_in(pkv_block_manager* bm, int seq, int32_t* blocks_out, int cap,
                       int* n_out);
int pkv_bm_seq_is_swapped(const pkv_block_manager* bm, int seq);   /* 1, 0, or error */

/* Automatic prefix caching ([lesson] "Sharing, and the reference counting it
 * needs": block-aligned prefixes of token ids are looked up in a global table
 * and shared on a hit, only when every token id is equal; [claims] "Paged
 * Attention": a hit needs an unbroken matching prefix).
 * pkv_bm_seq_admit_prompt admits an empty sequence with its prompt token ids
 * (host int32 [n_tokens]): the longest cached prefix of full blocks is shared
 * (count + 1), the remaining ceil(n / B) - hits blocks are allocated (all or
 * none: PKV_ERR_NO_FREE_BLOCK changes nothing), and the new full blocks are
 * entered under their prefixes.  *cached_tokens_out = hits * B: the caller
 * writes positions cached .. n-1 (paged_kv_append_tokens) before any
 * attention reads them, and may run prefill for those positions only
 * (paged_prefill_attention with context n and chunk n - cached).
 * Cache keys chain a 64-bit mix over the prefix; an entry also keeps its own
 * token ids and its parent key, both checked on a hit.  A cached block whose
 * count falls to 0 stays hittable; it is evicted, oldest first, when an
 * allocation finds no plain free block.  pkv_bm_num_free counts both kinds. */
int pkv_bm_seq_admit_prompt(pkv_block_manager* bm, int seq, const int32_t* tokens, int n_tokens,
                            int* cached_tokens_out);
int pkv_bm_num_cached(const pkv_block_manager* bm);   /* cached blocks, or error */
int pkv_bm_seq_len(const pkv_block_manager* bm, int seq);   /* >= 0, or error */
int pkv_bm_seq_num_blocks(const pkv_block_manager* bm, int seq);
/* Copy up to cap table entries of seq into out; returns the count copied. */
int pkv_bm_seq_table(const pkv_block_manager* bm, int seq, int32_t* out, int cap);
/* Host rows of block_tables for seqs[0..n): row i gets seqs[i]'s table padded
 * with -1 to ld entries, lens_out[i] its length.  A table longer than ld is
 * PKV_ERR_INVALID_ARG. */
int pkv_bm_export_tables(const pkv_block_manager* bm, const int* seqs, int n, int32_t* out,
                         int ld, int32_t* lens_out);

/* pkv_bm_export_cascade_groups - groups for paged_decode_attention_cascade,
 * read off the tables of the batch seqs[0..n) (row i = seqs[i], the row
 * order of pkv_bm_export_tables).  [lesson] "Sharing, and the reference
 * counting it needs": sequences with a common prompt prefix (forks, prefix
 * cache hits) hold the same physical blocks for it.  Rows whose first table
 * entry is the same block form a candidate group, in order of first
 * appearance; its prefix is the longest run of leading entries all its
 * members share, cut to the full blocks of its shortest member (a partial
 * block may still be written).  A candidate of at least 2 rows whose prefix
 * holds at least min_prefix_tokens tokens, and whose prefix tokens times
 * member count reach min_shared_tokens, is written out: members_out lists
 * its rows (batch row indices, ascending) from offsets_out[z] to
 * offsets_out[z+1], prefix_blocks_out[z] its prefix blocks.  Room:
 * offsets_out n + 1 entries, members_out n, prefix_blocks_out n.  A
 * negative min_prefix_tokens takes PKV_CASCADE_MIN_PREFIX_TOKENS, a
 * negative min_shared_tokens pkv_cascade_min_shared_tokens(8, 128, 2).
 * Rows in no group get plain decode attention from the cascade. */
int pkv_bm_export_cascade_groups(const pkv_block_manager* bm, const int* seqs, int n,
                                 int min_prefix_tokens, long long min_shared_tokens,
                                 int32_t* offsets_out, int32_t* members_out,
                                 int32_t* prefix_blocks_out, int* num_groups_out,
                                 int* num_members_out);

/* When the cascade pays.  It spends a fixed ~25 us of extra launches plus a
 * little per member and saves plain decode's re-reads of the shared prefix,
 * one per member.  Measured on MI355X (32 query / 8 KV heads of 128, fp16,
 * B 16, private suffixes of U[1, 512] tokens, plain decode with
 * cache-retaining loads), members x prefix tokens decides it: at 196,608
 * and above the cascade won everywhere (128 x 1536: 1.13x, 64 x 3072:
 * 1.29x, 256 x 1024: 1.17x), at 98,304 and below plain decode did or tied
 * (64 x 1536: 1.00x, 16 x 4096: 0.81x), and at 131,072 it went both ways
 * (64 x 2048: 1.12x, 128 x 1024: 0.96x).  The threshold sits between, at
 * 163,840 token rows, and is kept as bytes of K and V re-read (x 4 KiB =
 * 640 MiB) so that it carries over to other head shapes; no prefix under
 * 1024 tokens was measured to pay. */
#define PKV_CASCADE_MIN_PREFIX_TOKENS 1024
#define PKV_CASCADE_MIN_SHARED_BYTES (640LL << 20)
/* members x prefix tokens at which the cascade pays for num_kv_heads heads of
 * head_dim elements of elem_bytes bytes: PKV_CASCADE_MIN_SHARED_BYTES over
 * the K and V bytes of one token, rounded up; -1 for invalid arguments. */
long long pkv_cascade_min_shared_tokens(int num_kv_heads, int head_dim, int elem_bytes);

/*
 * pkv_validate_tables - host check of the block-id contract of a batch: every
 * entry below ceil(lens[s] / block_size) lies in [0, num_blocks) and fits in the
 * row.  Host pointers.  Returns PKV_OK, or PKV_ERR_INVALID_ARG and the first bad
 * sequence in *bad_seq_out (may be NULL).
 */
int pkv_validate_tables(const int32_t* block_tables, int max_blocks_per_seq,
                        const int32_t* context_lens, int num_seqs, int num_blocks,
                        int block_size, int* bad_seq_out);

/*
 * pkv_validate_cascade_groups - host check of the group contract of
 * paged_decode_attention_cascade (host pointers): offsets rise within
 * [0, num_members]; member ids lie in [0, num_seqs), each in at most one
 * group; 0 <= group_prefix_blocks[z] <= max_blocks_per_seq; every member is
 * at least its group's prefix long, and its first group_prefix_blocks[z]
 * table entries equal the group's first member's.  Returns PKV_OK, or
 * PKV_ERR_INVALID_ARG and the first bad group in *bad_group_out (may be NULL).
 */
int pkv_validate_cascade_groups(const int32_t* block_tables, int max_blocks_per_seq,
                                const int32_t* context_lens, int num_seqs, int block_size,
                                const int32_t* group_offsets, const int32_t* group_members,
                                int num_members, const int32_t* group_prefix_blocks,
                                int num_groups, int* bad_group_out);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
