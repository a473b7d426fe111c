/*
 * pagedkv.h -- C ABI of libpagedkv.so: paged KV-cache attention on AMD
 * Instinct MI355X (gfx950).
 *
 * The method: every sequence's KV cache is cut into fixed-size blocks of
 * block_size tokens; a per-sequence block table maps logical block i to a
 * physical block id in one global pool, and the attention kernels reach keys
 * and values by following that table ("Paged Attention for Efficient Memory
 * Management", The Daily Triptych: "At a glance", technical summary, "Look
 * closer / Logical blocks, physical frames"; "PagedAttention and
 * RadixAttention: Let's Talk About KV Cache", section "PagedAttention: Memory
 * Like an Operating System").  The block manager that decides which block a
 * token goes to lives on the host; these calls are the device side.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - All tensor arguments are DEVICE pointers owned by the caller.  The
 *    library allocates nothing, frees nothing and never synchronises.
 *  - Every call is enqueued on `stream` (a hipStream_t; NULL = the null
 *    stream) and returns once the work is enqueued.
 *  - Return value: PKV_OK (0) or a negative PKV_ERR_* code; on error nothing
 *    was enqueued and paged_kv_last_error() describes the problem (a
 *    per-thread string, valid until the next call on that thread).
 *  - dtype: PKV_DTYPE_FP32 (IEEE binary32) or PKV_DTYPE_BF16 (bfloat16).
 *    Every floating-point tensor of one call has that dtype, except the
 *    decode workspace (fp32).
 *  - block_size: 16 (the pages' default, "PagedAttention 与 RadixAttention",
 *    section "PagedAttention") or 32 (the alternative they name, "PagedAttention
 *    and RadixAttention: Let's Talk About KV Cache", section "PagedAttention:
 *    Memory Like an Operating System").  head_dim: 64 or 128.  num_q_heads must be
 *    a multiple of num_kv_heads with a group of at most 16 query heads per
 *    KV head (query head j uses KV head j / (num_q_heads / num_kv_heads)).
 *  - Device memory is addressed with 64-bit offsets: pools of any size.
 *
 * Pool layout (both pools hold num_blocks blocks; e = element):
 *    k_pool  [num_blocks][num_kv_heads][block_size][head_dim]
 *            -- a key vector is one contiguous row.
 *    v_pool  [num_blocks][num_kv_heads] slabs of head_dim x block_size
 *            elements -- values are stored transposed, in 16-token halves
 *            [block_size / 16][head_dim][16]: one row of 16 tokens per
 *            channel in each half (a 32-token block is two halves, one
 *            after the other), and in a row the token at offset `off` of
 *            its half sits at position v_pos(off) = off with bits 2 and 3
 *            exchanged (order 0-3, 8-11, 4-7, 12-15; the map is its own
 *            inverse).  This is the order in which the matrix cores consume
 *            a block's tokens, two 8-byte halves per lane, and the values
 *            of any 16 consecutive tokens of a block are contiguous.
 *  A slot is phys_block * block_size + offset_in_block.
 *
 * Safety: kernels never touch memory outside the ranges the arguments
 * describe.  Table entries or slots outside [0, num_blocks) are skipped
 * (append, copy) or read as block 0 (attention); results are then
 * unspecified but no out-of-range access happens.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_OK              0
#define PKV_ERR_INVALID    -1  /* null pointer, bad size, bad head ratio      */
#define PKV_ERR_UNSUPPORTED -2 /* dtype / head_dim / block_size / group size  */
#define PKV_ERR_WORKSPACE  -3  /* decode workspace missing or too small       */
#define PKV_ERR_LAUNCH     -4  /* the HIP runtime refused a kernel launch     */

#define PKV_DTYPE_FP32 0
#define PKV_DTYPE_BF16 1

/* Message for the last failing call on this thread ("" if none). */
const char* paged_kv_last_error(void);

/*
 * paged_kv_append -- write new tokens' keys and values into their pool slots.
 *
 * Passage: a new token's keys and values go into the next slot of the
 * sequence's current block, a fresh block being taken when the current one
 * is full (Triptych page, technical summary and "The story").  The host
 * allocator chooses the slots; this call only writes.
 *
 *   k_new, v_new   [num_tokens][num_kv_heads][head_dim]   (dtype)
 *   slot_mapping   [num_tokens] int32; slot < 0 = skip the token
 *   k_pool, v_pool pools as laid out above (written in place)
 *
 * Every head of token t goes to slot_mapping[t].  Slots within one call must
 * be distinct (else which write wins is unspecified).  num_tokens == 0 is a
 * no-op.  Result is a bit copy: no value changes.
 */
int paged_kv_append(const void* k_new, const void* v_new,
                    const int32_t* slot_mapping, int32_t num_tokens,
                    void* k_pool, void* v_pool, int32_t num_blocks,
                    int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                    int32_t dtype, void* stream);

/*
 * copy_blocks -- copy-on-write of shared blocks.
 *
 * Passage: once a forked sequence writes into a block other sequences still
 * reference, that block is copied first so the other references keep their
 * contents (Triptych page, technical summary, "Look closer / Sharing is a
 * pointer change" and "The story").
 *
 *   block_mapping  [num_pairs][2] int32 (src, dst), device memory
 *
 * For every pair the whole K block and the whole V block (all heads, all
 * block_size slots) of src are copied to dst, bit for bit.  Destinations must
 * be distinct and no destination may also be a source of the same call (the
 * result is then independent of pair order).  num_pairs == 0 is a no-op.
 */
int copy_blocks(void* k_pool, void* v_pool, int32_t num_blocks,
                const int32_t* block_mapping, int32_t num_pairs,
                int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                int32_t dtype, void* stream);

/*
 * swap_blocks -- copy whole blocks (K and V) from one pool to another, where
 * either pool may live in pinned host memory: the tier below HBM, for blocks
 * moved out of the GPU and back ("PagedAttention and RadixAttention: Let's
 * Talk About KV Cache", section "Beyond the Two Techniques", hierarchical
 * memory: hot blocks in GPU memory, recently used ones in host RAM).
 *
 *   dst_k, dst_v   pools of dst_num_blocks blocks in the layout above (K
 *                  [..][num_kv_heads][block_size][head_dim], V
 *                  [..][num_kv_heads] slabs of head_dim x block_size), written
 *   src_k, src_v   pools of src_num_blocks blocks, same layout, read
 *   block_mapping  [num_pairs][2] int32, device memory: (src block, dst block)
 *
 * Each pool is device memory or pinned host memory (hipHostMalloc, or a
 * pinned torch tensor); host pools are accessed through their device
 * mapping by the copy kernel, so the call is asynchronous on stream like the
 * others.  Bit-exact.  Pairs with a block id out of range are skipped;
 * destination blocks should be distinct (if not, which copy wins is
 * unspecified).  PKV_ERR_INVALID for memory that is neither device memory
 * nor pinned host memory.
 */
int swap_blocks(void* dst_k, void* dst_v, int32_t dst_num_blocks, const void* src_k,
                const void* src_v, int32_t src_num_blocks, const int32_t* block_mapping,
                int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                int32_t dtype, void* stream);

/*
 * Size in bytes of the workspace paged_attention_decode needs for these
 * arguments; partition_size as in paged_attention_decode (0 = the library's
 * choice).  Returns 0 only for invalid arguments (the decode call reports
 * those).
 */
size_t paged_attention_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                             int32_t num_kv_heads, int32_t head_dim,
                                             int32_t max_context_len,
                                             int32_t partition_size);

/*
 * paged_attention_decode -- one query token per sequence attends to its
 * whole paged context.
 *
 * Passage: the attention kernel walks the block table and gathers the
 * sequence's physical blocks; the result equals attention over the same
 * tokens stored contiguously (Triptych page, technical summary, "The story",
 * "The surprising detail").  Contexts are split along the sequence into
 * pieces computed in parallel and merged by the log-sum-exp rule
 * ("RadixAttention: Tree-Based KV Cache Reuse in SGLang Guide", section "3.
 * Integrating FlashInfer for Sub-Millisecond Paged Kernel Lookups",
 * split-KV decode).
 *
 *   out            [num_seqs][num_q_heads][head_dim]  (dtype), written
 *   q              [num_seqs][num_q_heads][head_dim]  (dtype)
 *   block_tables   [num_seqs][max_blocks_per_seq] int32; row s, entries
 *                  0 .. ceil(context_lens[s]/block_size)-1 are read
 *   context_lens   [num_seqs] int32, tokens in each context (the decoded
 *                  token's own key/value included); 0 gives a zero row
 *   max_context_len  host-side upper bound of context_lens (sizes the
 *                  workspace).  A precondition: a longer context is cut to
 *                  the (P - 1) x partition_size tokens the workspace can
 *                  hold (P below), never read past it
 *   scale          softmax scale applied to q.k
 *   partition_size the smallest piece of a context computed on its own
 *                  (tokens, a multiple of block_size; 0 = 512).  bf16: the
 *                  call's (sequence, KV head, block) triples, sequence-major,
 *                  are dealt in equal contiguous ranges of
 *                  C = max(partition_size / block_size, ceil(total / W))
 *                  blocks to W = 2 x (compute units) workgroups; a (sequence,
 *                  KV head) that meets several ranges is computed in pieces,
 *                  which a second kernel on the same stream merges.  fp32:
 *                  fixed partitions of partition_size tokens, then a merge
 *                  pass.
 *   workspace      device memory of at least
 *                  paged_attention_decode_workspace_size(...) bytes, 8-byte
 *                  aligned, owned by the caller, any contents (no clearing
 *                  is needed between calls; see count below).  Layout,
 *                  P = ceil(max_context_len / partition_size) + 1 pieces
 *                  per context:
 *                    o_part [num_seqs][num_q_heads][P][head_dim]  fp32, a
 *                                                  piece's normalised output
 *                    m_part [num_seqs][num_q_heads][P]  fp32, max scaled score
 *                    l_part [num_seqs][num_q_heads][P]  fp32, sum exp(score - m)
 *                    count  [num_seqs][num_kv_heads]  uint64, written for
 *                                  a (sequence, KV head) computed in several
 *                                  pieces: bits 24..63 a per-call tag, bits
 *                                  0..23 its piece count.  A word with
 *                                  another call's tag counts as one piece
 *                                  (nothing to merge), so old contents are
 *                                  harmless; arbitrary contents
 *                                  are misread only if a word holds exactly
 *                                  the call's 40-bit tag (tags run in one
 *                                  process-wide sequence from a random start
 *                                  with the top bit set).  A workspace
 *                                  zero-filled when it is allocated and used
 *                                  with one layout (same num_seqs,
 *                                  num_q_heads, head_dim and P) is never
 *                                  misread: no tag is zero, and these words
 *                                  only ever receive tagged values.
 *                  Piece k of a context is the k-th range it meets.  Calls
 *                  that share a workspace must not overlap in time.
 *                  Returns PKV_ERR_UNSUPPORTED (bf16) when one merge's
 *                  weights, 2 x group x P + group fp32 words, exceed the LDS
 *                  (160 KB): a larger partition_size lowers P.
 *
 * out[s][j] = sum_t softmax_t(scale * q[s][j] . k_t) v_t over t < context_lens[s],
 * with k_t, v_t from KV head j / (num_q_heads/num_kv_heads).  Arithmetic:
 * fp32 accumulation (bf16 products on the matrix cores for bf16 input).
 */
int paged_attention_decode(void* out, const void* q,
                           const void* k_pool, const void* v_pool, int32_t num_blocks,
                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* context_lens, int32_t num_seqs,
                           int32_t max_context_len, int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           float scale, int32_t partition_size,
                           void* workspace, size_t workspace_bytes,
                           int32_t dtype, void* stream);

/*
 * paged_attention_decode_noalloc -- paged_attention_decode for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Same arguments, kernels and
 * result as paged_attention_decode, without the workspace arguments: the
 * call's pieces and piece-count words live in a fixed array the library holds
 * on every GPU it runs on (64 MiB, kept until the process ends).  The call
 * allocates nothing.
 *
 * Limits: num_seqs * num_kv_heads <= 32768, and the partials,
 * num_seqs * num_q_heads * P * (head_dim + 2) * 4 bytes with P as in
 * paged_attention_decode, at most 64 MiB - 256 KiB (a larger partition_size
 * lowers P).  Beyond them the call returns PKV_ERR_WORKSPACE, with both
 * sizes in the message, and enqueues nothing.
 *
 * Every call on a GPU shares that GPU's array, which keeps the last call's
 * contents: calls in order on one stream are fine, but calls that overlap in
 * time on one GPU (other streams, other host threads) race and give wrong
 * results.  The first call on a GPU also enqueues, on `stream`, a small
 * kernel that clears the array's piece-count words.
 */
int paged_attention_decode_noalloc(void* out, const void* q, const void* k_pool,
                                   const void* v_pool, int32_t num_blocks,
                                   const int32_t* block_tables, int32_t max_blocks_per_seq,
                                   const int32_t* context_lens, int32_t num_seqs,
                                   int32_t max_context_len, int32_t num_q_heads,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                   float scale, int32_t partition_size, int32_t dtype,
                                   void* stream);

/*
 * Size in bytes of the workspace paged_attention_decode_shared needs for
 * these arguments (it depends on the device's compute-unit count, which
 * sets the prefix pass's key split).  Returns 0 for invalid arguments.
 */
size_t paged_attention_decode_shared_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                                    int32_t num_kv_heads, int32_t head_dim,
                                                    int32_t max_context_len, int32_t partition_size,
                                                    int32_t num_groups, int32_t max_group_size,
                                                    int32_t max_prefix_blocks);

/*
 * paged_attention_decode_shared -- paged_attention_decode for a batch in
 * which groups of sequences share the leading physical blocks of their
 * tables (a common system prompt, parallel samples forked from one parent).
 *
 * Passage: sharing a prefix is a pointer change, every sharer's table
 * pointing at the same physical blocks (Triptych page, technical summary
 * and "Look closer"); prefix caches hand the same blocks to every request
 * that starts with the same tokens ("PagedAttention and RadixAttention:
 * Let's Talk About KV Cache", "Two Layers, Not Two Rivals").  The pages do
 * not describe decoding such a batch; here the attention over a shared
 * prefix is computed once per (group, KV head) for all members' query heads
 * together, on the matrix cores, and combined with each member's attention
 * over the rest of its context by the log-sum-exp rule ("RadixAttention:
 * Tree-Based KV Cache Reuse in SGLang Guide", section "3. Integrating
 * FlashInfer ...", split-KV decode).  The result is the same function as
 * paged_attention_decode's.
 *
 * Arguments as paged_attention_decode, plus (device memory unless noted):
 *   group_offsets  [num_groups+1] int32: group i's members are
 *                  group_seqs[group_offsets[i] .. group_offsets[i+1]-1]
 *   group_seqs     sequence indices; a sequence belongs to at most one group
 *   group_prefix_blocks [num_groups] int32: the number of leading table
 *                  entries every member of the group has in common (the same
 *                  physical block ids, read from the first member's row)
 *   num_groups, max_group_size, max_prefix_blocks  host-side: the group
 *                  count, the largest member count and the largest
 *                  group_prefix_blocks (they size the prefix pass's grid)
 *   workspace      at least paged_attention_decode_shared_workspace_size(...)
 *                  bytes, 8-byte aligned: the paged_attention_decode layout
 *                  (o, m, l pieces, then one 64-bit word per (sequence, KV
 *                  head) holding the unit's piece count), then seq_prefix
 *                  [num_seqs] 64-bit words (where each sequence's own pass
 *                  starts, in 16-token granules, in bits 0..19, and how
 *                  many prefix partials it folds in, in bits 20..23), then
 *                  at the next 256-byte boundary the prefix partials o
 *                  [num_seqs][num_q_heads][NS][head_dim], m and l
 *                  [num_seqs][num_q_heads][NS] fp32 (NS key splits).  Every
 *                  64-bit word carries the writing call's tag in bits 24..63,
 *                  as paged_attention_decode's piece-count words do, and a word
 *                  with another tag reads as zero: nothing is cleared
 *                  between calls, and the same guarantee holds (a workspace
 *                  zero-filled at allocation is never misread).
 *
 * A member sees the shared blocks up to, not including, the block that holds
 * its last token (that block is always in its own pass): its first
 * min(prefix_blocks, (context_len - 1) / block_size) table entries must be
 * the first member's (the call reads the prefix blocks from the first
 * member's row only), and the first member must hold all prefix_blocks.
 * Otherwise the result is undefined, but every access stays inside the
 * pool.  Block sizes 16 and 32 (group_prefix_blocks counts table entries of
 * block_size tokens); fp32 inputs, or no groups, run paged_attention_decode
 * unchanged.  Errors as paged_attention_decode; PKV_ERR_UNSUPPORTED when the
 * merge weights, 2 x group x (P + NS) + group fp32 words, exceed the LDS;
 * PKV_ERR_INVALID when the prefix splits cover 2^20 granules of 16 tokens or
 * more (the start would not fit its 20 bits).
 */
int paged_attention_decode_shared(void* out, const void* q, const void* k_pool,
                                  const void* v_pool, int32_t num_blocks,
                                  const int32_t* block_tables, int32_t max_blocks_per_seq,
                                  const int32_t* context_lens, int32_t num_seqs,
                                  int32_t max_context_len, int32_t num_q_heads,
                                  int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                  float scale, const int32_t* group_offsets,
                                  const int32_t* group_seqs, const int32_t* group_prefix_blocks,
                                  int32_t num_groups, int32_t max_group_size,
                                  int32_t max_prefix_blocks, int32_t partition_size,
                                  void* workspace, size_t workspace_bytes, int32_t dtype,
                                  void* stream);

/*
 * paged_attention_extend -- new tokens of each request (a chunked prefill
 * after a cached prefix) attend causally to the prefix plus themselves.
 *
 * Passage: with the prefix's keys and values already in the pool, only the
 * unseen suffix is computed ("RadixAttention: Tree-Based KV Cache Reuse in
 * SGLang Guide", "RadixAttention Architecture", longest-prefix search and
 * prefill bypass; "PagedAttention and RadixAttention: Let's Talk About KV
 * Cache", section "RadixAttention: A Tree That Does Not Forget").  Prefill
 * is the compute-bound phase (same guide, "1. The Quadratic Cost ...").
 *
 *   out, q         [total_q][num_q_heads][head_dim]  (dtype)
 *   cu_seqlens_q   [num_reqs+1] int32: request r owns rows cu[r] .. cu[r+1]-1
 *                  (none when it has no new token, whatever its prefix)
 *   seq_lens       [num_reqs] int32: prefix + new tokens of request r; the
 *                  new tokens' keys/values must already be in the pool
 *   max_q_len      host-side bound of cu[r+1]-cu[r]   (sizes the grid)
 *   max_seq_len    host-side bound of seq_lens         (informational)
 *   block_tables   [num_reqs][max_blocks_per_seq] int32
 *
 * New token i of request r (position P_r + i, P_r = seq_lens[r] - n_r)
 * attends to positions 0 .. P_r + i.  Arithmetic: bf16 matrix-core products
 * with fp32 accumulation for bf16; fp32 throughout for fp32.
 */
int paged_attention_extend(void* out, const void* q,
                           const int32_t* cu_seqlens_q, const int32_t* seq_lens,
                           int32_t num_reqs, int32_t total_q, int32_t max_q_len,
                           int32_t max_seq_len,
                           const void* k_pool, const void* v_pool, int32_t num_blocks,
                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                           int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                           int32_t block_size, float scale, int32_t dtype, void* stream);

/*
 * paged_kv_gather -- copy one sequence's keys and values, in logical order,
 * out of the pool (the kernel-side walk of the block table, exposed so that
 * tests can check device-side indexing bit for bit).
 *
 *   k_out, v_out   [context_len][num_kv_heads][head_dim]  (dtype), written
 *   block_table_row [ceil(context_len/block_size)] int32, device memory
 */
int paged_kv_gather(void* k_out, void* v_out, const void* k_pool, const void* v_pool,
                    int32_t num_blocks, const int32_t* block_table_row,
                    int32_t context_len, int32_t num_kv_heads, int32_t head_dim,
                    int32_t block_size, int32_t dtype, void* stream);

/*
 * pinned_upload -- copy `bytes` bytes from src to dst with a kernel on
 * `stream`, for the host block manager's per-step outputs (slot mapping,
 * context lengths, block tables).  The pages put that bookkeeping beside the
 * attention kernels, not in them ("Paged Attention for Efficient Memory
 * Management", The Daily Triptych, technical summary: block tables and
 * reference counts are the scheme's bookkeeping cost; "PagedAttention 与
 * RadixAttention", section "RadixAttention": the tree lives in CPU memory),
 * so its results cross to the device every step.  A kernel that reads the
 * pinned buffer through its device mapping keeps that crossing on the
 * compute queue, where a copy-engine transfer would add a hand-off between
 * queues to every step.
 *
 *   dst    device memory (or pinned host memory), written
 *   src    pinned host memory (hipHostMalloc, torch pin_memory) or device
 *          memory; read by the kernel when it runs, so the caller keeps it
 *          unchanged until the stream has passed the call
 *   bytes  >= 0; 0 is a no-op.  Any alignment (16-byte pieces when both
 *          pointers are 16-byte aligned).
 *
 * PKV_ERR_INVALID for a negative size, a null pointer, or memory that is
 * neither device memory nor pinned host memory.  The ranges must not overlap.
 */
int pinned_upload(void* dst, const void* src, int64_t bytes, void* stream);

/*
 * upload_and_append -- pinned_upload and paged_kv_append in one call, for a
 * decode step whose staging buffer carries the slot mapping among its index
 * arrays.  The kernel copies `bytes` bytes of `staging` to `dst` and, at the
 * same time, writes the new tokens' keys and values into their slots
 * ("Paged Attention for Efficient Memory Management", The Daily Triptych,
 * "The story": a new token's keys and values go into the next slot of its
 * sequence's block), reading each token's slot from `staging` itself, so
 * the two parts do not wait for each other.  From 512 tokens on it runs as
 * the upload followed by paged_kv_append's bulk path (which reads the slots
 * from the device copy), i.e. two launches.
 *
 *   dst, staging, bytes   as pinned_upload (bytes >= 0; 0 is a no-op)
 *   slots_offset          byte offset of the slot mapping, int32
 *                         [num_tokens], inside staging: a multiple of 4,
 *                         slots_offset + 4 * num_tokens <= bytes
 *   k_new, v_new, num_tokens, k_pool, v_pool, num_blocks, num_kv_heads,
 *   head_dim, block_size, dtype   as paged_kv_append
 *
 * The pool writes happen after every earlier call on `stream` (a
 * copy_blocks for the step's copy-on-write pairs goes first).  Errors as
 * pinned_upload and paged_kv_append, plus PKV_ERR_INVALID for a slot
 * mapping outside the staged bytes.
 */
int upload_and_append(void* dst, const void* staging, int64_t bytes, int64_t slots_offset,
                      const void* k_new, const void* v_new, int32_t num_tokens, void* k_pool,
                      void* v_pool, int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                      int32_t block_size, int32_t dtype, void* stream);

/*
 * upload_and_append_tables -- upload_and_append for a caller that keeps its
 * block tables resident on the device and sends only the entries a step
 * changed.  In a decode step only a sequence's last table entry can change
 * (a fresh block when the last one is full, or its copy-on-write
 * replacement: "Paged Attention for Efficient Memory Management", The Daily
 * Triptych, "The story" and technical summary), so a step's update is one
 * (index, value) pair per sequence instead of the whole table.
 *
 *   dst, staging, bytes, slots_offset, and the append arguments
 *                 as upload_and_append
 *   block_tables  device int32 array of table_words words (for example the
 *                 [num_seqs][max_blocks_per_seq] tables a decode call reads)
 *   num_updates   >= 0 pairs of int32 (index, value), stored in staging right
 *                 after its first `bytes` bytes (bytes a multiple of 4);
 *                 block_tables[index] = value, indexes outside
 *                 [0, table_words) are skipped.  Pairs with the same index
 *                 leave one of their values, unspecified which.
 *
 * The table writes happen in the same launch as the upload (from 512 tokens
 * on, in the upload launch that precedes the bulk append) and are complete
 * for every later call on `stream`.  Errors as upload_and_append, plus
 * PKV_ERR_INVALID for negative counts, or updates without block_tables or
 * with bytes not a multiple of 4.
 */
int upload_and_append_tables(void* dst, const void* staging, int64_t bytes, int64_t slots_offset,
                             int32_t* block_tables, int64_t table_words, int32_t num_updates,
                             const void* k_new, const void* v_new, int32_t num_tokens,
                             void* k_pool, void* v_pool, int32_t num_blocks, int32_t num_kv_heads,
                             int32_t head_dim, int32_t block_size, int32_t dtype, void* stream);

/*
 * block_manager_append_step -- HOST call, the one exception to the device
 * conventions above: every pointer is host memory, nothing is enqueued and
 * no GPU is touched.  The decode step of the host block manager: one new
 * token for each sequence in sids, in that order ("Paged Attention for
 * Efficient Memory Management", The Daily Triptych, "The story" and
 * technical summary: a token fills the next slot of the sequence's last
 * block; a full last block is followed by a fresh block from the free pool;
 * a write into a block that other sequences still reference goes to a
 * fresh copy, and the last remaining owner writes in place).
 *
 * State (the block manager's own arrays, updated in place):
 *   tables      [max_seqs][max_blocks_per_seq] int32; row = sequence id;
 *               entries past a sequence's block count are -1
 *   lens, nblk  [max_seqs] int32: tokens and blocks per sequence
 *               (nblk = ceil(lens / block_size))
 *   live, on_host [max_seqs] uint8 (0/1): sequence exists / is on the host tier
 *   ref         [num_blocks] int32 references per block
 *   sealed      [num_blocks] uint8 (0/1): contents frozen (a prefix cache
 *               indexes the block)
 *   free_ring   [num_blocks] int32 FIFO ring of free block ids
 *   free_state  [2] int64: head index and count of the ring
 * Arguments:
 *   sids        [num_sids] int64 sequence ids, distinct
 * Results:
 *   slots_out   [num_sids] int32 slot of each sequence's new token
 *   pairs_out   [num_sids][2] int32 (src, dst) block copies to make before
 *               the new tokens are written (copy_blocks); *num_pairs_out of
 *               them are valid, in sequence order
 *
 * A sequence whose last block is full takes the block at the ring's head;
 * one whose last block has a count above one takes the head block as a
 * copy destination and drops one count from the old block.  Fresh blocks
 * are taken in sequence order and get a count of 1.
 *
 * Returns PKV_OK; PKV_ERR_INVALID (message set) for a null pointer, bad
 * sizes, a repeated, out-of-range, dead or host-tier sequence, a table
 * entry out of range, or a sequence that would exceed max_blocks_per_seq;
 * PKV_STEP_SEALED if a sequence would write into a sealed block, and
 * PKV_STEP_SHORT if the step needs more blocks than the ring holds.  On any
 * return but PKV_OK nothing was changed.
 */
#define PKV_STEP_SEALED 1
#define PKV_STEP_SHORT  2
int block_manager_append_step(int32_t* tables, int32_t* lens, int32_t* nblk,
                              const uint8_t* live, const uint8_t* on_host, int32_t max_seqs,
                              int32_t max_blocks_per_seq, int32_t* ref, const uint8_t* sealed,
                              int32_t num_blocks, int32_t block_size, const int64_t* sids,
                              int32_t num_sids, int32_t* free_ring, int64_t* free_state,
                              int32_t* slots_out, int32_t* pairs_out, int32_t* num_pairs_out);

/*
 * hbm_read_probe -- measurement support, not a step of the method: reads
 * num_chunks chunks of chunk_bytes bytes from buf with non-temporal 16-byte
 * loads, in the order chunk_order gives (num_chunks int32 entries in
 * [0, num_chunks), device memory; NULL = address order), and folds what it
 * read into sink[0 .. num_workgroups-1] (device uint32 words, XORed into).
 * The buffer holds num_chunks * chunk_bytes bytes.  Timing it over a random
 * order of 4 KB chunks gives the practical rate of the scattered 4 KB reads
 * a paged pool makes (a bf16 (block, KV head) slab at head_dim 128 is 4 KB),
 * the ceiling the decode kernels' bandwidth is reported against beside the
 * HBM peak.  Out-of-range order entries read chunk 0.  PKV_ERR_INVALID for
 * null pointers, negative counts or sizes and pointers that are not
 * multiples of 16 bytes.
 */
int hbm_read_probe(const void* buf, int64_t num_chunks, int32_t chunk_bytes,
                   const int32_t* chunk_order, uint32_t* sink, int32_t num_workgroups,
                   void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
