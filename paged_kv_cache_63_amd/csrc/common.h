// Internal helpers shared by the gfx950 kernels and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// ---- vector types for the matrix-core builtins and wide memory accesses ----
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// bf16 word -> fp32 (exact)
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t w) { return __uint_as_float((uint32_t)w << 16); }

// Position of a token's offset `off` (0..15) inside a 16-token V channel
// row: bits 2 and 3 exchanged, so a row holds tokens 0-3, 8-11, 4-7, 12-15.
// A matrix-core operand that needs tokens {4G..4G+3, 8+4G..8+4G+3} then
// reads 16 contiguous bytes.  The map is its own inverse.
__host__ __device__ __forceinline__ int v_pos(int off) {
  return (off & ~12) | ((off & 4) << 1) | ((off & 8) >> 1);
}

// V slab of one (block, head): the block's values transposed, in 16-token
// halves ([B/16][D][16]: a 32-token block is two of them, so the values of
// any 16-token granule are one contiguous run of 16 x D elements).  Element
// offset of (in-block token off, channel c); channel rows are kVRow apart.
constexpr int kVRow = 16;
__host__ __device__ __forceinline__ int64_t v_elem(int off, int c, int d) {
  return (int64_t)(off & ~15) * d + (int64_t)c * kVRow + v_pos(off & 15);
}

// fp32 -> bf16 word, round to nearest even (the gfx950 conversion instruction)
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

}  // namespace pkv

// ---- C++ launchers implemented in the kernel translation units ----
// Each returns 0 on success or a PKV_ERR_* code; arguments are already
// validated by the C-ABI layer.
namespace pkv {

int launch_append(const void* k_new, const void* v_new, const int32_t* slots, int32_t num_tokens,
                  void* k_pool, void* v_pool, int32_t num_blocks, int32_t hkv, int32_t d,
                  int32_t bs, int32_t elem_bytes, hipStream_t st);

int launch_copy_blocks(void* k_pool, void* v_pool, int32_t num_blocks, const int32_t* mapping,
                       int32_t num_pairs, int32_t hkv, int32_t d, int32_t bs, int32_t elem_bytes,
                       hipStream_t st);
// Block-table entries written by an upload kernel: table[pairs[2i]] =
// pairs[2i + 1], i < n (pairs device-readable; none when n is 0).
struct TableUpdates {
  int32_t* table = nullptr;
  int64_t words = 0;
  const int32_t* pairs = nullptr;
  int64_t n = 0;
};

int launch_upload(void* dst, const void* src, int64_t bytes, hipStream_t st,
                  TableUpdates u = TableUpdates{});
int launch_upload_append(void* dst, const void* src, int64_t bytes, int64_t slots_offset,
                         const void* k_new, const void* v_new, int32_t num_tokens, void* k_pool,
                         void* v_pool, int32_t num_blocks, int32_t hkv, int32_t d, int32_t bs,
                         int32_t elem_bytes, hipStream_t st, TableUpdates u = TableUpdates{});
int launch_swap_blocks(void* dst_k, void* dst_v, int32_t num_dst, const void* src_k,
                       const void* src_v, int32_t num_src, const int32_t* mapping,
                       int32_t num_pairs, int32_t hkv, int32_t d, int32_t bs, int32_t elem_bytes,
                       hipStream_t st);

int launch_gather(void* k_out, void* v_out, const void* k_pool, const void* v_pool,
                  int32_t num_blocks, const int32_t* row, int32_t ctx, int32_t hkv, int32_t d,
                  int32_t bs, int32_t elem_bytes, hipStream_t st);

struct DecodeArgs {
  void* out;
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float* part_o;   // [S][Hq][P][D]
  float* part_m;   // [S][Hq][P]
  float* part_l;   // [S][Hq][P]
  // [S][Hkv] piece-count words: a unit computed in several pieces gets,
  // from its first piece, bits 24..63 the call's tag and bits 0..23 its
  // piece count, which the fold reads; a word with another tag counts as
  // zero (the unit was finished in one piece), so the words need no
  // clearing between calls.
  uint64_t* arrive;
  uint64_t tag;       // this call's tag, already in bits 24..63
  int32_t num_blocks;
  int32_t max_blocks_per_seq;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t partition_blocks;  // smallest piece (bf16) / partition (fp32), in 16-token granules
  int32_t bs_shift;          // log2(block_size / 16): a table entry covers 16 << bs_shift tokens
  int32_t max_partitions;    // P: pieces per (sequence, query head) the workspace holds
  int32_t num_workgroups;    // bf16 grid
  float scale;
  // Shared-prefix decode only (null / 0 otherwise): per sequence, the first
  // block its own pass starts at and how many prefix partials (pre_*, one
  // per key split of the prefix pass) its result folds in, as one word that
  // the prefix pass writes for each group member: this call's tag in bits
  // 24..63, the start block in bits 0..19, the partial count in bits 20..23.
  // A word with another tag (a sequence in no group) means 0 and 0.
  const uint64_t* seq_prefix; // [S]
  const float* pre_o;        // [S][Hq][num_splits][D]
  const float* pre_m;        // [S][Hq][num_splits]
  const float* pre_l;        // [S][Hq][num_splits]
  int32_t num_splits;
};

int launch_decode(const DecodeArgs& a, int32_t dtype, hipStream_t st);

// The decode workspace the allocation-free entry uses: one fixed device
// array per GPU, kScratchBytes long, whose first kScratchArriveBytes hold the
// piece-count words (one per (sequence, KV head), so at most
// kScratchArriveBytes / 8 units) and the rest the pieces' partials.
constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr size_t kScratchArriveBytes = size_t(256) << 10;
// Device address of the current device's array; the first call on a device
// looks it up and clears its piece-count words with a kernel on st.  0 or a
// PKV_ERR_* code.
int decode_scratch(hipStream_t st, uint8_t** base);

struct ExtendArgs {
  void* out;
  const void* q;
  const int32_t* cu_seqlens_q;
  const int32_t* seq_lens;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_tables;
  int32_t num_reqs;
  int32_t total_q;
  int32_t max_q_len;
  int32_t max_seq_len;
  int32_t num_blocks;
  int32_t max_blocks_per_seq;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t block_size;   // 16 or 32
  float scale;
};

int launch_extend(const ExtendArgs& a, int32_t dtype, hipStream_t st);

// Prefix pass of the shared-prefix decode: for every group of sequences
// whose tables begin with the same prefix_blocks physical blocks, attention
// of all the members' query heads over those blocks, split along the keys
// into pieces of split_blocks blocks; writes each piece's (normalised o, m,
// l) per (sequence, query head) and each member's seq_prefix entry.
struct PrefixArgs {
  const void* q;             // [S][Hq][D]
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* group_offsets;       // [G+1]
  const int32_t* group_seqs;          // members, group-major
  const int32_t* group_prefix_blocks; // [G]
  float* pre_o;
  float* pre_m;
  float* pre_l;
  uint64_t* seq_prefix;      // [S] tagged words, as DecodeArgs::seq_prefix
  uint64_t tag;              // the decode call's tag (bits 24..63)
  int32_t num_groups;
  int32_t max_group_size;
  int32_t num_seqs;
  int32_t num_blocks;
  int32_t max_blocks_per_seq;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t block_size;        // tokens per table entry (16 or 32)
  int32_t split_blocks;      // table entries per key split, a multiple of 4
  int32_t num_splits;
  float scale;
};

int launch_prefix(const PrefixArgs& a, hipStream_t st);

// Set the per-thread message of paged_kv_last_error (entry points outside
// the file that owns it); set_error returns code, clear_error PKV_OK.
int set_error(int code, const char* msg);
int clear_error();

}  // namespace pkv
