// C-ABI entry points: argument checks, workspace sizing and dispatch to the
// kernel launchers.  Nothing here allocates or synchronises.
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <atomic>
#include <random>

#include "../../include/pagedkv.h"
#include "common.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = 0;
  return PKV_OK;
}

int elem_bytes(int32_t dtype) { return dtype == PKV_DTYPE_FP32 ? 4 : dtype == PKV_DTYPE_BF16 ? 2 : 0; }

// Shared shape checks; returns PKV_OK or an error code (message set).
int check_common(int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t dtype) {
  if (!elem_bytes(dtype)) return fail(PKV_ERR_UNSUPPORTED, "dtype %d not supported (0=fp32, 1=bf16)", dtype);
  if (block_size != 16 && block_size != 32)
    return fail(PKV_ERR_UNSUPPORTED, "block_size %d not supported (16 or 32)", block_size);
  if (head_dim != 64 && head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "head_dim %d not supported (64, 128)", head_dim);
  if (num_kv_heads <= 0) return fail(PKV_ERR_INVALID, "num_kv_heads must be positive");
  return PKV_OK;
}

int check_heads(int32_t num_q_heads, int32_t num_kv_heads) {
  if (num_q_heads <= 0 || num_q_heads % num_kv_heads)
    return fail(PKV_ERR_INVALID, "num_q_heads %d is not a positive multiple of num_kv_heads %d",
                num_q_heads, num_kv_heads);
  if (num_q_heads / num_kv_heads > 16)
    return fail(PKV_ERR_UNSUPPORTED, "query heads per KV head %d > 16", num_q_heads / num_kv_heads);
  return PKV_OK;
}

constexpr int32_t kDefaultPieceTokens = 512;
constexpr int32_t kMaxPieces = 1 << 20;      // pieces per (sequence, query head)

// Smallest piece of a context one workgroup computes (tokens): the caller's
// choice or 512.  Longer contexts are split further only as the balance of
// the call requires.
int32_t choose_piece(int32_t partition_size) {
  return partition_size > 0 ? partition_size : kDefaultPieceTokens;
}

// Pieces per (sequence, query head) the workspace must hold: a context of
// nb blocks meets at most ceil(nb / piece) + 1 workgroup ranges.
int64_t max_pieces(int32_t max_context_len, int32_t ptok) {
  const int64_t nblk_tok = max_context_len > 0 ? max_context_len : 0;
  return (nblk_tok + ptok - 1) / ptok + 1;
}

// Two workgroups per compute unit: what the bf16 decode kernel keeps
// resident at once (cached per device).
int decode_workgroups() {
  static std::atomic<int> cached[64];   // zero-initialised (static storage)
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  if (dev < 64) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  if (dev < 64) cached[dev].store(2 * cus, std::memory_order_relaxed);
  return 2 * cus;
}

// Key split of the shared-prefix pass: enough splits that the pass's
// workgroups (groups x KV heads x 256-row tiles x splits) about fill the
// compute units once, in multiples of the kernel's 4-block key tile.
struct PrefixSplit {
  int32_t blocks;   // per split
  int32_t count;    // splits of the longest prefix
};
PrefixSplit prefix_split(int32_t num_groups, int32_t max_group_size, int32_t max_prefix_blocks,
                         int32_t g, int32_t num_kv_heads) {
  if (num_groups <= 0 || max_group_size <= 0 || max_prefix_blocks <= 0) return {4, 0};
  const int64_t row_tiles = ((int64_t)max_group_size * g + 255) / 256;
  const int64_t base = (int64_t)num_groups * num_kv_heads * row_tiles;
  const int64_t cus = decode_workgroups() / 2;
  // at most 8 splits: each member's merge folds in every split's partial
  const int64_t want = base >= cus ? 1 : (cus / base < 8 ? cus / base : 8);
  int64_t blocks = (max_prefix_blocks + want - 1) / want;
  blocks = (blocks + 3) / 4 * 4;
  return {(int32_t)blocks, (int32_t)((max_prefix_blocks + blocks - 1) / blocks)};
}

// A tag per decode call for its tagged words (bits 24..63 of a word; a
// count sits below: a split unit's pieces).  Tags come from one
// process-wide sequence that starts at a random point with its top bit set:
// a word written by an earlier call carries an earlier tag, and a word the
// library never wrote matches only if it happens to hold this exact tag.
uint64_t next_call_tag() {
  static std::atomic<uint64_t> next{[] {
    std::random_device rd;
    return ((uint64_t)rd() << 32) ^ (uint64_t)rd();
  }()};
  constexpr uint64_t kLow = (1ull << 39) - 1;
  return ((1ull << 39) | (next.fetch_add(1, std::memory_order_relaxed) & kLow)) << 24;
}

// Byte offsets of the shared-prefix decode's workspace regions.
struct SharedLayout {
  size_t seq_prefix, pre_o, pre_m, pre_l, total;
};
SharedLayout shared_layout(int64_t S, int64_t hq, int64_t hkv, int64_t D, int64_t P, int64_t NS) {
  SharedLayout l{};
  // the plain decode's layout (pieces, then piece-count words), then one tagged
  // word per sequence (8-byte aligned: D + 2 is even)
  const size_t dec = (size_t)S * hq * P * (D + 2) * 4 + (size_t)S * hkv * 8;
  l.seq_prefix = dec;
  const size_t after = dec + (size_t)S * 8;
  l.pre_o = (after + 255) / 256 * 256;
  l.pre_m = l.pre_o + (size_t)S * hq * NS * D * 4;
  l.pre_l = l.pre_m + (size_t)S * hq * NS * 4;
  l.total = l.pre_l + (size_t)S * hq * NS * 4;
  return l;
}

// The address a kernel uses for p: p itself for device memory, the device
// mapping for pinned host memory.  Non-zero for memory HIP does not know.
int device_view(const void* p, void** out) {
  hipPointerAttribute_t at{};
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();
    return 1;
  }
  if (at.type == hipMemoryTypeHost) {
    if (!at.devicePointer) return 1;
    *out = (uint8_t*)at.devicePointer + ((const uint8_t*)p - (const uint8_t*)at.hostPointer);
    return 0;
  }
  if (at.type == hipMemoryTypeDevice || at.type == hipMemoryTypeManaged) {
    *out = const_cast<void*>(p);
    return 0;
  }
  return 1;
}

}  // namespace

namespace pkv {
// Error reporting for entry points defined in other files.
int set_error(int code, const char* msg) { return fail(code, "%s", msg); }
int clear_error() { return ok(); }
}  // namespace pkv

extern "C" {

const char* paged_kv_last_error(void) { return g_err; }

int paged_kv_append(const void* k_new, const void* v_new, const int32_t* slot_mapping,
                    int32_t num_tokens, void* k_pool, void* v_pool, int32_t num_blocks,
                    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t dtype,
                    void* stream) {
  int rc = check_common(num_kv_heads, head_dim, block_size, dtype);
  if (rc) return rc;
  if (num_tokens < 0 || num_blocks <= 0) return fail(PKV_ERR_INVALID, "bad num_tokens/num_blocks");
  if (num_tokens == 0) return ok();
  if (!k_new || !v_new || !slot_mapping || !k_pool || !v_pool)
    return fail(PKV_ERR_INVALID, "null pointer argument");
  if ((int64_t)num_blocks * block_size > INT32_MAX)
    return fail(PKV_ERR_INVALID, "num_blocks * block_size exceeds the int32 slot range");
  rc = pkv::launch_append(k_new, v_new, slot_mapping, num_tokens, k_pool, v_pool, num_blocks,
                          num_kv_heads, head_dim, block_size, elem_bytes(dtype), (hipStream_t)stream);
  return rc ? fail(rc, "append launch failed: %s", hipGetErrorString(hipGetLastError())) : ok();
}

int copy_blocks(void* k_pool, void* v_pool, int32_t num_blocks, const int32_t* block_mapping,
                int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                int32_t dtype, void* stream) {
  int rc = check_common(num_kv_heads, head_dim, block_size, dtype);
  if (rc) return rc;
  if (num_pairs < 0 || num_blocks <= 0) return fail(PKV_ERR_INVALID, "bad num_pairs/num_blocks");
  if (num_pairs == 0) return ok();
  if (num_pairs > 65535) return fail(PKV_ERR_INVALID, "num_pairs %d > 65535 per call", num_pairs);
  if (!k_pool || !v_pool || !block_mapping) return fail(PKV_ERR_INVALID, "null pointer argument");
  rc = pkv::launch_copy_blocks(k_pool, v_pool, num_blocks, block_mapping, num_pairs, num_kv_heads,
                               head_dim, block_size, elem_bytes(dtype), (hipStream_t)stream);
  return rc ? fail(rc, "copy_blocks launch failed") : ok();
}

int swap_blocks(void* dst_k, void* dst_v, int32_t dst_num_blocks, const void* src_k,
                const void* src_v, int32_t src_num_blocks, const int32_t* block_mapping,
                int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                int32_t dtype, void* stream) {
  int rc = check_common(num_kv_heads, head_dim, block_size, dtype);
  if (rc) return rc;
  if (num_pairs < 0 || dst_num_blocks <= 0 || src_num_blocks <= 0)
    return fail(PKV_ERR_INVALID, "bad num_pairs/num_blocks");
  if (num_pairs == 0) return ok();
  if (!dst_k || !dst_v || !src_k || !src_v || !block_mapping)
    return fail(PKV_ERR_INVALID, "null pointer argument");
  void* dk = nullptr;
  void* dv = nullptr;
  void* sk = nullptr;
  void* sv = nullptr;
  if (device_view(dst_k, &dk) || device_view(dst_v, &dv) || device_view(src_k, &sk) ||
      device_view(src_v, &sv))
    return fail(PKV_ERR_INVALID, "pools must be device memory or pinned host memory");
  rc = pkv::launch_swap_blocks(dk, dv, dst_num_blocks, sk, sv, src_num_blocks, block_mapping,
                               num_pairs, num_kv_heads, head_dim, block_size, elem_bytes(dtype),
                               (hipStream_t)stream);
  return rc ? fail(rc, "swap_blocks launch failed") : ok();
}

int pinned_upload(void* dst, const void* src, int64_t bytes, void* stream) {
  if (bytes < 0) return fail(PKV_ERR_INVALID, "negative byte count");
  if (bytes == 0) return ok();
  if (!dst || !src) return fail(PKV_ERR_INVALID, "null pointer argument");
  void* d = nullptr;
  void* sv = nullptr;
  if (device_view(dst, &d) || device_view(src, &sv))
    return fail(PKV_ERR_INVALID, "buffers must be device memory or pinned host memory");
  const int rc = pkv::launch_upload(d, sv, bytes, (hipStream_t)stream);
  return rc ? fail(rc, "upload launch failed") : ok();
}

int upload_and_append_tables(void* dst, const void* staging, int64_t bytes, int64_t slots_offset,
                             int32_t* block_tables, int64_t table_words, int32_t num_updates,
                             const void* k_new, const void* v_new, int32_t num_tokens,
                             void* k_pool, void* v_pool, int32_t num_blocks, int32_t num_kv_heads,
                             int32_t head_dim, int32_t block_size, int32_t dtype, void* stream) {
  int rc = check_common(num_kv_heads, head_dim, block_size, dtype);
  if (rc) return rc;
  if (bytes < 0 || num_tokens < 0 || num_blocks <= 0 || num_updates < 0 || table_words < 0)
    return fail(PKV_ERR_INVALID, "bad bytes/num_tokens/num_blocks/num_updates/table_words");
  if (slots_offset < 0 || slots_offset % 4 || slots_offset + 4 * (int64_t)num_tokens > bytes)
    return fail(PKV_ERR_INVALID, "slot mapping (offset %lld, %d tokens) not inside the %lld staged bytes",
                (long long)slots_offset, num_tokens, (long long)bytes);
  if (num_updates > 0 && (bytes % 4 || !block_tables))
    return fail(PKV_ERR_INVALID, "table updates need block_tables and a staged size that is a "
                "multiple of 4 (%lld)", (long long)bytes);
  if (bytes == 0 && num_updates == 0) return ok();
  if (!dst || !staging) return fail(PKV_ERR_INVALID, "null pointer argument");
  if (num_tokens > 0 && (!k_new || !v_new || !k_pool || !v_pool))
    return fail(PKV_ERR_INVALID, "null pointer argument");
  void* d = nullptr;
  void* sv = nullptr;
  if (device_view(dst, &d) || device_view(staging, &sv))
    return fail(PKV_ERR_INVALID, "buffers must be device memory or pinned host memory");
  pkv::TableUpdates u;
  if (num_updates > 0) {
    void* tv = nullptr;
    if (device_view(block_tables, &tv))
      return fail(PKV_ERR_INVALID, "block_tables must be device memory");
    u.table = (int32_t*)tv;
    u.words = table_words;
    u.pairs = (const int32_t*)((const uint8_t*)sv + bytes);
    u.n = num_updates;
  }
  rc = pkv::launch_upload_append(d, sv, bytes, slots_offset, k_new, v_new, num_tokens, k_pool,
                                 v_pool, num_blocks, num_kv_heads, head_dim, block_size,
                                 elem_bytes(dtype), (hipStream_t)stream, u);
  return rc ? fail(rc, "upload_and_append launch failed") : ok();
}

int upload_and_append(void* dst, const void* staging, int64_t bytes, int64_t slots_offset,
                      const void* k_new, const void* v_new, int32_t num_tokens, void* k_pool,
                      void* v_pool, int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                      int32_t block_size, int32_t dtype, void* stream) {
  return upload_and_append_tables(dst, staging, bytes, slots_offset, nullptr, 0, 0, k_new, v_new,
                                  num_tokens, k_pool, v_pool, num_blocks, num_kv_heads, head_dim,
                                  block_size, dtype, stream);
}

int paged_kv_gather(void* k_out, void* v_out, const void* k_pool, const void* v_pool,
                    int32_t num_blocks, const int32_t* block_table_row, int32_t context_len,
                    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t dtype,
                    void* stream) {
  int rc = check_common(num_kv_heads, head_dim, block_size, dtype);
  if (rc) return rc;
  if (context_len < 0 || num_blocks <= 0) return fail(PKV_ERR_INVALID, "bad context_len/num_blocks");
  if (context_len == 0) return ok();
  if (!k_out || !v_out || !k_pool || !v_pool || !block_table_row)
    return fail(PKV_ERR_INVALID, "null pointer argument");
  rc = pkv::launch_gather(k_out, v_out, k_pool, v_pool, num_blocks, block_table_row, context_len,
                          num_kv_heads, head_dim, block_size, elem_bytes(dtype), (hipStream_t)stream);
  return rc ? fail(rc, "gather launch failed") : ok();
}

size_t paged_attention_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                             int32_t num_kv_heads, int32_t head_dim,
                                             int32_t max_context_len, int32_t partition_size) {
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || max_context_len < 0)
    return 0;
  const int32_t ptok = choose_piece(partition_size);
  if (ptok <= 0) return 0;
  const int64_t P = max_pieces(max_context_len, ptok);
  return (size_t)num_seqs * num_q_heads * P * (head_dim + 2) * sizeof(float) +
         (size_t)num_seqs * num_kv_heads * sizeof(uint64_t);
}

namespace {

// The bf16 decode kernels number the call's (sequence, KV head, block)
// triples, and the ranges of up to 4 x decode_workgroups() workgroups over
// them, in 32-bit arithmetic: refuse calls whose list could reach 2^31.
int check_positions(int32_t num_seqs, int32_t num_kv_heads, int32_t max_blocks_per_seq,
                    int64_t P, int32_t ptok, int32_t block_size) {
  // the kernels count 16-token granules (a 32-token block is two)
  const int64_t piece_blocks = ptok / 16;
  const int64_t nb = std::min<int64_t>((int64_t)max_blocks_per_seq * (block_size / 16),
                                       (P - 1) * piece_blocks);
  const int64_t list = (int64_t)num_seqs * num_kv_heads * nb;
  const int64_t wgs = 4 * (int64_t)decode_workgroups();
  if (list + wgs >= INT32_MAX || wgs * (piece_blocks + 1) >= INT32_MAX)
    return fail(PKV_ERR_INVALID,
                "%lld (sequence, KV head, block) triples in one call (2^31 at most); split the "
                "batch", (long long)list);
  return PKV_OK;
}

// Checks shared by the decode entries; sets *P (pieces per context the
// partials hold) and *ptok (piece tokens) on success.
int decode_prepare(const void* out, const void* q, const void* k_pool, const void* v_pool,
                   int32_t num_blocks, const int32_t* block_tables, int32_t max_blocks_per_seq,
                   const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
                   int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                   int32_t block_size, int32_t partition_size, int32_t dtype, int64_t* P,
                   int32_t* ptok) {
  int rc = check_common(num_kv_heads, head_dim, block_size, dtype);
  if (rc) return rc;
  rc = check_heads(num_q_heads, num_kv_heads);
  if (rc) return rc;
  if (num_seqs < 0 || num_blocks <= 0 || max_blocks_per_seq <= 0 || max_context_len < 0)
    return fail(PKV_ERR_INVALID, "bad num_seqs/num_blocks/max_blocks_per_seq/max_context_len");
  if (num_seqs == 0) return ok();
  if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens)
    return fail(PKV_ERR_INVALID, "null pointer argument");
  if ((int64_t)num_seqs * num_kv_heads > INT32_MAX) return fail(PKV_ERR_INVALID, "too many sequences");
  *ptok = choose_piece(partition_size);
  if (*ptok < 0 || *ptok % block_size)
    return fail(PKV_ERR_INVALID, "partition_size %d must be a multiple of %d", partition_size,
                block_size);
  *P = max_pieces(max_context_len, *ptok);
  if (*P > kMaxPieces || (dtype == 0 && *P - 1 > 65535))
    return fail(PKV_ERR_INVALID, "max_context_len %d needs %lld pieces per context (too many)",
                max_context_len, (long long)*P);
  // a merge stages [2][group][P] + [group] fp32 weights in LDS (160 KB)
  if (dtype == 1 && (2 * (num_q_heads / num_kv_heads) * *P + 16) * 4 > 160 * 1024 - 256)
    return fail(PKV_ERR_UNSUPPORTED,
                "max_context_len %d over partition_size %d gives %lld pieces per context; use a "
                "larger partition_size", max_context_len, *ptok, (long long)*P);
  return check_positions(num_seqs, num_kv_heads, max_blocks_per_seq, *P, *ptok, block_size);
}

pkv::DecodeArgs decode_args(void* out, const void* q, const void* k_pool, const void* v_pool,
                            int32_t num_blocks, const int32_t* block_tables,
                            int32_t max_blocks_per_seq, const int32_t* context_lens,
                            int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t block_size, float scale, int32_t ptok,
                            int64_t P, float* part_o, uint64_t* arrive) {
  pkv::DecodeArgs a{};
  a.out = out;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  const int64_t rows = (int64_t)num_seqs * num_q_heads * P;
  a.part_o = part_o;
  a.part_m = part_o + rows * head_dim;
  a.part_l = a.part_m + rows;
  a.arrive = arrive;
  a.tag = next_call_tag();
  a.num_blocks = num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.partition_blocks = ptok / 16;   // in 16-token granules
  a.bs_shift = block_size == 32 ? 1 : 0;
  a.max_partitions = (int32_t)P;
  a.num_workgroups = decode_workgroups();
  a.scale = scale;
  return a;
}

}  // namespace

int paged_attention_decode(void* out, const void* q, const void* k_pool, const void* v_pool,
                           int32_t num_blocks, const int32_t* block_tables,
                           int32_t max_blocks_per_seq, const int32_t* context_lens,
                           int32_t num_seqs, int32_t max_context_len, int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size, float scale,
                           int32_t partition_size, void* workspace, size_t workspace_bytes,
                           int32_t dtype, void* stream) {
  int64_t P = 0;
  int32_t ptok = 0;
  int rc = decode_prepare(out, q, k_pool, v_pool, num_blocks, block_tables, max_blocks_per_seq,
                          context_lens, num_seqs, max_context_len, num_q_heads, num_kv_heads,
                          head_dim, block_size, partition_size, dtype, &P, &ptok);
  if (rc || num_seqs == 0) return rc;
  const size_t need = paged_attention_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads,
                                                            head_dim, max_context_len, ptok);
  if (!workspace || workspace_bytes < need)
    return fail(PKV_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace_bytes);
  if ((uintptr_t)workspace % 8)
    return fail(PKV_ERR_WORKSPACE, "workspace must be 8-byte aligned");
  float* ws = (float*)workspace;
  const int64_t rows = (int64_t)num_seqs * num_q_heads * P;
  // rows * (D + 2) floats: a multiple of 8 bytes, so the words are aligned
  uint64_t* arrive = (uint64_t*)(ws + rows * (head_dim + 2));
  const pkv::DecodeArgs a =
      decode_args(out, q, k_pool, v_pool, num_blocks, block_tables, max_blocks_per_seq,
                  context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, scale,
                  ptok, P, ws, arrive);
  rc = pkv::launch_decode(a, dtype, (hipStream_t)stream);
  return rc ? fail(rc, "decode launch failed: %s", hipGetErrorString(hipGetLastError())) : ok();
}

int paged_attention_decode_noalloc(void* out, const void* q, const void* k_pool,
                                   const void* v_pool, int32_t num_blocks,
                                   const int32_t* block_tables, int32_t max_blocks_per_seq,
                                   const int32_t* context_lens, int32_t num_seqs,
                                   int32_t max_context_len, int32_t num_q_heads,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                   float scale, int32_t partition_size, int32_t dtype,
                                   void* stream) {
  int64_t P = 0;
  int32_t ptok = 0;
  int rc = decode_prepare(out, q, k_pool, v_pool, num_blocks, block_tables, max_blocks_per_seq,
                          context_lens, num_seqs, max_context_len, num_q_heads, num_kv_heads,
                          head_dim, block_size, partition_size, dtype, &P, &ptok);
  if (rc || num_seqs == 0) return rc;
  const int64_t units = (int64_t)num_seqs * num_kv_heads;
  const int64_t part_bytes = (int64_t)num_seqs * num_q_heads * P * (head_dim + 2) * 4;
  constexpr int64_t kMaxUnits = (int64_t)(pkv::kScratchArriveBytes / 8);
  constexpr int64_t kPartMax = (int64_t)(pkv::kScratchBytes - pkv::kScratchArriveBytes);
  if (units > kMaxUnits || part_bytes > kPartMax)
    return fail(PKV_ERR_WORKSPACE,
                "the allocation-free decode's fixed workspace is too small: %lld (sequence, KV "
                "head) units (at most %lld) and %lld bytes of partials (at most %lld); a larger "
                "partition_size or fewer sequences per call fit, or use paged_attention_decode",
                (long long)units, (long long)kMaxUnits, (long long)part_bytes,
                (long long)kPartMax);
  uint8_t* base = nullptr;
  rc = pkv::decode_scratch((hipStream_t)stream, &base);
  if (rc) return fail(rc, "allocation-free decode: no workspace on this device (%s)",
                      hipGetErrorString(hipGetLastError()));
  const pkv::DecodeArgs a =
      decode_args(out, q, k_pool, v_pool, num_blocks, block_tables, max_blocks_per_seq,
                  context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, scale,
                  ptok, P, (float*)(base + pkv::kScratchArriveBytes), (uint64_t*)base);
  rc = pkv::launch_decode(a, dtype, (hipStream_t)stream);
  return rc ? fail(rc, "decode launch failed: %s", hipGetErrorString(hipGetLastError())) : ok();
}

size_t paged_attention_decode_shared_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                                    int32_t num_kv_heads, int32_t head_dim,
                                                    int32_t max_context_len, int32_t partition_size,
                                                    int32_t num_groups, int32_t max_group_size,
                                                    int32_t max_prefix_blocks) {
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      max_context_len < 0 || num_groups < 0 || max_group_size < 0 || max_prefix_blocks < 0 ||
      num_q_heads % num_kv_heads)
    return 0;
  const int32_t ptok = choose_piece(partition_size);
  if (ptok <= 0) return 0;
  const int64_t P = max_pieces(max_context_len, ptok);
  const PrefixSplit sp = prefix_split(num_groups, max_group_size, max_prefix_blocks,
                                      num_q_heads / num_kv_heads, num_kv_heads);
  return shared_layout(num_seqs, num_q_heads, num_kv_heads, head_dim, P, sp.count).total;
}

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
                                  void* stream) {
  int rc = check_common(num_kv_heads, head_dim, block_size, dtype);
  if (rc) return rc;
  if (num_groups < 0 || max_group_size < 0 || max_prefix_blocks < 0)
    return fail(PKV_ERR_INVALID, "negative group argument");
  if (dtype != PKV_DTYPE_BF16 || num_groups == 0 || max_group_size == 0 ||
      max_prefix_blocks == 0)
    // nothing shared (or fp32, which has no prefix pass): the plain decode
    return paged_attention_decode(out, q, k_pool, v_pool, num_blocks, block_tables,
                                  max_blocks_per_seq, context_lens, num_seqs, max_context_len,
                                  num_q_heads, num_kv_heads, head_dim, block_size, scale,
                                  partition_size, workspace, workspace_bytes, dtype, stream);
  rc = check_heads(num_q_heads, num_kv_heads);
  if (rc) return rc;
  if (num_seqs < 0 || num_blocks <= 0 || max_blocks_per_seq <= 0 || max_context_len < 0)
    return fail(PKV_ERR_INVALID, "bad num_seqs/num_blocks/max_blocks_per_seq/max_context_len");
  if (num_seqs == 0) return ok();
  if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens || !group_offsets ||
      !group_seqs || !group_prefix_blocks)
    return fail(PKV_ERR_INVALID, "null pointer argument");
  if (max_group_size > num_seqs || max_prefix_blocks > max_blocks_per_seq)
    return fail(PKV_ERR_INVALID, "max_group_size %d > num_seqs or max_prefix_blocks %d > "
                "max_blocks_per_seq", max_group_size, max_prefix_blocks);
  if ((int64_t)num_seqs * num_q_heads > INT32_MAX / 2) return fail(PKV_ERR_INVALID, "too many sequences");
  const int32_t ptok = choose_piece(partition_size);
  if (ptok < 0 || ptok % block_size)
    return fail(PKV_ERR_INVALID, "partition_size %d must be a multiple of %d", partition_size,
                block_size);
  const int64_t P = max_pieces(max_context_len, ptok);
  const int32_t g = num_q_heads / num_kv_heads;
  const PrefixSplit sp = prefix_split(num_groups, max_group_size, max_prefix_blocks, g, num_kv_heads);
  if (P > kMaxPieces || (2 * g * (P + sp.count) + 16) * 4 > 160 * 1024 - 256)
    return fail(PKV_ERR_UNSUPPORTED,
                "max_context_len %d over partition_size %d gives %lld pieces per context; use a "
                "larger partition_size", max_context_len, ptok, (long long)P);
  // a sequence's start (in 16-token granules) travels in 20 bits of its tagged word
  if ((int64_t)sp.count * sp.blocks * (block_size / 16) >= (1 << 20))
    return fail(PKV_ERR_INVALID, "max_prefix_blocks %d too large", max_prefix_blocks);
  rc = check_positions(num_seqs, num_kv_heads, max_blocks_per_seq, P, ptok, block_size);
  if (rc) return rc;
  const SharedLayout lay = shared_layout(num_seqs, num_q_heads, num_kv_heads, head_dim, P, sp.count);
  if (!workspace || workspace_bytes < lay.total)
    return fail(PKV_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", lay.total,
                workspace_bytes);
  if ((uintptr_t)workspace % 8)
    return fail(PKV_ERR_WORKSPACE, "workspace must be 8-byte aligned");

  uint8_t* ws = (uint8_t*)workspace;
  pkv::DecodeArgs a{};
  a.out = out;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  {
    const int64_t rows = (int64_t)num_seqs * num_q_heads * P;
    a.part_o = (float*)ws;
    a.part_m = a.part_o + rows * head_dim;
    a.part_l = a.part_m + rows;
    a.arrive = (uint64_t*)(a.part_l + rows);
    a.tag = next_call_tag();
  }
  a.num_blocks = num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.partition_blocks = ptok / 16;   // in 16-token granules
  a.bs_shift = block_size == 32 ? 1 : 0;
  a.max_partitions = (int32_t)P;
  a.num_workgroups = decode_workgroups();
  a.scale = scale;
  a.seq_prefix = (uint64_t*)(ws + lay.seq_prefix);
  a.pre_o = (float*)(ws + lay.pre_o);
  a.pre_m = (float*)(ws + lay.pre_m);
  a.pre_l = (float*)(ws + lay.pre_l);
  a.num_splits = sp.count;

  pkv::PrefixArgs p{};
  p.q = q;
  p.k_pool = k_pool;
  p.v_pool = v_pool;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.group_offsets = group_offsets;
  p.group_seqs = group_seqs;
  p.group_prefix_blocks = group_prefix_blocks;
  p.pre_o = (float*)a.pre_o;
  p.pre_m = (float*)a.pre_m;
  p.pre_l = (float*)a.pre_l;
  p.seq_prefix = (uint64_t*)a.seq_prefix;
  p.tag = a.tag;
  p.num_groups = num_groups;
  p.max_group_size = max_group_size;
  p.num_seqs = num_seqs;
  p.num_blocks = num_blocks;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.head_dim = head_dim;
  p.block_size = block_size;
  p.split_blocks = sp.blocks;
  p.num_splits = sp.count;
  p.scale = scale;

  hipStream_t st = (hipStream_t)stream;
  // nothing to clear: the prefix pass tags the words it writes with this
  // call's tag, and the decode reads any other word as "no prefix"
  rc = pkv::launch_prefix(p, st);
  if (!rc) rc = pkv::launch_decode(a, dtype, st);
  return rc ? fail(rc, "shared-prefix decode launch failed: %s", hipGetErrorString(hipGetLastError()))
            : ok();
}

int paged_attention_extend(void* out, const void* q, const int32_t* cu_seqlens_q,
                           const int32_t* seq_lens, int32_t num_reqs, int32_t total_q,
                           int32_t max_q_len, int32_t max_seq_len, const void* k_pool,
                           const void* v_pool, int32_t num_blocks, const int32_t* block_tables,
                           int32_t max_blocks_per_seq, int32_t num_q_heads, int32_t num_kv_heads,
                           int32_t head_dim, int32_t block_size, float scale, int32_t dtype,
                           void* stream) {
  int rc = check_common(num_kv_heads, head_dim, block_size, dtype);
  if (rc) return rc;
  rc = check_heads(num_q_heads, num_kv_heads);
  if (rc) return rc;
  if (num_reqs < 0 || total_q < 0 || max_q_len < 0 || max_seq_len < 0 || num_blocks <= 0 ||
      max_blocks_per_seq <= 0)
    return fail(PKV_ERR_INVALID, "negative size argument");
  if (num_reqs == 0 || total_q == 0) return ok();
  if (!out || !q || !cu_seqlens_q || !seq_lens || !k_pool || !v_pool || !block_tables)
    return fail(PKV_ERR_INVALID, "null pointer argument");
  if (max_q_len > 65535 && dtype == PKV_DTYPE_FP32)
    return fail(PKV_ERR_INVALID, "max_q_len %d > 65535 for fp32", max_q_len);
  pkv::ExtendArgs a{};
  a.out = out;
  a.q = q;
  a.cu_seqlens_q = cu_seqlens_q;
  a.seq_lens = seq_lens;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_tables = block_tables;
  a.num_reqs = num_reqs;
  a.total_q = total_q;
  a.max_q_len = max_q_len;
  a.max_seq_len = max_seq_len;
  a.num_blocks = num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.block_size = block_size;
  a.scale = scale;
  rc = pkv::launch_extend(a, dtype, (hipStream_t)stream);
  return rc ? fail(rc, "extend launch failed: %s", hipGetErrorString(hipGetLastError())) : ok();
}

}  // extern "C"
