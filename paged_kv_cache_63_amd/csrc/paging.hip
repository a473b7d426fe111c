// Pool writes and reads that move bits only: append (token -> slot),
// copy-on-write block copy, and the gather of one sequence's blocks.
//
// Pool layout: K [num_blocks][Hkv][B][D]; V [num_blocks][Hkv] slabs of
// B/16 channel-major 16-token halves [D][16], the tokens of a channel row in
// the order v_pos (bits 2 and 3 of the offset exchanged: 0-3, 8-11, 4-7,
// 12-15), see v_elem.  Every thread moves one 16-byte piece of a key or
// value row; all offsets are 64-bit.
#include "common.h"

namespace pkv {
namespace {

constexpr int kThreads = 256;
constexpr int kBulkTokens = 512;  // appends of at least this many tokens look for full-block runs

// One thread per 16-byte piece of one (token, head) row of k_new/v_new.
// The key piece is stored as it is (rows are contiguous in the K pool); the
// value piece is split into its 16/E elements, each going to its channel's
// row of the transposed V block.
// (Workgroup wg of nwg doing this work.)
template <int E>
__device__ __forceinline__ void append_pieces(
    const uint8_t* __restrict__ k_new, const uint8_t* __restrict__ v_new,
    const int32_t* __restrict__ slots, int64_t pieces, int32_t pieces_per_row, int32_t hkv,
    int32_t d, int32_t bs, int32_t num_blocks, uint8_t* __restrict__ k_pool,
    uint8_t* __restrict__ v_pool, int64_t wg, int64_t nwg) {
  constexpr int kPer = 16 / E;  // elements per piece
  const int64_t row_bytes = (int64_t)d * E;
  for (int64_t i = wg * kThreads + threadIdx.x; i < pieces; i += nwg * kThreads) {
    const int64_t row = i / pieces_per_row;        // token * hkv + head
    const int32_t piece = (int32_t)(i - row * pieces_per_row);
    const int64_t t = row / hkv;
    const int32_t h = (int32_t)(row - t * hkv);
    const int32_t slot = slots[t];
    if (slot < 0 || slot >= num_blocks * bs) continue;
    const int32_t blk = slot / bs, off = slot - blk * bs;
    const int64_t src = row * row_bytes + (int64_t)piece * 16;
    const u32x4 kv = *reinterpret_cast<const u32x4*>(k_new + src);
    const u32x4 vv = *reinterpret_cast<const u32x4*>(v_new + src);
    const int64_t head_base = ((int64_t)blk * hkv + h) * bs * row_bytes;  // bytes
    *reinterpret_cast<u32x4*>(k_pool + head_base + (int64_t)off * row_bytes + piece * 16) = kv;
    const int32_t c0 = piece * kPer;  // first channel of the piece
    uint8_t* vrow = v_pool + head_base + v_elem(off, c0, d) * E;
    if constexpr (E == 2) {
      const uint32_t w[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
      for (int e = 0; e < kPer; ++e) {
        const uint16_t x = (uint16_t)(w[e >> 1] >> ((e & 1) * 16));
        *reinterpret_cast<uint16_t*>(vrow + (int64_t)e * kVRow * E) = x;
      }
    } else {
      const uint32_t w[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
      for (int e = 0; e < kPer; ++e) *reinterpret_cast<uint32_t*>(vrow + (int64_t)e * kVRow * E) = w[e];
    }
  }
}

template <int E>
__global__ __launch_bounds__(kThreads) void append_kernel(
    const uint8_t* __restrict__ k_new, const uint8_t* __restrict__ v_new,
    const int32_t* __restrict__ slots, int64_t pieces, int32_t pieces_per_row, int32_t hkv,
    int32_t d, int32_t bs, int32_t num_blocks, uint8_t* __restrict__ k_pool,
    uint8_t* __restrict__ v_pool) {
  append_pieces<E>(k_new, v_new, slots, pieces, pieces_per_row, hkv, d, bs, num_blocks, k_pool,
                   v_pool, blockIdx.x, gridDim.x);
}

// grid.y = pair; each thread copies 16-byte pieces of the K block and of the
// V block of that pair.
__global__ __launch_bounds__(kThreads) void copy_blocks_kernel(
    uint8_t* __restrict__ k_pool, uint8_t* __restrict__ v_pool, const int32_t* __restrict__ map,
    int32_t num_blocks, int64_t block_bytes) {
  const int32_t src = map[2 * blockIdx.y], dst = map[2 * blockIdx.y + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  const int64_t pieces = block_bytes / 16;
  const int64_t s0 = (int64_t)src * block_bytes, d0 = (int64_t)dst * block_bytes;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < pieces;
       i += (int64_t)gridDim.x * kThreads) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(k_pool + s0 + i * 16);
    const u32x4 b = *reinterpret_cast<const u32x4*>(v_pool + s0 + i * 16);
    *reinterpret_cast<u32x4*>(k_pool + d0 + i * 16) = a;
    *reinterpret_cast<u32x4*>(v_pool + d0 + i * 16) = b;
  }
}

// Does token j start a full-block run: slot % 16 == 0 and the next 15
// tokens take the following slots of the same block?  The 16 loads are
// independent so that they are in flight together.
__device__ __forceinline__ bool full_run_at(const int32_t* slots, int64_t j, int64_t n,
                                            int32_t num_blocks) {
  if (j < 0 || j + 16 > n) return false;
  const int32_t s0 = slots[j];
  bool ok = s0 >= 0 && s0 < num_blocks * 16 && (s0 & 15) == 0;
#pragma unroll
  for (int i = 1; i < 16; ++i) ok &= slots[j + i] == s0 + i;
  return ok;
}

// Bulk append (block size 16), one launch in two parts.  Workgroups
// [0, n_win) take one window of 16 input tokens each and handle the
// full-block run that starts in it, if any (at most one can): the 16 tokens'
// key rows are copied as whole rows, and their value rows are staged in LDS
// in input order and read back transposed, so that every (head, channel) row
// of the V block leaves as whole 16-byte stores instead of 16 scattered
// element stores.  In the remaining workgroups each wave takes one token
// and, unless the token is skipped or inside a full run, writes it as
// append_kernel does.  Every pool word is written by exactly one thread.
// Below kBulkTokens tokens (a decode step's one token per sequence) runs are
// rare and append_kernel alone is faster.
constexpr int kBulkLds = 32768;   // V staging: [16 tokens][heads of one chunk][D] elements
constexpr int kWaves = kThreads / 64;

template <int E>
__global__ __launch_bounds__(kThreads) void append_bulk_kernel(
    const uint8_t* __restrict__ k_new, const uint8_t* __restrict__ v_new,
    const int32_t* __restrict__ slots, int64_t num_tokens, int64_t n_win, int32_t pieces_per_row,
    int32_t hkv, int32_t d, int32_t num_blocks, uint8_t* __restrict__ k_pool,
    uint8_t* __restrict__ v_pool) {
  constexpr int bs = 16;
  constexpr int kPer = 16 / E;
  constexpr int kB = 4;                      // loads in flight per thread per batch
  extern __shared__ __attribute__((aligned(16))) uint8_t vbuf[];
  const int64_t row_bytes = (int64_t)d * E;
  if (blockIdx.x < n_win) {
    const int64_t w0 = (int64_t)blockIdx.x * bs;
    __shared__ int64_t run_j;
    if (threadIdx.x < 64) {   // lane i of wave 0 tests a run starting at w0 + i
      const int i = threadIdx.x;
      const bool ok = i < bs && full_run_at(slots, w0 + i, num_tokens, num_blocks);
      const unsigned long long m = __ballot(ok);
      if (i == 0) run_j = m ? w0 + __ffsll((long long)m) - 1 : -1;
    }
    __syncthreads();
    const int64_t j0 = run_j;
    if (j0 < 0) return;
    const int32_t blk = slots[j0] >> 4;
    const int32_t ppr = pieces_per_row;
    // K: piece i of the run's input (rows (tok, h), contiguous) goes to row
    // (h, tok) of the block
    const uint8_t* ksrc = k_new + j0 * hkv * row_bytes;
    uint8_t* kblk = k_pool + (int64_t)blk * hkv * bs * row_bytes;
    const int32_t kpieces = bs * hkv * ppr;
    for (int32_t b0 = threadIdx.x; b0 < kpieces; b0 += kB * kThreads) {
      u32x4 r[kB];
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        const int32_t i = b0 + u * kThreads;
        if (i < kpieces) r[u] = *reinterpret_cast<const u32x4*>(ksrc + (int64_t)i * 16);
      }
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        const int32_t i = b0 + u * kThreads;
        if (i < kpieces) {
          const int32_t row = i / ppr, piece = i - row * ppr;
          const int32_t tok = row / hkv, h = row - tok * hkv;
          *reinterpret_cast<u32x4*>(kblk + ((int64_t)h * bs + tok) * row_bytes + piece * 16) = r[u];
        }
      }
    }
    // V: heads in chunks of hc whose [16][hc][D] staging fits kBulkLds
    const uint8_t* vsrc = v_new + j0 * hkv * row_bytes;
    const int hc_max = max(1, (int)(kBulkLds / (bs * row_bytes)));
    for (int h0 = 0; h0 < hkv; h0 += hc_max) {
      const int hc = min(hc_max, hkv - h0);
      const int32_t cpr = hc * ppr;          // pieces of one token's chunk
      const int32_t vpieces = bs * cpr;
      for (int32_t b0 = threadIdx.x; b0 < vpieces; b0 += kB * kThreads) {
        u32x4 r[kB];
#pragma unroll
        for (int u = 0; u < kB; ++u) {
          const int32_t i = b0 + u * kThreads;
          if (i < vpieces) {
            const int32_t tok = i / cpr, rest = i - tok * cpr;
            r[u] = *reinterpret_cast<const u32x4*>(vsrc + ((int64_t)tok * hkv + h0) * row_bytes +
                                                   (int64_t)rest * 16);
          }
        }
#pragma unroll
        for (int u = 0; u < kB; ++u) {
          const int32_t i = b0 + u * kThreads;
          if (i < vpieces) *reinterpret_cast<u32x4*>(vbuf + (int64_t)i * 16) = r[u];
        }
      }
      __syncthreads();
      // channel rows out: the element of (token tok, head hl, channel c)
      // sits at staging index (tok * hc + hl) * d + c; position p of a row
      // holds token v_pos(p)
      const uint32_t* w32 = reinterpret_cast<const uint32_t*>(vbuf);
      uint8_t* vblk = v_pool + ((int64_t)blk * hkv + h0) * d * bs * E;
      if constexpr (E == 2) {
        // one task = channels c, c + 1 of one head: one dword per token
        // holds both, and the two rows are 64 contiguous bytes
        const int32_t tasks = hc * d / 2;
        for (int32_t q = threadIdx.x; q < tasks; q += kThreads) {
          const int32_t hl = q / (d / 2), c = 2 * (q - hl * (d / 2));
          uint32_t w[bs];
#pragma unroll
          for (int p = 0; p < bs; ++p) w[p] = w32[((v_pos(p) * hc + hl) * d + c) >> 1];
          uint32_t lo[bs / 2], hi[bs / 2];
#pragma unroll
          for (int k = 0; k < bs / 2; ++k) {
            lo[k] = (w[2 * k] & 0xffffu) | (w[2 * k + 1] << 16);
            hi[k] = (w[2 * k] >> 16) | (w[2 * k + 1] & 0xffff0000u);
          }
          u32x4* dst = reinterpret_cast<u32x4*>(vblk + ((int64_t)hl * d + c) * bs * E);
          dst[0] = u32x4{lo[0], lo[1], lo[2], lo[3]};
          dst[1] = u32x4{lo[4], lo[5], lo[6], lo[7]};
          dst[2] = u32x4{hi[0], hi[1], hi[2], hi[3]};
          dst[3] = u32x4{hi[4], hi[5], hi[6], hi[7]};
        }
      } else {
        const int32_t tasks = hc * d;        // one task = one channel row
        for (int32_t q = threadIdx.x; q < tasks; q += kThreads) {
          const int32_t hl = q / d, c = q - hl * d;
          uint32_t w[bs];
#pragma unroll
          for (int p = 0; p < bs; ++p) w[p] = w32[(v_pos(p) * hc + hl) * d + c];
          u32x4* dst = reinterpret_cast<u32x4*>(vblk + ((int64_t)hl * d + c) * bs * E);
#pragma unroll
          for (int k = 0; k < 4; ++k) dst[k] = u32x4{w[4 * k], w[4 * k + 1], w[4 * k + 2], w[4 * k + 3]};
        }
      }
      __syncthreads();
    }
    return;
  }
  // one token per wave, outside full runs
  const int64_t t = (int64_t)(blockIdx.x - n_win) * kWaves + threadIdx.x / 64;
  if (t >= num_tokens) return;
  // lane k < 16 tests a run starting at t - 15 + k: all loads in flight together
  const int lane = threadIdx.x & 63;
  const bool starts = lane < bs && full_run_at(slots, t - 15 + lane, num_tokens, num_blocks);
  if (__ballot(starts)) return;
  const int32_t slot = slots[t];
  if (slot < 0 || slot >= num_blocks * bs) return;
  const int32_t blk = slot >> 4, off = slot & 15;
  const int32_t pieces = hkv * pieces_per_row;
  for (int32_t i = threadIdx.x % 64; i < pieces; i += 64) {
    const int32_t h = i / pieces_per_row, piece = i - h * pieces_per_row;
    const int64_t src = (t * hkv + h) * row_bytes + (int64_t)piece * 16;
    const u32x4 kv = *reinterpret_cast<const u32x4*>(k_new + src);
    const u32x4 vv = *reinterpret_cast<const u32x4*>(v_new + src);
    const int64_t head_base = ((int64_t)blk * hkv + h) * bs * row_bytes;
    *reinterpret_cast<u32x4*>(k_pool + head_base + (int64_t)off * row_bytes + piece * 16) = kv;
    const int32_t c0 = piece * kPer;
    uint8_t* vrow = v_pool + head_base + v_elem(off, c0, d) * E;
    const uint32_t w[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      if constexpr (E == 2)
        *reinterpret_cast<uint16_t*>(vrow + (int64_t)e * kVRow * E) = (uint16_t)(w[e >> 1] >> ((e & 1) * 16));
      else
        *reinterpret_cast<uint32_t*>(vrow + (int64_t)e * kVRow * E) = w[e];
    }
  }
}

// Byte copy into device memory from a source the device can read (the
// device mapping of pinned host memory): 16-byte pieces when both ends are
// 16-byte aligned, then the remaining bytes one by one.
__device__ __forceinline__ void upload_bytes(uint8_t* __restrict__ dst,
                                             const uint8_t* __restrict__ src, int64_t bytes,
                                             int vec, int64_t wg, int64_t nwg) {
  const int64_t stride = nwg * kThreads;
  const int64_t t0 = wg * kThreads + threadIdx.x;
  int64_t done = 0;
  if (vec) {
    const int64_t n16 = bytes / 16;
    for (int64_t i = t0; i < n16; i += stride)
      reinterpret_cast<u32x4*>(dst)[i] = reinterpret_cast<const u32x4*>(src)[i];
    done = n16 * 16;
  }
  for (int64_t i = done + t0; i < bytes; i += stride) dst[i] = src[i];
}

// Block-table updates that travel with an upload: table[pairs[2i]] =
// pairs[2i + 1] for i < n (the pairs read through the staging buffer's
// device mapping); an index outside [0, words) is skipped.
__device__ __forceinline__ void apply_updates(const TableUpdates& u, int64_t wg, int64_t nwg) {
  for (int64_t i = wg * kThreads + threadIdx.x; i < u.n; i += nwg * kThreads) {
    const int32_t idx = u.pairs[2 * i];
    const int32_t val = u.pairs[2 * i + 1];
    if (idx >= 0 && idx < u.words) u.table[idx] = val;
  }
}

__global__ __launch_bounds__(kThreads) void upload_kernel(uint8_t* __restrict__ dst,
                                                          const uint8_t* __restrict__ src,
                                                          int64_t bytes, int vec, TableUpdates u) {
  upload_bytes(dst, src, bytes, vec, blockIdx.x, gridDim.x);
  apply_updates(u, blockIdx.x, gridDim.x);
}

// A decode step's host->device traffic in one launch: workgroups
// [0, up_wgs) copy the staging buffer as upload_kernel does, the others
// write the new tokens as append_kernel does, reading each token's slot
// from the staging buffer itself (through its device mapping), so neither
// part waits for the other.
template <int E>
__global__ __launch_bounds__(kThreads) void upload_append_kernel(
    uint8_t* __restrict__ dst, const uint8_t* __restrict__ src, int64_t bytes, int vec,
    int32_t up_wgs, const uint8_t* __restrict__ k_new, const uint8_t* __restrict__ v_new,
    const int32_t* __restrict__ slots, int64_t pieces, int32_t pieces_per_row, int32_t hkv,
    int32_t d, int32_t bs, int32_t num_blocks, uint8_t* __restrict__ k_pool,
    uint8_t* __restrict__ v_pool, TableUpdates u) {
  if ((int32_t)blockIdx.x < up_wgs) {
    upload_bytes(dst, src, bytes, vec, blockIdx.x, up_wgs);
    apply_updates(u, blockIdx.x, up_wgs);
  } else
    append_pieces<E>(k_new, v_new, slots, pieces, pieces_per_row, hkv, d, bs, num_blocks, k_pool,
                     v_pool, blockIdx.x - up_wgs, gridDim.x - up_wgs);
}

// Block copy between two pools (one of them may be pinned host memory, seen
// through its device mapping): every (pair, 16-byte piece) of the K and V
// blocks, grid-stride; each thread has kSwapU pieces of K and of V in flight
// before it stores any (host-link reads have long latency).
constexpr int kSwapU = 4;
__global__ __launch_bounds__(kThreads) void swap_blocks_kernel(
    uint8_t* __restrict__ dst_k, uint8_t* __restrict__ dst_v, const uint8_t* __restrict__ src_k,
    const uint8_t* __restrict__ src_v, const int32_t* __restrict__ map, int32_t num_src,
    int32_t num_dst, int64_t block_pieces, int64_t total) {
  const int64_t step = (int64_t)gridDim.x * kThreads;
  for (int64_t i0 = (int64_t)blockIdx.x * kThreads + threadIdx.x; i0 < total; i0 += step * kSwapU) {
    u32x4 a[kSwapU], b[kSwapU];
    int64_t so[kSwapU], dof[kSwapU];
    bool ok[kSwapU];
#pragma unroll
    for (int u = 0; u < kSwapU; ++u) {
      const int64_t i = i0 + u * step;
      const int64_t pair = i / block_pieces;
      const int64_t piece = i - pair * block_pieces;
      const int32_t src = i < total ? map[2 * pair] : -1;
      const int32_t dst = i < total ? map[2 * pair + 1] : -1;
      ok[u] = src >= 0 && src < num_src && dst >= 0 && dst < num_dst;
      so[u] = ((int64_t)(ok[u] ? src : 0) * block_pieces + piece) * 16;
      dof[u] = ((int64_t)(ok[u] ? dst : 0) * block_pieces + piece) * 16;
      if (ok[u]) {
        a[u] = *reinterpret_cast<const u32x4*>(src_k + so[u]);
        b[u] = *reinterpret_cast<const u32x4*>(src_v + so[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < kSwapU; ++u)
      if (ok[u]) {
        *reinterpret_cast<u32x4*>(dst_k + dof[u]) = a[u];
        *reinterpret_cast<u32x4*>(dst_v + dof[u]) = b[u];
      }
  }
}

// One thread per 16-byte piece of the output rows [ctx][hkv][d].
template <int E>
__global__ __launch_bounds__(kThreads) void gather_kernel(
    uint8_t* __restrict__ k_out, uint8_t* __restrict__ v_out, const uint8_t* __restrict__ k_pool,
    const uint8_t* __restrict__ v_pool, const int32_t* __restrict__ table, int64_t pieces,
    int32_t pieces_per_row, int32_t hkv, int32_t d, int32_t bs, int32_t num_blocks) {
  constexpr int kPer = 16 / E;
  const int64_t row_bytes = (int64_t)d * E;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < pieces;
       i += (int64_t)gridDim.x * kThreads) {
    const int64_t row = i / pieces_per_row;
    const int32_t piece = (int32_t)(i - row * pieces_per_row);
    const int64_t t = row / hkv;
    const int32_t h = (int32_t)(row - t * hkv);
    int32_t blk = table[t / bs];
    if (blk < 0 || blk >= num_blocks) blk = 0;
    const int32_t off = (int32_t)(t % bs);
    const int64_t head_base = ((int64_t)blk * hkv + h) * bs * row_bytes;
    const int64_t dst = row * row_bytes + (int64_t)piece * 16;
    *reinterpret_cast<u32x4*>(k_out + dst) =
        *reinterpret_cast<const u32x4*>(k_pool + head_base + (int64_t)off * row_bytes + piece * 16);
    const uint8_t* vrow = v_pool + head_base + v_elem(off, piece * kPer, d) * E;
    uint32_t w[4];
    if constexpr (E == 2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t lo = *reinterpret_cast<const uint16_t*>(vrow + (int64_t)(2 * e) * kVRow * E);
        const uint32_t hi = *reinterpret_cast<const uint16_t*>(vrow + (int64_t)(2 * e + 1) * kVRow * E);
        w[e] = lo | (hi << 16);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = *reinterpret_cast<const uint32_t*>(vrow + (int64_t)e * kVRow * E);
    }
    *reinterpret_cast<u32x4*>(v_out + dst) = u32x4{w[0], w[1], w[2], w[3]};
  }
}

int grid_for(int64_t work) {
  const int64_t g = (work + kThreads - 1) / kThreads;
  return (int)(g < 65536 ? (g > 0 ? g : 1) : 65536);
}

int status_of(hipError_t e) { return e == hipSuccess ? 0 : -4; }

}  // namespace

int launch_append(const void* k_new, const void* v_new, const int32_t* slots, int32_t num_tokens,
                  void* k_pool, void* v_pool, int32_t num_blocks, int32_t hkv, int32_t d,
                  int32_t bs, int32_t elem_bytes, hipStream_t st) {
  const int32_t ppr = d * elem_bytes / 16;
  const int64_t pieces = (int64_t)num_tokens * hkv * ppr;
  if (pieces == 0) return 0;
  const int grid = grid_for(pieces);
  if (num_tokens >= kBulkTokens && bs == 16) {
    // full-block runs through LDS, the other tokens one per wave, in one launch
    const int64_t n_win = (num_tokens + 15) / 16;
    const int64_t g = n_win + (num_tokens + kWaves - 1) / kWaves;
    if (g > 0x7fffffff) return -1;
    const size_t lds = kBulkLds;
    if (elem_bytes == 2)
      append_bulk_kernel<2><<<(unsigned)g, kThreads, lds, st>>>(
          (const uint8_t*)k_new, (const uint8_t*)v_new, slots, num_tokens, n_win, ppr, hkv, d,
          num_blocks, (uint8_t*)k_pool, (uint8_t*)v_pool);
    else
      append_bulk_kernel<4><<<(unsigned)g, kThreads, lds, st>>>(
          (const uint8_t*)k_new, (const uint8_t*)v_new, slots, num_tokens, n_win, ppr, hkv, d,
          num_blocks, (uint8_t*)k_pool, (uint8_t*)v_pool);
    return status_of(hipGetLastError());
  }
  if (elem_bytes == 2)
    append_kernel<2><<<grid, kThreads, 0, st>>>((const uint8_t*)k_new, (const uint8_t*)v_new, slots,
                                                pieces, ppr, hkv, d, bs, num_blocks,
                                                (uint8_t*)k_pool, (uint8_t*)v_pool);
  else
    append_kernel<4><<<grid, kThreads, 0, st>>>((const uint8_t*)k_new, (const uint8_t*)v_new, slots,
                                                pieces, ppr, hkv, d, bs, num_blocks,
                                                (uint8_t*)k_pool, (uint8_t*)v_pool);
  return status_of(hipGetLastError());
}

int launch_copy_blocks(void* k_pool, void* v_pool, int32_t num_blocks, const int32_t* mapping,
                       int32_t num_pairs, int32_t hkv, int32_t d, int32_t bs, int32_t elem_bytes,
                       hipStream_t st) {
  if (num_pairs == 0) return 0;
  const int64_t block_bytes = (int64_t)hkv * bs * d * elem_bytes;
  int gx = grid_for(block_bytes / 16);
  if (gx > 64) gx = 64;
  copy_blocks_kernel<<<dim3(gx, num_pairs), kThreads, 0, st>>>(
      (uint8_t*)k_pool, (uint8_t*)v_pool, mapping, num_blocks, block_bytes);
  return status_of(hipGetLastError());
}

int launch_swap_blocks(void* dst_k, void* dst_v, int32_t num_dst, const void* src_k,
                       const void* src_v, int32_t num_src, const int32_t* mapping,
                       int32_t num_pairs, int32_t hkv, int32_t d, int32_t bs, int32_t elem_bytes,
                       hipStream_t st) {
  if (num_pairs == 0) return 0;
  const int64_t block_pieces = (int64_t)hkv * bs * d * elem_bytes / 16;
  const int64_t total = block_pieces * num_pairs;
  int64_t grid = (total + (int64_t)kThreads * kSwapU - 1) / ((int64_t)kThreads * kSwapU);
  if (grid > 4096) grid = 4096;
  swap_blocks_kernel<<<(unsigned)grid, kThreads, 0, st>>>(
      (uint8_t*)dst_k, (uint8_t*)dst_v, (const uint8_t*)src_k, (const uint8_t*)src_v, mapping,
      num_src, num_dst, block_pieces, total);
  return status_of(hipGetLastError());
}

int launch_gather(void* k_out, void* v_out, const void* k_pool, const void* v_pool,
                  int32_t num_blocks, const int32_t* row, int32_t ctx, int32_t hkv, int32_t d,
                  int32_t bs, int32_t elem_bytes, hipStream_t st) {
  const int32_t ppr = d * elem_bytes / 16;
  const int64_t pieces = (int64_t)ctx * hkv * ppr;
  if (pieces == 0) return 0;
  const int grid = grid_for(pieces);
  if (elem_bytes == 2)
    gather_kernel<2><<<grid, kThreads, 0, st>>>((uint8_t*)k_out, (uint8_t*)v_out,
                                                (const uint8_t*)k_pool, (const uint8_t*)v_pool, row,
                                                pieces, ppr, hkv, d, bs, num_blocks);
  else
    gather_kernel<4><<<grid, kThreads, 0, st>>>((uint8_t*)k_out, (uint8_t*)v_out,
                                                (const uint8_t*)k_pool, (const uint8_t*)v_pool, row,
                                                pieces, ppr, hkv, d, bs, num_blocks);
  return status_of(hipGetLastError());
}

// The upload's grid: one round of 16-byte pieces for the sizes a step's
// index arrays have, at most 1024 workgroups beyond that.
static int upload_vec(const void* dst, const void* src) {
  return (((uintptr_t)dst | (uintptr_t)src) & 15) == 0;
}

static int64_t upload_grid(int64_t bytes, int vec) {
  const int64_t work = vec ? bytes / 16 + 16 : bytes;
  const int64_t g = (work + kThreads - 1) / kThreads;
  return g < 1 ? 1 : (g > 1024 ? 1024 : g);
}

int launch_upload(void* dst, const void* src, int64_t bytes, hipStream_t st, TableUpdates u) {
  const int vec = upload_vec(dst, src);
  const int64_t g = max(upload_grid(bytes, vec), min((u.n + kThreads - 1) / kThreads, (int64_t)1024));
  upload_kernel<<<(unsigned)max(g, (int64_t)1), kThreads, 0, st>>>(
      (uint8_t*)dst, (const uint8_t*)src, bytes, vec, u);
  return status_of(hipGetLastError());
}

int launch_upload_append(void* dst, const void* src, int64_t bytes, int64_t slots_offset,
                         const void* k_new, const void* v_new, int32_t num_tokens, void* k_pool,
                         void* v_pool, int32_t num_blocks, int32_t hkv, int32_t d, int32_t bs,
                         int32_t elem_bytes, hipStream_t st, TableUpdates u) {
  if (num_tokens == 0) return bytes > 0 || u.n > 0 ? launch_upload(dst, src, bytes, st, u) : 0;
  if (num_tokens >= kBulkTokens && bs == 16) {
    // bulk: the window scans read the slots many times, from the device copy
    int rc = bytes > 0 || u.n > 0 ? launch_upload(dst, src, bytes, st, u) : 0;
    if (rc) return rc;
    return launch_append(k_new, v_new, (const int32_t*)((const uint8_t*)dst + slots_offset),
                         num_tokens, k_pool, v_pool, num_blocks, hkv, d, bs, elem_bytes, st);
  }
  const int vec = upload_vec(dst, src);
  const int64_t up = max(upload_grid(bytes, vec), min((u.n + kThreads - 1) / kThreads, (int64_t)1024));
  const int32_t ppr = d * elem_bytes / 16;
  const int64_t pieces = (int64_t)num_tokens * hkv * ppr;
  const int64_t g = up + grid_for(pieces);
  const int32_t* slots = (const int32_t*)((const uint8_t*)src + slots_offset);
  if (elem_bytes == 2)
    upload_append_kernel<2><<<(unsigned)g, kThreads, 0, st>>>(
        (uint8_t*)dst, (const uint8_t*)src, bytes, vec, (int32_t)up, (const uint8_t*)k_new,
        (const uint8_t*)v_new, slots, pieces, ppr, hkv, d, bs, num_blocks, (uint8_t*)k_pool,
        (uint8_t*)v_pool, u);
  else
    upload_append_kernel<4><<<(unsigned)g, kThreads, 0, st>>>(
        (uint8_t*)dst, (const uint8_t*)src, bytes, vec, (int32_t)up, (const uint8_t*)k_new,
        (const uint8_t*)v_new, slots, pieces, ppr, hkv, d, bs, num_blocks, (uint8_t*)k_pool,
        (uint8_t*)v_pool, u);
  return status_of(hipGetLastError());
}

}  // namespace pkv
