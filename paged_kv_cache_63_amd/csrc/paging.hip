// Pool writes and reads that move bits only: append (token -> slot),
// copy-on-write block copy, and the gather of one sequence's blocks.
//
// Pool layout: K [num_blocks][Hkv][B][D], V [num_blocks][Hkv][D][B] with
// the tokens of a V channel row in the order v_pos (bits 2 and 3 of the
// in-block offset exchanged: 0-3, 8-11, 4-7, 12-15).  Every thread moves one
// 16-byte piece of a key or value row; all offsets are 64-bit.
#include "common.h"

namespace pkv {
namespace {

constexpr int kThreads = 256;

// One thread per 16-byte piece of one (token, head) row of k_new/v_new.
// The key piece is stored as it is (rows are contiguous in the K pool); the
// value piece is split into its 16/E elements, each going to its channel's
// row of the transposed V block.
template <int E>
__global__ __launch_bounds__(kThreads) void append_kernel(
    const uint8_t* __restrict__ k_new, const uint8_t* __restrict__ v_new,
    const int32_t* __restrict__ slots, int64_t pieces, int32_t pieces_per_row, int32_t hkv,
    int32_t d, int32_t bs, int32_t num_blocks, uint8_t* __restrict__ k_pool,
    uint8_t* __restrict__ v_pool) {
  constexpr int kPer = 16 / E;  // elements per piece
  const int64_t row_bytes = (int64_t)d * E;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < pieces;
       i += (int64_t)gridDim.x * kThreads) {
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
    uint8_t* vrow = v_pool + head_base + ((int64_t)c0 * bs + v_pos(off)) * E;
    if constexpr (E == 2) {
      const uint32_t w[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
      for (int e = 0; e < kPer; ++e) {
        const uint16_t x = (uint16_t)(w[e >> 1] >> ((e & 1) * 16));
        *reinterpret_cast<uint16_t*>(vrow + (int64_t)e * bs * E) = x;
      }
    } else {
      const uint32_t w[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
      for (int e = 0; e < kPer; ++e) *reinterpret_cast<uint32_t*>(vrow + (int64_t)e * bs * E) = w[e];
    }
  }
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
    const uint8_t* vrow = v_pool + head_base + ((int64_t)piece * kPer * bs + v_pos(off)) * E;
    uint32_t w[4];
    if constexpr (E == 2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t lo = *reinterpret_cast<const uint16_t*>(vrow + (int64_t)(2 * e) * bs * E);
        const uint32_t hi = *reinterpret_cast<const uint16_t*>(vrow + (int64_t)(2 * e + 1) * bs * E);
        w[e] = lo | (hi << 16);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = *reinterpret_cast<const uint32_t*>(vrow + (int64_t)e * bs * E);
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

}  // namespace pkv
