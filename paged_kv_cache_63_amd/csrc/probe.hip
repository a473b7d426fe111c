// HBM read-rate probe: the measured ceiling the attention kernels' bandwidth
// is compared with.  Reads a device buffer in fixed-size chunks, in the
// order a chunk list gives (a random permutation stands for a pool whose
// blocks are scattered, as paging scatters them) or in address order, with
// non-temporal 16-byte loads, and folds the words it read into one word per
// workgroup so that no load can be dropped.  It is measurement support,
// not a step of the method.
#include "../../include/pagedkv.h"
#include "common.h"

namespace pkv {
namespace {

constexpr int kThreads = 256;
constexpr int kInFlight = 4;   // chunks each workgroup has in flight

// Chunk c of the read order is order[c] (or c when order is null); a chunk
// of chunk_bytes bytes is read by the workgroup's threads in 16-byte pieces.
__global__ __launch_bounds__(kThreads) void read_probe_kernel(const uint8_t* buf,
                                                              const int32_t* order,
                                                              int64_t num_chunks,
                                                              int32_t chunk_bytes,
                                                              uint32_t* sink) {
  const int pieces = chunk_bytes / 16;
  u32x4 acc = u32x4{0u, 0u, 0u, 0u};
  const int64_t stride = (int64_t)gridDim.x * kInFlight;
  for (int64_t c0 = (int64_t)blockIdx.x * kInFlight; c0 < num_chunks; c0 += stride) {
    u32x4 v[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) v[u] = u32x4{0u, 0u, 0u, 0u};
    for (int p = threadIdx.x; p < pieces; p += kThreads) {
#pragma unroll
      for (int u = 0; u < kInFlight; ++u) {
        const int64_t c = c0 + u;
        if (c < num_chunks) {
          int64_t chunk = order ? (int64_t)order[c] : c;
          chunk = chunk >= 0 && chunk < num_chunks ? chunk : 0;
          v[u] ^= __builtin_nontemporal_load(
              reinterpret_cast<const u32x4*>(buf + chunk * chunk_bytes) + p);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) acc ^= v[u];
  }
  uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
  for (int k = kWave / 2; k > 0; k >>= 1) x ^= __shfl_xor(x, k, kWave);
  if ((threadIdx.x & (kWave - 1)) == 0) atomicXor(&sink[blockIdx.x], x);
}

}  // namespace
}  // namespace pkv

extern "C" int hbm_read_probe(const void* buf, int64_t num_chunks, int32_t chunk_bytes,
                              const int32_t* chunk_order, uint32_t* sink, int32_t num_workgroups,
                              void* stream) {
  if (!buf || !sink || num_chunks < 0 || num_workgroups <= 0)
    return pkv::set_error(PKV_ERR_INVALID, "hbm_read_probe: null buffer or sink, or bad counts");
  if (chunk_bytes <= 0 || chunk_bytes % 16 || (uintptr_t)buf % 16)
    return pkv::set_error(PKV_ERR_INVALID,
                          "hbm_read_probe: chunk_bytes and the buffer must be 16-byte multiples");
  if (num_chunks == 0) return pkv::clear_error();
  pkv::read_probe_kernel<<<num_workgroups, pkv::kThreads, 0, (hipStream_t)stream>>>(
      (const uint8_t*)buf, chunk_order, num_chunks, chunk_bytes, sink);
  if (hipGetLastError() != hipSuccess)
    return pkv::set_error(PKV_ERR_LAUNCH, "hbm_read_probe: launch failed");
  return pkv::clear_error();
}
