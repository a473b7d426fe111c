// Paged extend (chunked prefill over a cached prefix) for gfx950.
//
// Request r has n new tokens at positions P..P+n-1 (P = seq_len - n); token
// i attends to keys 0..P+i.  Their keys/values are already in the pool.
//
// bf16 kernel: one workgroup = 4 waves = one KV head of one request x a tile
// of ROWS query rows, where a row is (new token, query head of the group) and
// rows of consecutive tokens are adjacent (row = token * g + head), so every
// staged K/V tile serves the whole GQA group.  Each wave owns 16*CT rows.
// Keys are consumed 64 at a time (four 16-token blocks): the workgroup copies
// the four K blocks and four V blocks of the next tile from the pool into a
// second LDS buffer while it computes on the current one (global loads are
// issued before the compute, LDS writes after it, one barrier per tile).
// Per 64-key tile and 16 rows a wave issues, on the matrix cores,
//   S^T[key x row]  = K[key x D] . Q^T[D x row]        (16x16x32 bf16)
//   O^T[D x row]   += V^T[D x key] . P^T[key x row]    (16x16x32 bf16)
// The score tile's register layout is the layout P^T needs as an operand
// (row = lane column, four consecutive keys per lane and block), and V is
// stored channel-major in the pool, so neither product needs a transpose.
// Softmax is online (running max / sum per row, base-2 exponentials with
// the scale folded in), fp32.  The causal mask is applied only on the tiles
// that cross a wave's diagonal; tiles wholly in a wave's future are skipped.
// K rows are XOR-swizzled in LDS (16-byte chunk c of row i stored at chunk
// c ^ i) so the 16 rows a fragment load touches hit distinct banks.
//
// Work order: all query tiles of one (request, KV head) read the same keys,
// so they are given workgroup ids that land on the same XCD (ids are dealt
// round-robin over the 8 XCDs) and hence share that XCD's L2; within a unit
// the tiles with the most keys start first.
//
// fp32 kernel: one wave per (new token, KV head) over its causal context,
// exact expf; it serves fp32 inputs.
#include <math.h>

#include "common.h"

namespace pkv {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kBs = 16;
constexpr int kXcds = 8;
constexpr int kTabCache = 1024;  // table entries kept in LDS (16K tokens)

__device__ __forceinline__ float wave_xor(float x, int mask) { return __shfl_xor(x, mask, kWave); }

template <int D, int CT, int NW>
__global__ __launch_bounds__(NW * kWave) void extend_bf16_kernel(ExtendArgs a, int tiles_per_unit,
                                                                 int units) {
  constexpr int ROWS = NW * 16 * CT;
  constexpr int NBT = 4;                  // blocks per key tile
  constexpr int KT = NBT * kBs;           // keys per tile
  constexpr int KQ = D / 32;
  constexpr int KV = D / 16;
  constexpr int ROWB = D * 2;             // bytes of one key row
  constexpr int CPR = D / 8;              // 16-byte chunks per key row
  constexpr int BLKB = kBs * ROWB;        // bytes of one (block, head) slab
  constexpr int TILEB = NBT * BLKB;       // bytes of a K (or V) tile
  constexpr int CHUNKS = 2 * TILEB / 16;  // K + V chunks per tile
  constexpr int PER_T = CHUNKS / (NW * kWave);
  static_assert(PER_T * NW * kWave == CHUNKS, "tile must split evenly over the threads");

  __shared__ __attribute__((aligned(16))) uint8_t kv_s[2][2][TILEB];  // [buf][K,V]
  __shared__ int32_t tab_s[kTabCache];

  const int hkv = a.num_kv_heads;
  const int hq = a.num_q_heads;
  const int g = hq / hkv;
  const int bid = blockIdx.x;
  const int slot = bid / kXcds;
  const int unit = bid % kXcds + kXcds * (slot / tiles_per_unit);
  if (unit >= units) return;
  const int tile = tiles_per_unit - 1 - slot % tiles_per_unit;
  const int r = unit / hkv;
  const int h = unit - r * hkv;
  const int q0 = a.cu_seqlens_q[r];
  const int n = a.cu_seqlens_q[r + 1] - q0;
  int L = a.seq_lens[r];
  const int row0 = tile * ROWS;
  if (n <= 0 || row0 >= n * g || q0 < 0 || q0 + n > a.total_q) return;
  if (L > a.max_blocks_per_seq * kBs) L = a.max_blocks_per_seq * kBs;
  const int P = L - n;
  if (P < 0) return;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int nblk = (L + kBs - 1) / kBs;
  const int32_t* trow = a.block_tables + (int64_t)r * a.max_blocks_per_seq;

  for (int i = tid; i < nblk && i < kTabCache; i += NW * kWave) {
    const int b = trow[i];
    tab_s[i] = (b >= 0 && b < a.num_blocks) ? b : 0;
  }

  // Rows of this workgroup and their last visible key.
  const int last_row = min(row0 + ROWS, n * g) - 1;
  const int kend = P + last_row / g + 1;                   // keys 0..kend-1 are needed
  const int ntiles = (kend + KT - 1) / KT;
  const int wrow0 = row0 + wave * 16 * CT;
  const int wq_min = P + min(wrow0, last_row) / g;         // smallest query position of the wave
  const int wq_max = P + min(wrow0 + 16 * CT - 1, last_row) / g;

  // Q^T operands.
  const uint16_t* qp = (const uint16_t*)a.q;
  bf16x8 qf[CT][KQ];
  int qpos[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int rr = wrow0 + ct * 16 + col;
    const bool live = rr <= last_row;
    const int t = live ? rr / g : 0;
    const int j = live ? rr - (rr / g) * g : 0;
    qpos[ct] = P + (live ? t : last_row / g);
    const uint16_t* qrow = qp + ((int64_t)(q0 + t) * hq + h * g + j) * D + grp * 8;
#pragma unroll
    for (int kk = 0; kk < KQ; ++kk) {
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(qrow + kk * 32);
      qf[ct][kk] = live ? v : bf16x8{};
    }
  }
  __syncthreads();  // table cache ready

  const uint8_t* kpool = (const uint8_t*)a.k_pool;
  const uint8_t* vpool = (const uint8_t*)a.v_pool;
  auto entry = [&](int b) -> int {
    if (b < kTabCache) return tab_s[b];
    const int e = trow[b];
    return (e >= 0 && e < a.num_blocks) ? e : 0;
  };

  u32x4 stg[PER_T];
  auto issue = [&](int tk) {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int c = tid + i * NW * kWave;
      const int which = c / (TILEB / 16);
      const int cc = c - which * (TILEB / 16);
      const int blk = cc / (BLKB / 16);
      const int within = cc - blk * (BLKB / 16);
      const int kb = tk * NBT + blk;
      if (kb < nblk) {
        const int phys = entry(kb);
        const uint8_t* src = (which ? vpool : kpool) + ((int64_t)phys * hkv + h) * BLKB + within * 16;
        stg[i] = *reinterpret_cast<const u32x4*>(src);
      } else {
        stg[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto commit = [&](int tk, int buf) {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int c = tid + i * NW * kWave;
      const int which = c / (TILEB / 16);
      const int cc = c - which * (TILEB / 16);
      const int blk = cc / (BLKB / 16);
      const int within = cc - blk * (BLKB / 16);
      u32x4 v = stg[i];
      int off;
      if (which == 0) {
        const int row = within / CPR;
        const int ch = within - row * CPR;
        off = blk * BLKB + row * ROWB + ((ch ^ (row % CPR)) * 16);
      } else {
        // 16 bytes = 8 consecutive keys of one channel row; clear keys past
        // the end of the sequence (the pool holds arbitrary bits there).
        off = blk * BLKB + within * 16;
        const int k0 = (tk * NBT + blk) * kBs + (within & 1) * 8;
        const int nv = L - k0;
        if (nv < 8) {
          uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t lo = (2 * e < nv) ? 0x0000ffffu : 0u;
            const uint32_t hi = (2 * e + 1 < nv) ? 0xffff0000u : 0u;
            w[e] &= (lo | hi);
          }
          v = u32x4{w[0], w[1], w[2], w[3]};
        }
      }
      *reinterpret_cast<u32x4*>(&kv_s[buf][which][off]) = v;
    }
  };

  const float sl2 = a.scale * kLog2e;
  float m_run[CT], l_run[CT];
  f32x4 o[CT][KV];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    m_run[ct] = -INFINITY;
    l_run[ct] = 0.f;
#pragma unroll
    for (int m = 0; m < KV; ++m) o[ct][m] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  issue(0);
  commit(0, 0);
  __syncthreads();

  for (int tk = 0; tk < ntiles; ++tk) {
    const int buf = tk & 1;
    const bool more = tk + 1 < ntiles;
    if (more) issue(tk + 1);

    const int kbase = tk * KT;
    if (kbase <= wq_max) {  // else the whole tile is in this wave's future
      const uint8_t* ks = kv_s[buf][0];
      const uint8_t* vs = kv_s[buf][1];
      f32x4 sc[CT][NBT];
#pragma unroll
      for (int blk = 0; blk < NBT; ++blk) {
        bf16x8 kf[KQ];
        const int row = col;
#pragma unroll
        for (int kk = 0; kk < KQ; ++kk) {
          const int ch = kk * 4 + grp;
          kf[kk] = *reinterpret_cast<const bf16x8*>(ks + blk * BLKB + row * ROWB +
                                                   ((ch ^ (row % CPR)) * 16));
        }
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < KQ; ++kk)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kk], qf[ct][kk], acc, 0, 0, 0);
          sc[ct][blk] = acc;
        }
      }

      const bool need_mask = kbase + KT - 1 > wq_min;
      bf16x8 pf[CT][NBT / 2];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        float z[NBT][4];
        float mb = -INFINITY;
#pragma unroll
        for (int blk = 0; blk < NBT; ++blk)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int kpos = kbase + blk * kBs + grp * 4 + e;
            float x = sc[ct][blk][e] * sl2;
            if (need_mask && kpos > qpos[ct]) x = -INFINITY;
            z[blk][e] = x;
            mb = fmaxf(mb, x);
          }
        mb = fmaxf(mb, wave_xor(mb, 16));
        mb = fmaxf(mb, wave_xor(mb, 32));
        const float m_new = fmaxf(m_run[ct], mb);
        const float alpha = exp2f(m_run[ct] - m_new);
        float ps = 0.f;
        float p[NBT][4];
#pragma unroll
        for (int blk = 0; blk < NBT; ++blk)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            p[blk][e] = exp2f(z[blk][e] - m_new);
            ps += p[blk][e];
          }
        l_run[ct] = l_run[ct] * alpha + ps;
        m_run[ct] = m_new;
#pragma unroll
        for (int m = 0; m < KV; ++m) o[ct][m] *= alpha;
#pragma unroll
        for (int pr = 0; pr < NBT / 2; ++pr)
          pf[ct][pr] = bf16x8{(__bf16)p[2 * pr][0], (__bf16)p[2 * pr][1], (__bf16)p[2 * pr][2],
                              (__bf16)p[2 * pr][3], (__bf16)p[2 * pr + 1][0],
                              (__bf16)p[2 * pr + 1][1], (__bf16)p[2 * pr + 1][2],
                              (__bf16)p[2 * pr + 1][3]};
      }

#pragma unroll
      for (int pr = 0; pr < NBT / 2; ++pr) {
#pragma unroll
        for (int m = 0; m < KV; ++m) {
          const int drow = m * 16 + col;
          const u32x2 lo = *reinterpret_cast<const u32x2*>(vs + (2 * pr) * BLKB + drow * 32 + grp * 8);
          const u32x2 hi =
              *reinterpret_cast<const u32x2*>(vs + (2 * pr + 1) * BLKB + drow * 32 + grp * 8);
          const bf16x8 vf = __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
#pragma unroll
          for (int ct = 0; ct < CT; ++ct)
            o[ct][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[ct][pr], o[ct][m], 0, 0, 0);
        }
      }
    }

    if (more) {
      commit(tk + 1, buf ^ 1);
    }
    __syncthreads();
  }

  // Normalise and store: lane (row column col, group grp) holds channels
  // m*16 + grp*4 .. +3 of its row.
  uint16_t* out = (uint16_t*)a.out;
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    float l = l_run[ct];
    l += wave_xor(l, 16);
    l += wave_xor(l, 32);
    const int rr = wrow0 + ct * 16 + col;
    if (rr > last_row) continue;
    const int t = rr / g;
    const int j = rr - t * g;
    const float inv = 1.f / l;
    uint16_t* orow = out + ((int64_t)(q0 + t) * hq + h * g + j) * D + grp * 4;
#pragma unroll
    for (int m = 0; m < KV; ++m) {
      const uint32_t w0 = (uint32_t)f32_to_bf16(o[ct][m][0] * inv) |
                          ((uint32_t)f32_to_bf16(o[ct][m][1] * inv) << 16);
      const uint32_t w1 = (uint32_t)f32_to_bf16(o[ct][m][2] * inv) |
                          ((uint32_t)f32_to_bf16(o[ct][m][3] * inv) << 16);
      *reinterpret_cast<u32x2*>(orow + m * 16) = u32x2{w0, w1};
    }
  }
}

// fp32: one wave per (new token, KV head); the g query heads of the group
// are processed together, exactly like a decode step with the context cut at
// the token's own position.
template <int D>
__global__ __launch_bounds__(kWave) void extend_f32_kernel(ExtendArgs a) {
  constexpr int DPL = D / kWave;
  __shared__ float q_s[16][D];
  __shared__ float sc_s[16][kBs];
  const int hkv = a.num_kv_heads;
  const int hq = a.num_q_heads;
  const int g = hq / hkv;
  const int i = blockIdx.x;  // token within the request
  const int h = blockIdx.y;
  const int r = blockIdx.z;
  const int q0 = a.cu_seqlens_q[r];
  const int n = a.cu_seqlens_q[r + 1] - q0;
  if (i >= n || q0 < 0 || q0 + n > a.total_q) return;
  int L = a.seq_lens[r];
  if (L > a.max_blocks_per_seq * kBs) L = a.max_blocks_per_seq * kBs;
  const int P = L - n;
  if (P < 0) return;
  const int ctx = P + i + 1;
  const int lane = threadIdx.x;
  const float* qp = (const float*)a.q + ((int64_t)(q0 + i) * hq + h * g) * D;
  for (int k = lane; k < g * D; k += kWave) q_s[k / D][k % D] = qp[k];
  __syncthreads();

  const int32_t* trow = a.block_tables + (int64_t)r * a.max_blocks_per_seq;
  const float* kpool = (const float*)a.k_pool;
  const float* vpool = (const float*)a.v_pool;
  float m_run[16], l_run[16], o[16][DPL];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    m_run[j] = -INFINITY;
    l_run[j] = 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[j][e] = 0.f;
  }
  const int nb = (ctx + kBs - 1) / kBs;
  for (int b = 0; b < nb; ++b) {
    int phys = trow[b];
    phys = (phys >= 0 && phys < a.num_blocks) ? phys : 0;
    const int64_t base = ((int64_t)phys * hkv + h) * kBs * D;
    const float* kb = kpool + base;
    const float* vb = vpool + base;
    const int nvalid = min(kBs, ctx - b * kBs);
    for (int idx = lane; idx < kBs * g; idx += kWave) {
      const int t = idx & (kBs - 1);
      const int j = idx / kBs;
      float acc = 0.f;
      for (int d = 0; d < D; ++d) acc = fmaf(q_s[j][d], kb[t * D + d], acc);
      sc_s[j][t] = t < nvalid ? acc * a.scale : -INFINITY;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (j >= g) continue;
      float mb = -INFINITY;
      for (int t = 0; t < nvalid; ++t) mb = fmaxf(mb, sc_s[j][t]);
      const float m_new = fmaxf(m_run[j], mb);
      const float alpha = expf(m_run[j] - m_new);
      float psum = 0.f, acc[DPL];
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[e] = 0.f;
      for (int t = 0; t < nvalid; ++t) {
        const float pt = expf(sc_s[j][t] - m_new);
        psum += pt;
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[e] = fmaf(pt, vb[(lane + e * kWave) * kBs + t], acc[e]);
      }
      l_run[j] = l_run[j] * alpha + psum;
      m_run[j] = m_new;
#pragma unroll
      for (int e = 0; e < DPL; ++e) o[j][e] = o[j][e] * alpha + acc[e];
    }
    __syncthreads();
  }
  float* out = (float*)a.out;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (j >= g) continue;
#pragma unroll
    for (int e = 0; e < DPL; ++e)
      out[((int64_t)(q0 + i) * hq + h * g + j) * D + lane + e * kWave] = o[j][e] / l_run[j];
  }
}

template <int D>
int launch_e(const ExtendArgs& a, int32_t dtype, hipStream_t st) {
  if (dtype == 1) {
    constexpr int NW = 4, CT = 2;
    constexpr int ROWS = NW * 16 * CT;
    const int g = a.num_q_heads / a.num_kv_heads;
    const int tiles = (a.max_q_len * g + ROWS - 1) / ROWS;
    const int units = a.num_reqs * a.num_kv_heads;
    const int unit_groups = (units + kXcds - 1) / kXcds;
    const int64_t grid = (int64_t)kXcds * unit_groups * tiles;
    if (grid == 0) return 0;
    if (grid > 0x7fffffff) return -1;
    extend_bf16_kernel<D, CT, NW><<<(unsigned)grid, NW * kWave, 0, st>>>(a, tiles, units);
  } else {
    if (a.max_q_len == 0) return 0;
    extend_f32_kernel<D><<<dim3(a.max_q_len, a.num_kv_heads, a.num_reqs), kWave, 0, st>>>(a);
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace

int launch_extend(const ExtendArgs& a, int32_t dtype, hipStream_t st) {
  if (a.num_reqs == 0 || a.total_q == 0) return 0;
  if (a.head_dim == 128) return launch_e<128>(a, dtype, st);
  return launch_e<64>(a, dtype, st);
}

}  // namespace pkv
