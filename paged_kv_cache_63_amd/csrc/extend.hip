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
constexpr int kTabLdsMax = 12288;  // block-table entries that fit in LDS beside the K/V ring

__device__ __forceinline__ float wave_xor(float x, int mask) { return __shfl_xor(x, mask, kWave); }

// s_waitcnt with only the vector-memory counter constrained (expcnt and
// lgkmcnt left at their maxima), gfx9 encoding.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// TAB_LDS: the request's whole block table sits in LDS (tab_cap entries,
// dynamic shared memory), so the loop issues no global loads other than
// the direct-to-LDS tile copies and every wait on the vector-memory counter
// is exact.  Otherwise table entries are read from global memory per tile
// (for contexts too long for the LDS table; the waits then cover them).
//
// Matrix-core layout (v_mfma_f32_32x32x16_bf16, A 32x16, B 16x32, C 32x32;
// lane l: A/B row-or-column l%32, k slots 8*(l/32)..+7; C column l%32, rows
// 8*(v/4) + 4*(l/32) + v%4 for its 16 values v):
//   S^T[32 keys x 32 rows] = K[32 keys x D] . Q^T[D x 32 rows]  (D/16 steps)
//   O^T[32 ch x 32 rows]  += V^T[32 ch x 16 keys] . P^T[16 keys x 32 rows]
// A lane's 16 score values for a 32-key chunk are keys 8b + 4G + e
// (b = v/4, e = v%4, G = l/32); values 0..7 cover the chunk's first 16-key
// block and 8..15 the second, in exactly the slot order P^T needs when V^T
// slot (hb, e) holds key 8*hb + 4G + e, i.e. two 8-byte reads of a
// channel's 32-byte row.  No shuffles between the two products.
template <int D, int NW, bool TAB_LDS>
__global__ __launch_bounds__(NW * kWave) void extend_bf16_kernel(ExtendArgs a, int tiles_per_unit,
                                                                 int units, int tab_cap) {
  constexpr int RPW = 32;                 // query rows per wave
  constexpr int ROWS = NW * RPW;
  constexpr int NBT = 4;                  // blocks per key tile
  constexpr int KT = NBT * kBs;           // keys per tile
  constexpr int KS = D / 16;              // QK k-steps per 32-key chunk
  constexpr int DT = D / 32;              // 32-channel tiles of O
  constexpr int ROWB = D * 2;             // bytes of one key row
  constexpr int CPR = D / 8;              // 16-byte chunks per key row
  constexpr int BLKB = kBs * ROWB;        // bytes of one (block, head) slab
  constexpr int TILEB = NBT * BLKB;       // bytes of a K (or V) tile
  constexpr int CHUNKS = 2 * TILEB / 16;  // K + V chunks per tile
  constexpr int PER_T = CHUNKS / (NW * kWave);  // direct-to-LDS loads per thread per tile
  constexpr int NST = 3;                  // LDS ring stages (loads run two tiles ahead)
  static_assert(PER_T * NW * kWave == CHUNKS, "tile must split evenly over the threads");
  // Rescale the accumulators only when a row's maximum has grown by more
  // than this many powers of two since the reference used for its
  // exponentials (the exponentials stay below 2^kLazy in between).
  constexpr float kLazy = 8.0f;

  __shared__ __attribute__((aligned(16))) uint8_t kv_s[NST][2 * TILEB];  // [stage][K tile | V tile]
  extern __shared__ int32_t tab_s[];      // [tab_cap] when TAB_LDS

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
  if (TAB_LDS && L > tab_cap * kBs) L = tab_cap * kBs;
  const int P = L - n;
  if (P < 0) return;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int c32 = lane & 31;    // A/B row-or-column, C column
  const int G = lane >> 5;      // k-slot group / C row group
  const int nblk = (L + kBs - 1) / kBs;
  const int32_t* trow = a.block_tables + (int64_t)r * a.max_blocks_per_seq;

  // Rows of this workgroup and their last visible key.
  const int last_row = min(row0 + ROWS, n * g) - 1;
  const int kend = P + last_row / g + 1;                   // keys 0..kend-1 are needed
  const int ntiles = (kend + KT - 1) / KT;
  const int wrow0 = row0 + wave * RPW;
  const int wq_min = P + min(wrow0, last_row) / g;         // smallest query position of the wave
  const int wq_max = P + min(wrow0 + RPW - 1, last_row) / g;

  // Q^T operand: lane (row c32, group G) holds channels ks*16 + G*8 .. +7.
  const uint16_t* qp = (const uint16_t*)a.q;
  bf16x8 qf[KS];
  int qpos;
  {
    const int rr = wrow0 + c32;
    const bool live = rr <= last_row;
    const int t = live ? rr / g : 0;
    const int j = live ? rr - (rr / g) * g : 0;
    qpos = P + (live ? t : last_row / g);
    const uint16_t* qrow = qp + ((int64_t)(q0 + t) * hq + h * g + j) * D + G * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(qrow + ks * 16);
      qf[ks] = live ? v : bf16x8{};
    }
  }
  if (TAB_LDS)
    for (int i = tid; i < nblk; i += NW * kWave) {
      const int b = trow[i];
      tab_s[i] = (b >= 0 && b < a.num_blocks) ? b : 0;
    }
  __syncthreads();  // table in LDS, Q loaded (no vector loads outstanding)

  const uint8_t* kpool = (const uint8_t*)a.k_pool;
  const uint8_t* vpool = (const uint8_t*)a.v_pool;
  auto entry = [&](int b) -> int {
    if (TAB_LDS) return tab_s[b];
    const int e = trow[b];
    return (e >= 0 && e < a.num_blocks) ? e : 0;
  };

  // Copy tile tk into stage st with direct-to-LDS loads.  Load i of wave w
  // fills LDS chunks (i*NW + w)*64 + lane; the global chunk each lane reads
  // is chosen so that K rows land XOR-swizzled (chunk c of row r at c ^ r)
  // and each V channel row's two 16-byte halves are swapped on rows 4..7
  // mod 8 (so 8 consecutive lanes reading half G of 8 rows hit distinct
  // banks).  Which pool, which block of the tile and the byte offset inside
  // the (block, head) slab do not change from tile to tile: computed once.
  // Blocks past the end of the sequence read block 0 of the pool (masked
  // out when used).
  int64_t src_off[PER_T];   // byte offset inside the (K or V) pool, block 0
  int src_blk[PER_T];
  bool src_v[PER_T];
#pragma unroll
  for (int i = 0; i < PER_T; ++i) {
    const int c = (i * NW + wave) * kWave + lane;
    const int which = c / (TILEB / 16);
    const int cc = c - which * (TILEB / 16);
    const int blk = cc / (BLKB / 16);
    const int within = cc - blk * (BLKB / 16);
    int src_chunk;
    if (which == 0) {
      const int row = within / CPR;
      const int pos = within - row * CPR;
      src_chunk = row * CPR + (pos ^ (row % CPR));
    } else {
      src_chunk = within ^ ((within >> 3) & 1);
    }
    src_off[i] = (int64_t)h * BLKB + src_chunk * 16;
    src_blk[i] = blk;
    src_v[i] = which != 0;
  }
  const int64_t blk_stride = (int64_t)hkv * BLKB;   // bytes between physical blocks
  auto issue = [&](int tk, int st) {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int c0 = (i * NW + wave) * kWave;  // first LDS chunk of this load
      const int kb = tk * NBT + src_blk[i];
      const int phys = kb < nblk ? entry(kb) : 0;
      const uint8_t* src = (src_v[i] ? vpool : kpool) + src_off[i] + (int64_t)phys * blk_stride;
      __builtin_amdgcn_global_load_lds(
          src,
          (__attribute__((address_space(3))) void*)(&kv_s[st][c0 * 16]), 16, 0, 0);
    }
  };

  const float c2 = a.scale * kLog2e;   // scores -> base-2 exponent units
  float m_ref = -INFINITY, l_run = 0.f;
  f32x16 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[dt][v] = 0.f;
  const bf16x2 ones = bf16x2{(__bf16)1.0f, (__bf16)1.0f};

  // One barrier per tile: after it, tile tk is in LDS and every wave has
  // finished tile tk-1, so stage (tk+2)%3 = (tk-1)%3 may be refilled.
  issue(0, 0);
  if (ntiles > 1) issue(1, 1);

  for (int tk = 0; tk < ntiles; ++tk) {
    const int st = tk % NST;
    if (tk + 1 < ntiles) wait_vm<PER_T>();   // tile tk landed; tk+1 may be in flight
    else wait_vm<0>();
    __builtin_amdgcn_s_barrier();
    if (tk + 2 < ntiles) issue(tk + 2, (tk + 2) % NST);

    const int kbase = tk * KT;
    if (kbase <= wq_max) {  // else the whole tile is in this wave's future
      const uint8_t* ks_ = kv_s[st];
      const uint8_t* vs = kv_s[st] + TILEB;
      // S^T for the two 32-key chunks of the tile
      f32x16 sc[2];
#pragma unroll
      for (int ch = 0; ch < 2; ++ch) {
        const int blk = 2 * ch + (c32 >> 4);
        const int row = c32 & 15;
        const uint8_t* krow = ks_ + blk * BLKB + row * ROWB;
        f32x16 acc;
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[v] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int cix = ks * 2 + G;
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(krow + ((cix ^ (row % CPR)) * 16));
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], acc, 0, 0, 0);
        }
        sc[ch] = acc;
      }

      if (kbase + KT - 1 > wq_min) {   // tile crosses the diagonal of some row
#pragma unroll
        for (int ch = 0; ch < 2; ++ch)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            if (kbase + ch * 32 + (v >> 2) * 8 + G * 4 + (v & 3) > qpos) sc[ch][v] = -INFINITY;
      }
      float mb = -INFINITY;
#pragma unroll
      for (int ch = 0; ch < 2; ++ch)
#pragma unroll
        for (int v = 0; v < 16; v += 2) mb = fmaxf(mb, fmaxf(sc[ch][v], sc[ch][v + 1]));
      mb = fmaxf(mb, wave_xor(mb, 32));
      const float m_new = mb * c2;
      const bool grow = m_new > m_ref + kLazy;
      if (__any(grow)) {   // rare after the first tile
        const float target = grow ? m_new : m_ref;
        const float alpha = __builtin_amdgcn_exp2f(m_ref - target);
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
        m_ref = target;
      }
      const float nm = -m_ref;
      bf16x8 pf[NBT];
#pragma unroll
      for (int b = 0; b < NBT; ++b) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) p[e] = __builtin_amdgcn_exp2f(fmaf(sc[b >> 1][(b & 1) * 8 + e], c2, nm));
        const bf16x8 pb = bf16x8{(__bf16)p[0], (__bf16)p[1], (__bf16)p[2], (__bf16)p[3],
                                 (__bf16)p[4], (__bf16)p[5], (__bf16)p[6], (__bf16)p[7]};
        pf[b] = pb;
        // row sum of the rounded probabilities the PV product uses
        const bf16x2* pp = reinterpret_cast<const bf16x2*>(&pb);
#pragma unroll
        for (int e = 0; e < 4; ++e) l_run = __builtin_amdgcn_fdot2_f32_bf16(pp[e], ones, l_run, false);
      }

      // Keys at or past the end of the sequence (tail of the last block,
      // blocks read as block 0) hold arbitrary bits: p is 0 there but 0 * NaN
      // is not, so their value words are cleared (last tile only).
      // V^T operand of block b, channel tile dt: the lane's 16 bytes are
      // keys 4G..4G+3 and 8+4G..8+4G+3 of channel dt*32 + c32 (positions
      // 8G..8G+7 of the row), i.e. half G of the row, stored at half
      // G ^ ((row >> 2) & 1).
      auto vptr = [&](int b, int dt) {
        const int row = dt * 32 + c32;
        return vs + b * BLKB + row * 32 + ((G ^ ((row >> 2) & 1)) * 16);
      };
      if (kbase + KT > L) {
#pragma unroll
        for (int b = 0; b < NBT; ++b) {
          uint32_t mk[4];
#pragma unroll
          for (int hb = 0; hb < 2; ++hb) {
            const int k0 = kbase + b * kBs + hb * 8 + G * 4;
            mk[2 * hb] = (k0 < L ? 0x0000ffffu : 0u) | (k0 + 1 < L ? 0xffff0000u : 0u);
            mk[2 * hb + 1] = (k0 + 2 < L ? 0x0000ffffu : 0u) | (k0 + 3 < L ? 0xffff0000u : 0u);
          }
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            const u32x4 w = *reinterpret_cast<const u32x4*>(vptr(b, dt));
            const bf16x8 vf = __builtin_bit_cast(
                bf16x8, u32x4{w.x & mk[0], w.y & mk[1], w.z & mk[2], w.w & mk[3]});
            o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[b], o[dt], 0, 0, 0);
          }
        }
      } else {
#pragma unroll
        for (int b = 0; b < NBT; ++b)
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            const bf16x8 vf = *reinterpret_cast<const bf16x8*>(vptr(b, dt));
            o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[b], o[dt], 0, 0, 0);
          }
      }
    }
  }

  // Normalise and store: lane (row c32, group G) holds channels
  // dt*32 + 8*(v/4) + 4*G + v%4 of its row.
  float l = l_run;
  l += wave_xor(l, 32);
  const int rr = wrow0 + c32;
  if (rr > last_row) return;
  const int t = rr / g;
  const int j = rr - t * g;
  const float inv = 1.f / l;
  uint16_t* orow = (uint16_t*)a.out + ((int64_t)(q0 + t) * hq + h * g + j) * D + G * 4;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint32_t w0 = (uint32_t)f32_to_bf16(o[dt][4 * b + 0] * inv) |
                          ((uint32_t)f32_to_bf16(o[dt][4 * b + 1] * inv) << 16);
      const uint32_t w1 = (uint32_t)f32_to_bf16(o[dt][4 * b + 2] * inv) |
                          ((uint32_t)f32_to_bf16(o[dt][4 * b + 3] * inv) << 16);
      *reinterpret_cast<u32x2*>(orow + dt * 32 + b * 8) = u32x2{w0, w1};
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
        for (int e = 0; e < DPL; ++e) acc[e] = fmaf(pt, vb[(lane + e * kWave) * kBs + v_pos(t)], acc[e]);
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
    constexpr int NW = 8;
    constexpr int ROWS = NW * 32;
    const int g = a.num_q_heads / a.num_kv_heads;
    const int tiles = (a.max_q_len * g + ROWS - 1) / ROWS;
    const int units = a.num_reqs * a.num_kv_heads;
    const int unit_groups = (units + kXcds - 1) / kXcds;
    const int64_t grid = (int64_t)kXcds * unit_groups * tiles;
    if (grid == 0) return 0;
    if (grid > 0x7fffffff) return -1;
    // block table of the longest request in LDS when it fits next to the
    // 96 KB K/V ring (up to 12288 blocks = 196608 tokens)
    int tab_cap = (a.max_seq_len + kBs - 1) / kBs;
    if (tab_cap < 1) tab_cap = 1;
    if (tab_cap <= kTabLdsMax) {
      auto kern = extend_bf16_kernel<D, NW, true>;
      const size_t lds = (size_t)tab_cap * sizeof(int32_t);
      static bool attr_set = false;
      if (!attr_set) {
        if (hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                kTabLdsMax * (int)sizeof(int32_t)) != hipSuccess)
          return -4;
        attr_set = true;
      }
      kern<<<(unsigned)grid, NW * kWave, lds, st>>>(a, tiles, units, tab_cap);
    } else {
      extend_bf16_kernel<D, NW, false><<<(unsigned)grid, NW * kWave, 0, st>>>(a, tiles, units,
                                                                                  tab_cap);
    }
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
