// Paged decode attention for gfx950: one query token per sequence against
// its whole paged context, split along the sequence into partitions that run
// as separate workgroups, then merged with the log-sum-exp rule.
//
// Pass 1 (one workgroup per sequence x KV head x partition)
//   bf16: four waves; each wave takes every fourth block of the partition.
//     Per 16-token block the wave issues two matrix-core products:
//       S^T[16 tok x 16 heads] = K[16 tok x D] . Q^T[D x 16 heads]
//            (v_mfma_f32_16x16x32_bf16, D/32 of them)
//       O^T[D x 16 heads]     += V^T[D x 16 tok] . P^T[16 tok x 16 heads]
//            (v_mfma_f32_16x16x16_bf16, D/16 of them)
//     The query heads that share the KV head (the GQA group, g <= 16) fill
//     the 16 columns, so one read of a K/V block serves the whole group.
//     The score tile comes out of the first product in exactly the register
//     layout the second product wants for P^T (lane = head column, four
//     consecutive tokens per lane), and V is stored transposed in the pool
//     (channel-major inside a block), so the V^T operand is a plain
//     coalesced 8-byte load per lane: no LDS staging, no shuffles.
//     Online softmax (running max / sum per head) lives in registers; the
//     per-block max needs two cross-lane steps.  Block-table entries of the
//     partition are fetched up front, one per lane, and the next block's K/V
//     loads are issued before the current block is computed.
//   fp32: a plain vector-ALU kernel (one wave per workgroup) with the same
//     partition structure and exact expf; it exists for fp32 inputs.
// Pass 2 (one workgroup per sequence x query head, only when a sequence has
//   more than one partition): out = sum_p o_p l_p e^(m_p-M) / sum_p l_p e^(m_p-M).
#include <math.h>

#include "common.h"

namespace pkv {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kBs = 16;  // tokens per block

__device__ __forceinline__ float wave_xor(float x, int mask) {
  return __shfl_xor(x, mask, kWave);
}

__device__ __forceinline__ int clamp_block(int b, int num_blocks) {
  return (b >= 0 && b < num_blocks) ? b : 0;
}

// Context length as the kernels use it: cut to what the table and the
// partition grid can describe (both are preconditions; the cut keeps every
// access in range if a caller breaks them).
__device__ __forceinline__ int usable_len(const DecodeArgs& a, int s) {
  int L = a.context_lens[s];
  L = L < 0 ? 0 : L;
  const int cap_tab = a.max_blocks_per_seq * kBs;
  const int cap_part = a.max_partitions * a.partition_blocks * kBs;
  L = L < cap_tab ? L : cap_tab;
  return L < cap_part ? L : cap_part;
}

// ---------------------------------------------------------------- bf16 pass 1
// Workgroup = NW waves on one (sequence, KV head, partition); wave w takes
// blocks w, w+NW, w+2NW, ... of the partition.  Each wave keeps DEPTH blocks
// of K/V loads in flight in a ring of DEPTH+1 register buffers (indices fixed
// by unrolling) while it computes on the oldest; the loads are non-temporal
// (every K/V byte is read once per call).  No load is conditional: the trip
// count is padded to a multiple of the ring size, padded slots re-read the
// wave's last block and are computed fully masked.  Scheduling barriers keep
// the compiler from hoisting a later block's products (and hence its load
// wait) above the current block.
template <int D, int NW, int DEPTH>
__global__ __launch_bounds__(NW * kWave) void decode_bf16_kernel(DecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) float smem[];
  constexpr int KQ = D / 32;  // QK products per block
  constexpr int KV = D / 16;  // PV products per block
  constexpr int NBUF = DEPTH + 1;
  const int hkv = a.num_kv_heads;
  const int hq = a.num_q_heads;
  const int g = hq / hkv;
  const int s = blockIdx.x / hkv;
  const int h = blockIdx.x - s * hkv;
  const int part = blockIdx.y;
  const int L = usable_len(a, s);
  const int ptok = a.partition_blocks * kBs;
  const int n_part = (L + ptok - 1) / ptok;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int col = lane & 15;  // head column (B/C operands) or token/channel row (A operand)
  const int grp = lane >> 4;  // k-group of the lane
  uint16_t* out = (uint16_t*)a.out;

  if (L == 0) {  // empty context: a zero row (written by the first partition only)
    if (part == 0)
      for (int i = threadIdx.x; i < g * D; i += NW * kWave)
        out[((int64_t)s * hq + h * g) * D + i] = 0;
    return;
  }
  if (part >= n_part) return;

  const int nblk = (L + kBs - 1) / kBs;
  const int b0 = part * a.partition_blocks;
  const int b1 = min(b0 + a.partition_blocks, nblk);
  const int my_cnt = (b1 - b0 - wave + NW - 1) / NW;  // blocks this wave handles (may be <= 0)

  // Block-table entries for this wave's blocks, one per lane.
  const int32_t* trow = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
  int my_entry = 0;
  if (lane < my_cnt) my_entry = clamp_block(trow[b0 + wave + lane * NW], a.num_blocks);

  // Q^T operand: lane (head column col, group grp) holds 8 channels per product.
  const uint16_t* qp = (const uint16_t*)a.q;
  bf16x8 qf[KQ];
  {
    const bool live = col < g;
    const uint16_t* qrow = qp + ((int64_t)s * hq + h * g + (live ? col : 0)) * D;
#pragma unroll
    for (int kk = 0; kk < KQ; ++kk) {
      bf16x8 v = *reinterpret_cast<const bf16x8*>(qrow + kk * 32 + grp * 8);
      qf[kk] = live ? v : bf16x8{};
    }
  }

  const uint16_t* kpool = (const uint16_t*)a.k_pool;
  const uint16_t* vpool = (const uint16_t*)a.v_pool;
  const int64_t head_elems = (int64_t)kBs * D;  // one (block, head) slab
  const float sl2 = a.scale * kLog2e;

  float m_run = -INFINITY;
  float l_run = 0.f;
  f32x4 o[KV];
#pragma unroll
  for (int m = 0; m < KV; ++m) o[m] = f32x4{0.f, 0.f, 0.f, 0.f};

  bf16x8 kb[NBUF][KQ];
  u32x2 vb[NBUF][KV];
  auto load = [&](int i, bf16x8* kd, u32x2* vd) {
    const int phys = __builtin_amdgcn_readlane(my_entry, i);
    const int64_t base = ((int64_t)phys * hkv + h) * head_elems;
    const uint16_t* kr = kpool + base + col * D + grp * 8;    // token row = col
    // channel row = col; tokens 4grp..4grp+3 sit at v_pos(4grp)
    const uint16_t* vr = vpool + base + col * kBs + v_pos(grp * 4);
#pragma unroll
    for (int kk = 0; kk < KQ; ++kk)
      kd[kk] = __builtin_bit_cast(
          bf16x8, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kr + kk * 32)));
#pragma unroll
    for (int m = 0; m < KV; ++m)
      vd[m] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(vr + m * 16 * kBs));
  };
  auto compute = [&](int i, const bf16x8* kd, const u32x2* vd) {
    // tokens of this block inside the context; 0 for a padded slot
    const int nvalid = i < my_cnt ? L - (b0 + wave + i * NW) * kBs : 0;
    f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KQ; ++kk)
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kd[kk], qf[kk], sc, 0, 0, 0);
    float z[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) z[r] = (grp * 4 + r < nvalid) ? sc[r] * sl2 : -INFINITY;
    float mb = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
    mb = fmaxf(mb, wave_xor(mb, 16));
    mb = fmaxf(mb, wave_xor(mb, 32));
    // a padded slot leaves every value as it is (its mb is -inf)
    const float m_new = fmaxf(m_run, mb);
    const float alpha = exp2f(m_run - m_new);
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = exp2f(z[r] - m_new);
    l_run = l_run * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
    m_run = m_new;
#pragma unroll
    for (int m = 0; m < KV; ++m) o[m] *= alpha;
    // Tail tokens of a partly filled block hold arbitrary bits (possibly
    // NaN); p is 0 there but 0 * NaN is not, so clear those value words.
    const int t0 = grp * 4;
    const uint32_t mx = (t0 + 0 < nvalid ? 0x0000ffffu : 0u) | (t0 + 1 < nvalid ? 0xffff0000u : 0u);
    const uint32_t my = (t0 + 2 < nvalid ? 0x0000ffffu : 0u) | (t0 + 3 < nvalid ? 0xffff0000u : 0u);
    const bf16x4 pf = bf16x4{(__bf16)p[0], (__bf16)p[1], (__bf16)p[2], (__bf16)p[3]};
#pragma unroll
    for (int m = 0; m < KV; ++m) {
      const u32x2 vm = u32x2{vd[m].x & mx, vd[m].y & my};
      o[m] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, vm), pf, o[m],
                                                       0, 0, 0);
    }
  };

  if (my_cnt > 0) {
    const int cnt_pad = (my_cnt + NBUF - 1) / NBUF * NBUF;
#pragma unroll
    for (int j = 0; j < DEPTH; ++j) {
      load(min(j, my_cnt - 1), kb[j], vb[j]);
      __builtin_amdgcn_sched_barrier(0);  // buffers complete in ring order
    }
    for (int i = 0; i < cnt_pad; i += NBUF) {
#pragma unroll
      for (int j = 0; j < NBUF; ++j) {
        const int bi = i + j;
        load(min(bi + DEPTH, my_cnt - 1), kb[(j + DEPTH) % NBUF], vb[(j + DEPTH) % NBUF]);
        compute(bi, kb[j], vb[j]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // Combine the four k-groups' partial sums of the same head column.
  l_run += wave_xor(l_run, 16);
  l_run += wave_xor(l_run, 32);

  // Merge the waves of the workgroup through LDS.
  float* sm_o = smem;                  // [NW][g][D]
  float* sm_m = smem + NW * g * D;     // [NW][16]
  float* sm_l = sm_m + NW * 16;        // [NW][16]
  if (col < g) {
#pragma unroll
    for (int m = 0; m < KV; ++m)
      *reinterpret_cast<f32x4*>(&sm_o[(wave * g + col) * D + m * 16 + grp * 4]) = o[m];
    if (grp == 0) {
      sm_m[wave * 16 + col] = m_run;
      sm_l[wave * 16 + col] = l_run;
    }
  }
  __syncthreads();

  const int P = a.max_partitions;
  for (int idx = threadIdx.x; idx < g * D; idx += NW * kWave) {
    const int c = idx / D;
    const int dd = idx - c * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_m[w * 16 + c]);
    float lsum = 0.f, acc = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = exp2f(sm_m[w * 16 + c] - M);  // 0 for a wave that saw no block
      lsum += sm_l[w * 16 + c] * f;
      acc += sm_o[(w * g + c) * D + dd] * f;
    }
    const float res = acc / lsum;
    const int64_t row = (int64_t)s * hq + h * g + c;
    if (n_part == 1) {
      out[row * D + dd] = f32_to_bf16(res);
    } else {
      a.part_o[(row * P + part) * D + dd] = res;
      if (dd == 0) {
        a.part_m[row * P + part] = M * kLn2;  // back to natural-log units
        a.part_l[row * P + part] = lsum;
      }
    }
  }
}

// ---------------------------------------------------------------- fp32 pass 1
template <int D>
__global__ __launch_bounds__(kWave) void decode_f32_kernel(DecodeArgs a) {
  constexpr int DPL = D / kWave;  // channels per lane
  __shared__ float q_s[16][D];
  __shared__ float sc_s[16][kBs];
  const int hkv = a.num_kv_heads;
  const int hq = a.num_q_heads;
  const int g = hq / hkv;
  const int s = blockIdx.x / hkv;
  const int h = blockIdx.x - s * hkv;
  const int part = blockIdx.y;
  const int L = usable_len(a, s);
  const int ptok = a.partition_blocks * kBs;
  const int n_part = (L + ptok - 1) / ptok;
  const int lane = threadIdx.x;
  float* out = (float*)a.out;

  if (L == 0) {
    if (part == 0)
      for (int i = lane; i < g * D; i += kWave) out[((int64_t)s * hq + h * g) * D + i] = 0.f;
    return;
  }
  if (part >= n_part) return;

  const float* qp = (const float*)a.q + ((int64_t)s * hq + h * g) * D;
  for (int i = lane; i < g * D; i += kWave) q_s[i / D][i % D] = qp[i];
  __syncthreads();

  const int nblk = (L + kBs - 1) / kBs;
  const int b0 = part * a.partition_blocks;
  const int b1 = min(b0 + a.partition_blocks, nblk);
  const int32_t* trow = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
  const float* kpool = (const float*)a.k_pool;
  const float* vpool = (const float*)a.v_pool;

  float m_run[16], l_run[16], o[16][DPL];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    m_run[j] = -INFINITY;
    l_run[j] = 0.f;
#pragma unroll
    for (int i = 0; i < DPL; ++i) o[j][i] = 0.f;
  }

  for (int b = b0; b < b1; ++b) {
    const int phys = clamp_block(trow[b], a.num_blocks);
    const int64_t base = ((int64_t)phys * hkv + h) * kBs * D;
    const float* kb = kpool + base;
    const float* vb = vpool + base;
    const int nvalid = min(kBs, L - b * kBs);
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
      float psum = 0.f;
      float acc[DPL];
#pragma unroll
      for (int i = 0; i < DPL; ++i) acc[i] = 0.f;
      for (int t = 0; t < nvalid; ++t) {
        const float pt = expf(sc_s[j][t] - m_new);
        psum += pt;
#pragma unroll
        for (int i = 0; i < DPL; ++i) acc[i] = fmaf(pt, vb[(lane + i * kWave) * kBs + v_pos(t)], acc[i]);
      }
      l_run[j] = l_run[j] * alpha + psum;
      m_run[j] = m_new;
#pragma unroll
      for (int i = 0; i < DPL; ++i) o[j][i] = o[j][i] * alpha + acc[i];
    }
    __syncthreads();
  }

  const int P = a.max_partitions;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (j >= g) continue;
    const int64_t row = (int64_t)s * hq + h * g + j;
#pragma unroll
    for (int i = 0; i < DPL; ++i) {
      const int d = lane + i * kWave;
      const float res = o[j][i] / l_run[j];
      if (n_part == 1) out[row * D + d] = res;
      else a.part_o[(row * P + part) * D + d] = res;
    }
    if (n_part > 1 && lane == 0) {
      a.part_m[row * P + part] = m_run[j];
      a.part_l[row * P + part] = l_run[j];
    }
  }
}

// ------------------------------------------------------------------ pass 2
// One wave per (sequence, query head).  Lanes read the partitions' (m, l) in
// strides of 64, the wave reduces M and the weights w_p = l_p e^(m_p - M);
// each lane then accumulates its D/64 channels over the partitions, the
// weights broadcast lane by lane.
template <int D, bool BF16>
__global__ __launch_bounds__(kWave) void decode_merge_kernel(DecodeArgs a) {
  constexpr int CPL = D / kWave;  // channels per lane (adjacent)
  const int j = blockIdx.x;       // query head
  const int s = blockIdx.y;
  const int hq = a.num_q_heads;
  const int L = usable_len(a, s);
  const int ptok = a.partition_blocks * kBs;
  const int n_part = (L + ptok - 1) / ptok;
  if (n_part <= 1) return;        // pass 1 wrote this row directly
  const int P = a.max_partitions;
  const int64_t row = (int64_t)s * hq + j;
  const float* m = a.part_m + row * P;
  const float* l = a.part_l + row * P;
  const float* o = a.part_o + row * P * D + threadIdx.x * CPL;
  const int lane = threadIdx.x;

  float M = -INFINITY;
  for (int p = lane; p < n_part; p += kWave) M = fmaxf(M, m[p]);
  for (int k = kWave / 2; k > 0; k >>= 1) M = fmaxf(M, wave_xor(M, k));

  float W = 0.f;
  float acc[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
  for (int p0 = 0; p0 < n_part; p0 += kWave) {
    const int p = p0 + lane;
    const float w = p < n_part ? l[p] * expf(m[p] - M) : 0.f;
    W += w;
    const int cnt = min(kWave, n_part - p0);
    for (int k = 0; k < cnt; ++k) {
      const float wk = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), k));
      const float* op = o + (int64_t)(p0 + k) * D;
      if constexpr (CPL == 2) {
        const float2 v = *reinterpret_cast<const float2*>(op);
        acc[0] = fmaf(wk, v.x, acc[0]);
        acc[1] = fmaf(wk, v.y, acc[1]);
      } else {
        acc[0] = fmaf(wk, op[0], acc[0]);
      }
    }
  }
  for (int k = kWave / 2; k > 0; k >>= 1) W += wave_xor(W, k);
  const float inv = 1.f / W;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int d = lane * CPL + c;
    if (BF16) ((uint16_t*)a.out)[row * D + d] = f32_to_bf16(acc[c] * inv);
    else ((float*)a.out)[row * D + d] = acc[c] * inv;
  }
}

int status_of(hipError_t e) { return e == hipSuccess ? 0 : -4; }

template <int D>
int launch_d(const DecodeArgs& a, int32_t dtype, hipStream_t st) {
  const dim3 grid(a.num_seqs * a.num_kv_heads, a.max_partitions);
  const int g = a.num_q_heads / a.num_kv_heads;
  if (dtype == 1) {
    // 8 waves per workgroup, no register prefetch (4 waves per SIMD resident):
    // the fastest of the depth / width combinations measured on MI355X.
    constexpr int NW = 8;
    const size_t lds = (size_t)(NW * g * D + 2 * NW * 16) * sizeof(float);
    decode_bf16_kernel<D, NW, 0><<<grid, NW * kWave, lds, st>>>(a);
  } else {
    decode_f32_kernel<D><<<grid, kWave, 0, st>>>(a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return -4;
  if (a.max_partitions > 1) {
    const dim3 mgrid(a.num_q_heads, a.num_seqs);
    if (dtype == 1) decode_merge_kernel<D, true><<<mgrid, kWave, 0, st>>>(a);
    else decode_merge_kernel<D, false><<<mgrid, kWave, 0, st>>>(a);
    e = hipGetLastError();
  }
  return status_of(e);
}

}  // namespace

int launch_decode(const DecodeArgs& a, int32_t dtype, hipStream_t st) {
  if (a.num_seqs == 0) return 0;
  if (a.head_dim == 128) return launch_d<128>(a, dtype, st);
  return launch_d<64>(a, dtype, st);
}

}  // namespace pkv
