// Paged decode attention for gfx950: one query token per sequence against
// its whole paged context.
//
// bf16: the call's K/V blocks are dealt out in equal contiguous ranges to a
// fixed grid of workgroups; a (sequence, KV head) unit that straddles
// ranges is computed in pieces, each leaving a partial, and a small second
// kernel (the fold) merges every split unit's pieces by the log-sum-exp rule.
// Shared-prefix variant (bf16): each sequence's pass starts after the blocks
// a prefix pass has already covered, every piece leaves a partial, and the
// fold merges each unit's pieces with the prefix partials.
// fp32: a plain vector-ALU pass over fixed partitions (one wave per
// workgroup, exact expf), then a merge pass for contexts with more than one
// partition: out = sum_p o_p l_p e^(m_p-M) / sum_p l_p e^(m_p-M).
#include <math.h>

#include <atomic>
#include <mutex>

#include "common.h"

// Workspace of the allocation-free decode entry: a fixed array on every GPU
// the library runs on, held until the process ends.  Host code never uses
// this name as an address: the per-device address comes from
// hipGetSymbolAddress (decode_scratch below).
static __device__ __align__(256) uint8_t scratch[pkv::kScratchBytes];

namespace pkv {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr size_t kDecodeLdsMax = 160 * 1024 - 256;   // dynamic LDS: a CU's 160 KB less the static part
constexpr int kBs = 16;  // tokens per block
constexpr uint64_t kTagLow = (1ull << 24) - 1;   // bits below a call's tag
// The softmax reference moves only when a block's maximum exceeds it by more
// than this many powers of two (the weights stay below 2^kLazy in between).
constexpr float kLazy = 8.0f;

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
  const int cap_tab = a.max_blocks_per_seq * (kBs << a.bs_shift);
  // the workspace holds max_partitions pieces per unit: at most
  // ceil(nb / partition_blocks) + 1 of them for nb blocks
  const int cap_part = (a.max_partitions - 1) * a.partition_blocks * kBs;
  L = L < cap_tab ? L : cap_tab;
  return L < cap_part ? L : cap_part;
}


// A wave-uniform value the compiler may hold in a vector register, moved to
// a scalar one (inline-assembly "s" operands must be scalar registers).
__device__ __forceinline__ uint32_t uni(uint32_t x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ const uint8_t* uni(const uint8_t* p) {
  const uint64_t v = (uint64_t)p;
  return (const uint8_t*)(((uint64_t)uni((uint32_t)(v >> 32)) << 32) | uni((uint32_t)v));
}

// Direct-to-LDS copies of one 16-token granule of one head into this wave's
// LDS slot: dma_k moves the K rows (16 x D bf16, 32*D bytes at kbase),
// dma_v the V rows (D channel rows of 16 tokens, 32 bytes each at
// vbase + row * vrow_bytes).  Every instruction moves 1 KB: lane l writes
// slot bytes i*1024 + 16*l and reads the global chunk that belongs there
// (koff, voff per lane; the K chunk positions are XOR-swizzled by row, so
// instruction i's lane offset is koff with the row-group bits flipped).
// M0 is saved and restored; each s_nop covers the M0-write hazard.
template <int D>
__device__ __forceinline__ void dma_k(const uint8_t* kbase, uint32_t koff, uint32_t lds_k) {
  constexpr int NI = D / 32;   // 1 KB instructions
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0" : "=s"(saved));
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const uint32_t ko = koff ^ (uint32_t)((i * (1024 / (2 * D))) % (D / 8) * 16);
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2 nt"
        :
        : "s"(uni(lds_k + i * 1024)), "v"(ko), "s"(uni(kbase + i * 1024))
        : "memory");
  }
  asm volatile("s_mov_b32 m0, %0" : : "s"(saved) : "memory");
}
template <int D>
__device__ __forceinline__ void dma_v(const uint8_t* vbase, uint32_t voff, uint32_t lds_v,
                                      uint32_t vrow_bytes) {
  constexpr int NI = D / 32;
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0" : "=s"(saved));
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2 nt"
        :
        : "s"(uni(lds_v + i * 1024)), "v"(voff), "s"(uni(vbase + i * 32 * vrow_bytes))
        : "memory");
  }
  asm volatile("s_mov_b32 m0, %0" : : "s"(saved) : "memory");
}

// Wait until at most N vector-memory operations of this wave are in flight;
// also a compiler barrier, so that LDS reads of the copied data stay after it.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// ---------------------------------------------------------------- bf16 decode
// Balanced split: the work of the call is the list of (sequence, KV head,
// block) triples, sequence-major; unit (s, h) owns nb(s) = ceil(L_s / 16)
// consecutive positions of that list.  The grid has a fixed number W of
// workgroups (the number resident at once: two 8-wave ones per compute
// unit, eight 2-wave ones in the shared-prefix own pass)
// and workgroup w takes positions [w*C, (w+1)*C) with
// C = max(partition_blocks, ceil(total / W)), so every workgroup streams
// the same number of K/V blocks and all of them finish together (a grid of
// fixed-size partitions leaves compute units idle while ragged sequences
// finish).  A unit that falls into one workgroup's range is finished there;
// a unit split over several ranges is computed in pieces, each piece
// writes its (o, m, l) to the workspace, and the fold kernel merges them by
// the log-sum-exp rule once the call's pieces are all written (a merge
// inside this launch, by the piece that arrived last, left every
// workgroup's last piece waiting for its stores, an atomic count and the
// merge's loads at the end of the kernel).
//
// Per piece the NW waves take blocks b, b+NW, ... of the piece; per 16-token
// block a wave issues two matrix-core products:
//   S^T[16 tok x 16 heads] = K[16 tok x D] . Q^T[D x 16 heads]
//        (v_mfma_f32_16x16x32_bf16, D/32 of them)
//   O^T[D x 16 heads]     += V^T[D x 16 tok] . P^T[16 tok x 16 heads]
//        (v_mfma_f32_16x16x16_bf16, D/16 of them)
// The query heads of the GQA group (g <= 16) fill the 16 columns, so one
// read of a K/V block serves the whole group; the score tile comes out in
// the register layout P^T needs, and the channel-major V rows make the V^T
// operand one 8-byte read per lane.  Each wave stages its blocks in an LDS
// slot of its own: direct-to-LDS copies bring block i+1's keys while the wave
// computes on block i's (and its values once block i's have been read), so
// a copy is in flight through most of the wave's compute without holding
// registers.  The copies are non-temporal (each byte is read once per call).
// Block-table entries are fetched one per lane, 64 blocks per wave at a
// time, and broadcast with readlane.

// Sum over the workgroup (all threads get the result); uses red[NW].
template <int NW>
__device__ __forceinline__ int wg_sum(int v, int* red) {
  for (int k = kWave / 2; k > 0; k >>= 1) v += __shfl_xor(v, k, kWave);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = v;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) t += red[i];
  return t;
}

// Inclusive prefix sum over the workgroup's threads; *total gets the sum.
template <int NW>
__device__ __forceinline__ int wg_scan(int v, int* red, int* total) {
  const int lane = threadIdx.x & (kWave - 1);
  for (int k = 1; k < kWave; k <<= 1) {
    const int u = __shfl_up(v, k, kWave);
    if (lane >= k) v += u;
  }
  __syncthreads();
  if (lane == kWave - 1) red[threadIdx.x / kWave] = v;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    if (i < (int)(threadIdx.x / kWave)) before += red[i];
    all += red[i];
  }
  *total = all;
  return v + before;
}

// At most 128 VGPRs (four waves per SIMD): two workgroups per compute unit
// stay resident, the number the grid is sized for.
// SHARED: the shared-prefix variant (seq_prefix and the prefix partials are
// read); a template flag so that the plain decode's code is unaffected.
template <int D, int NW, bool SHARED, int BS>
__global__ __launch_bounds__(NW * kWave, 4) void decode_bf16_kernel(DecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) float smem[];
  __shared__ int red[NW];
  __shared__ int sh_first_g;
  __shared__ int sh_first_s;
  constexpr int KQ = D / 32;  // QK products per block
  constexpr int KV = D / 16;  // PV products per block
  constexpr int NT = NW * kWave;
  const int hkv = a.num_kv_heads;
  const int hq = a.num_q_heads;
  const int g = hq / hkv;
  const int S = a.num_seqs;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int col = lane & 15;  // head column (B/C operands) or token/channel row (A operand)
  const int grp = lane >> 4;  // k-group of the lane
  const int W = gridDim.x;
  const int w = blockIdx.x;
  uint16_t* out = (uint16_t*)a.out;
  // Shared-prefix decode: sequence s's own pass covers its 16-token
  // granules from start_block(s) on (the prefix pass covers those before);
  // the start sits in the sequence's word, which counts only if the prefix
  // pass of this call wrote it.
  auto start_block = [&](int s, int nb) {
    if constexpr (SHARED) {
      const uint64_t v = a.seq_prefix[s];
      const int st = (v & ~kTagLow) == a.tag ? (int)(v & 0xfffff) : 0;
      return min(st, max(nb - 1, 0));
    } else {
      return 0;
    }
  };
  auto nblocks = [&](int s) {
    const int nb = (usable_len(a, s) + kBs - 1) / kBs;
    return nb - start_block(s, nb);
  };

  // Plan, part 1: total work; empty contexts get a zero row (workgroup
  // s mod W writes it).
  // Positions of the (sequence, KV head, block) list fit 32 bits: the host
  // refuses calls whose list could reach 2^31 positions.
  int mine = 0;
  for (int s = tid; s < S; s += NT) {
    const int nb = nblocks(s);
    mine += nb;
    if (nb == 0 && s % W == w)
      for (int i = 0; i < hq * D; ++i) out[(int64_t)s * hq * D + i] = 0;
  }
  const int total = hkv * wg_sum<NW>(mine, red);
  const int C = max(a.partition_blocks, (int)(((uint32_t)total + W - 1) / (uint32_t)W));
  const int lo = w * C;   // below 2^31: w < W and (W - 1) * C < total + W
  if (lo >= total) return;
  const int hi = min(lo + C, total);

  // Plan, part 2: the sequence whose units contain position lo (a prefix
  // sum over the sequences, NT at a time).
  if (tid == 0) sh_first_s = -1;
  int base = 0;
  for (int c0 = 0; c0 < S; c0 += NT) {
    const int s = c0 + tid;
    const int v = s < S ? hkv * nblocks(s) : 0;
    int chunk;
    const int incl = wg_scan<NW>(v, red, &chunk);
    const int st = base + incl - v;
    if (v > 0 && st <= lo && lo < st + v) {
      sh_first_s = s;
      sh_first_g = st;
    }
    __syncthreads();
    if (sh_first_s >= 0) break;
    base += chunk;
  }
  int s = sh_first_s;
  int G = sh_first_g;

  const uint16_t* qp = (const uint16_t*)a.q;
  const uint16_t* kpool = (const uint16_t*)a.k_pool;
  const uint16_t* vpool = (const uint16_t*)a.v_pool;
  // The kernel walks 16-token granules; a table entry covers 1 << sh of
  // them (block_size 16 << sh).  Granule b is part b & (2^sh - 1) of the
  // entry b >> sh: its keys are that part's 16 rows of the (block, head) K
  // slab, its values that part's 16-token half of the V slab ([D][16]):
  // both one contiguous run of 16 x D elements.
  constexpr int sh = BS == 32 ? 1 : 0;
  static_assert(BS == 16 || BS == 32, "block sizes 16 and 32");
  const int64_t head_elems = (int64_t)kBs * D;           // one granule of one head
  const int64_t slab_elems = head_elems << sh;           // one (block, head) slab
  const int vrow = kVRow;                                // V channel row, elements
  const float sl2 = a.scale * kLog2e;
  const int P = a.max_partitions;
  float* sm_o = smem;                  // [NW][g][D]
  float* sm_m = smem + NW * g * D;     // [NW][16] each wave's reference
  float* sm_l = sm_m + NW * 16;        // [NW][16]
  float* sm_x = sm_l + NW * 16;        // [NW][16] each wave's maximum

  // Each wave's LDS slot for one granule: K rows [16][D] (16-byte chunk c
  // of row r at position c ^ (r % (D/8))), then V channel rows [D][16]
  // (the two 16-byte halves of row ch swapped where bit 3 of ch is set), so
  // that the matrix-core operand reads hit distinct banks.  The slots alias
  // the wave-merge area (a barrier separates the uses).
  constexpr int ROWB = 2 * D;
  constexpr int CPR = D / 8;
  constexpr uint32_t SLOT = 64 * D;   // bytes: 32*D of K, 32*D of V
  const char* slot_bytes = reinterpret_cast<const char*>(smem);
  const uint32_t smem_lds = (uint32_t)(size_t)(__attribute__((address_space(3))) float*)smem;
  const uint32_t lds_k = smem_lds + wave * SLOT;
  const uint32_t lds_v = lds_k + 32 * D;
  // Per-lane offsets, recomputed from the lane id where used (an opaque
  // copy of the id keeps the compiler from holding them in registers across
  // the block loop).
  auto opaque_lane = [] {
    uint32_t l = __lane_id();
    asm volatile("" : "+v"(l));
    return (int)l;
  };
  auto rk_off = [&](int l) {   // K fragment 0 of lane l
    const int c = l & 15, gq = l >> 4;
    return (uint32_t)(wave * SLOT + c * ROWB + ((gq ^ (c % CPR)) * 16));
  };
  auto rv_off = [&](int l) {   // V fragment 0 of lane l
    const int c = l & 15, gq = l >> 4;
    return (uint32_t)(wave * SLOT + 32 * D + c * 32 + (((gq & 1) ^ ((c >> 3) & 1)) * 16) + (gq >> 1) * 8);
  };
  auto dma_koff = [&](int l) {   // source of the slot bytes lane l copies in instruction 0
    const int p = 16 * l;
    const int r = p / ROWB, cp = (p % ROWB) / 16;
    return (uint32_t)(r * ROWB + ((cp ^ (r % CPR)) * 16));
  };
  auto dma_voff = [&](int l) {
    return (uint32_t)((l / 2) * (vrow * 2) + (((l & 1) ^ ((l >> 4) & 1)) * 16));
  };

  // One piece: blocks [bb, be) of unit (s, h); piece k of np.
  auto piece = [&](int s, int h, int L, int bb, int be, int k, int np) {
    // Q^T operand: lane (head column col, group grp) holds 8 channels per product.
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
    const int32_t* trow = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
    // Online softmax with a lazily moved reference: p = 2^(z - m_ref), and
    // m_ref moves (rescaling o and l) only when a block's maximum exceeds it
    // by more than kLazy, so p stays below 2^kLazy; m_max is the true
    // running maximum, which the piece's statistics are reported against.
    float m_ref = -INFINITY;
    float m_max = -INFINITY;
    float l_run = 0.f;
    f32x4 o[KV];
#pragma unroll
    for (int m = 0; m < KV; ++m) o[m] = f32x4{0.f, 0.f, 0.f, 0.f};

    // this wave's blocks: bb + wave + i*NW, i < cnt.  Each block's K and V
    // granule is copied straight into the wave's LDS slot while the wave
    // computes on the previous one, then read into registers.
    const int cnt = (be - bb - wave + NW - 1) / NW;
    constexpr int NI = D / 32;   // copy instructions per K (or V) granule
    auto kaddr = [&](int j, int phys) {
      const int b = bb + wave + j * NW;
      return (const uint8_t*)(kpool + ((int64_t)phys * hkv + h) * slab_elems +
                              (b & ((1 << sh) - 1)) * head_elems);
    };
    auto vaddr = [&](int j, int phys) {
      const int b = bb + wave + j * NW;
      return (const uint8_t*)(vpool + ((int64_t)phys * hkv + h) * slab_elems +
                              (b & ((1 << sh) - 1)) * head_elems);
    };
    auto issue_k = [&](int j, int phys) { dma_k<D>(kaddr(j, phys), dma_koff(opaque_lane()), lds_k); };
    auto issue_v = [&](int j, int phys) {
      dma_v<D>(vaddr(j, phys), dma_voff(opaque_lane()), lds_v, (uint32_t)vrow * 2);
    };
    __syncthreads();   // the slots alias the previous piece's merge area
    for (int i0 = 0; i0 < cnt; i0 += kWave) {
      const int n_here = min(kWave, cnt - i0);
      int my_entry = 0;
      if (lane < n_here)
        my_entry = clamp_block(trow[(bb + wave + (i0 + lane) * NW) >> sh], a.num_blocks);
      {
        const int e0 = __builtin_amdgcn_readlane(my_entry, 0);
        issue_k(i0, e0);
        issue_v(i0, e0);
      }
      for (int i = 0; i < n_here; ++i) {
        const int b = bb + wave + (i0 + i) * NW;
        const bool more = i + 1 < n_here;
        const int e_next = __builtin_amdgcn_readlane(my_entry, more ? i + 1 : i);
        // K of this block is in the slot (its V may still be in flight)
        wait_vm<NI>();
        bf16x8 kd[KQ];
        {
          // (the per-product addresses are recomputed here rather than kept
          // live across the loop)
          const uint32_t rk = rk_off(opaque_lane());
#pragma unroll
          for (int kk = 0; kk < KQ; ++kk)
            kd[kk] = *reinterpret_cast<const bf16x8*>(slot_bytes + (rk ^ (uint32_t)(64 * kk)));
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // K slot free
        if (more) issue_k(i0 + i + 1, e_next);
        const int nvalid = L - b * kBs;   // tokens of this block inside the context
        f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KQ; ++kk)
          sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kd[kk], qf[kk], sc, 0, 0, 0);
        float z[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) z[r] = sc[r] * sl2;
        const bool partial = nvalid < kBs;   // the same for the whole wave
        if (partial) {
#pragma unroll
          for (int r = 0; r < 4; ++r) z[r] = (grp * 4 + r < nvalid) ? z[r] : -INFINITY;
        }
        float mb = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
        mb = fmaxf(mb, wave_xor(mb, 16));
        mb = fmaxf(mb, wave_xor(mb, 32));
        m_max = fmaxf(m_max, mb);
        const bool grow = mb > m_ref + kLazy;
        if (__any(grow)) {   // rare after a piece's first block
          const float target = grow ? mb : m_ref;
          const float alpha = exp2f(m_ref - target);   // 0 on the first block
          l_run *= alpha;
#pragma unroll
          for (int m = 0; m < KV; ++m) o[m] *= alpha;
          m_ref = target;
        }
        float p[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) p[r] = exp2f(z[r] - m_ref);
        const bf16x4 pf = bf16x4{(__bf16)p[0], (__bf16)p[1], (__bf16)p[2], (__bf16)p[3]};
        {
          // the sum of exactly the rounded weights the value product uses
          const u32x2 pw = __builtin_bit_cast(u32x2, pf);
          l_run += (bf16_lo(pw.x) + bf16_hi(pw.x)) + (bf16_lo(pw.y) + bf16_hi(pw.y));
        }
        // V of this block is in the slot (the next block's K may be in flight)
        if (more) wait_vm<NI>();
        else wait_vm<0>();
        u32x2 vd[KV];
#pragma unroll
        for (int m = 0; m < KV; ++m)
          vd[m] = *reinterpret_cast<const u32x2*>(slot_bytes + rv_off(opaque_lane()) + m * 512);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // V slot free
        if (more) issue_v(i0 + i + 1, e_next);
        if (partial) {
          // Tail tokens of a partly filled block hold arbitrary bits
          // (possibly NaN); p is 0 there but 0 * NaN is not, so clear those
          // value words.
          const int t0 = grp * 4;
          const uint32_t mx = (t0 + 0 < nvalid ? 0x0000ffffu : 0u) | (t0 + 1 < nvalid ? 0xffff0000u : 0u);
          const uint32_t my = (t0 + 2 < nvalid ? 0x0000ffffu : 0u) | (t0 + 3 < nvalid ? 0xffff0000u : 0u);
#pragma unroll
          for (int m = 0; m < KV; ++m) vd[m] = u32x2{vd[m].x & mx, vd[m].y & my};
        }
#pragma unroll
        for (int m = 0; m < KV; ++m)
          o[m] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, vd[m]), pf,
                                                           o[m], 0, 0, 0);
      }
    }

    // Combine the four k-groups' partial sums of the same head column, then
    // the waves of the workgroup through LDS.
    l_run += wave_xor(l_run, 16);
    l_run += wave_xor(l_run, 32);
    __syncthreads();   // the previous piece's readers are done with the LDS
    if (col < g) {
#pragma unroll
      for (int m = 0; m < KV; ++m)
        *reinterpret_cast<f32x4*>(&sm_o[(wave * g + col) * D + m * 16 + grp * 4]) = o[m];
      if (grp == 0) {
        sm_m[wave * 16 + col] = m_ref;
        sm_l[wave * 16 + col] = l_run;
        sm_x[wave * 16 + col] = m_max;
      }
    }
    __syncthreads();
    // (with 32-token blocks the thread id is taken opaque here, so that the
    // compiler does not keep this loop's addresses live across the piece
    // loop: they would not fit the register budget)
    int tid_m = tid;
    if constexpr (BS == 32) asm volatile("" : "+v"(tid_m));
    for (int idx = tid_m; idx < g * D; idx += NT) {
      const int c = idx / D;
      const int dd = idx - c * D;
      // the piece's maximum; each wave's o and l are relative to its own
      // reference, weighted by 2^(reference - M) (0 for a wave that saw no
      // block)
      float M = -INFINITY;
#pragma unroll
      for (int v = 0; v < NW; ++v) M = fmaxf(M, sm_x[v * 16 + c]);
      float lsum = 0.f, acc = 0.f;
#pragma unroll
      for (int v = 0; v < NW; ++v) {
        const float f = exp2f(sm_m[v * 16 + c] - M);  // 0 for a wave that saw no block
        lsum += sm_l[v * 16 + c] * f;
        acc += sm_o[(v * g + c) * D + dd] * f;
      }
      const int64_t row = (int64_t)s * hq + h * g + c;
      if (!SHARED && np == 1) {
        out[row * D + dd] = f32_to_bf16(acc / lsum);
      } else {
        // a partial for the fold (in the shared-prefix variant every piece
        // is one: the fold adds the prefix pass's partials)
        a.part_o[(row * P + k) * D + dd] = acc / lsum;
        if (dd == 0) {
          a.part_m[row * P + k] = M * kLn2;  // natural-log units
          a.part_l[row * P + k] = lsum;
        }
      }
    }
    // the unit's piece count, for the fold (kernel order makes the pieces
    // visible to it)
    if (k == 0 && (SHARED || np > 1) && tid == 0)
      a.arrive[(int64_t)s * hkv + h] = a.tag | (uint64_t)np;
  };

  // Walk the units that intersect [lo, hi).  Only the first and the last
  // of them can be split (the others lie wholly inside the range).
  while (G < hi && s < S) {
    const int L = usable_len(a, s);
    const int nb_all = (L + kBs - 1) / kBs;
    const int st = start_block(s, nb_all);
    const int nb = nb_all - st;
    for (int h = 0; h < hkv; ++h) {
      const int Gh = G + h * nb;
      const int a0 = max(lo, Gh), a1 = min(hi, Gh + nb);
      if (a0 < a1) {
        // A unit inside the range is one piece; only the range's first and
        // last unit can be split, and only they need the divisions.
        int k = 0, np = 1;
        if (Gh < lo || Gh + nb > hi) {
          const int first = (int)((uint32_t)Gh / (uint32_t)C);
          k = w - first;
          np = (int)((uint32_t)(Gh + nb - 1) / (uint32_t)C) - first + 1;
        }
        piece(s, h, L, st + (int)(a0 - Gh), st + (int)(a1 - Gh), k, np);
      }
    }
    G += hkv * nb;
    ++s;
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

  // 16-token granules; a table entry covers 1 << sh of them (as in the bf16
  // kernel)
  const int sh = a.bs_shift;
  const int vrow = kVRow;
  for (int b = b0; b < b1; ++b) {
    const int phys = clamp_block(trow[b >> sh], a.num_blocks);
    const int part = b & ((1 << sh) - 1);
    const int64_t base = ((int64_t)phys * hkv + h) * (kBs << sh) * D;
    const float* kb = kpool + base + part * kBs * D;   // the granule's keys and values:
    const float* vb = vpool + base + part * kBs * D;   // 16 x D elements each
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
        for (int i = 0; i < DPL; ++i) acc[i] = fmaf(pt, vb[(lane + i * kWave) * vrow + v_pos(t)], acc[i]);
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

// Raises a kernel's dynamic-LDS limit to the CU's 160 KB (needed above 64
// KB) once per device; *done holds one bit per device id below 64 (ids from
// 64 on set it on every call).  Safe to call from several host threads.
int raise_lds_limit(const void* kern, std::atomic<uint64_t>* done) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -4;
  const uint64_t bit = dev >= 0 && dev < 64 ? 1ull << dev : 0;
  if (bit && (done->load(std::memory_order_acquire) & bit)) return 0;
  if (hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kDecodeLdsMax) !=
      hipSuccess)
    return -4;
  done->fetch_or(bit, std::memory_order_release);
  return 0;
}

// Fold, the bf16 decode's last step: for every (sequence, KV head) whose
// context was split, its pieces (and, in the shared-prefix decode, the
// prefix pass's partials) are combined by the log-sum-exp rule,
// out = sum_j o_j l_j e^(m_j - M) / sum_j l_j e^(m_j - M) (natural-log
// statistics).  The unit's piece count and the sequence's prefix-partial
// count come from words tagged by this call's kernels; a word with another
// tag means 0 (a unit the decode kernel finished in one piece or gave its
// zero rows, or a sequence in no group).
template <int D>
__global__ __launch_bounds__(256) void decode_fold_kernel(DecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) float fold_s[];   // [g][n] m, [g][n] weights, [g] 1/sum
  const int hkv = a.num_kv_heads;
  const int hq = a.num_q_heads;
  const int g = hq / hkv;
  const int unit = blockIdx.x;
  const int s = unit / hkv;
  const int h = unit - s * hkv;
  const uint64_t cw = a.arrive[unit];
  const int np = (cw & ~kTagLow) == a.tag ? (int)(cw & kTagLow) : 0;
  if (np <= 0) return;
  const int NS = a.num_splits;
  const int P = a.max_partitions;
  const uint64_t pw = a.seq_prefix ? a.seq_prefix[s] : 0;
  const int nsp = (pw & ~kTagLow) == a.tag ? min((int)((pw >> 20) & 0xf), NS) : 0;
  const int n = np + nsp;
  const int tid = threadIdx.x;
  if (nsp == 0 && np <= 8) {
    // a few pieces: every thread loads its pieces' m, l and o at once and
    // forms the weights itself (one round trip, no LDS)
    uint16_t* out = (uint16_t*)a.out;
    for (int idx = tid; idx < g * D; idx += 256) {
      const int c = idx / D;
      const int dd = idx - c * D;
      const int64_t row = (int64_t)s * hq + h * g + c;
      float mv[8], lv[8], ov[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int jj = min(j, np - 1);
        mv[j] = a.part_m[row * P + jj];
        lv[j] = a.part_l[row * P + jj];
        ov[j] = a.part_o[(row * P + jj) * D + dd];
      }
      float M = -INFINITY;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j < np) M = fmaxf(M, mv[j]);
      float wsum = 0.f, acc = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j < np) {
          const float wt = lv[j] * expf(mv[j] - M);
          wsum += wt;
          acc = fmaf(wt, ov[j], acc);
        }
      out[row * D + dd] = f32_to_bf16(acc / wsum);
    }
    return;
  }
  for (int idx = tid; idx < g * n; idx += 256) {
    const int c = idx / n;
    const int j = idx - c * n;
    const int64_t row = (int64_t)s * hq + h * g + c;
    fold_s[idx] = j < np ? a.part_m[row * P + j] : a.pre_m[row * NS + j - np];
    fold_s[g * n + idx] = j < np ? a.part_l[row * P + j] : a.pre_l[row * NS + j - np];
  }
  __syncthreads();
  // weights l_j e^(m_j - M) per head: one wave per head, lanes over pieces
  const int lane = tid & (kWave - 1);
  for (int c = tid / kWave; c < g; c += 256 / kWave) {
    float M = -INFINITY;
    for (int j = lane; j < n; j += kWave) M = fmaxf(M, fold_s[c * n + j]);
    for (int k = kWave / 2; k > 0; k >>= 1) M = fmaxf(M, __shfl_xor(M, k, kWave));
    float wsum = 0.f;
    for (int j = lane; j < n; j += kWave) {
      const float wt = fold_s[g * n + c * n + j] * expf(fold_s[c * n + j] - M);
      fold_s[g * n + c * n + j] = wt;
      wsum += wt;
    }
    for (int k = kWave / 2; k > 0; k >>= 1) wsum += __shfl_xor(wsum, k, kWave);
    if (lane == 0) fold_s[2 * g * n + c] = 1.f / wsum;
  }
  __syncthreads();
  // Each thread's partial outputs are loaded eight at a time, all in
  // flight together (one latency per eight partials, not one each).
  uint16_t* out = (uint16_t*)a.out;
  for (int idx = tid; idx < g * D; idx += 256) {
    const int c = idx / D;
    const int dd = idx - c * D;
    const int64_t row = (int64_t)s * hq + h * g + c;
    const float* wts = fold_s + g * n + c * n;
    float acc = 0.f;
    for (int j0 = 0; j0 < n; j0 += 8) {
      float ov[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j = min(j0 + u, n - 1);
        ov[u] = j < np ? a.part_o[(row * P + j) * D + dd] : a.pre_o[(row * NS + j - np) * D + dd];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (j0 + u < n) acc = fmaf(wts[j0 + u], ov[u], acc);
    }
    out[row * D + dd] = f32_to_bf16(acc * fold_s[2 * g * n + c]);
  }
}

template <int D>
int launch_d(const DecodeArgs& a, int32_t dtype, hipStream_t st) {
  const int g = a.num_q_heads / a.num_kv_heads;
  if (dtype == 1) {
    // Plain decode: 8-wave workgroups, two per CU.  The shared-prefix own
    // pass walks many short suffixes (tens of blocks): there 2-wave
    // workgroups, eight per CU, so that a piece is spread over fewer waves
    // and each wave streams longer (measured: 188-190 us per call against
    // 200 for 8 waves x 4 per CU, 191 for 4 waves x 4, 194 for 1 wave x 16).
    constexpr int NW = 8, NWS = 2;
    const int nw = a.seq_prefix ? NWS : NW;
    // wave-merge area [nw][g][D] + [nw][16] x 3 (reference, l, maximum),
    // aliased with the per-wave granule slots (K + V of 16 tokens)
    const size_t wave_area = (size_t)nw * g * D + 3 * nw * 16;
    const size_t lds = max(wave_area * sizeof(float), (size_t)nw * 64 * D);
    // the fold's general path stages [2][g][pieces + prefix partials] + [g] weights
    const size_t flds = (size_t)(2 * g * (a.max_partitions + a.num_splits) + g) * sizeof(float);
    if (lds > kDecodeLdsMax || flds > kDecodeLdsMax) return -2;
    auto kern = a.seq_prefix ? (a.bs_shift ? decode_bf16_kernel<D, NWS, true, 32>
                                           : decode_bf16_kernel<D, NWS, true, 16>)
                : a.bs_shift ? decode_bf16_kernel<D, NW, false, 32>
                             : decode_bf16_kernel<D, NW, false, 16>;
    const int variant = (a.seq_prefix ? 2 : 0) + (a.bs_shift ? 1 : 0);
    static std::atomic<uint64_t> attr_set[4];   // per variant, one bit per device
    static std::atomic<uint64_t> fold_attr;
    if (raise_lds_limit((const void*)kern, &attr_set[variant]) ||
        raise_lds_limit((const void*)decode_fold_kernel<D>, &fold_attr))
      return -4;
    const int64_t units = (int64_t)a.num_seqs * a.num_kv_heads;
    // (tagged words, nothing to clear)
    kern<<<a.seq_prefix ? 4 * a.num_workgroups : a.num_workgroups, nw * kWave, lds, st>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return -4;
    decode_fold_kernel<D><<<(unsigned)units, 256, flds, st>>>(a);
    return status_of(hipGetLastError());
  }
  const int n_part = a.max_partitions - 1;   // fixed partitions of the fp32 path
  const dim3 grid(a.num_seqs * a.num_kv_heads, n_part);
  decode_f32_kernel<D><<<grid, kWave, 0, st>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return -4;
  if (n_part > 1) {
    const dim3 mgrid(a.num_q_heads, a.num_seqs);
    decode_merge_kernel<D, false><<<mgrid, kWave, 0, st>>>(a);
    e = hipGetLastError();
  }
  return status_of(e);
}

__global__ __launch_bounds__(256) void zero_words_kernel(uint64_t* w, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    w[i] = 0;
}

}  // namespace

int decode_scratch(hipStream_t st, uint8_t** base) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static uint8_t* addr[kMaxDevices];   // per device, set once
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -2;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return -4;
    // piece-count words start at zero (no call's tag is zero); the partials need
    // no initial value
    constexpr int64_t words = (int64_t)(kScratchArriveBytes / 8);
    zero_words_kernel<<<(unsigned)(words / 256 / 8), 256, 0, st>>>((uint64_t*)p, words);
    if (hipGetLastError() != hipSuccess) return -4;
    addr[dev] = (uint8_t*)p;
  }
  *base = addr[dev];
  return 0;
}

int launch_decode(const DecodeArgs& a, int32_t dtype, hipStream_t st) {
  if (a.num_seqs == 0) return 0;
  if (a.head_dim == 128) return launch_d<128>(a, dtype, st);
  return launch_d<64>(a, dtype, st);
}

}  // namespace pkv
