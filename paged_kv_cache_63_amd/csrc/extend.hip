// Paged extend (chunked prefill over a cached prefix) for gfx950.
//
// Request r has n new tokens at positions P..P+n-1 (P = seq_len - n); token
// i attends to keys 0..P+i.  Their keys/values are already in the pool.
//
// bf16 kernel: one workgroup = 8 waves = one KV head of one request x a tile
// of 256 query rows, where a row is (new token, query head of the group) and
// rows of consecutive tokens are adjacent (row = token * g + head), so every
// staged K/V tile serves the whole GQA group.  Each wave owns 32 rows.
// Keys are consumed 64 at a time (four 16-token blocks), copied from the
// pool by direct-to-LDS loads into a 5-stage LDS ring (160 KB for D = 128),
// three tiles ahead of their first use.  Per 64-key tile a wave issues, on
// the matrix cores (v_mfma_f32_32x32x16_bf16),
//   S^T[key x row]  = K[key x D] . Q^T[D x row]
//   O^T[D x row]   += V^T[D x key] . P^T[key x row]
// The score tile's register layout is the layout P^T needs as an operand,
// and V is stored channel-major in the pool, so neither product needs a
// transpose.  Softmax is online (running max / sum per row, base-2
// exponentials with the scale folded in), fp32.
//
// Ping-pong: waves w and w+4 share a SIMD.  Every wave alternates a matrix
// phase (PV of the previous tile, then QK of the current one: 32 MFMAs fed
// from LDS) and a vector phase (softmax of the current tile, plus the tile
// copies, table lookups and the first LDS reads of the next matrix phase),
// and waves 4..7 run one phase behind waves 0..3.  A workgroup barrier
// follows every second phase (one per tile): between two barriers, waves
// 0..3 run a matrix then a vector phase and waves 4..7 a vector then a
// matrix phase.  So while one wave of a SIMD keeps its matrix core busy,
// the other runs its exponentials on the vector ALU; the matrix
// phase runs at raised issue priority so that the older wave's VALU work
// cannot starve it.  The softmax uses no instruction that executes on the
// matrix pipeline (bf16 dot products would wait for the other wave's
// MFMAs): row sums are taken by the matrix core itself, as small 4x4x4
// products with an all-ones operand.  The probabilities are pinned to the
// vector phase (the compiler would otherwise sink them into the matrix
// phase that consumes them).
//
// LDS layouts (16-byte chunks; reads hit 64 distinct banks per 16 lanes):
// K rows are XOR-swizzled (chunk c of row i at c ^ f(i)); each V channel
// row's two 16-byte halves are swapped where bit 2 xor bit 3 of the channel
// is set.  The direct-to-LDS copy writes LDS contiguously, so each lane reads
// the global chunk that belongs at its LDS position.
//
// Work order: all query tiles of one (request, KV head) read the same keys,
// so they are given workgroup ids that land on the same XCD (ids are dealt
// round-robin over the 8 XCDs) and hence share that XCD's L2; within a unit
// the tiles with the most keys start first.
//
// fp32 kernel: one wave per (new token, KV head) over its causal context,
// exact expf; it serves fp32 inputs.
#include <math.h>

#include <type_traits>

#include "common.h"

namespace pkv {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kBs = 16;
constexpr int kXcds = 8;

// Maximum of x over lanes l and l ^ 32, through the VALU (no LDS).
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// s_waitcnt with only the vector-memory counter constrained (expcnt and
// lgkmcnt left at their maxima), gfx9 encoding.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Workgroup barrier that also keeps the compiler from moving memory
// operations across it (the hardware barrier alone does not wait for
// anything; the LDS data it publishes was waited for explicitly).
__device__ __forceinline__ void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

typedef const __attribute__((address_space(4))) int32_t const_i32;

// Marks a register value as produced here: the computation of x cannot be
// moved past this point (the compiler otherwise sinks pure ALU work across
// workgroup barriers towards its first use).
template <typename T>
__device__ __forceinline__ void materialize(T& x) {
  asm volatile("" : "+v"(x));
}

// Two direct-to-LDS copies, the K and the V slab of one block: every lane
// loads 16 bytes from kbase + koff (then vbase + voff), bases wave-uniform,
// and the wave writes them to LDS at lds_k + lane*16 (then lds_v +
// lane*16).  Issued as inline assembly so that the compiler neither hoists
// 64-bit per-lane addresses out of the loop nor adds waits for these copies
// before unrelated LDS reads; the kernel waits for them itself (vmcnt).  M0
// (the LDS base of a copy) is saved once and restored after both; each
// s_nop covers the M0-write hazard.
__device__ __forceinline__ void lds_dma16_kv(const uint8_t* kbase, uint32_t koff,
                                             const uint8_t* vbase, uint32_t voff, uint32_t lds_k,
                                             uint32_t lds_v) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %5\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %6\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %3, %4\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(koff), "s"(kbase), "v"(voff), "s"(vbase), "s"(lds_k), "s"(lds_v)
      : "memory");
}

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
//
// PREFIX: the prefix pass of the shared-prefix decode.  A unit is (group,
// KV head, key split); its rows are (member, query head of the group), the
// member's single query token taking the place of a new token; its keys are
// the split's range of the prefix blocks (read through the first member's
// table), starting at key tile kt0.  A member sees the prefix keys below
// its own start block (keys past it are masked like causal ones), and a row
// may see no key of a split at all, so the exponent reference of such a row
// is taken as 0 instead of -inf.  Output: the normalised partial (o, m in
// natural-log units, l) per (member, query head, split).
template <int D, bool PREFIX, typename Args, int BS>
__global__ __launch_bounds__(8 * kWave) void extend_bf16_kernel(Args a, int tiles_per_unit,
                                                                int units) {
  constexpr int NW = 8;
  constexpr int HALF = NW / 2;            // waves per group: one per SIMD
  constexpr int RPW = 32;                 // query rows per wave
  constexpr int ROWS = NW * RPW;
  // A key tile is 64 keys: four 16-key sub-blocks (the unit of the
  // products), i.e. NBT table blocks of BS tokens (BS = 16 or 32).
  constexpr int NSB = 4;                  // 16-key sub-blocks per key tile
  constexpr int SPB = BS / kBs;           // sub-blocks per table block
  constexpr int NBT = NSB / SPB;          // table blocks per key tile
  constexpr int KT = NSB * kBs;           // keys per tile
  constexpr int KS = D / 16;              // QK k-steps per 32-key chunk
  constexpr int DT = D / 32;              // 32-channel tiles of O
  constexpr int ROWB = D * 2;             // bytes of one key row
  constexpr int CPR = D / 8;              // 16-byte chunks per key row
  constexpr int SWZ = 16 / CPR;           // consecutive key rows sharing one swizzle value
  constexpr int SUBB = kBs * ROWB;        // bytes of one 16-key sub-block of one head
  constexpr int BLKB = BS * ROWB;         // bytes of one (block, head) slab
  constexpr int VROWB = kVRow * 2;        // bytes of one V channel row (a 16-token half of a slab)
  constexpr int TILEB = NSB * SUBB;       // bytes of a K (or V) tile
  constexpr int SEGS = TILEB / 16 / kWave;  // 64-chunk segments per K (or V) tile
  constexpr int PER_T = 2 * SEGS / NW;    // direct-to-LDS loads per thread per tile
  constexpr int NST = 5;                  // LDS ring stages (160 KB for D = 128)
  static_assert(PER_T * NW == 2 * SEGS, "tile must split evenly over the waves");
  static_assert(BS == 16 || BS == 32, "block sizes 16 and 32");
  // V rows in LDS: the two 16-byte chunks of channel row c are exchanged
  // where vswz(c) is set, so that the 16 lanes of one read phase (channels
  // c..c+15, the same chunk) hit 16 distinct 4-bank groups (32-byte rows
  // repeat the banks every 8 channels).  A slab's 16-token halves lie one
  // after the other, [D][16] each, in the pool and in LDS alike.
  auto vswz = [](int c) -> int { return ((c >> 2) ^ (c >> 3)) & 1; };
  // Rescale the accumulators only when a row's maximum has grown by more
  // than this many powers of two since the reference used for its
  // exponentials (the exponentials stay below 2^kLazy in between).
  constexpr float kLazy = 8.0f;

  __shared__ __attribute__((aligned(16))) uint8_t kv_s[NST][2 * TILEB];  // [stage][K tile | V tile]

  const int hkv = a.num_kv_heads;
  const int hq = a.num_q_heads;
  const int g = hq / hkv;
  const int bid = blockIdx.x;
  const int slot = bid / kXcds;
  const int unit = bid % kXcds + kXcds * (slot / tiles_per_unit);
  if (unit >= units) return;
  const int tile = tiles_per_unit - 1 - slot % tiles_per_unit;
  const int row0 = tile * ROWS;
  int r, h, n, L, P = 0, q0 = 0;
  int kt0 = 0;                        // first key tile of the unit
  int goff = 0, split = 0, pblk = 0;  // prefix pass: group's first member, split, prefix blocks
  if constexpr (!PREFIX) {
    r = unit / hkv;
    h = unit - r * hkv;
    q0 = a.cu_seqlens_q[r];
    n = a.cu_seqlens_q[r + 1] - q0;
    L = a.seq_lens[r];
    if (n <= 0 || row0 >= n * g || q0 < 0 || q0 + n > a.total_q) return;
    if (L > a.max_blocks_per_seq * BS) L = a.max_blocks_per_seq * BS;
    P = L - n;
    if (P < 0) return;
  } else {
    const int per_group = hkv * a.num_splits;
    const int grp = unit / per_group;
    const int rem = unit - grp * per_group;
    h = rem / a.num_splits;
    split = rem - h * a.num_splits;
    goff = a.group_offsets[grp];
    n = a.group_offsets[grp + 1] - goff;   // members
    // (at most what the splits cover: the host sized them for the longest prefix)
    pblk = min(min(max(a.group_prefix_blocks[grp], 0), a.max_blocks_per_seq),
               a.num_splits * a.split_blocks);
    if (goff < 0 || n <= 0 || n > a.max_group_size || row0 >= n * g) return;
    if (row0 == 0 && h == 0 && split == 0) {
      // each member's own pass starts at its first block past the prefix
      // that still leaves it one token (the decoded one): its last block
      // (the word holds that start in 16-token granules, the decode's unit)
      for (int m = threadIdx.x; m < n; m += NW * kWave) {
        const int s = a.group_seqs[goff + m];
        if (s < 0 || s >= a.num_seqs) continue;
        const int Ls = a.context_lens[s];
        const uint64_t start = Ls >= 1 ? min(pblk, (Ls - 1) / BS) : 0;
        const uint64_t nsp = Ls >= 1 ? (pblk + a.split_blocks - 1) / a.split_blocks : 0;
        a.seq_prefix[s] = a.tag | (nsp << 20) | (start * SPB);
      }
    }
    const int klo = split * a.split_blocks * BS;
    L = min(pblk * BS, klo + a.split_blocks * BS);   // keys at or past L are masked
    if (klo >= L) return;
    kt0 = klo / KT;
    r = a.group_seqs[goff];     // the first member's table supplies the prefix blocks
    if (r < 0 || r >= a.num_seqs) return;
  }

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const bool lead = wave < HALF;
  const int c32 = lane & 31;    // A/B row-or-column, C column
  const int G = lane >> 5;      // k-slot group / C row group
  const int nblk = (L + BS - 1) / BS;   // table blocks holding keys 0 .. L-1
  const_i32* trow = (const_i32*)(a.block_tables + (int64_t)r * a.max_blocks_per_seq);

  // Rows of this workgroup and their last visible key.
  const int last_row = min(row0 + ROWS, n * g) - 1;
  const int wrow0 = row0 + wave * RPW;
  const bool has_rows = wrow0 <= last_row;
  int ntiles, wq_min, wq_max;

  // Q^T operand: lane (row c32, group G) holds channels ks*16 + G*8 .. +7
  // (loaded after the first tile copies have been issued).
  const uint16_t* qp = (const uint16_t*)a.q;
  bf16x8 qf[KS];
  int qpos;                 // the row's last visible key
  const uint16_t* qrow;
  bool qlive;
  if constexpr (!PREFIX) {
    const int kend = P + last_row / g + 1;                 // keys 0..kend-1 are needed
    ntiles = (kend + KT - 1) / KT;
    wq_min = P + min(wrow0, last_row) / g;                 // smallest query position of the wave
    wq_max = has_rows ? P + min(wrow0 + RPW - 1, last_row) / g : -1;
    const int rr = wrow0 + c32;
    const bool live = rr <= last_row;
    const int t = live ? rr / g : 0;
    const int j = live ? rr - (rr / g) * g : 0;
    qpos = P + (live ? t : last_row / g);
    qrow = qp + ((int64_t)(q0 + t) * hq + h * g + j) * D + G * 8;
    qlive = live;
  } else {
    ntiles = (L - kt0 * KT + KT - 1) / KT;
    const int rr = wrow0 + c32;
    int s = rr <= last_row ? a.group_seqs[goff + rr / g] : -1;
    const bool live = s >= 0 && s < a.num_seqs;
    const int j = rr - (rr / g) * g;
    const int Ls = live ? a.context_lens[s] : 0;
    const int start = Ls >= 1 ? min(pblk, (Ls - 1) / BS) : 0;
    qpos = live ? min(start * BS, L) - 1 : -1;
    qrow = qp + ((int64_t)(live ? s : 0) * hq + h * g + (live ? j : 0)) * D + G * 8;
    qlive = live;
    int lo = live ? qpos : (1 << 30), hi = live ? qpos : -1;
#pragma unroll
    for (int k = 1; k < 32; k <<= 1) {
      lo = min(lo, __shfl_xor(lo, k, kWave));
      hi = max(hi, __shfl_xor(hi, k, kWave));
    }
    wq_min = __builtin_amdgcn_readfirstlane(lo);
    wq_max = __builtin_amdgcn_readfirstlane(hi);
  }

  const uint8_t* kpool = (const uint8_t*)a.k_pool;
  const uint8_t* vpool = (const uint8_t*)a.v_pool;
  // Table word of logical block kb; past the end of the sequence, the
  // sequence's last block (its keys there are masked where used).  The word
  // is loaded well before its copy is issued and range-checked only then
  // (an entry outside the pool reads block 0), so the scalar load's latency
  // stays off the critical path.
  auto entry_raw = [&](int kb) -> int { return trow[min(kb, nblk - 1)]; };
  auto entry_ok = [&](int e) -> uint32_t {
    return (uint32_t)e < (uint32_t)a.num_blocks ? (uint32_t)e : 0u;
  };

  // Direct-to-LDS copy of tile t into stage t % NST ([K tile | V tile]).
  // Wave w copies, for each i < NBW, the 64-chunk segment s = i*NW + w of
  // the K tile and the same segment of the V tile: both lie in block
  // src_blk[i] of the tile, so each block's address is formed once.  Each
  // lane's byte offsets inside the head's K and V slabs are fixed per
  // (i, w): computed once.
  constexpr int NBW = PER_T / 2;
  static_assert(NBW * NW == SEGS, "a wave's K and V segments pair up block by block");
  uint32_t src_off_k[NBW], src_off_v[NBW];
  int src_blk[NBW];
#pragma unroll
  for (int i = 0; i < NBW; ++i) {
    const int c0 = (i * NW + wave) * kWave;      // first chunk of the segment in its tile
    const int blk = c0 / (BLKB / 16);
    const int within = c0 - blk * (BLKB / 16) + lane;
    const int row = within / CPR;
    const int pos = within - row * CPR;
    src_off_k[i] = (uint32_t)(h * BLKB + (row * CPR + (pos ^ (((row & 15) / SWZ) % CPR))) * 16);
    // V: LDS chunk q' of channel row c holds the slab's chunk q' ^ vswz(c)
    constexpr int CPV = VROWB / 16;       // 16-byte chunks per V channel row
    const int vc = within / CPV;
    src_off_v[i] = (uint32_t)(h * BLKB + (vc * CPV + ((within % CPV) ^ vswz(vc))) * 16);
    src_blk[i] = blk;
  }
  const uint32_t blk_stride = (uint32_t)(hkv * BLKB);   // bytes between physical blocks
  auto fetch_entries = [&](int t, int (&e)[NBW]) {
#pragma unroll
    for (int i = 0; i < NBW; ++i) e[i] = entry_raw((t + kt0) * NBT + src_blk[i]);
  };
  auto issue = [&](int t, const int (&e)[NBW]) {
    const uint32_t lds0 = (uint32_t)(size_t)(__attribute__((address_space(3))) uint8_t*)(
        &kv_s[t % NST][wave * kWave * 16]);
#pragma unroll
    for (int i = 0; i < NBW; ++i) {
      const uint64_t off = (uint64_t)entry_ok(e[i]) * blk_stride;
      const uint32_t lk = lds0 + i * NW * kWave * 16;
      lds_dma16_kv(kpool + off, src_off_k[i], vpool + off, src_off_v[i], lk, lk + TILEB);
    }
  };

  // LDS read offsets (stage 0).  K: key row c32 % 16 of block
  // 2*chunk + c32 / 16, logical chunk 2*ks + G.  V: channel dt*32 + c32,
  // half G of the row.
  uint32_t koff[KS];
  {
    const int row = c32 & 15;
    const int f = (row / SWZ) % CPR;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      koff[ks] = (uint32_t)((c32 >> 4) * SUBB + row * ROWB + (((ks * 2 + G) ^ f) * 16));
  }
  // V: channel row c32 of a 16-key sub-block, chunk G (sub-block b of the
  // tile at b * SUBB)
  const uint32_t voff = (uint32_t)(TILEB + c32 * VROWB + ((G ^ vswz(c32)) * 16));

  const float c2 = a.scale * kLog2e;   // scores -> base-2 exponent units
  float m_ref = -INFINITY;
  // Row sums: each lane sums its own probabilities (every value of lsA and
  // lsB holds the running sum of one half of the lane's keys); the two lanes
  // of a row are added at the end.
  f32x4 lsA = f32x4{0.f, 0.f, 0.f, 0.f}, lsB = f32x4{0.f, 0.f, 0.f, 0.f};
  const bf16x4 ones4 = bf16x4{(__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f};
  f32x16 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[dt][v] = 0.f;
  f32x16 sc[2];
  bf16x8 pf[NSB];

  // Matrix-phase streams.  Fragment reads and MFMAs are interleaved with
  // a fixed lookahead, so LDS latency hides behind the matrix core and only
  // a few fragments are live at once.
  // PV reads: V fragment (block b, channel tile dt) for i = b*DT + dt.
  // QK reads: K fragment (k-step ks, 32-key chunk ch) for i = ks*2 + ch.
  constexpr int NPV = NSB * DT;
  constexpr int NQK = 2 * KS;
  constexpr int LA = 6;          // lookahead of the QK-only stream
  constexpr int NPRE = NPV / 2;  // V fragments read at the end of the vector phase
  auto vread = [&](int st, int i) {
    const int b = i / DT;   // sub-block
    return *reinterpret_cast<const bf16x8*>(kv_s[st] + voff + b * SUBB + (i % DT) * 32 * VROWB);
  };
  auto kread = [&](int st, int i) {
    return *reinterpret_cast<const bf16x8*>(kv_s[st] + koff[i / 2] + (i % 2) * 2 * SUBB);
  };
  auto pv_mfma = [&](int i, bf16x8 f) {
    o[i % DT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, pf[i / DT], o[i % DT], 0, 0, 0);
  };
  // Row sums of the rounded probabilities (exactly the weights PV uses) on
  // the matrix core: v_mfma_f32_4x4x4_16b_bf16 with an all-ones A operand
  // gives each lane the sum of its own four B values (16 blocks of 4x4: lane
  // l supplies column l % 4 of block l / 4), issuing every ~9 cycles against
  // 32 for a 32x32x16 product.  Two per 16-key sub-block, on two chains.
  // The vector phase then needs no adds, and no bf16 dot instructions (those
  // run on the matrix pipeline and would wait behind the other wave's MFMAs).
  auto sum_mfma = [&](int b) {
    const bf16x4 lo = __builtin_shufflevector(pf[b], pf[b], 0, 1, 2, 3);
    const bf16x4 hi = __builtin_shufflevector(pf[b], pf[b], 4, 5, 6, 7);
    lsA = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(ones4, lo, lsA, 0, 0, 0);
    lsB = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(ones4, hi, lsB, 0, 0, 0);
  };
  auto qk_mfma = [&](int i, bf16x8 f) {
    sc[i % 2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, qf[i / 2], sc[i % 2], 0, 0, 0);
  };
  auto clear_sc = [&]() {
#pragma unroll
    for (int ch = 0; ch < 2; ++ch)
#pragma unroll
      for (int v = 0; v < 16; ++v) sc[ch][v] = 0.f;
  };
  // The first NPRE V fragments of the next PV, read while this wave is in
  // its vector phase (their tile is already in LDS), so the matrix phase
  // starts on MFMAs rather than on LDS latency.
  bf16x8 vpre[NPRE];
  auto pre_read = [&](int sp) {
#pragma unroll
    for (int i = 0; i < NPRE; ++i) vpre[i] = vread(sp, i);
  };
  // PV of the tile in stage sp (fragments 0..NPRE-1 already read), then QK
  // of the tile in stage sq.  Stream read j is issued after MFMA j and
  // consumed by MFMA j + NPRE.
  auto pv_qk = [&](int sp, int sq) {
    constexpr int NR = NPV - NPRE + NQK;
    // Higher issue priority while feeding the matrix core: the other wave of
    // the SIMD (in its vector phase) would otherwise win every issue slot
    // and delay the MFMAs whenever it is the older wave.
    __builtin_amdgcn_s_setprio(1);
    bf16x8 fr[NR];
#pragma unroll
    for (int j = 0; j < NPV - NPRE; ++j) fr[j] = vread(sp, NPRE + j);
#pragma unroll
    for (int j = 0; j < NQK; ++j) fr[NPV - NPRE + j] = kread(sq, j);
    clear_sc();
#pragma unroll
    for (int i = 0; i < NPRE; ++i) pv_mfma(i, vpre[i]);
#pragma unroll
    for (int b = 0; b < NSB; ++b) sum_mfma(b);
#pragma unroll
    for (int i = NPRE; i < NPV; ++i) pv_mfma(i, fr[i - NPRE]);
#pragma unroll
    for (int i = 0; i < NQK; ++i) qk_mfma(i, fr[NPV - NPRE + i]);
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, NPRE + 2 * NSB, 0);
    __builtin_amdgcn_s_setprio(0);
  };
  // QK alone (first tile): LA reads, then (MFMA, read) pairs.
  auto qk = [&](int sq) {
    bf16x8 fr[NQK];
#pragma unroll
    for (int i = 0; i < NQK; ++i) fr[i] = kread(sq, i);
    clear_sc();
#pragma unroll
    for (int i = 0; i < NQK; ++i) qk_mfma(i, fr[i]);
    __builtin_amdgcn_sched_group_barrier(0x100, LA, 0);
#pragma unroll
    for (int i = 0; i < NQK - LA; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, LA, 0);
  };

  // Probabilities of tile t (keys kbase..) from its scores.
  auto softmax = [&](int kbase, auto masked) {
    if constexpr (decltype(masked)::value) {   // tile crosses the diagonal of some row
#pragma unroll
      for (int ch = 0; ch < 2; ++ch)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (kbase + ch * 32 + (v >> 2) * 8 + G * 4 + (v & 3) > qpos) sc[ch][v] = -INFINITY;
    }
    // row maximum as a depth-4 tree of three-input maxima
    auto x = [&](int i) { return sc[i >> 4][i & 15]; };
    float m1[11];
#pragma unroll
    for (int i = 0; i < 10; ++i) m1[i] = fmaxf(fmaxf(x(3 * i), x(3 * i + 1)), x(3 * i + 2));
    m1[10] = fmaxf(x(30), x(31));
    const float m2a = fmaxf(fmaxf(m1[0], m1[1]), m1[2]);
    const float m2b = fmaxf(fmaxf(m1[3], m1[4]), m1[5]);
    const float m2c = fmaxf(fmaxf(m1[6], m1[7]), m1[8]);
    const float m2d = fmaxf(m1[9], m1[10]);
    const float mb = max_halves(fmaxf(fmaxf(m2a, m2b), fmaxf(m2c, m2d)));
    const float m_new = mb * c2;
    const bool grow = m_new > m_ref + kLazy;
    if (__any(grow)) {   // rare after the first tile
      const float target = grow ? m_new : m_ref;
      float alpha = __builtin_amdgcn_exp2f(m_ref - target);
      // a row that has seen no key keeps m_ref = -inf: exp2(-inf - -inf) is
      // not 1, so rows that do not grow take alpha = 1 explicitly
      if constexpr (PREFIX) alpha = grow ? alpha : 1.f;
      lsA *= alpha;
      lsB *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
      m_ref = target;
    }
    float nm = -m_ref;
    if constexpr (PREFIX) nm = m_ref == -INFINITY ? 0.f : nm;   // a row with no key yet
#pragma unroll
    for (int b = 0; b < NSB; ++b) {
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) p[e] = __builtin_amdgcn_exp2f(fmaf(sc[b >> 1][(b & 1) * 8 + e], c2, nm));
      pf[b] = bf16x8{(__bf16)p[0], (__bf16)p[1], (__bf16)p[2], (__bf16)p[3],
                     (__bf16)p[4], (__bf16)p[5], (__bf16)p[6], (__bf16)p[7]};
    }
    // The probabilities are computed in this (vector) phase, not in the
    // matrix phase that consumes them.
#pragma unroll
    for (int b = 0; b < NSB; ++b) materialize(pf[b]);
  };

  // PV alone (the last tile of the workgroup).  V^T operand of block b,
  // channel tile dt: the lane's 16 bytes are keys 4G..4G+3 and 8+4G..8+4G+3
  // of channel dt*32 + c32 (positions 8G..8G+7 of the row).  Keys at or past
  // the end of the sequence (tail of the last block, blocks read as block
  // 0) hold arbitrary bits: p is 0 there but 0 * NaN is not, so their value
  // words are cleared.
  auto pv = [&](int sp, int kbase) {
    bf16x8 fr[NPV];
#pragma unroll
    for (int i = 0; i < NPV; ++i) fr[i] = vread(sp, i);
    if (kbase + KT > L) {
#pragma unroll
      for (int b = 0; b < NSB; ++b) {
        uint32_t mk[4];
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          const int k0 = kbase + b * kBs + hb * 8 + G * 4;
          mk[2 * hb] = (k0 < L ? 0x0000ffffu : 0u) | (k0 + 1 < L ? 0xffff0000u : 0u);
          mk[2 * hb + 1] = (k0 + 2 < L ? 0x0000ffffu : 0u) | (k0 + 3 < L ? 0xffff0000u : 0u);
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const u32x4 w = __builtin_bit_cast(u32x4, fr[b * DT + dt]);
          fr[b * DT + dt] = __builtin_bit_cast(
              bf16x8, u32x4{w.x & mk[0], w.y & mk[1], w.z & mk[2], w.w & mk[3]});
        }
      }
    }
#pragma unroll
    for (int i = 0; i < NPV; ++i) pv_mfma(i, fr[i]);
#pragma unroll
    for (int b = 0; b < NSB; ++b) sum_mfma(b);
  };

  // Slots: waves 0..3 run matrix phase j in slot 2j and vector phase j in
  // slot 2j+1; waves 4..7 one slot later.  Matrix phase j holds PV of tile
  // j-1 and QK of tile j; vector phase t the softmax of tile t, the copy of
  // tile t+3 (tiles 0..2 are copied before the loop) and the table lookups
  // for tile t+4, whether or not this wave computes on those tiles (all
  // eight waves share each copy).  A barrier ends every odd slot, so slots
  // 2j and 2j+1 form one window: there waves 0..3 run matrix phase j and
  // vector phase j, waves 4..7 vector phase j-1 and matrix phase j.  Tile t
  // occupies stage t % 5 from its copy until the PV in matrix phase t+1
  // (window t+1); the first copy that refills the stage is issued in vector
  // phase t+2, which no wave starts before window t+2.
  //
  // Phase boundary after the phase in slot s.  Odd slots end where tile
  // (s+1)/2 must be in LDS for everyone (matrix phase (s+1)/2 reads it in
  // the next window): this wave waits for its share, leaving in flight only
  // the copies it issued after that tile (waves 0..3 have issued up to tile
  // u+3 by then, waves 4..7 up to u+2), and the barrier follows.  Even slots
  // end without one.
  auto end_phase = [&](int s) {
    if (s & 1) {
      const int u = s >> 1;
      const int n_out = min(u + (lead ? 3 : 2), ntiles - 1) - (u + 1);
      if (n_out >= 2) wait_vm<2 * PER_T>();
      else if (n_out == 1) wait_vm<PER_T>();
      else wait_vm<0>();
      wg_barrier();
    }
  };
  int e_nxt[NBW];   // table words of the next tile to copy
  auto copy_and_lookup = [&](int t) {
    if (t + 3 < ntiles) issue(t + 3, e_nxt);
    if (t + 4 < ntiles) fetch_entries(t + 4, e_nxt);
  };

  // This wave computes on tiles 0..nt-1 (later tiles are in the future of
  // all its rows), with the causal mask from tile td on; a tile past the end
  // of the sequence can only be the last one, whose PV has no QK after it.
  const int nt = has_rows && wq_max >= kt0 * KT ? min(ntiles, (wq_max - kt0 * KT) / KT + 1) : 0;
  const int td = wq_min + 1 >= kt0 * KT ? (wq_min + 1 - kt0 * KT) / KT : 0;
  {
    int e0[NBW], e1[NBW], e2[NBW];
    fetch_entries(0, e0);
    fetch_entries(1, e1);
    fetch_entries(2, e2);
    if (ntiles > 3) fetch_entries(3, e_nxt);
    issue(0, e0);
    if (ntiles > 1) issue(1, e1);
    if (ntiles > 2) issue(2, e2);
  }
  // Q after the first copies, so both latencies overlap; waiting for all
  // of them (the compiler's own wait for Q would do the same) also covers
  // tiles 0..2 before the first barrier.
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(qrow + ks * 16);
    qf[ks] = qlive ? v : bf16x8{};
  }
  wait_vm<0>();
  wg_barrier();
  const int lag = lead ? 0 : 1;
  if (nt > 0) qk(0);
  int t = 0;
  const int t_plain = min(td, nt - 1);
  for (; t < t_plain; ++t) {          // no mask, PV and QK
    end_phase(2 * t + lag);
    copy_and_lookup(t);
    softmax((t + kt0) * KT, std::false_type{});
    pre_read(t % NST);
    end_phase(2 * t + 1 + lag);
    pv_qk(t % NST, (t + 1) % NST);
  }
  for (; t < nt - 1; ++t) {           // masked, PV and QK
    end_phase(2 * t + lag);
    copy_and_lookup(t);
    softmax((t + kt0) * KT, std::true_type{});
    pre_read(t % NST);
    end_phase(2 * t + 1 + lag);
    pv_qk(t % NST, (t + 1) % NST);
  }
  if (t < nt) {                        // last tile of this wave: PV only
    end_phase(2 * t + lag);
    copy_and_lookup(t);
    if (t < td) softmax((t + kt0) * KT, std::false_type{});
    else softmax((t + kt0) * KT, std::true_type{});
    end_phase(2 * t + 1 + lag);
    pv(t % NST, (t + kt0) * KT);
    ++t;
  }
  for (; t < ntiles; ++t) {           // copies and barriers only
    end_phase(2 * t + lag);
    copy_and_lookup(t);
    end_phase(2 * t + 1 + lag);
  }

  // Normalise and store: lane (row c32, group G) holds channels
  // dt*32 + 8*(v/4) + 4*G + v%4 of its row.
  const float l = [&] {   // lanes l and l ^ 32 hold the two halves of the row's keys
    const float part = lsA[0] + lsB[0];
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }();
  const int rr = wrow0 + c32;
  if (rr > last_row) return;
  if constexpr (PREFIX) {
    if (!qlive) return;
    const int s = a.group_seqs[goff + rr / g];
    const int64_t prow = ((int64_t)s * hq + h * g + (rr - (rr / g) * g)) * a.num_splits + split;
    const float inv = l > 0.f ? 1.f / l : 0.f;   // a row that saw no key: o = 0, weight 0
    float* orow = a.pre_o + prow * D + G * 4;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int b = 0; b < 4; ++b)
        *reinterpret_cast<f32x4*>(orow + dt * 32 + b * 8) =
            f32x4{o[dt][4 * b] * inv, o[dt][4 * b + 1] * inv, o[dt][4 * b + 2] * inv,
                  o[dt][4 * b + 3] * inv};
    if (G == 0) {
      a.pre_m[prow] = l > 0.f ? m_ref * kLn2 : -INFINITY;   // natural-log units
      a.pre_l[prow] = l;
    }
    return;
  } else {
  const int tok = rr / g;
  const int jh = rr - tok * g;
  const float inv = 1.f / l;
  uint16_t* orow = (uint16_t*)a.out + ((int64_t)(q0 + tok) * hq + h * g + jh) * D + G * 4;
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
  const int bsz = a.block_size;
  if (L > a.max_blocks_per_seq * bsz) L = a.max_blocks_per_seq * bsz;
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
  // 16-token granules; granule b is part b % (bsz/16) of table block b / (bsz/16)
  const int spb = bsz / kBs;
  const int nb = (ctx + kBs - 1) / kBs;
  for (int b = 0; b < nb; ++b) {
    int phys = trow[b / spb];
    phys = (phys >= 0 && phys < a.num_blocks) ? phys : 0;
    const int part = b % spb;
    const int64_t base = ((int64_t)phys * hkv + h) * bsz * D;
    const float* kb = kpool + base + part * kBs * D;   // the granule's keys and values:
    const float* vb = vpool + base + part * kBs * D;   // 16 x D elements each
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
        for (int e = 0; e < DPL; ++e) acc[e] = fmaf(pt, vb[(lane + e * kWave) * kVRow + v_pos(t)], acc[e]);
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
    if (a.block_size == 32)
      extend_bf16_kernel<D, false, ExtendArgs, 32><<<(unsigned)grid, NW * kWave, 0, st>>>(a, tiles,
                                                                                         units);
    else
      extend_bf16_kernel<D, false, ExtendArgs, 16><<<(unsigned)grid, NW * kWave, 0, st>>>(a, tiles,
                                                                                         units);
  } else {
    if (a.max_q_len == 0) return 0;
    extend_f32_kernel<D><<<dim3(a.max_q_len, a.num_kv_heads, a.num_reqs), kWave, 0, st>>>(a);
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

template <int D>
int launch_p(const PrefixArgs& a, hipStream_t st) {
  constexpr int ROWS = 8 * 32;
  const int g = a.num_q_heads / a.num_kv_heads;
  const int tiles = (a.max_group_size * g + ROWS - 1) / ROWS;
  const int64_t units = (int64_t)a.num_groups * a.num_kv_heads * a.num_splits;
  const int64_t unit_groups = (units + kXcds - 1) / kXcds;
  const int64_t grid = (int64_t)kXcds * unit_groups * tiles;
  if (grid == 0) return 0;
  if (grid > 0x7fffffff || units > 0x7fffffff) return -1;
  if (a.block_size == 32)
    extend_bf16_kernel<D, true, PrefixArgs, 32><<<(unsigned)grid, 8 * kWave, 0, st>>>(a, tiles,
                                                                                     (int)units);
  else
    extend_bf16_kernel<D, true, PrefixArgs, 16><<<(unsigned)grid, 8 * kWave, 0, st>>>(a, tiles,
                                                                                     (int)units);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace

int launch_prefix(const PrefixArgs& a, hipStream_t st) {
  if (a.num_groups == 0 || a.max_group_size == 0) return 0;
  if (a.head_dim == 128) return launch_p<128>(a, st);
  return launch_p<64>(a, st);
}

int launch_extend(const ExtendArgs& a, int32_t dtype, hipStream_t st) {
  if (a.num_reqs == 0 || a.total_q == 0) return 0;
  if (a.head_dim == 128) return launch_e<128>(a, dtype, st);
  return launch_e<64>(a, dtype, st);
}

}  // namespace pkv
