// Host code: the decode step of the block manager (one new token for each
// sequence of a batch), run natively on the block manager's own arrays.
//
// Per sequence: if its last block is full it gets a fresh block from the
// free list; if it writes into a block that other sequences also reference
// (count above one), it gets a fresh block to copy into and the old block
// loses one reference; the token's slot is the next one of its last block
// ("Paged Attention for Efficient Memory Management", The Daily Triptych,
// "The story": a new token fills the current block, a full block is
// followed by a fresh one from the pool, and a write into a shared block
// goes to a copy).  Sequences are handled in the order given, so of several
// sequences sharing one partial block every one but the last copies it and
// the last writes in place.  No GPU call is made.
#include <vector>

#include "../../include/pagedkv.h"
#include "common.h"

extern "C" int block_manager_append_step(
    int32_t* tables, int32_t* lens, int32_t* nblk, const uint8_t* live, const uint8_t* on_host,
    int32_t max_seqs, int32_t max_blocks_per_seq, int32_t* ref, const uint8_t* sealed,
    int32_t num_blocks, int32_t block_size, const int64_t* sids, int32_t num_sids,
    int32_t* free_ring, int64_t* free_state, int32_t* slots_out, int32_t* pairs_out,
    int32_t* num_pairs_out) {
  using pkv::set_error;
  if (!tables || !lens || !nblk || !live || !on_host || !ref || !sealed || !free_ring ||
      !free_state || !num_pairs_out || (num_sids > 0 && (!sids || !slots_out || !pairs_out)))
    return set_error(PKV_ERR_INVALID, "block_manager_append_step: null pointer");
  if (max_seqs <= 0 || max_blocks_per_seq <= 0 || num_blocks <= 0 || block_size <= 0 ||
      num_sids < 0 || num_sids > max_seqs)
    return set_error(PKV_ERR_INVALID, "block_manager_append_step: bad sizes");
  const int64_t head0 = free_state[0], count0 = free_state[1];
  if (head0 < 0 || head0 >= num_blocks || count0 < 0 || count0 > num_blocks)
    return set_error(PKV_ERR_INVALID, "block_manager_append_step: bad free-list state");
  *num_pairs_out = 0;
  if (num_sids == 0) return pkv::clear_error();

  std::vector<uint8_t> seen(max_seqs, 0);
  for (int32_t i = 0; i < num_sids; ++i) {
    const int64_t s = sids[i];
    if (s < 0 || s >= max_seqs) return set_error(PKV_ERR_INVALID, "sequence id out of range");
    if (seen[s]) return set_error(PKV_ERR_INVALID, "a sequence may appear once per step");
    seen[s] = 1;
    if (!live[s]) return set_error(PKV_ERR_INVALID, "append_step on a sequence that is not live");
    if (on_host[s]) return set_error(PKV_ERR_INVALID, "append_step on a sequence on the host tier");
  }

  // Pass 1: what each sequence needs.  Copy-on-write drops the old block's
  // count as it goes (so the last sharer writes in place); the drops are
  // undone if the step cannot be completed.
  enum : uint8_t { kInPlace, kNew, kCopy };
  std::vector<uint8_t> kind(num_sids);
  std::vector<int32_t> old(num_sids, -1);
  std::vector<int32_t> dropped;   // blocks whose count was dropped, one entry per drop
  auto undo = [&]() {
    for (int32_t b : dropped) ref[b] += 1;
  };
  int64_t need = 0;
  bool too_long = false;
  for (int32_t i = 0; i < num_sids; ++i) {
    const int64_t s = sids[i];
    const int32_t pos = lens[s], nb = nblk[s];
    if (pos % block_size == 0) {
      kind[i] = kNew;
      ++need;
      if (nb + 1 > max_blocks_per_seq) too_long = true;
      continue;
    }
    if (nb <= 0) {
      undo();
      return set_error(PKV_ERR_INVALID, "block table shorter than the sequence");
    }
    const int32_t b = tables[s * (int64_t)max_blocks_per_seq + nb - 1];
    if (b < 0 || b >= num_blocks) {
      undo();
      return set_error(PKV_ERR_INVALID, "block table entry out of range");
    }
    if (sealed[b]) {
      undo();
      return PKV_STEP_SEALED;
    }
    old[i] = b;
    if (ref[b] > 1) {
      kind[i] = kCopy;
      ref[b] -= 1;
      dropped.push_back(b);
      ++need;
    } else {
      kind[i] = kInPlace;
    }
  }
  if (need > count0) {
    undo();
    return PKV_STEP_SHORT;
  }
  if (too_long) {
    undo();
    return set_error(PKV_ERR_INVALID, "sequence would exceed max_blocks_per_seq");
  }

  // Pass 2: take fresh blocks in sequence order from the front of the free
  // list, update the tables, emit copy pairs and slots.
  int64_t head = head0;
  int32_t np = 0;
  for (int32_t i = 0; i < num_sids; ++i) {
    const int64_t s = sids[i];
    int32_t* row = tables + s * (int64_t)max_blocks_per_seq;
    const int32_t pos = lens[s], nb = nblk[s];
    if (kind[i] != kInPlace) {
      const int32_t got = free_ring[head];
      head = head + 1 == num_blocks ? 0 : head + 1;
      ref[got] = 1;
      if (kind[i] == kNew) {
        row[nb] = got;
        nblk[s] = nb + 1;
      } else {
        row[nb - 1] = got;
        pairs_out[2 * np] = old[i];
        pairs_out[2 * np + 1] = got;
        ++np;
      }
    }
    slots_out[i] = row[pos / block_size] * block_size + pos % block_size;
    lens[s] = pos + 1;
  }
  free_state[0] = head;
  free_state[1] = count0 - need;
  *num_pairs_out = np;
  return pkv::clear_error();
}
