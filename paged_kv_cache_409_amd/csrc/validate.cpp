// Debug checks of index-buffer values on the host (C ABI in include/pkv_validate.h; what
// each check follows on the pages is listed there). Plain loops over host arrays; the
// device entry point copies the buffers here first (api.hip).
#include <cstdint>
#include <unordered_map>
#include <vector>

#include "pkv.h"
#include "pkv_validate.h"

namespace {

void fail(pkv_validation* r, int check, int64_t index, int64_t value) {
  r->check = check;
  r->index = index;
  r->value = value;
}

}  // namespace

extern "C" int pkv_validate_inputs_host(const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
                                        int max_blocks_per_seq, int block_size, int64_t num_blocks,
                                        const int64_t* slot_mapping, int num_tokens, int decode_step,
                                        const int32_t* cow_src, const int64_t* src_dst_pairs, int num_pairs,
                                        pkv_validation* result) {
  if (!result) return PKV_ERR_NULL;
  if (num_seqs < 0 || num_tokens < 0 || num_pairs < 0 || num_blocks <= 0) return PKV_ERR_SHAPE;
  if (block_size != 16 && block_size != 32 && block_size != 64) return PKV_ERR_UNSUPPORTED;
  const bool tables = block_tables != nullptr || context_lens != nullptr;
  if (tables && (!block_tables || !context_lens)) return PKV_ERR_NULL;
  if (tables && max_blocks_per_seq <= 0) return PKV_ERR_SHAPE;
  if (decode_step && (!tables || !slot_mapping)) return PKV_ERR_NULL;
  if (decode_step && num_tokens != num_seqs) return PKV_ERR_SHAPE;
  if (cow_src && !decode_step) return PKV_ERR_SHAPE;
  fail(result, PKV_CHECK_OK, -1, 0);

  const int64_t P = block_size;
  const int64_t max_ctx = (int64_t)max_blocks_per_seq * P;
  if (tables) {
    for (int s = 0; s < num_seqs; ++s) {
      const int64_t c = context_lens[s];
      if (c < 0 || c > max_ctx) {
        fail(result, PKV_CHECK_CONTEXT_LEN, s, c);
        return PKV_OK;
      }
    }
    for (int s = 0; s < num_seqs; ++s) {
      const int64_t used = (context_lens[s] + P - 1) / P;   // entries that hold context
      for (int64_t i = 0; i < used; ++i) {
        const int64_t b = block_tables[(int64_t)s * max_blocks_per_seq + i];
        if (b < 0 || b >= num_blocks) {
          fail(result, PKV_CHECK_BLOCK_ID, (int64_t)s * max_blocks_per_seq + i, b);
          return PKV_OK;
        }
      }
    }
  }

  if (slot_mapping) {
    const int64_t num_slots = num_blocks * P;
    for (int t = 0; t < num_tokens; ++t) {
      if (slot_mapping[t] >= num_slots) {
        fail(result, PKV_CHECK_SLOT_RANGE, t, slot_mapping[t]);
        return PKV_OK;
      }
    }
    std::unordered_map<int64_t, int> taken;
    taken.reserve((size_t)num_tokens * 2);
    for (int t = 0; t < num_tokens; ++t) {
      if (slot_mapping[t] < 0) continue;
      if (!taken.emplace(slot_mapping[t], t).second) {
        fail(result, PKV_CHECK_SLOT_DUPLICATE, t, slot_mapping[t]);
        return PKV_OK;
      }
    }
    if (decode_step) {
      for (int s = 0; s < num_seqs; ++s) {
        const int64_t slot = slot_mapping[s];
        if (slot < 0) continue;
        const int64_t pos = (int64_t)context_lens[s] - 1;
        const bool ok = pos >= 0 &&
                        slot == (int64_t)block_tables[(int64_t)s * max_blocks_per_seq + pos / P] * P + pos % P;
        if (!ok) {
          fail(result, PKV_CHECK_SLOT_NOT_LAST, s, slot);
          return PKV_OK;
        }
      }
      // Which sequences read each block that a new token goes into.
      std::unordered_map<int64_t, int> target;   // block -> writing sequence
      for (int s = 0; s < num_seqs; ++s)
        if (slot_mapping[s] >= 0) target.emplace(slot_mapping[s] / P, s);
      for (int s = 0; s < num_seqs; ++s) {
        const int64_t used = (context_lens[s] + P - 1) / P;
        for (int64_t i = 0; i < used; ++i) {
          const auto it = target.find(block_tables[(int64_t)s * max_blocks_per_seq + i]);
          if (it != target.end() && it->second != s) {
            fail(result, PKV_CHECK_SLOT_SHARED_BLOCK, it->second, s);
            return PKV_OK;
          }
        }
      }
    }
  }

  if (cow_src) {
    // The step's copies: each sequence's last block (the destination) becomes a copy of
    // cow_src[s] before its new token lands there.
    for (int s = 0; s < num_seqs; ++s) {
      const int64_t b = cow_src[s];
      if (b < -1 || b >= num_blocks) {
        fail(result, PKV_CHECK_COW_RANGE, s, b);
        return PKV_OK;
      }
      if (b >= 0 && context_lens[s] == 0) {
        fail(result, PKV_CHECK_COW_NO_CONTEXT, s, b);
        return PKV_OK;
      }
    }
    std::unordered_map<int64_t, int> dst_of;   // destination block -> copying sequence
    for (int s = 0; s < num_seqs; ++s) {
      if (cow_src[s] < 0) continue;
      const int64_t dst = block_tables[(int64_t)s * max_blocks_per_seq + (context_lens[s] - 1) / P];
      if (dst != cow_src[s]) dst_of.emplace(dst, s);   // a copy onto itself is a no-op
    }
    for (int t = 0; t < num_seqs; ++t) {
      const int64_t used = (context_lens[t] + P - 1) / P;
      for (int64_t i = 0; i < used; ++i) {
        const auto it = dst_of.find(block_tables[(int64_t)t * max_blocks_per_seq + i]);
        if (it != dst_of.end() && it->second != t) {
          fail(result, PKV_CHECK_COW_SHARED_DST, it->second, t);
          return PKV_OK;
        }
      }
    }
    for (int t = 0; t < num_seqs; ++t) {
      if (cow_src[t] < 0) continue;
      const auto it = dst_of.find(cow_src[t]);
      if (it != dst_of.end() && it->second != t) {
        fail(result, PKV_CHECK_COW_DST_IS_SRC, it->second, t);
        return PKV_OK;
      }
    }
    // A copy takes every row of its source but its own new token's; another sequence's new
    // token may land in the source only in that row (beams that shared the block hold the
    // same number of tokens in it, so their new tokens share the row).
    std::unordered_map<int64_t, std::vector<int>> copies_from;   // source block -> copying sequences
    for (const auto& [dst, s] : dst_of) copies_from[cow_src[s]].push_back(s);
    for (int t = 0; t < num_seqs; ++t) {
      const int64_t slot = slot_mapping[t];
      if (slot < 0) continue;
      const auto it = copies_from.find(slot / P);
      if (it == copies_from.end()) continue;
      for (const int s : it->second) {
        if (s == t) continue;
        const int64_t dst = block_tables[(int64_t)s * max_blocks_per_seq + (context_lens[s] - 1) / P];
        const int64_t own = slot_mapping[s];
        const int64_t skip = (own >= 0 && own / P == dst) ? own % P : -1;
        if (slot % P != skip) {
          fail(result, PKV_CHECK_COW_SRC_WRITTEN, s, t);
          return PKV_OK;
        }
      }
    }
  }

  if (num_pairs > 0) {
    if (!src_dst_pairs) return PKV_ERR_NULL;
    for (int p = 0; p < num_pairs; ++p) {
      const int64_t src = src_dst_pairs[2 * p], dst = src_dst_pairs[2 * p + 1];
      if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) {
        fail(result, PKV_CHECK_PAIR_RANGE, p, (src < 0 || src >= num_blocks) ? src : dst);
        return PKV_OK;
      }
    }
    std::unordered_map<int64_t, int> dsts;
    dsts.reserve((size_t)num_pairs * 2);
    for (int p = 0; p < num_pairs; ++p) {
      const int64_t src = src_dst_pairs[2 * p], dst = src_dst_pairs[2 * p + 1];
      if (src == dst) continue;   // a no-op copy
      if (!dsts.emplace(dst, p).second) {
        fail(result, PKV_CHECK_PAIR_DUPLICATE_DST, p, dst);
        return PKV_OK;
      }
    }
    for (int p = 0; p < num_pairs; ++p) {
      const int64_t src = src_dst_pairs[2 * p], dst = src_dst_pairs[2 * p + 1];
      if (src == dst) continue;
      const auto it = dsts.find(src);
      if (it != dsts.end()) {
        fail(result, PKV_CHECK_PAIR_DST_IS_SRC, it->second, src);
        return PKV_OK;
      }
    }
  }
  return PKV_OK;
}
