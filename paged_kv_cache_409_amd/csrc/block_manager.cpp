// Host-side KV block manager (C ABI in include/pkv_block_manager.h).
//
// What it follows on the pages is listed in the header. Choices of this implementation:
// * free GPU and host blocks are FIFO queues, lowest id first at the start;
// * prefix caching keys a full block by a 64-bit chain hash of its tokens and its
//   predecessor's key (SplitMix64 as the mixing step, Steele, Lea and Flood, OOPSLA 2014);
//   a hit is confirmed by comparing the block's stored tokens and its predecessor block id,
//   so a hash collision can only cost a miss;
// * a known block whose last holder ends waits in a least-recently-freed queue and is
//   reused as a free block only when the free queue is empty;
// * every call checks what it needs (sequence ids, blocks, output room) before it changes
//   anything, so a failed call leaves the manager as it was.
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <deque>
#include <list>
#include <new>
#include <unordered_map>
#include <vector>

#include "pkv.h"
#include "pkv_block_manager.h"

namespace {

constexpr uint64_t kChainSeed = 0x70616765645f6b76ull;   // key "before" the first block

uint64_t splitmix64(uint64_t x) {
  x += 0x9E3779B97F4A7C15ull;
  x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
  x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
  return x ^ (x >> 31);
}

uint64_t chain_key(uint64_t prev, const int32_t* tokens, int n) {
  uint64_t h = splitmix64(prev);
  for (int i = 0; i < n; ++i) h = splitmix64(h ^ (uint64_t)(uint32_t)tokens[i]);
  return h;
}

struct Seq {
  std::vector<int> blocks;          // GPU blocks (on the GPU) or host blocks (swapped out), logical order
  int num_tokens = 0;
  bool on_gpu = true;
  bool has_tokens = false;          // every token id is known, so filled blocks can be registered
  std::vector<int32_t> partial;     // token ids of the partial last block
  uint64_t last_key = kChainSeed;   // key of the last full block
  int last_full = -1;               // GPU block of the last full block (-1: none, or not registered)
};

}  // namespace

struct pkv_block_manager {
  int nb_gpu, nb_host, P;
  bool caching;
  std::vector<int> ref;                       // holders of each GPU block
  std::deque<int> free_gpu, free_host;
  // prefix cache
  std::unordered_map<uint64_t, int> by_key;
  std::vector<uint8_t> known;
  std::vector<uint64_t> key_of;
  std::vector<int> parent_of;
  std::vector<int32_t> tokens_of;             // [nb_gpu * P]
  std::list<int> lru;                         // known blocks without holders, least recently freed first
  std::vector<std::list<int>::iterator> lru_pos;
  std::vector<uint8_t> in_lru;
  std::unordered_map<int64_t, Seq> seqs;

  int available_gpu() const { return (int)(free_gpu.size() + lru.size()); }

  int take_gpu() {   // caller checked availability
    int b;
    if (!free_gpu.empty()) {
      b = free_gpu.front();
      free_gpu.pop_front();
    } else {
      b = lru.front();
      lru.pop_front();
      in_lru[b] = 0;
      forget(b);
    }
    ref[b] = 1;
    return b;
  }

  void forget(int b) {
    if (!known[b]) return;
    auto it = by_key.find(key_of[b]);
    if (it != by_key.end() && it->second == b) by_key.erase(it);
    known[b] = 0;
  }

  void decref(int b) {
    if (--ref[b] > 0) return;
    if (known[b]) {
      lru.push_back(b);
      lru_pos[b] = std::prev(lru.end());
      in_lru[b] = 1;
    } else {
      free_gpu.push_back(b);
    }
  }

  void hold(int b) {   // one more holder; a known block waiting for reuse leaves the queue
    if (ref[b] == 0 && in_lru[b]) {
      lru.erase(lru_pos[b]);
      in_lru[b] = 0;
    }
    ++ref[b];
  }

  void remember(int b, uint64_t key, int parent, const int32_t* tokens) {
    if (!caching || by_key.count(key)) return;   // the first block with this content stays the known one
    by_key[key] = b;
    known[b] = 1;
    key_of[b] = key;
    parent_of[b] = parent;
    std::memcpy(&tokens_of[(size_t)b * P], tokens, sizeof(int32_t) * P);
  }

  int lookup(uint64_t key, int parent, const int32_t* tokens) const {
    auto it = by_key.find(key);
    if (it == by_key.end()) return -1;
    const int b = it->second;
    if (parent_of[b] != parent || std::memcmp(&tokens_of[(size_t)b * P], tokens, sizeof(int32_t) * P) != 0)
      return -1;
    return b;
  }
};

extern "C" {

int pkv_bm_create(int num_gpu_blocks, int num_host_blocks, int block_size, int enable_prefix_caching,
                  pkv_block_manager** out) {
  if (!out) return PKV_ERR_NULL;
  if (num_gpu_blocks <= 0 || num_host_blocks < 0 || block_size <= 0 || block_size > 4096 ||
      (enable_prefix_caching != 0 && enable_prefix_caching != 1))
    return PKV_ERR_SHAPE;
  if ((int64_t)num_gpu_blocks * block_size > (int64_t)1 << 40) return PKV_ERR_SHAPE;
  auto* bm = new (std::nothrow) pkv_block_manager();
  if (!bm) return PKV_ERR_NO_BLOCKS;
  bm->nb_gpu = num_gpu_blocks;
  bm->nb_host = num_host_blocks;
  bm->P = block_size;
  bm->caching = enable_prefix_caching != 0;
  bm->ref.assign(num_gpu_blocks, 0);
  for (int b = 0; b < num_gpu_blocks; ++b) bm->free_gpu.push_back(b);
  for (int b = 0; b < num_host_blocks; ++b) bm->free_host.push_back(b);
  bm->known.assign(num_gpu_blocks, 0);
  bm->in_lru.assign(num_gpu_blocks, 0);
  bm->lru_pos.resize(num_gpu_blocks);
  if (bm->caching) {
    bm->key_of.assign(num_gpu_blocks, 0);
    bm->parent_of.assign(num_gpu_blocks, -1);
    bm->tokens_of.assign((size_t)num_gpu_blocks * block_size, 0);
  }
  *out = bm;
  return PKV_OK;
}

void pkv_bm_destroy(pkv_block_manager* bm) { delete bm; }

int pkv_bm_add_sequence(pkv_block_manager* bm, int64_t seq_id, const int32_t* tokens, int num_tokens,
                        int64_t* slots_out, int* num_cached_tokens) {
  if (!bm) return PKV_ERR_NULL;
  if (num_tokens < 0) return PKV_ERR_SHAPE;
  if (num_tokens > 0 && !slots_out) return PKV_ERR_NULL;
  if (bm->seqs.count(seq_id)) return PKV_ERR_SEQ;
  const int P = bm->P;
  const int nblocks = (num_tokens + P - 1) / P, nfull = num_tokens / P;
  const bool use_cache = bm->caching && tokens != nullptr;

  // Leading full blocks already known.
  std::vector<int> matched;
  std::vector<uint64_t> keys;   // key of every full block, matched or not
  uint64_t key = kChainSeed;
  int prev = -1;
  if (use_cache) {
    for (int j = 0; j < nfull; ++j) {
      key = chain_key(key, tokens + (size_t)j * P, P);
      keys.push_back(key);
      if ((int)matched.size() == j) {
        const int b = bm->lookup(key, prev, tokens + (size_t)j * P);
        if (b >= 0) {
          matched.push_back(b);
          prev = b;
        }
      }
    }
    // A prompt known to its last token still recomputes its last block.
    if (!matched.empty() && (int)matched.size() == nblocks) matched.pop_back();
  }
  int waiting = 0;   // matched blocks that would leave the reuse queue
  for (int b : matched) waiting += (bm->ref[b] == 0 && bm->in_lru[b]) ? 1 : 0;
  if (nblocks - (int)matched.size() > bm->available_gpu() - waiting) return PKV_ERR_NO_BLOCKS;

  Seq s;
  for (int b : matched) {
    bm->hold(b);
    s.blocks.push_back(b);
  }
  int parent = matched.empty() ? -1 : matched.back();
  for (int j = (int)matched.size(); j < nblocks; ++j) {
    const int b = bm->take_gpu();
    s.blocks.push_back(b);
    if (use_cache && j < nfull) {
      bm->remember(b, keys[j], parent, tokens + (size_t)j * P);
      parent = b;
    }
  }
  for (int t = 0; t < num_tokens; ++t) slots_out[t] = (int64_t)s.blocks[t / P] * P + t % P;
  s.num_tokens = num_tokens;
  s.has_tokens = use_cache;
  if (use_cache) {
    s.partial.assign(tokens + (size_t)nfull * P, tokens + num_tokens);
    s.last_key = nfull > 0 ? keys[nfull - 1] : kChainSeed;
    s.last_full = nfull > 0 ? s.blocks[nfull - 1] : -1;
  }
  if (num_cached_tokens) *num_cached_tokens = (int)matched.size() * P;
  bm->seqs.emplace(seq_id, std::move(s));
  return PKV_OK;
}

int pkv_bm_append(pkv_block_manager* bm, int64_t seq_id, const int32_t* tokens, int n, int64_t* slots_out,
                  int64_t* cow_pairs, int cow_cap, int* num_cow) {
  if (!bm) return PKV_ERR_NULL;
  if (n < 0 || cow_cap < 0) return PKV_ERR_SHAPE;
  if (n > 0 && !slots_out) return PKV_ERR_NULL;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end() || !it->second.on_gpu) return PKV_ERR_SEQ;
  Seq& s = it->second;
  const int P = bm->P;
  const bool cow = n > 0 && s.num_tokens % P != 0 && bm->ref[s.blocks.back()] > 1;
  const int grow = (s.num_tokens + n + P - 1) / P - (s.num_tokens + P - 1) / P;
  if (cow && (cow_cap < 1 || !cow_pairs)) return PKV_ERR_CAPACITY;
  if (grow + (cow ? 1 : 0) > bm->available_gpu()) return PKV_ERR_NO_BLOCKS;

  int ncow = 0;
  if (cow) {
    const int old = s.blocks.back();
    const int fresh = bm->take_gpu();
    bm->decref(old);
    s.blocks.back() = fresh;
    cow_pairs[0] = old;
    cow_pairs[1] = fresh;
    ncow = 1;
  }
  const bool track = s.has_tokens && tokens != nullptr && bm->caching;
  if (!track) {
    s.has_tokens = false;
    s.partial.clear();
  }
  for (int i = 0; i < n; ++i) {
    if (s.num_tokens % P == 0) s.blocks.push_back(bm->take_gpu());
    slots_out[i] = (int64_t)s.blocks.back() * P + s.num_tokens % P;
    ++s.num_tokens;
    if (track) {
      s.partial.push_back(tokens[i]);
      if ((int)s.partial.size() == P) {   // the block is full: make it known
        const uint64_t key = chain_key(s.last_key, s.partial.data(), P);
        bm->remember(s.blocks.back(), key, s.last_full, s.partial.data());
        s.last_key = key;
        s.last_full = s.blocks.back();
        s.partial.clear();
      }
    }
  }
  if (num_cow) *num_cow = ncow;
  return PKV_OK;
}

int pkv_bm_append_batch(pkv_block_manager* bm, const int64_t* seq_ids, int n, const int32_t* tokens,
                        int64_t* slots_out, int64_t* cow_pairs, int cow_cap, int* num_cow) {
  if (!bm) return PKV_ERR_NULL;
  if (n < 0 || cow_cap < 0) return PKV_ERR_SHAPE;
  if (n == 0) {
    if (num_cow) *num_cow = 0;
    return PKV_OK;
  }
  if (!seq_ids || !slots_out) return PKV_ERR_NULL;
  // Check the whole step first: ids, blocks (copies counted as the holders drop in order), room.
  const int P = bm->P;
  std::unordered_map<int64_t, int> seen;
  std::unordered_map<int, int> dropped;   // holders a block loses to earlier copies in this step
  int need = 0, copies = 0;
  std::vector<Seq*> seq(n);
  for (int i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end() || !it->second.on_gpu || !seen.emplace(seq_ids[i], i).second) return PKV_ERR_SEQ;
    Seq& s = it->second;
    seq[i] = &s;
    if (s.num_tokens % P == 0) {
      ++need;
    } else {
      const int last = s.blocks.back();
      int& d = dropped[last];
      if (bm->ref[last] - d > 1) {
        ++need;
        ++copies;
        ++d;
      }
    }
  }
  if (copies > cow_cap || (copies > 0 && !cow_pairs)) return PKV_ERR_CAPACITY;
  if (need > bm->available_gpu()) return PKV_ERR_NO_BLOCKS;
  int ncow = 0;
  for (int i = 0; i < n; ++i) {
    int c = 0;
    const int st = pkv_bm_append(bm, seq_ids[i], tokens ? tokens + i : nullptr, 1, slots_out + i,
                                 cow_pairs ? cow_pairs + 2 * ncow : nullptr, cow_cap - ncow, &c);
    if (st != PKV_OK) return st;   // cannot happen after the checks above
    ncow += c;
  }
  if (num_cow) *num_cow = ncow;
  return PKV_OK;
}

int pkv_bm_append_step(pkv_block_manager* bm, const int64_t* seq_ids, int n, const int32_t* tokens,
                       int64_t* slots_out, int32_t* cow_src_out) {
  if (!bm) return PKV_ERR_NULL;
  if (n < 0) return PKV_ERR_SHAPE;
  if (n > 0 && !cow_src_out) return PKV_ERR_NULL;
  // At most one copy per sequence; the batch call checks everything before changing anything.
  std::vector<int64_t> pairs(2 * (size_t)std::max(n, 1));
  int ncow = 0;
  const int st = pkv_bm_append_batch(bm, seq_ids, n, tokens, slots_out, pairs.data(), n, &ncow);
  if (st != PKV_OK) return st;
  // Each pair's fresh block holds the new token of exactly one sequence of the step.
  std::unordered_map<int64_t, int64_t> src_of;   // fresh block -> its source
  for (int k = 0; k < ncow; ++k) src_of[pairs[2 * k + 1]] = pairs[2 * k];
  for (int i = 0; i < n; ++i) {
    const auto it = src_of.find(slots_out[i] / bm->P);
    cow_src_out[i] = it == src_of.end() ? -1 : (int32_t)it->second;
  }
  return PKV_OK;
}

int pkv_bm_fork(pkv_block_manager* bm, int64_t parent_id, int64_t child_id) {
  if (!bm) return PKV_ERR_NULL;
  auto it = bm->seqs.find(parent_id);
  if (it == bm->seqs.end() || !it->second.on_gpu || bm->seqs.count(child_id)) return PKV_ERR_SEQ;
  Seq child = it->second;
  for (int b : child.blocks) bm->hold(b);
  bm->seqs.emplace(child_id, std::move(child));
  return PKV_OK;
}

int pkv_bm_free(pkv_block_manager* bm, int64_t seq_id) {
  if (!bm) return PKV_ERR_NULL;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PKV_ERR_SEQ;
  if (it->second.on_gpu) {
    for (int b : it->second.blocks) bm->decref(b);
  } else {
    for (int b : it->second.blocks) bm->free_host.push_back(b);
  }
  bm->seqs.erase(it);
  return PKV_OK;
}

int pkv_bm_block_tables(pkv_block_manager* bm, const int64_t* seq_ids, int n, int32_t* tables, int max_blocks,
                        int32_t pad_block, int32_t* context_lens) {
  if (!bm) return PKV_ERR_NULL;
  if (n < 0 || max_blocks < 0) return PKV_ERR_SHAPE;
  if (n == 0) return PKV_OK;
  if (!seq_ids || !tables) return PKV_ERR_NULL;
  for (int i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end() || !it->second.on_gpu) return PKV_ERR_SEQ;
    if ((int)it->second.blocks.size() > max_blocks) return PKV_ERR_CAPACITY;
  }
  for (int i = 0; i < n; ++i) {
    const Seq& s = bm->seqs.find(seq_ids[i])->second;
    int32_t* row = tables + (size_t)i * max_blocks;
    const int nb = (int)s.blocks.size();
    for (int j = 0; j < nb; ++j) row[j] = s.blocks[j];
    for (int j = nb; j < max_blocks; ++j) row[j] = pad_block;
    if (context_lens) context_lens[i] = s.num_tokens;
  }
  return PKV_OK;
}

int pkv_bm_swap_out(pkv_block_manager* bm, int64_t seq_id, int64_t* pairs, int cap, int* num_pairs) {
  if (!bm) return PKV_ERR_NULL;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end() || !it->second.on_gpu) return PKV_ERR_SEQ;
  Seq& s = it->second;
  const int nb = (int)s.blocks.size();
  if (nb > cap || (nb > 0 && !pairs)) return PKV_ERR_CAPACITY;
  if (nb > (int)bm->free_host.size()) return PKV_ERR_NO_BLOCKS;
  std::vector<int> host(nb);
  for (int j = 0; j < nb; ++j) {
    host[j] = bm->free_host.front();
    bm->free_host.pop_front();
    pairs[2 * j] = s.blocks[j];
    pairs[2 * j + 1] = host[j];
  }
  for (int b : s.blocks) bm->decref(b);
  s.blocks = std::move(host);
  s.on_gpu = false;
  s.last_full = -1;   // the GPU copies of its full blocks are no longer its own
  if (num_pairs) *num_pairs = nb;
  return PKV_OK;
}

int pkv_bm_swap_in(pkv_block_manager* bm, int64_t seq_id, int64_t* pairs, int cap, int* num_pairs) {
  if (!bm) return PKV_ERR_NULL;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end() || it->second.on_gpu) return PKV_ERR_SEQ;
  Seq& s = it->second;
  const int nb = (int)s.blocks.size();
  if (nb > cap || (nb > 0 && !pairs)) return PKV_ERR_CAPACITY;
  if (nb > bm->available_gpu()) return PKV_ERR_NO_BLOCKS;
  std::vector<int> gpu(nb);
  for (int j = 0; j < nb; ++j) {
    gpu[j] = bm->take_gpu();
    pairs[2 * j] = s.blocks[j];
    pairs[2 * j + 1] = gpu[j];
  }
  for (int b : s.blocks) bm->free_host.push_back(b);
  s.blocks = std::move(gpu);
  s.on_gpu = true;
  if (num_pairs) *num_pairs = nb;
  return PKV_OK;
}

int pkv_bm_num_free(const pkv_block_manager* bm, int* gpu_free, int* gpu_cached, int* host_free) {
  if (!bm) return PKV_ERR_NULL;
  if (gpu_free) *gpu_free = (int)bm->free_gpu.size();
  if (gpu_cached) *gpu_cached = (int)bm->lru.size();
  if (host_free) *host_free = (int)bm->free_host.size();
  return PKV_OK;
}

int pkv_bm_refcount(const pkv_block_manager* bm, int block, int* count) {
  if (!bm || !count) return PKV_ERR_NULL;
  if (block < 0 || block >= bm->nb_gpu) return PKV_ERR_SHAPE;
  *count = bm->ref[block];
  return PKV_OK;
}

int pkv_bm_sequence_info(const pkv_block_manager* bm, int64_t seq_id, int* num_tokens, int* num_blocks,
                         int* on_gpu) {
  if (!bm) return PKV_ERR_NULL;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PKV_ERR_SEQ;
  if (num_tokens) *num_tokens = it->second.num_tokens;
  if (num_blocks) *num_blocks = (int)it->second.blocks.size();
  if (on_gpu) *on_gpu = it->second.on_gpu ? 1 : 0;
  return PKV_OK;
}

}  // extern "C"
