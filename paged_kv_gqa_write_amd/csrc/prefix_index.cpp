// Host-side prefix-block index: which physical KV blocks already hold the
// leading full blocks of a token sequence ("Qwen3-4B / 8B / 32B", intro and
// Architecture Notes: prefix caching on by default, prefix matching against
// the GPU KV cache; section Warm Prefix-Cache TTFT: a repeated prompt lands
// as a warm hit).  The result feeds pa_prefill's prefix_lens (matched blocks
// x 16) and the sequence's block-table row.
//
// Structure: a trie of sealed (full, 16-token) blocks.  A node is keyed by
// (parent node, its 16 token ids), so a block is found only under its whole
// prefix and two prefixes never share a node.  Keys are compared in full --
// the hash only picks the bucket -- so a hash collision can cost a probe but
// never returns another prefix's blocks.  Nodes live in one vector with a
// free list; children lists make removing a block's subtree linear in its
// size.
#include <stdint.h>

#include <algorithm>
#include <array>
#include <new>
#include <unordered_map>
#include <vector>

#include "pa.h"

namespace {

constexpr int kBlockTokens = 16;

struct Key {
  int64_t parent;  // node index, -1 at the root
  std::array<int32_t, kBlockTokens> tokens;
  bool operator==(const Key& o) const { return parent == o.parent && tokens == o.tokens; }
};

// 64-bit multiply-xorshift mixing of the 17 words (the final avalanche is
// the fmix64 step of MurmurHash3).
struct KeyHash {
  size_t operator()(const Key& k) const {
    uint64_t h = 0x9E3779B97F4A7C15ull ^ static_cast<uint64_t>(k.parent);
    for (int32_t t : k.tokens) {
      h ^= static_cast<uint32_t>(t);
      h *= 0x100000001B3ull;
      h ^= h >> 29;
    }
    h ^= h >> 33;
    h *= 0xFF51AFD7ED558CCDull;
    h ^= h >> 33;
    h *= 0xC4CEB9FE1A85EC53ull;
    h ^= h >> 33;
    return static_cast<size_t>(h);
  }
};

struct Node {
  Key key;
  int32_t block;
  bool live;
  std::vector<int64_t> children;
};

Key key_of(int64_t parent, const int32_t* tokens) {
  Key k;
  k.parent = parent;
  std::copy(tokens, tokens + kBlockTokens, k.tokens.begin());
  return k;
}

}  // namespace

struct pa_prefix_index {
  int64_t capacity = 0;
  int64_t count = 0;
  std::vector<Node> nodes;
  std::vector<int64_t> free_nodes;
  std::unordered_map<Key, int64_t, KeyHash> by_key;
  std::unordered_map<int32_t, int64_t> by_block;

  int64_t find(int64_t parent, const int32_t* tokens) const {
    auto it = by_key.find(key_of(parent, tokens));
    return it == by_key.end() ? -1 : it->second;
  }

  // Drops the node holding `block` and its whole subtree; returns how many.
  int64_t remove_block(int32_t block) {
    auto it = by_block.find(block);
    if (it == by_block.end()) return 0;
    const int64_t root = it->second;
    const int64_t parent = nodes[root].key.parent;
    if (parent >= 0) {
      auto& ch = nodes[parent].children;
      ch.erase(std::find(ch.begin(), ch.end(), root));
    }
    int64_t removed = 0;
    std::vector<int64_t> stack{root};
    while (!stack.empty()) {
      const int64_t n = stack.back();
      stack.pop_back();
      Node& nd = nodes[n];
      for (int64_t c : nd.children) stack.push_back(c);
      by_key.erase(nd.key);
      by_block.erase(nd.block);
      nd.children.clear();
      nd.live = false;
      free_nodes.push_back(n);
      ++removed;
    }
    count -= removed;
    return removed;
  }

  int64_t add(int64_t parent, const int32_t* tokens, int32_t block) {
    int64_t n;
    if (!free_nodes.empty()) {
      n = free_nodes.back();
      free_nodes.pop_back();
    } else {
      nodes.emplace_back();
      n = static_cast<int64_t>(nodes.size()) - 1;
    }
    Node& nd = nodes[n];
    nd.key = key_of(parent, tokens);
    nd.block = block;
    nd.live = true;
    by_key.emplace(nd.key, n);
    by_block.emplace(block, n);
    if (parent >= 0) nodes[parent].children.push_back(n);
    ++count;
    return n;
  }
};

extern "C" {

int pa_prefix_index_create(int64_t capacity, pa_prefix_index** out) {
  if (!out || capacity <= 0) return PA_ERR_INVALID_ARG;
  *out = nullptr;
  pa_prefix_index* idx = new (std::nothrow) pa_prefix_index();
  if (!idx) return PA_ERR_NO_MEMORY;
  idx->capacity = capacity;
  *out = idx;
  return PA_OK;
}

void pa_prefix_index_destroy(pa_prefix_index* idx) { delete idx; }

int64_t pa_prefix_index_size(const pa_prefix_index* idx) { return idx ? idx->count : -1; }

int pa_prefix_index_match(const pa_prefix_index* idx, const int32_t* tokens, int32_t num_tokens,
                          int32_t* block_ids, int32_t* num_matched) {
  if (!idx || !num_matched || num_tokens < 0) return PA_ERR_INVALID_ARG;
  const int32_t nfull = num_tokens / kBlockTokens;
  if (nfull > 0 && (!tokens || !block_ids)) return PA_ERR_INVALID_ARG;
  int64_t cur = -1;
  int32_t i = 0;
  for (; i < nfull; ++i) {
    const int64_t n = idx->find(cur, tokens + (int64_t)i * kBlockTokens);
    if (n < 0) break;
    block_ids[i] = idx->nodes[n].block;
    cur = n;
  }
  *num_matched = i;
  return PA_OK;
}

int pa_prefix_index_insert(pa_prefix_index* idx, const int32_t* tokens, int32_t num_tokens,
                           const int32_t* block_ids, int32_t num_block_ids,
                           int32_t* num_inserted) {
  if (!idx || !num_inserted || num_tokens < 0 || num_block_ids < 0) return PA_ERR_INVALID_ARG;
  *num_inserted = 0;
  const int32_t nfull = std::min(num_tokens / kBlockTokens, num_block_ids);
  if (nfull > 0 && (!tokens || !block_ids)) return PA_ERR_INVALID_ARG;
  try {
    // The cached run, then the ids to register (up to the first negative).
    std::vector<int32_t> path;
    int64_t cur = -1;
    int32_t i = 0;
    for (; i < nfull; ++i) {
      const int64_t n = idx->find(cur, tokens + (int64_t)i * kBlockTokens);
      if (n < 0) break;
      path.push_back(idx->nodes[n].block);
      cur = n;
    }
    int32_t end = i;
    while (end < nfull && block_ids[end] >= 0) ++end;
    std::vector<int32_t> fresh(block_ids + i, block_ids + end);
    std::sort(fresh.begin(), fresh.end());
    if (std::adjacent_find(fresh.begin(), fresh.end()) != fresh.end()) return PA_ERR_INVALID_ARG;
    for (int32_t b : path)
      if (std::binary_search(fresh.begin(), fresh.end(), b)) return PA_ERR_INVALID_ARG;
    int32_t added = 0;
    for (int32_t j = i; j < end; ++j) {
      const int32_t b = block_ids[j];
      const bool reused = idx->by_block.count(b) != 0;
      if (idx->count >= idx->capacity && !reused) break;
      idx->remove_block(b);  // the block now holds other tokens
      cur = idx->add(cur, tokens + (int64_t)j * kBlockTokens, b);
      ++added;
    }
    *num_inserted = added;
    return PA_OK;
  } catch (const std::bad_alloc&) {
    return PA_ERR_NO_MEMORY;
  }
}

int pa_prefix_index_remove(pa_prefix_index* idx, int32_t block_id, int32_t* num_removed) {
  if (!idx || !num_removed) return PA_ERR_INVALID_ARG;
  *num_removed = static_cast<int32_t>(idx->remove_block(block_id));
  return PA_OK;
}

}  // extern "C"
