// Host prefix index: a radix tree over cached token sequences whose nodes own runs of whole
// KV blocks ("KV Cache Optimization and Management", section "RadixAttention: caching, not just
// packing, the prefix": sequences that share a prefix share its path from the root; a request
// is matched token by token and only the tokens past the divergence need a fresh prefill; the
// least recently used leaves are trimmed first, and reference counting keeps a branch that a
// running request still uses from being evicted).
//
// Every edge is labelled with whole blocks of B tokens (a partially filled block is not shared)
// and holds the physical block and the last-use time of each of them. Children are keyed by the
// tokens of their first block. The index holds one pool reference per cached block; a match
// takes one more per matched block for the caller. Times come from a logical clock that
// advances once per match or insert; every block on the matched or inserted path gets the new
// time, so times never increase towards the leaves and the oldest block of a path is its last.
// Eviction frees one block at a time: the last block of a leaf that only the index references,
// the oldest such (ties: lower block id); a leaf whose edge empties is removed and its parent
// may become a leaf in turn.
#include <algorithm>
#include <map>
#include <memory>
#include <new>
#include <vector>

#include "pagedkv.h"

namespace {

struct Node {
  Node* parent = nullptr;
  std::vector<int32_t> tokens;     // B tokens per block of the edge
  std::vector<int32_t> blocks;     // physical block of each edge block
  std::vector<uint64_t> stamps;    // last use of each edge block
  std::map<std::vector<int32_t>, std::unique_ptr<Node>> children;
};

std::vector<int32_t> first_block(const int32_t* t, int B) { return std::vector<int32_t>(t, t + B); }

bool same_block(const int32_t* a, const int32_t* b, int B) { return std::equal(a, a + B, b); }

}  // namespace

struct pkv_prefix_index {
  pkv_pool* pool = nullptr;
  int B = 0;
  Node root;
  uint64_t clock = 0;
  int64_t cached = 0;
};

namespace {

// Split `child` after its first j blocks: a new node takes those blocks and becomes child's
// parent (same key in the grandparent's map, since its first block is child's old one).
Node* split(pkv_prefix_index* x, Node* child, size_t j) {
  const int B = x->B;
  Node* parent = child->parent;
  auto key = first_block(child->tokens.data(), B);
  std::unique_ptr<Node> mid(new Node);
  mid->parent = parent;
  mid->tokens.assign(child->tokens.begin(), child->tokens.begin() + j * B);
  mid->blocks.assign(child->blocks.begin(), child->blocks.begin() + j);
  mid->stamps.assign(child->stamps.begin(), child->stamps.begin() + j);
  child->tokens.erase(child->tokens.begin(), child->tokens.begin() + j * B);
  child->blocks.erase(child->blocks.begin(), child->blocks.begin() + j);
  child->stamps.erase(child->stamps.begin(), child->stamps.begin() + j);
  std::unique_ptr<Node> owned = std::move(parent->children[key]);
  child->parent = mid.get();
  mid->children[first_block(child->tokens.data(), B)] = std::move(owned);
  Node* m = mid.get();
  parent->children[key] = std::move(mid);
  return m;
}

void release_all(pkv_prefix_index* x, Node* n) {
  for (int32_t b : n->blocks) pkv_pool_decref(x->pool, b, nullptr);
  for (auto& c : n->children) release_all(x, c.second.get());
}

// Oldest evictable block: the last block of a leaf that only the index references.
void find_victim(pkv_prefix_index* x, Node* n, Node*& best) {
  if (n != &x->root && n->children.empty()) {
    const int32_t b = n->blocks.back();
    if (pkv_pool_refcount(x->pool, b) == 1 &&
        (!best || n->stamps.back() < best->stamps.back() ||
         (n->stamps.back() == best->stamps.back() && b < best->blocks.back())))
      best = n;
    return;
  }
  for (auto& c : n->children) find_victim(x, c.second.get(), best);
}

}  // namespace

extern "C" {

pkv_prefix_index* pkv_prefix_index_create(pkv_pool* pool, int block_size) {
  if (!pool || block_size <= 0) return nullptr;
  pkv_prefix_index* x = new (std::nothrow) pkv_prefix_index;
  if (!x) return nullptr;
  x->pool = pool;
  x->B = block_size;
  return x;
}

void pkv_prefix_index_destroy(pkv_prefix_index* index) {
  if (!index) return;
  release_all(index, &index->root);
  delete index;
}

int pkv_prefix_index_match(pkv_prefix_index* index, const int32_t* tokens, int num_tokens,
                           int32_t* out_blocks, int max_blocks, int* matched_blocks) {
  if (!index || (!tokens && num_tokens > 0) || num_tokens < 0 || !matched_blocks ||
      (!out_blocks && max_blocks > 0) || max_blocks < 0)
    return PKV_ERR_INVALID_ARG;
  const int B = index->B;
  const uint64_t now = ++index->clock;
  int found = 0, pos = 0;
  Node* node = &index->root;
  try {
    while (pos + B <= num_tokens && found < max_blocks) {
      auto it = node->children.find(first_block(tokens + pos, B));
      if (it == node->children.end()) break;
      Node* child = it->second.get();
      size_t j = 0;
      while (j < child->blocks.size() && pos + B <= num_tokens && found < max_blocks &&
             same_block(child->tokens.data() + j * B, tokens + pos, B)) {
        child->stamps[j] = now;
        out_blocks[found++] = child->blocks[j];
        pos += B;
        ++j;
      }
      if (j < child->blocks.size()) break;
      node = child;
    }
  } catch (...) {
    return PKV_ERR_INVALID_ARG;
  }
  for (int i = 0; i < found; ++i) pkv_pool_incref(index->pool, out_blocks[i]);
  *matched_blocks = found;
  return PKV_OK;
}

int pkv_prefix_index_insert(pkv_prefix_index* index, const int32_t* tokens, int num_tokens,
                            const int32_t* blocks, int* inserted_blocks) {
  if (!index || num_tokens < 0 || (num_tokens > 0 && (!tokens || !blocks)) || !inserted_blocks)
    return PKV_ERR_INVALID_ARG;
  const int B = index->B;
  const int nb = num_tokens / B;
  for (int j = 0; j < nb; ++j)   // the index may only reference live blocks
    if (pkv_pool_refcount(index->pool, blocks[j]) < 1) return PKV_ERR_REFCOUNT;
  const uint64_t now = ++index->clock;
  int added = 0, pos = 0;
  Node* node = &index->root;
  try {
    while (pos + B <= num_tokens) {
      auto key = first_block(tokens + pos, B);
      auto it = node->children.find(key);
      if (it == node->children.end()) {
        std::unique_ptr<Node> c(new Node);
        c->parent = node;
        c->tokens.assign(tokens + pos, tokens + (size_t)nb * B);
        c->blocks.assign(blocks + pos / B, blocks + nb);
        c->stamps.assign(c->blocks.size(), now);
        for (int32_t b : c->blocks) pkv_pool_incref(index->pool, b);
        added += (int)c->blocks.size();
        node->children[key] = std::move(c);
        break;
      }
      Node* child = it->second.get();
      size_t j = 0;
      while (j < child->blocks.size() && pos + B <= num_tokens &&
             same_block(child->tokens.data() + j * B, tokens + pos, B)) {
        child->stamps[j] = now;
        pos += B;
        ++j;
      }
      if (j == child->blocks.size()) {
        node = child;
      } else if (pos + B > num_tokens) {
        break;   // the sequence ends inside this edge: all of it is cached
      } else {
        node = split(index, child, j);   // diverges inside the edge
      }
    }
  } catch (...) {
    return PKV_ERR_INVALID_ARG;
  }
  index->cached += added;
  *inserted_blocks = added;
  return PKV_OK;
}

int pkv_prefix_index_evict(pkv_prefix_index* index, int max_blocks, int32_t* freed_ids,
                           int* freed_blocks) {
  if (!index || max_blocks < 0 || !freed_blocks) return PKV_ERR_INVALID_ARG;
  const int B = index->B;
  int freed = 0;
  while (freed < max_blocks) {
    Node* leaf = nullptr;
    find_victim(index, &index->root, leaf);
    if (!leaf) break;
    const int32_t b = leaf->blocks.back();
    auto key = first_block(leaf->tokens.data(), B);
    leaf->blocks.pop_back();
    leaf->stamps.pop_back();
    leaf->tokens.resize(leaf->tokens.size() - B);
    pkv_pool_decref(index->pool, b, nullptr);
    if (freed_ids) freed_ids[freed] = b;
    ++freed;
    --index->cached;
    if (leaf->blocks.empty()) leaf->parent->children.erase(key);
  }
  *freed_blocks = freed;
  return PKV_OK;
}

int pkv_prefix_index_size(const pkv_prefix_index* index) {
  return index ? (int)index->cached : PKV_ERR_INVALID_ARG;
}

}  // extern "C"
