// Host block allocator of libpa: block tables, LIFO free list, per-block
// reference counts, fork and copy-on-write.
//
// Page "vLLM PagedAttention chuyên sâu: Phân mảnh bộ nhớ KV Cache, Prefill
// theo khối & Prefix Caching" (locionic.com), section "Tương tự phân trang bộ
// nhớ ảo": logical blocks of a fixed token count map to physical blocks
// through a per-sequence block table; physical blocks may be scattered and
// shared; growth maps new blocks without moving old ones.  Section "Cơ chế
// APC", item 3: a sequence leaving a shared prefix copies the shared block it
// writes into.  The exact policies are spelled out in include/pa.h.
//
// Automatic prefix caching (same page, section "Cơ chế APC", items 1-2, and
// its eviction advice for memory pressure): full blocks whose token ids are
// known are entered in a trie keyed by block contents, so that a new request
// whose prompt starts with the same tokens links those physical blocks into
// its table instead of recomputing them.  Cached blocks that no sequence holds
// are kept, and evicted least recently used first when the free list runs
// dry.  The policies are spelled out in include/pa.h.
//
// The allocator runs on the scheduler's thread; it owns host memory only.
// Every entry point validates first and mutates only once success is certain.

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <map>
#include <new>
#include <set>
#include <tuple>
#include <unordered_map>
#include <vector>

#include "../../include/pa.h"

namespace {

struct Seq {
  std::vector<int32_t> table;   // logical block -> physical block
  int32_t len = 0;              // tokens held
  bool known = true;            // token ids of [0, len) recorded in `tokens`
  std::vector<int32_t> tokens;  // (prefix caching only)
  int64_t trie_node = 0;        // trie node of the full blocks' tokens; -1: none
};

// One full block's worth of tokens under its parent in the prefix trie.
struct Node {
  int64_t parent = -1;
  int32_t depth = 0;  // logical block index + 1
  int32_t block = -1;
  std::map<std::vector<int32_t>, int64_t> children;
};

}  // namespace

struct pa_allocator {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<int32_t> free_stack;  // back() is handed out next
  std::vector<int32_t> refcount;
  std::unordered_map<int64_t, Seq> seqs;

  // prefix cache
  bool apc = false;
  int64_t tick = 0;
  int64_t next_node = 1;
  std::unordered_map<int64_t, Node> nodes;  // node 0 is the root
  std::vector<int64_t> block_node;          // 0: block not cached
  std::vector<int64_t> stamp;               // last use of a cached block
  // cached blocks no sequence holds, in eviction order: oldest first, deeper
  // first among equals, then by block id
  std::set<std::tuple<int64_t, int32_t, int32_t>> evictable;
  int64_t hit_tokens = 0, query_tokens = 0, evictions = 0;

  static int32_t ceil_div(int64_t a, int64_t b) { return static_cast<int32_t>((a + b - 1) / b); }

  int64_t available() const {
    return static_cast<int64_t>(free_stack.size()) + static_cast<int64_t>(evictable.size());
  }

  std::tuple<int64_t, int32_t, int32_t> evict_key(int32_t b) const {
    return std::make_tuple(stamp[b], -nodes.at(block_node[b]).depth, b);
  }

  // Drop node `id` and everything under it from the trie.  Blocks of dropped
  // nodes become ordinary blocks; those no sequence holds go to the free
  // list, in depth-first order (children by token order), except `keep`.
  void drop_subtree(int64_t id, int32_t keep) {
    std::vector<int64_t> order;
    std::vector<int64_t> todo{id};
    while (!todo.empty()) {
      int64_t x = todo.back();
      todo.pop_back();
      order.push_back(x);
      const Node& n = nodes.at(x);
      for (auto it = n.children.rbegin(); it != n.children.rend(); ++it) todo.push_back(it->second);
    }
    Node& top = nodes.at(id);
    if (top.parent >= 0) {
      Node& par = nodes.at(top.parent);
      for (auto it = par.children.begin(); it != par.children.end(); ++it)
        if (it->second == id) {
          par.children.erase(it);
          break;
        }
    }
    for (int64_t x : order) {
      const int32_t b = nodes.at(x).block;
      if (refcount[b] == 0) {
        evictable.erase(evict_key(b));
        if (b != keep) free_stack.push_back(b);
      }
      block_node[b] = 0;
    }
    for (int64_t x : order) nodes.erase(x);
  }

  // Caller has checked available() > 0.
  int32_t take() {
    if (!free_stack.empty()) return pop();
    const int32_t b = std::get<2>(*evictable.begin());
    drop_subtree(block_node[b], b);
    ++evictions;
    return b;
  }

  // A block no sequence holds any more: kept in the cache, or freed.
  void release(int32_t b) {
    if (apc && block_node[b] != 0) {
      stamp[b] = tick;
      evictable.insert(evict_key(b));
    } else {
      free_stack.push_back(b);
    }
  }

  // Enter the full blocks [from, to) of `s` (token ids known) in the trie.
  void register_blocks(Seq& s, int32_t from, int32_t to) {
    const int32_t bs = block_size;
    for (int32_t i = from; i < to; ++i) {
      if (s.trie_node < 0 || nodes.find(s.trie_node) == nodes.end()) {
        s.trie_node = -1;
        return;
      }
      std::vector<int32_t> key(s.tokens.begin() + static_cast<int64_t>(i) * bs,
                               s.tokens.begin() + static_cast<int64_t>(i + 1) * bs);
      Node& par = nodes.at(s.trie_node);
      auto it = par.children.find(key);
      if (it != par.children.end()) {  // same tokens already cached in another block
        s.trie_node = it->second;
        continue;
      }
      const int64_t id = next_node++;
      Node n;
      n.parent = s.trie_node;
      n.depth = i + 1;
      n.block = s.table[i];
      par.children.emplace(std::move(key), id);
      nodes.emplace(id, std::move(n));
      block_node[s.table[i]] = id;
      stamp[s.table[i]] = tick;
      s.trie_node = id;
    }
  }

  // Number of blocks an append of n tokens pops, and whether it copies first.
  void plan_append(const Seq& s, int32_t n, bool* cow, int64_t* grow) const {
    *cow = (s.len % block_size != 0) && refcount[s.table.back()] > 1;
    *grow = static_cast<int64_t>(ceil_div(static_cast<int64_t>(s.len) + n, block_size)) -
            static_cast<int64_t>(s.table.size());
  }

  int pop() {
    int32_t b = free_stack.back();
    free_stack.pop_back();
    return b;
  }

  int append(int64_t seq, int32_t n, int64_t* slots, int32_t* cow_pair, int32_t* n_cow,
             const int32_t* tokens = nullptr) {
    if (n_cow) *n_cow = 0;
    auto it = seqs.find(seq);
    if (it == seqs.end()) return PA_ERR_UNKNOWN_SEQ;
    if (n < 0 || (n > 0 && slots == nullptr)) return PA_ERR_INVALID_ARG;
    if (n == 0) return PA_OK;
    Seq& s = it->second;
    if (static_cast<int64_t>(s.len) + n > INT32_MAX) return PA_ERR_INVALID_ARG;
    bool cow;
    int64_t grow;
    plan_append(s, n, &cow, &grow);
    if (grow + (cow ? 1 : 0) > available()) return PA_ERR_NO_FREE_BLOCKS;
    ++tick;
    if (cow) {
      int32_t src = s.table.back();
      int32_t dst = take();
      refcount[src] -= 1;
      refcount[dst] = 1;
      s.table.back() = dst;
      if (cow_pair) {
        cow_pair[0] = src;
        cow_pair[1] = dst;
      }
      if (n_cow) *n_cow = 1;
    }
    for (int64_t k = 0; k < grow; ++k) {
      int32_t b = take();
      refcount[b] = 1;
      s.table.push_back(b);
    }
    const int64_t bs = block_size;
    for (int32_t i = 0; i < n; ++i) {
      int64_t p = static_cast<int64_t>(s.len) + i;
      slots[i] = static_cast<int64_t>(s.table[p / bs]) * bs + p % bs;
    }
    const int32_t old_len = s.len;
    s.len += n;
    if (apc) {
      if (tokens && s.known) {
        s.tokens.insert(s.tokens.end(), tokens, tokens + n);
        register_blocks(s, old_len / block_size, s.len / block_size);
      } else {
        s.known = false;
        s.tokens.clear();
        s.trie_node = -1;
      }
    }
    return PA_OK;
  }

  int new_cached(int64_t seq, const int32_t* tokens, int32_t n, int32_t* n_cached) {
    if (seqs.count(seq)) return PA_ERR_SEQ_EXISTS;
    ++tick;
    Seq s;
    int64_t node = 0;
    const int32_t bs = block_size;
    const int32_t max_blocks = n > 0 ? (n - 1) / bs : 0;  // leave the last token to compute
    for (int32_t i = 0; i < max_blocks; ++i) {
      std::vector<int32_t> key(tokens + static_cast<int64_t>(i) * bs,
                               tokens + static_cast<int64_t>(i + 1) * bs);
      const Node& cur = nodes.at(node);
      auto it = cur.children.find(key);
      if (it == cur.children.end()) break;
      node = it->second;
      const int32_t b = nodes.at(node).block;
      if (refcount[b] == 0) evictable.erase(evict_key(b));
      refcount[b] += 1;
      stamp[b] = tick;
      s.table.push_back(b);
    }
    s.len = static_cast<int32_t>(s.table.size()) * bs;
    s.tokens.assign(tokens, tokens + s.len);
    s.trie_node = node;
    hit_tokens += s.len;
    query_tokens += n;
    if (n_cached) *n_cached = s.len;
    seqs.emplace(seq, std::move(s));
    return PA_OK;
  }

  int export_rows(const int64_t* ids, int32_t count, int32_t* tables, int32_t width,
                  int32_t* lens) const {
    for (int32_t i = 0; i < count; ++i) {
      auto it = seqs.find(ids[i]);
      if (it == seqs.end()) return PA_ERR_UNKNOWN_SEQ;
      if (tables && static_cast<int64_t>(it->second.table.size()) > width) return PA_ERR_INVALID_ARG;
    }
    for (int32_t i = 0; i < count; ++i) {
      const Seq& s = seqs.find(ids[i])->second;
      if (tables) {
        int32_t* row = tables + static_cast<int64_t>(i) * width;
        std::copy(s.table.begin(), s.table.end(), row);
        std::fill(row + s.table.size(), row + width, -1);
      }
      if (lens) lens[i] = s.len;
    }
    return PA_OK;
  }
};

extern "C" {

int pa_alloc_enable_prefix_cache(pa_allocator* a) {
  if (a == nullptr || !a->seqs.empty()) return PA_ERR_INVALID_ARG;
  if (a->apc) return PA_OK;
  a->apc = true;
  a->nodes.clear();
  a->nodes.emplace(0, Node());
  a->block_node.assign(a->num_blocks, 0);
  a->stamp.assign(a->num_blocks, 0);
  return PA_OK;
}

int pa_seq_new_cached(pa_allocator* a, int64_t seq, const int32_t* tokens, int32_t n,
                      int32_t* n_cached_out) {
  if (a == nullptr || !a->apc || n < 0 || (n > 0 && tokens == nullptr)) return PA_ERR_INVALID_ARG;
  return a->new_cached(seq, tokens, n, n_cached_out);
}

int pa_seq_append_tokens(pa_allocator* a, int64_t seq, const int32_t* tokens, int32_t n,
                         int64_t* slots_out, int32_t* cow_pair_out, int32_t* n_cow_out) {
  if (a == nullptr || (n > 0 && tokens == nullptr)) return PA_ERR_INVALID_ARG;
  return a->append(seq, n, slots_out, cow_pair_out, n_cow_out, tokens);
}

int pa_prefix_cache_stats(const pa_allocator* a, int64_t out[5]) {
  if (a == nullptr || out == nullptr) return PA_ERR_INVALID_ARG;
  out[0] = a->hit_tokens;
  out[1] = a->query_tokens;
  out[2] = a->apc ? static_cast<int64_t>(a->nodes.size()) - 1 : 0;
  out[3] = static_cast<int64_t>(a->evictable.size());
  out[4] = a->evictions;
  return PA_OK;
}

int pa_prefix_cache_blocks(const pa_allocator* a, int32_t* blocks_out, int32_t* depths_out,
                           int32_t* evictable_out, int32_t cap, int32_t* n_out) {
  if (a == nullptr || n_out == nullptr || cap < 0 ||
      (cap > 0 && (blocks_out == nullptr || depths_out == nullptr)))
    return PA_ERR_INVALID_ARG;
  int32_t n = 0;
  if (a->apc) {
    for (int32_t b = 0; b < a->num_blocks; ++b) {
      if (a->block_node[b] == 0) continue;
      if (n < cap) {
        blocks_out[n] = b;
        depths_out[n] = a->nodes.at(a->block_node[b]).depth;
      }
      ++n;
    }
  }
  *n_out = n;
  if (evictable_out) {
    int32_t i = 0;
    for (const auto& k : a->evictable) {
      if (i >= cap) break;
      evictable_out[i++] = std::get<2>(k);
    }
  }
  return PA_OK;
}

int pa_alloc_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                    pa_allocator** out) {
  if (out == nullptr || num_blocks <= 0 || block_size <= 0) return PA_ERR_INVALID_ARG;
  *out = nullptr;
  std::vector<int32_t> order(num_blocks);
  if (free_order) {
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      int32_t b = free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) return PA_ERR_INVALID_ARG;
      seen[b] = 1;
      order[i] = b;
    }
  } else {
    for (int32_t i = 0; i < num_blocks; ++i) order[i] = i;
  }
  pa_allocator* a = new (std::nothrow) pa_allocator();
  if (a == nullptr) return PA_ERR_INVALID_ARG;
  a->num_blocks = num_blocks;
  a->block_size = block_size;
  a->free_stack.assign(order.rbegin(), order.rend());
  a->refcount.assign(num_blocks, 0);
  *out = a;
  return PA_OK;
}

void pa_alloc_destroy(pa_allocator* a) { delete a; }

int pa_seq_new(pa_allocator* a, int64_t seq) {
  if (a == nullptr) return PA_ERR_INVALID_ARG;
  if (a->seqs.count(seq)) return PA_ERR_SEQ_EXISTS;
  a->seqs.emplace(seq, Seq());
  return PA_OK;
}

int pa_seq_fork(pa_allocator* a, int64_t parent, int64_t child) {
  if (a == nullptr) return PA_ERR_INVALID_ARG;
  auto it = a->seqs.find(parent);
  if (it == a->seqs.end()) return PA_ERR_UNKNOWN_SEQ;
  if (a->seqs.count(child)) return PA_ERR_SEQ_EXISTS;
  Seq c = it->second;
  for (int32_t b : c.table) a->refcount[b] += 1;
  a->seqs.emplace(child, std::move(c));
  return PA_OK;
}

int pa_seq_append(pa_allocator* a, int64_t seq, int32_t n, int64_t* slots_out,
                  int32_t* cow_pair_out, int32_t* n_cow_out) {
  if (a == nullptr) return PA_ERR_INVALID_ARG;
  return a->append(seq, n, slots_out, cow_pair_out, n_cow_out);
}

int pa_seq_free(pa_allocator* a, int64_t seq) {
  if (a == nullptr) return PA_ERR_INVALID_ARG;
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) return PA_ERR_UNKNOWN_SEQ;
  const std::vector<int32_t>& t = it->second.table;
  ++a->tick;
  for (auto b = t.rbegin(); b != t.rend(); ++b) {
    if (--a->refcount[*b] == 0) a->release(*b);
  }
  a->seqs.erase(it);
  return PA_OK;
}

int pa_seq_len(const pa_allocator* a, int64_t seq, int32_t* len_out) {
  if (a == nullptr || len_out == nullptr) return PA_ERR_INVALID_ARG;
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) return PA_ERR_UNKNOWN_SEQ;
  *len_out = it->second.len;
  return PA_OK;
}

int pa_seq_block_table(const pa_allocator* a, int64_t seq, int32_t* out, int32_t cap,
                       int32_t* n_out) {
  if (a == nullptr || n_out == nullptr || cap < 0 || (cap > 0 && out == nullptr))
    return PA_ERR_INVALID_ARG;
  auto it = a->seqs.find(seq);
  if (it == a->seqs.end()) return PA_ERR_UNKNOWN_SEQ;
  const std::vector<int32_t>& t = it->second.table;
  int32_t n = static_cast<int32_t>(t.size());
  std::copy(t.begin(), t.begin() + std::min(n, cap), out);
  *n_out = n;
  return PA_OK;
}

int pa_block_refcount(const pa_allocator* a, int32_t block, int32_t* rc_out) {
  if (a == nullptr || rc_out == nullptr || block < 0 || block >= a->num_blocks)
    return PA_ERR_INVALID_ARG;
  *rc_out = a->refcount[block];
  return PA_OK;
}

int pa_num_free(const pa_allocator* a, int32_t* n_out) {
  if (a == nullptr || n_out == nullptr) return PA_ERR_INVALID_ARG;
  *n_out = static_cast<int32_t>(a->free_stack.size());
  return PA_OK;
}

int pa_free_list(const pa_allocator* a, int32_t* out, int32_t cap, int32_t* n_out) {
  if (a == nullptr || n_out == nullptr || cap < 0 || (cap > 0 && out == nullptr))
    return PA_ERR_INVALID_ARG;
  int32_t n = static_cast<int32_t>(a->free_stack.size());
  std::copy(a->free_stack.begin(), a->free_stack.begin() + std::min(n, cap), out);
  *n_out = n;
  return PA_OK;
}

int pa_batch_append(pa_allocator* a, const int64_t* seqs, int32_t num_seqs, const int32_t* n,
                    int64_t* slots_out, int32_t* cow_pairs_out, int32_t* n_cow_out,
                    int32_t* block_tables_out, int32_t max_blocks_per_seq,
                    int32_t* context_lens_out, int32_t* n_done_out) {
  if (n_done_out) *n_done_out = 0;
  if (n_cow_out) *n_cow_out = 0;
  if (a == nullptr || num_seqs < 0 || (num_seqs > 0 && (seqs == nullptr || n == nullptr)))
    return PA_ERR_INVALID_ARG;
  if (block_tables_out && max_blocks_per_seq <= 0) return PA_ERR_INVALID_ARG;
  int64_t total = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    if (n[i] < 0) return PA_ERR_INVALID_ARG;
    total += n[i];
  }
  if (total > 0 && slots_out == nullptr) return PA_ERR_INVALID_ARG;
  int64_t off = 0;
  int32_t ncow = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    int32_t pair[2];
    int32_t c = 0;
    int rc = a->append(seqs[i], n[i], slots_out ? slots_out + off : nullptr, pair, &c);
    if (rc != PA_OK) return rc;
    if (c) {
      if (cow_pairs_out) {
        cow_pairs_out[2 * ncow] = pair[0];
        cow_pairs_out[2 * ncow + 1] = pair[1];
      }
      ++ncow;
      if (n_cow_out) *n_cow_out = ncow;
    }
    off += n[i];
    if (n_done_out) *n_done_out = i + 1;
  }
  if (block_tables_out || context_lens_out)
    return a->export_rows(seqs, num_seqs, block_tables_out, max_blocks_per_seq, context_lens_out);
  return PA_OK;
}

int pa_export_tables(const pa_allocator* a, const int64_t* seqs, int32_t num_seqs,
                     int32_t* block_tables_out, int32_t max_blocks_per_seq,
                     int32_t* context_lens_out) {
  if (a == nullptr || num_seqs < 0 || (num_seqs > 0 && seqs == nullptr)) return PA_ERR_INVALID_ARG;
  if (block_tables_out && max_blocks_per_seq <= 0) return PA_ERR_INVALID_ARG;
  return a->export_rows(seqs, num_seqs, block_tables_out, max_blocks_per_seq, context_lens_out);
}

int pa_alloc_stats(const pa_allocator* a, int64_t out[5]) {
  if (a == nullptr || out == nullptr) return PA_ERR_INVALID_ARG;
  int64_t shared = 0, wasted = 0;
  for (int32_t rc : a->refcount) shared += rc > 1;
  for (const auto& kv : a->seqs)
    wasted += static_cast<int64_t>(kv.second.table.size()) * a->block_size - kv.second.len;
  out[0] = static_cast<int64_t>(a->free_stack.size());
  out[1] = a->num_blocks - out[0];
  out[2] = shared;
  out[3] = static_cast<int64_t>(a->seqs.size());
  out[4] = wasted;
  return PA_OK;
}

const char* pa_status_str(int status) {
  switch (status) {
    case PA_OK: return "PA_OK";
    case PA_ERR_INVALID_ARG: return "PA_ERR_INVALID_ARG";
    case PA_ERR_NO_FREE_BLOCKS: return "PA_ERR_NO_FREE_BLOCKS";
    case PA_ERR_UNKNOWN_SEQ: return "PA_ERR_UNKNOWN_SEQ";
    case PA_ERR_SEQ_EXISTS: return "PA_ERR_SEQ_EXISTS";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE";
    case PA_ERR_DEVICE: return "PA_ERR_DEVICE";
    default: return "PA_ERR_UNKNOWN_STATUS";
  }
}

int pa_version(void) { return 3; }

}  // extern "C"
