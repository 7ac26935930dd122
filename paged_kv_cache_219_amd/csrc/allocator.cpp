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
// The allocator runs on the scheduler's thread; it owns host memory only.
// Every entry point validates first and mutates only once success is certain.

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <new>
#include <unordered_map>
#include <vector>

#include "../../include/pa.h"

namespace {

struct Seq {
  std::vector<int32_t> table;  // logical block -> physical block
  int32_t len = 0;             // tokens held
};

}  // namespace

struct pa_allocator {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<int32_t> free_stack;  // back() is handed out next
  std::vector<int32_t> refcount;
  std::unordered_map<int64_t, Seq> seqs;

  static int32_t ceil_div(int64_t a, int64_t b) { return static_cast<int32_t>((a + b - 1) / b); }

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

  int append(int64_t seq, int32_t n, int64_t* slots, int32_t* cow_pair, int32_t* n_cow) {
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
    if (grow + (cow ? 1 : 0) > static_cast<int64_t>(free_stack.size())) return PA_ERR_NO_FREE_BLOCKS;
    if (cow) {
      int32_t src = s.table.back();
      int32_t dst = pop();
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
      int32_t b = pop();
      refcount[b] = 1;
      s.table.push_back(b);
    }
    const int64_t bs = block_size;
    for (int32_t i = 0; i < n; ++i) {
      int64_t p = static_cast<int64_t>(s.len) + i;
      slots[i] = static_cast<int64_t>(s.table[p / bs]) * bs + p % bs;
    }
    s.len += n;
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
  for (auto b = t.rbegin(); b != t.rend(); ++b) {
    if (--a->refcount[*b] == 0) a->free_stack.push_back(*b);
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

int pa_version(void) { return 1; }

}  // extern "C"
