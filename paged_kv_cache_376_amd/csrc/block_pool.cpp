// Host block pool and block tables (pure C++, no HIP dependency).
//
// The paging scheme of the 111cn.net page "大模型推理引擎高频优化：连续批处理、PagedAttention
// 与 KV Cache 实战拆解" §3.2-§3.3: a pool of equal physical blocks, a free list that
// allocation pops from the end, one block table per sequence, and a fresh block only when
// the last one is full.  Reference counts per block from the gtnt.cn page "vLLM推理加速框架：
// PagedAttention与连续批处理技术解析" §2.1, copy-on-write of shared blocks from its §2.2, and
// blocks returned to the pool when a request ends from the yunthe.com page "大模型推理显存
// 优化实战：PagedAttention机制原理与vLLM连续批处理配置", section
// "PagedAttention分页注意力机制原理".
//
// Every mutating call first computes how many blocks it needs and fails with
// PKV_ERR_OUT_OF_BLOCKS before touching anything if the free list is too short.  Each also
// makes every host allocation it needs before its first change to the pool, so that a failed
// allocation (PKV_ERR_HOST_MEMORY; no exception crosses the C ABI) leaves the pool unchanged.
#include <algorithm>
#include <cstring>
#include <memory>
#include <new>
#include <stdexcept>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "pkv_internal.h"

struct pkv_block_pool {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<int32_t> free_list;  // next allocation pops back()
  std::vector<int32_t> ref;        // per physical block
  struct Seq {
    std::vector<int32_t> table;    // logical -> physical
    int64_t num_tokens = 0;
  };
  std::unordered_map<int64_t, Seq> seqs;
};

namespace {

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Runs the body of an entry point; a host allocation that fails inside it becomes
// PKV_ERR_HOST_MEMORY.
template <typename F>
pkv_status host_call(F&& body) {
  try {
    return body();
  } catch (const std::bad_alloc&) {
    return pkv::fail(PKV_ERR_HOST_MEMORY, "host allocation failed");
  } catch (const std::length_error&) {
    return pkv::fail(PKV_ERR_HOST_MEMORY, "host allocation too large");
  }
}

// Blocks that appending n tokens to `s` takes from the free list (incl. a CoW copy).
int64_t blocks_needed(const pkv_block_pool* p, const pkv_block_pool::Seq& s, int64_t n) {
  const int64_t bs = p->block_size;
  int64_t need = ceil_div(s.num_tokens + n, bs) - ceil_div(s.num_tokens, bs);
  if (n > 0 && s.num_tokens % bs != 0 && p->ref[s.table.back()] > 1) need += 1;
  return need;
}

}  // namespace

extern "C" pkv_status pkv_pool_create(int32_t num_blocks, int32_t block_size,
                                      const int32_t* free_order, pkv_block_pool** out) {
  pkv::clear_error();
  if (!out) return pkv::fail(PKV_ERR_INVALID_ARGUMENT, "out is NULL");
  *out = nullptr;
  if (num_blocks <= 0) return pkv::fail(PKV_ERR_INVALID_ARGUMENT, "num_blocks=%d", num_blocks);
  if (block_size <= 0) return pkv::fail(PKV_ERR_INVALID_ARGUMENT, "block_size=%d", block_size);
  return host_call([&]() -> pkv_status {
    std::unique_ptr<pkv_block_pool> p(new pkv_block_pool());
    p->num_blocks = num_blocks;
    p->block_size = block_size;
    p->ref.assign(num_blocks, 0);
    p->free_list.resize(num_blocks);  // its capacity never drops below num_blocks: frees do not allocate
    if (free_order) {
      std::vector<char> seen(num_blocks, 0);
      for (int32_t i = 0; i < num_blocks; ++i) {
        int32_t b = free_order[i];
        if (b < 0 || b >= num_blocks || seen[b])
          return pkv::fail(PKV_ERR_INVALID_ARGUMENT,
                           "free_order is not a permutation of 0..%d (entry %d = %d)",
                           num_blocks - 1, i, b);
        seen[b] = 1;
        p->free_list[i] = b;
      }
    } else {
      for (int32_t i = 0; i < num_blocks; ++i) p->free_list[i] = i;
    }
    *out = p.release();
    return PKV_OK;
  });
}

extern "C" void pkv_pool_destroy(pkv_block_pool* pool) { delete pool; }

extern "C" int32_t pkv_pool_num_blocks(const pkv_block_pool* p) { return p ? p->num_blocks : -1; }
extern "C" int32_t pkv_pool_block_size(const pkv_block_pool* p) { return p ? p->block_size : -1; }
extern "C" int32_t pkv_pool_num_free(const pkv_block_pool* p) {
  return p ? static_cast<int32_t>(p->free_list.size()) : -1;
}
extern "C" int32_t pkv_pool_num_seqs(const pkv_block_pool* p) {
  return p ? static_cast<int32_t>(p->seqs.size()) : -1;
}

extern "C" int32_t pkv_pool_ref_count(const pkv_block_pool* p, int32_t block_id) {
  if (!p || block_id < 0 || block_id >= p->num_blocks) return -1;
  return p->ref[block_id];
}

extern "C" int32_t pkv_pool_free_list(const pkv_block_pool* p, int32_t* out, int32_t capacity) {
  if (!p) return -1;
  const int32_t n = static_cast<int32_t>(p->free_list.size());
  if (out && capacity > 0) {
    const int32_t m = capacity < n ? capacity : n;
    std::memcpy(out, p->free_list.data(), sizeof(int32_t) * m);
  }
  return n;
}

extern "C" pkv_status pkv_seq_allocate(pkv_block_pool* p, int64_t seq, int32_t num_tokens,
                                       int32_t* blocks_out) {
  pkv::clear_error();
  if (!p) return pkv::fail(PKV_ERR_INVALID_ARGUMENT, "pool is NULL");
  if (num_tokens < 0) return pkv::fail(PKV_ERR_INVALID_ARGUMENT, "num_tokens=%d", num_tokens);
  if (p->seqs.count(seq)) return pkv::fail(PKV_ERR_ALREADY_EXISTS, "sequence %lld exists", (long long)seq);
  const int64_t need = ceil_div(num_tokens, p->block_size);
  if (need > static_cast<int64_t>(p->free_list.size()))
    return pkv::fail(PKV_ERR_OUT_OF_BLOCKS, "allocate needs %lld blocks, %zu free",
                     (long long)need, p->free_list.size());
  return host_call([&]() -> pkv_status {
    pkv_block_pool::Seq fresh;
    fresh.table.reserve(need);
    pkv_block_pool::Seq& s = p->seqs.emplace(seq, std::move(fresh)).first->second;
    // no allocation from here on
    for (int64_t i = 0; i < need; ++i) {
      const int32_t b = p->free_list.back();
      p->free_list.pop_back();
      p->ref[b] = 1;
      s.table.push_back(b);
      if (blocks_out) blocks_out[i] = b;
    }
    s.num_tokens = num_tokens;
    return PKV_OK;
  });
}

extern "C" pkv_status pkv_seq_extend(pkv_block_pool* p, int64_t seq, int32_t n, int64_t* slots_out,
                                     int32_t* cow_out, int32_t* num_cow_out) {
  pkv::clear_error();
  if (num_cow_out) *num_cow_out = 0;
  if (!p) return pkv::fail(PKV_ERR_INVALID_ARGUMENT, "pool is NULL");
  if (n < 0) return pkv::fail(PKV_ERR_INVALID_ARGUMENT, "n=%d", n);
  auto it = p->seqs.find(seq);
  if (it == p->seqs.end()) return pkv::fail(PKV_ERR_NOT_FOUND, "sequence %lld", (long long)seq);
  pkv_block_pool::Seq& s = it->second;
  const int64_t need = blocks_needed(p, s, n);
  if (need > static_cast<int64_t>(p->free_list.size()))
    return pkv::fail(PKV_ERR_OUT_OF_BLOCKS, "extend by %d needs %lld blocks, %zu free", n,
                     (long long)need, p->free_list.size());
  try {
    s.table.reserve(s.table.size() + need);  // the loop below then allocates nothing
  } catch (const std::exception&) {
    return pkv::fail(PKV_ERR_HOST_MEMORY, "host allocation failed");
  }
  const int64_t bs = p->block_size;
  for (int32_t i = 0; i < n; ++i) {
    const int64_t offset = s.num_tokens % bs;
    if (offset == 0) {  // last block full, or no block yet: take a fresh one
      const int32_t b = p->free_list.back();
      p->free_list.pop_back();
      p->ref[b] = 1;
      s.table.push_back(b);
    } else if (p->ref[s.table.back()] > 1) {  // shared, partly filled: copy on write
      const int32_t src = s.table.back();
      const int32_t dst = p->free_list.back();
      p->free_list.pop_back();
      p->ref[src] -= 1;
      p->ref[dst] = 1;
      s.table.back() = dst;
      if (cow_out) {
        cow_out[0] = src;
        cow_out[1] = dst;
      }
      if (num_cow_out) *num_cow_out = 1;  // only the first appended token can trigger it
    }
    if (slots_out) slots_out[i] = static_cast<int64_t>(s.table.back()) * bs + offset;
    s.num_tokens += 1;
  }
  return PKV_OK;
}

extern "C" pkv_status pkv_seq_fork(pkv_block_pool* p, int64_t parent, int64_t child) {
  pkv::clear_error();
  if (!p) return pkv::fail(PKV_ERR_INVALID_ARGUMENT, "pool is NULL");
  auto it = p->seqs.find(parent);
  if (it == p->seqs.end()) return pkv::fail(PKV_ERR_NOT_FOUND, "sequence %lld", (long long)parent);
  if (p->seqs.count(child)) return pkv::fail(PKV_ERR_ALREADY_EXISTS, "sequence %lld exists", (long long)child);
  return host_call([&]() -> pkv_status {
    pkv_block_pool::Seq c = it->second;  // copy: table and token count
    const pkv_block_pool::Seq& added = p->seqs.emplace(child, std::move(c)).first->second;
    for (int32_t b : added.table) p->ref[b] += 1;
    return PKV_OK;
  });
}

extern "C" pkv_status pkv_seq_free(pkv_block_pool* p, int64_t seq) {
  pkv::clear_error();
  if (!p) return pkv::fail(PKV_ERR_INVALID_ARGUMENT, "pool is NULL");
  auto it = p->seqs.find(seq);
  if (it == p->seqs.end()) return pkv::fail(PKV_ERR_NOT_FOUND, "sequence %lld", (long long)seq);
  for (int32_t b : it->second.table) {
    if (--p->ref[b] == 0) p->free_list.push_back(b);
  }
  p->seqs.erase(it);
  return PKV_OK;
}

extern "C" int64_t pkv_seq_context_len(const pkv_block_pool* p, int64_t seq) {
  if (!p) return -1;
  auto it = p->seqs.find(seq);
  return it == p->seqs.end() ? -1 : it->second.num_tokens;
}

extern "C" pkv_status pkv_pool_block_tables(const pkv_block_pool* p, const int64_t* seqs, int32_t n,
                                            int32_t max_blocks_per_seq, int32_t* tables_out,
                                            int32_t* context_lens_out) {
  pkv::clear_error();
  if (!p) return pkv::fail(PKV_ERR_INVALID_ARGUMENT, "pool is NULL");
  if (n < 0 || (n > 0 && !seqs)) return pkv::fail(PKV_ERR_INVALID_ARGUMENT, "n=%d seqs=%p", n, (const void*)seqs);
  if (max_blocks_per_seq < 0) return pkv::fail(PKV_ERR_INVALID_ARGUMENT, "max_blocks_per_seq=%d", max_blocks_per_seq);
  // validate everything before writing anything
  for (int32_t i = 0; i < n; ++i) {
    auto it = p->seqs.find(seqs[i]);
    if (it == p->seqs.end()) return pkv::fail(PKV_ERR_NOT_FOUND, "sequence %lld", (long long)seqs[i]);
    if (static_cast<int64_t>(it->second.table.size()) > max_blocks_per_seq)
      return pkv::fail(PKV_ERR_INVALID_ARGUMENT, "sequence %lld has %zu blocks > max_blocks_per_seq %d",
                       (long long)seqs[i], it->second.table.size(), max_blocks_per_seq);
    if (it->second.num_tokens > INT32_MAX)
      return pkv::fail(PKV_ERR_INVALID_ARGUMENT, "context length overflows int32");
  }
  for (int32_t i = 0; i < n; ++i) {
    const auto& s = p->seqs.find(seqs[i])->second;
    if (tables_out) {
      int32_t* row = tables_out + static_cast<int64_t>(i) * max_blocks_per_seq;
      const int32_t len = static_cast<int32_t>(s.table.size());
      for (int32_t j = 0; j < len; ++j) row[j] = s.table[j];
      for (int32_t j = len; j < max_blocks_per_seq; ++j) row[j] = -1;
    }
    if (context_lens_out) context_lens_out[i] = static_cast<int32_t>(s.num_tokens);
  }
  return PKV_OK;
}

// Swap of whole sequences between two pools (the swap space of the yunthe.com page, section
// "生产部署注意事项": KV cache moved out to host memory when device memory runs short and back
// later).  The moved sequences' distinct blocks, in order of first use (sequences in the given
// order, each table in logical order), each get one fresh block of `dst`, popped from the end
// of its free list, that inherits the block's reference count; the sequences' tables are
// rewritten through that map and the sequences leave `src` as pkv_seq_free would leave it.
extern "C" pkv_status pkv_pool_move_seqs(pkv_block_pool* src, pkv_block_pool* dst, const int64_t* seqs, int32_t n,
                                         int32_t* pairs_out, int32_t capacity, int32_t* num_pairs_out) {
  pkv::clear_error();
  if (num_pairs_out) *num_pairs_out = 0;
  if (!src || !dst) return pkv::fail(PKV_ERR_INVALID_ARGUMENT, "pool is NULL");
  if (src == dst) return pkv::fail(PKV_ERR_INVALID_ARGUMENT, "source and destination are the same pool");
  if (src->block_size != dst->block_size)
    return pkv::fail(PKV_ERR_INVALID_ARGUMENT, "block sizes differ (%d, %d)", src->block_size, dst->block_size);
  if (n < 0 || (n > 0 && !seqs)) return pkv::fail(PKV_ERR_INVALID_ARGUMENT, "n=%d seqs=%p", n, (const void*)seqs);
  if (capacity < 0) return pkv::fail(PKV_ERR_INVALID_ARGUMENT, "capacity=%d", capacity);
  return host_call([&]() -> pkv_status {
    // validate everything, and make every allocation, before changing anything
    std::unordered_set<int64_t> seen;
    std::unordered_map<int32_t, int32_t> uses;  // block -> references held by the moving sequences
    std::vector<int32_t> order;                  // distinct blocks, first use first
    for (int32_t i = 0; i < n; ++i) {
      auto it = src->seqs.find(seqs[i]);
      if (it == src->seqs.end()) return pkv::fail(PKV_ERR_NOT_FOUND, "sequence %lld", (long long)seqs[i]);
      if (dst->seqs.count(seqs[i]))
        return pkv::fail(PKV_ERR_ALREADY_EXISTS, "sequence %lld exists in the destination", (long long)seqs[i]);
      if (!seen.insert(seqs[i]).second)
        return pkv::fail(PKV_ERR_INVALID_ARGUMENT, "sequence %lld listed twice", (long long)seqs[i]);
      for (int32_t b : it->second.table)
        if (uses[b]++ == 0) order.push_back(b);
    }
    for (int32_t b : order)
      if (src->ref[b] != uses[b])
        return pkv::fail(PKV_ERR_UNSUPPORTED, "block %d is also used by a sequence that does not move", b);
    if (order.size() > dst->free_list.size())
      return pkv::fail(PKV_ERR_OUT_OF_BLOCKS, "need %zu blocks, %zu free", order.size(), dst->free_list.size());
    if (static_cast<int64_t>(order.size()) > capacity || (!pairs_out && !order.empty()))
      return pkv::fail(PKV_ERR_INVALID_ARGUMENT, "pairs_out holds %d pairs, %zu needed", pairs_out ? capacity : 0,
                       order.size());
    // block k of `order` takes the k-th block from the end of dst's free list
    std::unordered_map<int32_t, int32_t> to;
    to.reserve(order.size());
    const size_t nfree = dst->free_list.size();
    for (size_t k = 0; k < order.size(); ++k) to.emplace(order[k], dst->free_list[nfree - 1 - k]);
    std::vector<std::vector<int32_t>> tables(n);
    for (int32_t i = 0; i < n; ++i) {
      const std::vector<int32_t>& t = src->seqs.find(seqs[i])->second.table;
      tables[i].reserve(t.size());
      for (int32_t b : t) tables[i].push_back(to.find(b)->second);
    }
    dst->seqs.reserve(dst->seqs.size() + n);  // the node moves below then never rehash
    // changes: no allocation from here on
    for (size_t k = 0; k < order.size(); ++k) {
      const int32_t b = order[k];
      const int32_t nb = dst->free_list.back();
      dst->free_list.pop_back();
      dst->ref[nb] = uses.find(b)->second;
      pairs_out[2 * k] = b;
      pairs_out[2 * k + 1] = nb;
    }
    for (int32_t i = 0; i < n; ++i) {
      auto node = src->seqs.extract(seqs[i]);
      for (int32_t b : node.mapped().table)
        if (--src->ref[b] == 0) src->free_list.push_back(b);
      node.mapped().table = std::move(tables[i]);
      dst->seqs.insert(std::move(node));
    }
    if (num_pairs_out) *num_pairs_out = static_cast<int32_t>(order.size());
    return PKV_OK;
  });
}

// Groups of batch entries whose contexts start with the same physical blocks (prefix sharing
// by reference, the yunthe.com page, section "PagedAttention分页注意力机制原理").  Entries are
// bucketed by their first block; a bucket of two or more shares its members' common leading
// table entries, counting only blocks every member fills completely; the shared prefix P is
// that many tokens rounded down to a multiple of 16.  Buckets with P below max(16,
// min_prefix_tokens) are not grouped.  Groups come in order of their first member.
extern "C" pkv_status pkv_pool_prefix_groups(const pkv_block_pool* p, const int64_t* seqs, int32_t n,
                                             int32_t min_prefix_tokens, int32_t* seq_prefix_out,
                                             int32_t* group_offsets_out, int32_t* group_members_out,
                                             int32_t* num_groups_out, int32_t* max_prefix_out) {
  pkv::clear_error();
  if (!p) return pkv::fail(PKV_ERR_INVALID_ARGUMENT, "pool is NULL");
  if (n < 0 || (n > 0 && !seqs)) return pkv::fail(PKV_ERR_INVALID_ARGUMENT, "n=%d seqs=%p", n, (const void*)seqs);
  if (min_prefix_tokens < 0) return pkv::fail(PKV_ERR_INVALID_ARGUMENT, "min_prefix_tokens=%d", min_prefix_tokens);
  if (!seq_prefix_out || !group_offsets_out || !group_members_out || !num_groups_out || !max_prefix_out)
    return pkv::fail(PKV_ERR_INVALID_ARGUMENT, "NULL output");
  return host_call([&]() -> pkv_status {
    std::vector<const pkv_block_pool::Seq*> rows(n);
    for (int32_t i = 0; i < n; ++i) {
      auto it = p->seqs.find(seqs[i]);
      if (it == p->seqs.end()) return pkv::fail(PKV_ERR_NOT_FOUND, "sequence %lld", (long long)seqs[i]);
      rows[i] = &it->second;
    }
    const int64_t bs = p->block_size;
    std::unordered_map<int32_t, std::vector<int32_t>> bucket;
    std::vector<int32_t> first_seen;  // first blocks in order of first appearance
    for (int32_t i = 0; i < n; ++i) {
      seq_prefix_out[i] = 0;
      if (rows[i]->num_tokens / bs < 1) continue;  // no full block
      const int32_t b0 = rows[i]->table[0];
      auto& v = bucket[b0];
      if (v.empty()) first_seen.push_back(b0);
      v.push_back(i);
    }
    int32_t ng = 0, off = 0, maxp = 0;
    for (int32_t b0 : first_seen) {
      const std::vector<int32_t>& mem = bucket[b0];
      if (mem.size() < 2) continue;
      int64_t K = INT64_MAX;
      for (int32_t i : mem) K = std::min<int64_t>(K, rows[i]->num_tokens / bs);
      const std::vector<int32_t>& lead = rows[mem[0]]->table;
      for (int64_t k = 1; k < K; ++k) {
        bool same = true;
        for (int32_t i : mem) same = same && rows[i]->table[k] == lead[k];
        if (!same) {
          K = k;
          break;
        }
      }
      const int64_t P = K * bs / 16 * 16;
      if (P < std::max<int64_t>(16, min_prefix_tokens) || P > INT32_MAX) continue;
      group_offsets_out[ng++] = off;
      for (int32_t i : mem) {
        group_members_out[off++] = i;
        seq_prefix_out[i] = static_cast<int32_t>(P);
      }
      maxp = std::max<int32_t>(maxp, static_cast<int32_t>(P));
    }
    group_offsets_out[ng] = off;
    *num_groups_out = ng;
    *max_prefix_out = maxp;
    return PKV_OK;
  });
}
