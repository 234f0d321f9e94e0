// Line-protocol driver of the host block pool (block_pool.cpp + status.cpp), built by the CPU
// tests with g++ and -fsanitize=address,undefined so that the pool's C ABI runs under the
// sanitizers.  The pool is the block manager of the 111cn.net page "大模型推理引擎高频优化：
// 连续批处理、PagedAttention 与 KV Cache 实战拆解" §3.3, with the per-block reference counts of
// the gtnt.cn page "vLLM推理加速框架：PagedAttention与连续批处理技术解析" §2.1.
//
// One command per input line, one answer line per command (the status name first, then the
// results), so a Python test can drive the same histories it drives through the library and
// compare every answer with the oracle's block manager:
//   create <pool> <num_blocks> <block_size> <k> <free_order x k>   (k = 0: default order)
//   destroy <pool>
//   alloc <pool> <seq> <tokens>                  -> status blocks...
//   extend <pool> <seq> <n>                      -> status S slots... C src dst (if copy-on-write)
//   fork <pool> <parent> <child>                 -> status
//   free <pool> <seq>                            -> status
//   len <pool> <seq>                             -> OK len
//   freelist <pool>                              -> OK entries...
//   refs <pool>                                  -> OK ref counts of blocks 0..num_blocks-1
//   nseqs <pool>                                 -> OK count
//   tables <pool> <maxb> <k> <seqs x k>          -> status T entries... L lens...
//   move <src> <dst> <capacity> <k> <seqs x k>   -> status pairs...
//   groups <pool> <min_prefix> <k> <seqs x k>    -> status P prefixes... O offsets... M members... X max
// Pools are numbered by the caller (0 .. 15).  Every pool left is destroyed at end of input, so
// that the leak checker sees a clean exit.
#include <cstdint>
#include <cstdio>
#include <iostream>
#include <sstream>
#include <string>
#include <vector>

#include "../../include/pagedkv.h"

namespace {

pkv_block_pool* g_pools[16] = {};

pkv_block_pool* pool_at(int i) { return (i >= 0 && i < 16) ? g_pools[i] : nullptr; }

std::vector<int64_t> read_seqs(std::istringstream& in, int k) {
  std::vector<int64_t> v(k > 0 ? k : 0);
  for (auto& x : v) in >> x;
  return v;
}

void put(std::ostringstream& out, const char* tag, const int32_t* p, int n) {
  out << ' ' << tag;
  for (int i = 0; i < n; ++i) out << ' ' << p[i];
}

std::string run(const std::string& line) {
  std::istringstream in(line);
  std::string cmd;
  in >> cmd;
  std::ostringstream out;
  if (cmd == "create") {
    int id, nb, bs, k;
    in >> id >> nb >> bs >> k;
    std::vector<int32_t> order(k > 0 ? k : 0);
    for (auto& x : order) in >> x;
    if (id < 0 || id >= 16) return "PKV_ERR_INVALID_ARGUMENT";
    if (g_pools[id]) pkv_pool_destroy(g_pools[id]);
    g_pools[id] = nullptr;
    const pkv_status s = pkv_pool_create(nb, bs, k > 0 ? order.data() : nullptr, &g_pools[id]);
    return pkv_status_string(s);
  }
  int id;
  in >> id;
  pkv_block_pool* p = pool_at(id);
  if (cmd == "destroy") {
    if (p) pkv_pool_destroy(p);
    if (id >= 0 && id < 16) g_pools[id] = nullptr;
    return "PKV_OK";
  }
  if (!p) return "NO_POOL";
  if (cmd == "alloc") {
    int64_t seq;
    int32_t n;
    in >> seq >> n;
    const int32_t bs = pkv_pool_block_size(p);
    std::vector<int32_t> blocks(n > 0 ? (n + bs - 1) / bs : 0);
    const pkv_status s = pkv_seq_allocate(p, seq, n, blocks.empty() ? nullptr : blocks.data());
    out << pkv_status_string(s);
    if (s == PKV_OK) put(out, "B", blocks.data(), static_cast<int>(blocks.size()));
  } else if (cmd == "extend") {
    int64_t seq;
    int32_t n;
    in >> seq >> n;
    std::vector<int64_t> slots(n > 0 ? n : 0);
    int32_t cow[2] = {-1, -1}, ncow = 0;
    const pkv_status s = pkv_seq_extend(p, seq, n, slots.empty() ? nullptr : slots.data(), cow, &ncow);
    out << pkv_status_string(s);
    if (s == PKV_OK) {
      out << " S";
      for (int64_t x : slots) out << ' ' << x;
      put(out, "C", cow, ncow > 0 ? 2 : 0);
    }
  } else if (cmd == "fork") {
    int64_t a, b;
    in >> a >> b;
    out << pkv_status_string(pkv_seq_fork(p, a, b));
  } else if (cmd == "free") {
    int64_t seq;
    in >> seq;
    out << pkv_status_string(pkv_seq_free(p, seq));
  } else if (cmd == "len") {
    int64_t seq;
    in >> seq;
    out << "PKV_OK " << pkv_seq_context_len(p, seq);
  } else if (cmd == "freelist") {
    const int32_t n = pkv_pool_free_list(p, nullptr, 0);
    std::vector<int32_t> v(n);
    pkv_pool_free_list(p, v.data(), n);
    out << "PKV_OK";
    put(out, "F", v.data(), n);
  } else if (cmd == "refs") {
    const int32_t nb = pkv_pool_num_blocks(p);
    out << "PKV_OK R";
    for (int32_t b = 0; b < nb; ++b) out << ' ' << pkv_pool_ref_count(p, b);
  } else if (cmd == "nseqs") {
    out << "PKV_OK " << pkv_pool_num_seqs(p);
  } else if (cmd == "tables") {
    int32_t maxb, k;
    in >> maxb >> k;
    const auto seqs = read_seqs(in, k);
    std::vector<int32_t> tables(static_cast<size_t>(k > 0 ? k : 0) * (maxb > 0 ? maxb : 0));
    std::vector<int32_t> lens(k > 0 ? k : 0);
    const pkv_status s = pkv_pool_block_tables(p, seqs.data(), k, maxb, tables.empty() ? nullptr : tables.data(),
                                               lens.empty() ? nullptr : lens.data());
    out << pkv_status_string(s);
    if (s == PKV_OK) {
      put(out, "T", tables.data(), static_cast<int>(tables.size()));
      put(out, "L", lens.data(), static_cast<int>(lens.size()));
    }
  } else if (cmd == "move") {
    int dst_id, cap, k;
    in >> dst_id >> cap >> k;
    const auto seqs = read_seqs(in, k);
    std::vector<int32_t> pairs(2 * static_cast<size_t>(cap > 0 ? cap : 1));
    int32_t npairs = 0;
    const pkv_status s = pkv_pool_move_seqs(p, pool_at(dst_id), seqs.data(), k, pairs.data(), cap, &npairs);
    out << pkv_status_string(s);
    if (s == PKV_OK) put(out, "P", pairs.data(), 2 * npairs);
  } else if (cmd == "groups") {
    int32_t minp, k;
    in >> minp >> k;
    const auto seqs = read_seqs(in, k);
    std::vector<int32_t> sp(k > 0 ? k : 1), offs(k + 1), mem(k > 0 ? k : 1);
    int32_t ng = 0, mx = 0;
    const pkv_status s = pkv_pool_prefix_groups(p, seqs.data(), k, minp, sp.data(), offs.data(), mem.data(), &ng, &mx);
    out << pkv_status_string(s);
    if (s == PKV_OK) {
      put(out, "P", sp.data(), k);
      put(out, "O", offs.data(), ng + 1);
      put(out, "M", mem.data(), offs[ng]);
      out << " X " << mx;
    }
  } else {
    out << "UNKNOWN_COMMAND";
  }
  return out.str();
}

}  // namespace

int main() {
  std::string line;
  while (std::getline(std::cin, line)) {
    if (line.empty()) continue;
    std::cout << run(line) << '\n' << std::flush;
  }
  for (auto& p : g_pools) {
    if (p) pkv_pool_destroy(p);
    p = nullptr;
  }
  return 0;
}
