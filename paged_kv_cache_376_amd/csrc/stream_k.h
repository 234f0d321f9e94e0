// Internal interface of the evenly split grouped-query decode path (paged_attn_sk.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace pkv {
namespace sk {

// Waves the work is spread over (about 8 per CU on a 256-CU MI355X).
constexpr int kSkTargetWaves = 2048;
// Largest batch the path takes (the prefix sum of block counts lives in LDS).
constexpr int kSkMaxSeqs = 8192;

struct SkParams {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float* ws_acc;   // [ranges][Hkv][2][16][D]  unnormalised acc of cut sequences
  float* ws_ml;    // [ranges][Hkv][2][16][2]  (running max, sum)
  int32_t* ws_cu;  // [B + 1] prefix sum of block counts, written by the decode kernel
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;
  int32_t head_dim;
  int32_t max_blocks_per_seq;
  int32_t max_context_len;
  int32_t num_blocks;
  int32_t ranges;  // equal tile ranges per KV head
  float scale_log2e;
};

// Ranges per KV head for these arguments (host).
int32_t sk_ranges(int32_t num_seqs, int32_t num_kv_heads, int32_t max_context_len);
// Workspace bytes the path needs (host).
size_t sk_workspace_bytes(int32_t num_seqs, int32_t num_kv_heads, int32_t head_dim, int32_t max_context_len);
// Enqueues the decode kernel and the merge kernel on `stream`.
hipError_t sk_launch(SkParams p, int32_t dtype, hipStream_t stream);

}  // namespace sk
}  // namespace pkv
