// Internal interface of the prefix-shared decode (paged_attn_prefix.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace pkv {
namespace sk {

// Prefix-shared decode: the tokens a group of sequences shares at the start of its contexts
// (the same physical blocks) are attended once per group by the prefix pass, the rest of each
// context by the even split in suffix and partial-result mode (both in one launch: each
// work-group takes its prefix units first, then its range of the split), and a finalize kernel
// merges the two (with the records of suffixes the split cut).  With a fused append the
// suffix pass takes each sequence's last token from the new rows, and the finalize kernel
// writes them to their slots (the launches that read the pool are then done).
constexpr int kPrefixChunkTiles = 32;  // 16-token tiles per prefix work-group (512 tokens)

struct PrefixParams {
  const void* q;
  void* k_cache;  // read by the prefix pass; written only by the finalize kernel with a fused
  void* v_cache;  // append (new_key != NULL)
  const int32_t* block_tables;
  const int32_t* context_lens;   // for a fused append: each sequence's last token is its new row
  const void* new_key;           // [B][Hkv][D] or NULL: with a fused append, the finalize kernel
  const void* new_value;         // writes each sequence's new row to its slot
  int32_t max_context_len;
  const int32_t* seq_prefix;     // [B] shared prefix tokens of each sequence (multiple of 16), 0 if none
  const int32_t* group_offsets;  // [num_groups + 1] into group_members
  const int32_t* group_members;  // batch positions; the first member's table holds the prefix blocks
  float* pre_acc;                // [B][Hq][chunks][D] unnormalised prefix partials
  float* pre_ml;                 // [B][Hq][chunks][2] (running max, sum)
  const float* part_out;         // suffix results of the even split (normalised fp32) ...
  const float* part_lse;         // ... and their log2-sum-exp, for suffixes inside one range
  const float* rec_acc;          // the even split's records (suffixes cut by its ranges):
  const float* rec_ml;           //   acc [ranges][Hkv][2][16][D], (m, l) [ranges][Hkv][2][16][2]
  const int32_t* cu;             // [B + 2] its tile-list prefix sum and ranges in use
  void* out;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;
  int32_t head_dim;
  int32_t max_blocks_per_seq;
  int32_t num_blocks;
  int32_t block_size;
  int32_t num_groups;
  int32_t chunks;  // prefix work-groups per group and KV head: ceil(max prefix tiles / kPrefixChunkTiles)
  float scale_log2e;
};

// Enqueues the finalize kernel (suffix results or records + prefix partials -> out; with a
// fused append also the new rows to their slots).
hipError_t finalize_launch(const PrefixParams& pp, int32_t dtype, hipStream_t stream);

}  // namespace sk
}  // namespace pkv
