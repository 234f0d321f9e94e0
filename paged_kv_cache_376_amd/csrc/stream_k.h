// Internal interface of the evenly split grouped-query decode path (paged_attn_sk.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace pkv {
namespace sk {

// Waves the work is spread over (about 8 per CU on a 256-CU MI355X).
constexpr int kSkTargetWaves = 2048;
// Bytes reserved at the start of the workspace for the status word (records follow, aligned).
constexpr int kStatusBytes = 256;
// Status word values.
constexpr int32_t kStatusOk = 0;
constexpr int32_t kStatusWaitGaveUp = 1;
// Default poll count of the merge kernel's waits on LDS flags: far beyond what co-resident
// waves of one work-group ever need, and still a bounded wait.
constexpr int32_t kDefaultSpinLimit = 1 << 22;
// Largest batch the path takes (the prefix sum of block counts lives in LDS).
constexpr int kSkMaxSeqs = 8192;
// LDS one work-group may hold on gfx950 (the whole 160 KiB of a CU).
constexpr int kLdsPerWorkgroup = 160 * 1024;

struct SkParams {
  void* out;
  const void* q;
  void* k_cache;  // written only with a fused append (new_key != NULL)
  void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const void* new_key;    // [B][Hkv][D] or NULL: with a fused append, each sequence's new
  const void* new_value;  // token (its last one) comes from here and is written to its slot
  float* ws_acc;     // [ranges][Hkv][2][16][D]  unnormalised acc of sequences cut by ranges
  float* ws_ml;      // [ranges][Hkv][2][16][2]  (running max, sum); ranges are per work-group
  int32_t* ws_desc;  // [ranges][4] per range: the sequence cut at its start whose merge it owns
                     // (or -1), with the first and last range holding tiles of that sequence
  int32_t* ws_status;  // one word at the start of the workspace: cleared by the decode kernel, set
                       // to kStatusWaitGaveUp by the merge kernel if one of its bounded waits ended
                       // without the flag it waited for
  int32_t spin_limit;  // polls of such a wait before it gives up
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;
  int32_t head_dim;
  int32_t max_blocks_per_seq;
  int32_t max_context_len;
  int32_t num_blocks;
  int32_t block_size;  // tokens per pool block: 8, 16 or 32 (a tile is always 16 tokens)
  int32_t ranges;  // equal tile ranges per KV head (one work-group of 4 waves each)
  float scale_log2e;
  // Suffix mode (prefix-shared decode): tokens at the start of each context that this launch
  // skips because they are attended elsewhere, [B], or NULL.
  const int32_t* seq_start;
  // Partial-result mode: when part_out is set, results go there as fp32 rows normalised by
  // their own sum, [B][Hq][D], with part_lse [B][Hq] = running max + log2(sum) (log2 units of
  // scale*log2(e)*logit; -inf for an empty context), instead of to out.
  float* part_out;
  float* part_lse;
  // Suffix mode: [B + 2] the tile-list prefix sum (B + 1 entries) and the ranges in use, written
  // by the first work-group for the finalize kernel; when set, the merge kernel is not launched
  // (the finalize kernel folds the records of cut suffixes).
  int32_t* ws_cu;
};

// KV heads per work-group of the even split (group: query heads per KV head).  The launch
// keeps about 256 work-groups, so the fewer heads a work-group takes, the fewer ranges each
// head's tile list is cut into, and the fewer records the cut sequences leave:
//   * 1 below 8 sequences: a small batch is cut into many ranges per sequence; one head with
//     eight sub-ranges merged in LDS leaves the merge kernel a quarter of the records;
//   * 2 below 32 sequences when a head serves a query-head group (4 sub-ranges): half the
//     ranges of 4 heads per work-group.  Measured, same process: 29.8 -> 23.4 us on 16
//     lognormal 70B-GQA sequences, 192.5 -> 190.1 us on 8 x 32768 tokens; from about 32
//     uniform long sequences up, the narrower 512-byte row slices cost more than they save;
//   * 2 as well with a single KV head (multi-query attention) at any batch: 4 heads per
//     work-group would leave 6 of its 8 waves without a head (256 x 8 query heads on one KV
//     head: 43.3 -> 32.1 us; 512 sequences: 71.2 -> 47.6 us);
//   * 4 otherwise, and with two KV heads at any batch: four adjacent 256-byte slices of each
//     token row, 2 sub-ranges.  (With two KV heads, 4 heads per work-group keeps 4 of its
//     waves busy and was 2-5% faster than 2 heads x 4 sub-ranges at 12 to 256 sequences.)
inline int32_t sk_heads(int32_t num_seqs, int32_t num_kv_heads, int32_t group) {
  return num_seqs < 8 ? 1 : (group >= 2 && num_kv_heads != 2 && (num_seqs < 32 || num_kv_heads == 1)) ? 2 : 4;
}
// Ranges per KV head for these arguments (host).
int32_t sk_ranges(int32_t num_seqs, int32_t num_kv_heads, int32_t group, int32_t max_context_len);
// LDS bytes of the decode kernel for these shapes (host), dynamic and static together;
// above 64 KiB needs no opt-in here.
int sk_lds_bytes_host(int32_t num_seqs, int32_t head_dim, int32_t group);
// Whether the path's kernels fit one work-group's LDS for these shapes (host).  The prefix
// sum takes about 8 bytes per sequence and the wave states 2 * 8 * group * head_dim * 4, so
// large batches with large groups do not fit (group 16, head_dim 128: up to 3807 sequences).
bool sk_fits(int32_t num_seqs, int32_t head_dim, int32_t group);
// Workspace bytes the path needs (host).
size_t sk_workspace_bytes(int32_t num_seqs, int32_t num_kv_heads, int32_t group, int32_t head_dim,
                          int32_t max_context_len);
// Enqueues the decode kernel and the merge kernel on `stream` (the decode kernel alone in suffix
// mode, where the prefix-shared decode's finalize kernel merges).
hipError_t sk_launch(SkParams p, int32_t dtype, hipStream_t stream);
struct PrefixParams;
// Enqueues the prefix-shared decode's prefix pass and suffix pass as one launch (suffix mode).
hipError_t sk_launch_prefix(SkParams p, const PrefixParams& pp, int32_t dtype, hipStream_t stream);

}  // namespace sk
}  // namespace pkv
