/*
 * pagedkv.h -- C ABI of libpagedkv: paged KV-cache decode attention for AMD MI355X (gfx950).
 *
 * The method follows three web pages on vLLM's PagedAttention, cited by title and section:
 *   [111cn]  "大模型推理引擎高频优化：连续批处理、PagedAttention 与 KV Cache 实战拆解"
 *   [gtnt]   "vLLM推理加速框架：PagedAttention与连续批处理技术解析"
 *   [yunthe] "大模型推理显存优化实战：PagedAttention机制原理与vLLM连续批处理配置"
 *
 * Terms.  The KV cache is cut into fixed blocks of block_size tokens (16 by default,
 * [111cn] §3.2, [yunthe] section "PagedAttention分页注意力机制原理").  Physical blocks sit
 * anywhere in a preallocated pool; each sequence's block table lists its physical block
 * ids in logical order ([111cn] §3.2).  A block's data has shape (block_size, heads,
 * head_dim) ([gtnt] §2.1), and there is one pool for K and one for V, so each pool is
 *
 *     cache[num_blocks][block_size][num_kv_heads][head_dim]     (row-major, contiguous)
 *
 * and token t of a sequence with table bt lives at block bt[t / block_size], offset
 * t % block_size.  A "slot" is physical_block * block_size + offset.
 *
 * Conventions for every call:
 *   - Return codes only; nothing throws across the ABI.  On failure pkv_last_error()
 *     (thread-local) holds a message.  A call that fails validation launches nothing and
 *     changes no state.
 *   - Device calls take caller-owned device pointers (any HIP device allocation, e.g.
 *     PyTorch tensors) that must be 16-byte aligned, and a stream (a hipStream_t passed
 *     as void*; NULL is the default stream).  They enqueue and return; errors inside the
 *     kernels are not reported (see each call's device-side contract).
 *   - The library never allocates device memory (no hipMalloc, no allocating library call):
 *     workspaces are the caller's, except that pkv_paged_attn_decode_append_noalloc takes its
 *     workspace from a fixed scratch array compiled into the library (one per GPU).
 *   - Host pool calls are not thread-safe: one owner per pool.
 *   - Supported by the kernels: dtype f32, f16, bf16; head_dim 64 or 128; block_size 16
 *     (decode of f16/bf16 pools also 8 and 32; appends and block copies any block size).
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define PKV_API __attribute__((visibility("default")))
#else
#define PKV_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARGUMENT = 1,   /* null/misaligned pointer, bad size, bad shape      */
  PKV_ERR_UNSUPPORTED = 2,        /* valid request the kernels do not implement         */
  PKV_ERR_OUT_OF_BLOCKS = 3,      /* pool cannot cover the request; pool unchanged       */
  PKV_ERR_NOT_FOUND = 4,          /* unknown sequence id                                 */
  PKV_ERR_WORKSPACE_TOO_SMALL = 5,
  PKV_ERR_HIP = 6,                /* the HIP runtime refused a launch                    */
  PKV_ERR_ALREADY_EXISTS = 7,     /* sequence id already in use                          */
  PKV_ERR_HOST_MEMORY = 8         /* a host allocation failed (the pool is left unchanged) */
} pkv_status;

typedef enum { PKV_F32 = 0, PKV_F16 = 1, PKV_BF16 = 2 } pkv_dtype;

/* Shape of one of the two pools (K and V share it). */
typedef struct {
  int32_t num_blocks;    /* physical blocks in the pool (> 0)                    */
  int32_t block_size;    /* tokens per block; the kernels implement 16            */
  int32_t num_kv_heads;  /* KV heads per token (> 0)                              */
  int32_t head_dim;      /* 64 or 128                                             */
  int32_t dtype;         /* pkv_dtype                                             */
} pkv_cache_desc;

/* ------------------------------------------------------------------------------------ */
/* Library                                                                               */
/* ------------------------------------------------------------------------------------ */

/* Message of the last failing call on this thread ("" if none).  Owned by the library,
 * valid until the next call on this thread. */
PKV_API const char* pkv_last_error(void);

/* Static name of a status code. */
PKV_API const char* pkv_status_string(int32_t status);

/* Library version string, static. */
PKV_API const char* pkv_version(void);

/* ------------------------------------------------------------------------------------ */
/* Device: KV append (the reshape-and-cache scatter)                                     */
/* ------------------------------------------------------------------------------------ */

/* Writes each new token's K and V row into its pool slot.
 *
 * Defined by the append step of [111cn] §3.3 (the new token goes to the end of the last
 * block, or into a freshly taken block when the last one is full -- the host pool below
 * decides which, and hands the result over as slots) and the block layout of [gtnt] §2.1.
 *
 *   key, value      device, [num_tokens][num_kv_heads][head_dim] of cache->dtype, read only
 *   k_cache,v_cache device pools laid out as described at the top, written in place
 *   cache           host descriptor of both pools
 *   slot_mapping    device int64 [num_tokens]; row i goes to block slot/bs, offset slot%bs
 *   num_tokens      >= 0 (0 is a no-op)
 *
 * For each i with 0 <= slot_mapping[i] < num_blocks*block_size the row is copied bit for
 * bit; other slots (negative = padding, or out of range) are skipped without any memory
 * access.  Two tokens with the same slot race (undefined which row wins).
 * Errors: INVALID_ARGUMENT (null or misaligned pointer, num_tokens < 0, bad descriptor),
 * UNSUPPORTED (dtype or head_dim outside the set above), HIP (launch failed). */
PKV_API pkv_status pkv_kv_cache_append(const void* key, const void* value,
                               void* k_cache, void* v_cache, const pkv_cache_desc* cache,
                               const int64_t* slot_mapping, int32_t num_tokens,
                               void* stream);

/* ------------------------------------------------------------------------------------ */
/* Device: paged decode attention                                                        */
/* ------------------------------------------------------------------------------------ */

/* Bytes of workspace pkv_paged_attn_decode needs for these arguments (0 when the chosen
 * work split needs none), partition_size and dtype (a pkv_dtype) as for the decode call.
 *   - partition_size 0 with f16/bf16 pools and at most 8192 sequences whose decode state fits
 *     one work-group's 160 KiB of LDS (about 8 bytes per sequence plus
 *     16 * group * head_dim * 4 bytes of wave states: every batch up to 8192 for groups up to
 *     8 at head_dim 128, up to 3807 sequences at group 16): the even split over the GPU.  The
 *     workspace holds a status word (the first 256 bytes are reserved for it, see below), then,
 *     per work range, fp32 records of sequences cut by the split (two per KV head,
 *     16*head_dim + 32 floats each) and one 16-byte descriptor; it does not depend on the
 *     context lengths beyond max_context_len nor on the block size.
 *     Status word: the first int32 of the workspace.  The decode launch clears it and the
 *     merge launch sets it to 1 if one of its bounded waits (a wave waiting on an LDS flag of
 *     another wave of its own work-group) ran out of polls; the call's output is then not
 *     reliable.  Read it once the stream has finished the call; 0 means every wait ended
 *     normally.  (Co-resident waves of one work-group always set their flags, so the limit
 *     only bounds the wait; pkv_set_merge_spin_limit lowers it to test this path.)
 *   - otherwise (f32 pools, or an explicit partition_size): fixed partitions; fp32 partials of
 *     split sequences, num_seqs * num_q_heads * P * (head_dim + 2) floats with P partitions
 *     of the longest context, 0 when nothing is split.
 * Returns 0 for arguments the decode call would reject. */
PKV_API size_t pkv_paged_attn_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                      int32_t num_kv_heads, int32_t head_dim,
                                      int32_t max_context_len, int32_t partition_size,
                                      int32_t dtype);

/* The fixed partition size (tokens) pkv_paged_attn_decode uses for these arguments: the
 * resolved value of partition_size 0 (auto) or -1 (never split: max_context_len rounded up
 * to the block size), or partition_size itself.  0 when the even split over the GPU is used
 * (partition_size 0 with f16/bf16 pools, see above) and on invalid arguments. */
PKV_API int32_t pkv_paged_attn_partition_size(int32_t num_seqs, int32_t num_q_heads,
                                      int32_t num_kv_heads, int32_t head_dim,
                                      int32_t max_context_len, int32_t partition_size,
                                      int32_t dtype);

/* Single-query attention of every sequence over its paged context.
 *
 * The kernel finds each token's physical block through the block table and attends over
 * the non-contiguous blocks ([yunthe] section "PagedAttention分页注意力机制原理"); the
 * result is scaled dot-product attention over the sequence's tokens in logical order:
 *
 *   out[s,h,:] = sum_t w_t V_s[t, h/G, :] / sum_t w_t,
 *   w_t = exp(scale * <q[s,h,:], K_s[t, h/G, :]> - max),  t = 0 .. context_lens[s]-1,
 *
 * with G = num_q_heads / num_kv_heads (query head h reads KV head h / G).  The argument
 * list extends the one of the CUDA kernel shown in [gtnt] §6.2 (out, q, k, v, block
 * tables; out shares q's element type) with context lengths, scale, workspace and stream.
 *
 *   out            device [num_seqs][num_q_heads][head_dim], cache->dtype, written
 *   q              device [num_seqs][num_q_heads][head_dim], cache->dtype
 *   k_cache,v_cache device pools (read only)
 *   block_tables   device int32 [num_seqs][max_blocks_per_seq]; entries past
 *                  ceil(context_len/bs) are never read (any value, e.g. -1)
 *   context_lens   device int32 [num_seqs]
 *   max_context_len host int, >= every context_lens[s], <= max_blocks_per_seq*block_size
 *   scale          logit scale (usually 1/sqrt(head_dim))
 *   workspace      device scratch of >= pkv_paged_attn_workspace_bytes(...) bytes, 16-byte
 *                  aligned (may be NULL when that is 0); contents on entry and return
 *                  unspecified (no state carries over between calls)
 *   partition_size 0 = auto; -1 = never split; else tokens per partition, a positive
 *                  multiple of block_size.  With 0 and f16/bf16 pools (at most 8192
 *                  sequences) the work is split evenly over the GPU: each KV head's list of
 *                  (sequence, 16-token tile) pairs is cut into equal ranges whatever the
 *                  length mix, and sequences cut by the ranges are merged exactly (log-sum-exp
 *                  combine in a fixed order) by a second kernel.  Otherwise (f32 pools, or an
 *                  explicit size) sequences longer than one partition are processed as
 *                  independent partitions and merged the same way.
 *
 * A sequence with context length 0 yields zeros.  Results are bitwise reproducible run to
 * run for identical inputs and arguments (no atomics; every merge has a fixed order).  With
 * the even split, two sequences with equal contents at different batch positions may be cut
 * differently and then agree up to rounding rather than bit for bit.
 * Device-side contract (not checked on the host): context_lens[s] in [0, max_context_len]
 * and table entries in [0, num_blocks).  To never touch memory outside the buffers, the
 * kernels clamp context lengths to max_context_len and skip blocks whose id is out of
 * range; the output is then unspecified, but nothing outside the buffers is read.
 * Block sizes: 8, 16 or 32 tokens on the even split (f16/bf16, partition_size 0; the block
 * size of 8 suits models under 7B, [gtnt] end of §6.2); 16 with fixed partitions and for f32.
 * Errors: INVALID_ARGUMENT, UNSUPPORTED (dtype/head_dim/block_size/group size outside the
 * implemented set: f32 supports G <= 2, f16/bf16 support G <= 16), WORKSPACE_TOO_SMALL,
 * HIP. */
PKV_API pkv_status pkv_paged_attn_decode(void* out, const void* q,
                                 const void* k_cache, const void* v_cache,
                                 const pkv_cache_desc* cache,
                                 const int32_t* block_tables, int32_t max_blocks_per_seq,
                                 const int32_t* context_lens, int32_t max_context_len,
                                 int32_t num_seqs, int32_t num_q_heads, float scale,
                                 void* workspace, size_t workspace_bytes,
                                 int32_t partition_size, void* stream);

/* One decode step in one call: the KV append of each sequence's new token, then the decode
 * of pkv_paged_attn_decode over contexts that include it.
 *
 * The new token of sequence s is its last one, position context_lens[s] - 1, whose slot the
 * block table gives (block block_tables[s][(ctx-1)/bs], offset (ctx-1) % bs): the append step
 * of [111cn] §3.3 after the host pool has taken that slot (pkv_seq_extend by one token).
 * The result equals pkv_kv_cache_append with those slots followed by pkv_paged_attn_decode,
 * bit for bit in the pools and in the output.  The wave that reads a sequence's last tile
 * takes the new row from new_key/new_value.  On the evenly split path the merge launch that
 * follows the decode writes the rows to their slots, so the step is the decode launch plus
 * the merge; with fixed partitions the work-group of each sequence's last partition writes
 * its KV head's row, so the step is the decode launch (plus the reduce when a sequence spans
 * several partitions).
 *
 *   new_key, new_value  device [num_seqs][num_kv_heads][head_dim] of cache->dtype, 16-byte
 *                       aligned, read only
 *   k_cache, v_cache    written at the new tokens' slots, read everywhere else
 *   all other arguments as for pkv_paged_attn_decode (max_blocks_per_seq must be > 0)
 * Sequences with context length 0 append nothing.  Block ids outside the pool are skipped
 * for the write as for the read.  Errors: as pkv_paged_attn_decode, plus INVALID_ARGUMENT
 * for missing or misaligned new_key/new_value. */
PKV_API pkv_status pkv_paged_attn_decode_append(void* out, const void* q,
                                        const void* new_key, const void* new_value,
                                        void* k_cache, void* v_cache,
                                        const pkv_cache_desc* cache,
                                        const int32_t* block_tables, int32_t max_blocks_per_seq,
                                        const int32_t* context_lens, int32_t max_context_len,
                                        int32_t num_seqs, int32_t num_q_heads, float scale,
                                        void* workspace, size_t workspace_bytes,
                                        int32_t partition_size, void* stream);

/* Allocation-free variant of pkv_paged_attn_decode_append, for callers that cannot allocate
 * device memory or pass a workspace: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  The same append and decode, on the same kernels, with the
 * workspace taken from a fixed scratch array that the library holds in device memory: one copy
 * per GPU (pkv_paged_attn_noalloc_scratch_bytes() bytes, 32 MiB), set up on the first call on
 * that GPU and kept until the process ends.  The call allocates nothing (no hipMalloc, no
 * library allocation).
 *
 * Arguments as for pkv_paged_attn_decode_append, without workspace and workspace_bytes.  The
 * stream must belong to the current device.  Every call on one GPU uses that GPU's one scratch
 * array, which keeps the last call's contents (nothing in it needs to start at zero: each call
 * clears its status word and writes every record before reading it); two calls that overlap on
 * one GPU (different streams, or different threads) race on it and give undefined results.
 * The status word of pkv_paged_attn_workspace_bytes lives at the start of the array, out of the
 * caller's reach.
 * Errors: as pkv_paged_attn_decode_append; WORKSPACE_TOO_SMALL when the arguments need more
 * workspace than the scratch array holds (every even-split decode with at most 2016 KV heads
 * fits; more KV heads, and large fixed-partition splits, e.g. f32 pools with long contexts and
 * many sequences, do not), with
 * the sizes in the message; HIP when the scratch array's address cannot be found on the
 * current device. */
PKV_API pkv_status pkv_paged_attn_decode_append_noalloc(void* out, const void* q,
                                                const void* new_key, const void* new_value,
                                                void* k_cache, void* v_cache,
                                                const pkv_cache_desc* cache,
                                                const int32_t* block_tables, int32_t max_blocks_per_seq,
                                                const int32_t* context_lens, int32_t max_context_len,
                                                int32_t num_seqs, int32_t num_q_heads, float scale,
                                                int32_t partition_size, void* stream);

/* Bytes of the scratch array pkv_paged_attn_decode_append_noalloc uses on each GPU. */
PKV_API size_t pkv_paged_attn_noalloc_scratch_bytes(void);

/* Decode attention with prefix sharing: the same result as pkv_paged_attn_decode (up to
 * rounding), computed so that a prefix shared by a group of sequences is read once per group.
 *
 * Sequences that share the physical blocks of the start of their contexts (prefix sharing by
 * reference to the same blocks, [yunthe] section "PagedAttention分页注意力机制原理"; one block
 * shared by several requests, [111cn] §3.2) attend over that shared prefix in one pass for
 * the whole group: a work-group takes 32 prefix tiles (512 tokens) of one KV head and its
 * waves take the group's query rows (member x query head), so every prefix tile is read once
 * for the group.
 * Each sequence's own remainder is attended by the even split over the GPU, in the same launch
 * (each work-group takes its prefix tiles first, then its range of the split), and a second
 * launch merges the two parts (and the pieces of remainders the split cut) exactly with the
 * log-sum-exp rule (fixed order: deterministic).
 *
 * Arguments as for pkv_paged_attn_decode (f16/bf16 pools, block size 8, 16 or 32, at most 8192
 * sequences; no partition_size), plus the group description that pkv_pool_prefix_groups
 * produces, copied to device memory:
 *   seq_prefix     device int32 [num_seqs]: shared prefix tokens of each sequence, a multiple
 *                  of 16, 0 for sequences in no group
 *   group_offsets  device int32 [num_groups + 1]: group i is group_members[offsets[i] ..
 *                  offsets[i+1])
 *   group_members  device int32: batch positions (0 .. num_seqs-1)
 *   num_groups     >= 0
 *   max_prefix_tokens  host int: >= every seq_prefix, a multiple of 16, <= max_context_len
 *   workspace      >= pkv_paged_attn_decode_prefix_workspace_bytes(...) bytes
 * Device-side contract: the members of a group have the same seq_prefix P <= their context
 * lengths, and the first P tokens of their tables name the same blocks (the kernels read a
 * group's prefix through its first member's table); sequences in no group have 0; each batch
 * position is in at most one group.  As for the other arguments, a description that breaks
 * this contract gives unspecified output but no access outside the buffers: offsets past
 * num_seqs and member positions outside [0, num_seqs) are skipped, prefix lengths are kept
 * inside [0, context length] on a 16-token boundary, and no more than
 * ceil(max_prefix_tokens / 512) prefix partials are read per row.
 * The workspace starts with the even split's status word (see
 * pkv_paged_attn_workspace_bytes).
 * Errors: as pkv_paged_attn_decode; UNSUPPORTED for f32 pools, more than 8192 sequences, or a
 * batch and group size whose decode state does not fit the LDS (see
 * pkv_paged_attn_workspace_bytes); INVALID_ARGUMENT for a bad group description (null
 * pointers, num_groups < 0, bad max_prefix_tokens). */
PKV_API pkv_status pkv_paged_attn_decode_prefix(void* out, const void* q,
                                        const void* k_cache, const void* v_cache,
                                        const pkv_cache_desc* cache,
                                        const int32_t* block_tables, int32_t max_blocks_per_seq,
                                        const int32_t* context_lens, int32_t max_context_len,
                                        int32_t num_seqs, int32_t num_q_heads, float scale,
                                        const int32_t* seq_prefix, const int32_t* group_offsets,
                                        const int32_t* group_members, int32_t num_groups,
                                        int32_t max_prefix_tokens, void* workspace,
                                        size_t workspace_bytes, void* stream);

/* One prefix-shared decode step in one call: the KV append of each sequence's new token, then
 * the decode of pkv_paged_attn_decode_prefix over contexts that include it.
 *
 * The new token of sequence s is its last one, position context_lens[s] - 1, in the slot its
 * block table gives: the append step of [111cn] §3.3 after the host pool has taken that slot
 * (pkv_seq_extend by one token, which copies a shared last block first), with the groups of
 * pkv_pool_prefix_groups computed on the extended tables.  The result equals pkv_kv_cache_append
 * with those slots followed by pkv_paged_attn_decode_prefix, bit for bit in the pools and in
 * the output: the suffix pass takes each sequence's last token from new_key/new_value, and the
 * finalize launch writes the rows to their slots after every read of the pool.  The step stays
 * two launches.
 *
 *   new_key, new_value  device [num_seqs][num_kv_heads][head_dim] of cache->dtype, 16-byte
 *                       aligned, read only
 *   k_cache, v_cache    written at the new tokens' slots, read everywhere else
 *   all other arguments as for pkv_paged_attn_decode_prefix
 * Device-side contract, beyond that of pkv_paged_attn_decode_prefix: a sequence's shared prefix
 * ends before its new token (seq_prefix[s] <= context_lens[s] - 1), as it does for groups found
 * on tables whose last blocks are private; otherwise the prefix pass reads the slot before the
 * write and the output is unspecified (no access outside the buffers).  Sequences with context
 * length 0 append nothing; block ids outside the pool are skipped for the write as for the read.
 * Errors: as pkv_paged_attn_decode_prefix, plus INVALID_ARGUMENT for missing or misaligned
 * new_key/new_value. */
PKV_API pkv_status pkv_paged_attn_decode_prefix_append(void* out, const void* q,
                                               const void* new_key, const void* new_value,
                                               void* k_cache, void* v_cache,
                                               const pkv_cache_desc* cache,
                                               const int32_t* block_tables, int32_t max_blocks_per_seq,
                                               const int32_t* context_lens, int32_t max_context_len,
                                               int32_t num_seqs, int32_t num_q_heads, float scale,
                                               const int32_t* seq_prefix, const int32_t* group_offsets,
                                               const int32_t* group_members, int32_t num_groups,
                                               int32_t max_prefix_tokens, void* workspace,
                                               size_t workspace_bytes, void* stream);

/* Test hook for the merge launch's bounded waits (see the status word under
 * pkv_paged_attn_workspace_bytes): sets the number of polls after which such a wait gives up,
 * for every later call in this process, and returns the previous value.  A negative limit
 * restores the default (2^22 polls).  With 0 every wait gives up at once: the call still ends
 * normally, its output is not reliable and the status word reads 1.  Not thread-safe with
 * respect to calls in flight on other threads. */
PKV_API int32_t pkv_set_merge_spin_limit(int32_t limit);

/* Bytes of workspace pkv_paged_attn_decode_prefix needs (the even split's, plus fp32
 * suffix results [num_seqs][num_q_heads][head_dim + 1], prefix partials
 * [num_seqs][num_q_heads][ceil(max_prefix_tokens / 512)][head_dim + 2] and num_seqs + 2 int32
 * of suffix bookkeeping, each region rounded up to 256 bytes).  0 for arguments the call would
 * reject. */
PKV_API size_t pkv_paged_attn_decode_prefix_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                                    int32_t num_kv_heads, int32_t head_dim,
                                                    int32_t max_context_len,
                                                    int32_t max_prefix_tokens, int32_t dtype);

/* ------------------------------------------------------------------------------------ */
/* Device: whole-block copies (copy-on-write, swap)                                      */
/* ------------------------------------------------------------------------------------ */

/* Copies whole blocks inside both pools: for each pair i, block pairs[2i] (source) is copied
 * onto block pairs[2i+1] (destination) in k_cache and in v_cache, bit for bit, all pairs in
 * one launch.
 *
 * This is the copy half of copy-on-write ([gtnt] §2.2, with the reference counts of §2.1):
 * before a sequence writes into a partly filled block it shares with others, it takes a fresh
 * block holding a copy.  pkv_seq_extend decides and reports the (source, destination) pairs;
 * the copies must run before the append that writes into the destinations.
 *
 *   k_cache, v_cache  device pools [num_blocks][block_size][num_kv_heads][head_dim], 16-byte
 *                     aligned, written at the destination blocks only
 *   cache             host descriptor (any dtype; block_size, num_kv_heads, head_dim > 0 with
 *                     a block of a multiple of 16 bytes)
 *   pairs             device int32 [num_pairs][2] (source, destination), 4-byte aligned
 *   num_pairs         >= 0 (0 is a no-op)
 * Pairs with an id outside [0, num_blocks), or with source == destination, are skipped
 * without any memory access.  A block that is the destination of one pair and the source or
 * destination of another in the same call races (undefined contents).
 * Errors: INVALID_ARGUMENT (null or misaligned pointer, num_pairs < 0, bad descriptor),
 * UNSUPPORTED (dtype, block of a size not a multiple of 16), HIP (launch failed). */
PKV_API pkv_status pkv_copy_blocks(void* k_cache, void* v_cache, const pkv_cache_desc* cache,
                           const int32_t* pairs, int32_t num_pairs, void* stream);

/* Copies whole blocks from one pair of pools into another pair of pools of the same block
 * shape: for each pair i, block pairs[2i] of (src_k, src_v) onto block pairs[2i+1] of
 * (dst_k, dst_v), bit for bit, in one launch.
 *
 * This moves the bytes of a swap: when device memory runs short, some requests' KV cache goes
 * out to host memory and comes back once memory frees up (the swap space of [yunthe] section
 * "生产部署注意事项"); here a sequence's blocks are moved whole, by block id.  Either
 * side may be device memory or pinned host memory that the GPU can address (for example a
 * PyTorch tensor made with pin_memory=True); both are read and written by the GPU over the
 * bus, one kernel per call.
 *
 *   dst_k, dst_v       destination pools (dst_num_blocks blocks each), 16-byte aligned
 *   src_k, src_v       source pools (src_num_blocks blocks each), 16-byte aligned, read only
 *   cache              host descriptor of the block shape (its num_blocks is not used)
 *   pairs              int32 [num_pairs][2] (source block, destination block), 4-byte
 *                      aligned, in device memory or GPU-addressable pinned host memory
 *   num_pairs          >= 0 (0 is a no-op)
 * Pairs with an id outside its pool are skipped.  The destination and source pools must be
 * different allocations (use pkv_copy_blocks inside one pool).  A destination block named
 * twice races.  The call checks with the HIP runtime that every pointer is device memory or
 * pinned host memory mapped for the current device.
 * Errors: INVALID_ARGUMENT (null, misaligned or unmapped pointer, same pool on both sides,
 * pool size <= 0, num_pairs < 0, bad descriptor), UNSUPPORTED (as pkv_copy_blocks),
 * HIP (launch failed). */
PKV_API pkv_status pkv_swap_blocks(void* dst_k, void* dst_v, int32_t dst_num_blocks,
                           const void* src_k, const void* src_v, int32_t src_num_blocks,
                           const pkv_cache_desc* cache, const int32_t* pairs,
                           int32_t num_pairs, void* stream);

/* ------------------------------------------------------------------------------------ */
/* Host: block pool and block tables                                                     */
/* ------------------------------------------------------------------------------------ */

/* The pool of [111cn] §3.2-§3.3 / [yunthe] "PagedAttention分页注意力机制原理": a free list
 * of physical block ids, a reference count per block ([gtnt] §2.1) and one block table per
 * sequence.  Pure host code.  Every operation is all-or-nothing: when the free list
 * cannot cover it (the admission check of the scheduler in [111cn] §2.2), it returns
 * PKV_ERR_OUT_OF_BLOCKS and nothing changes; when a host allocation fails, it returns
 * PKV_ERR_HOST_MEMORY and nothing changes either (no C++ exception leaves the library). */
typedef struct pkv_block_pool pkv_block_pool;

/* free_order: NULL for 0..num_blocks-1, else a permutation of 0..num_blocks-1; blocks are
 * popped from the END of this list ([111cn] §3.3).  *out receives the new pool. */
PKV_API pkv_status pkv_pool_create(int32_t num_blocks, int32_t block_size,
                           const int32_t* free_order, pkv_block_pool** out);
PKV_API void pkv_pool_destroy(pkv_block_pool* pool);

/* Pool queries.  Each returns -1 for a NULL pool.
 * Physical blocks in the preallocated pool ([111cn] §3.2: the cache is cut into fixed-size
 * blocks of one physical pool). */
PKV_API int32_t pkv_pool_num_blocks(const pkv_block_pool* pool);
/* Tokens per block ([111cn] §3.2 and [yunthe] "PagedAttention分页注意力机制原理": 16 by default). */
PKV_API int32_t pkv_pool_block_size(const pkv_block_pool* pool);
/* Entries of the free list ([111cn] §3.3 free_blocks): the admission check of [111cn] §2.2
 * compares a request's block count with this. */
PKV_API int32_t pkv_pool_num_free(const pkv_block_pool* pool);
/* Reference count of a block ([gtnt] §2.1 Block.ref_count: the number of sequences whose
 * tables name it), -1 if block_id is out of range. */
PKV_API int32_t pkv_pool_ref_count(const pkv_block_pool* pool, int32_t block_id);
/* Copies min(capacity, num_free) free-list entries (bottom first; the next pop takes the
 * last one, [111cn] §3.3 pop()) into out; returns num_free. */
PKV_API int32_t pkv_pool_free_list(const pkv_block_pool* pool, int32_t* out, int32_t capacity);
/* Number of live sequences: sequences holding a block table ([111cn] §3.3 block_tables). */
PKV_API int32_t pkv_pool_num_seqs(const pkv_block_pool* pool);

/* New sequence holding num_tokens (>= 0) tokens: ceil(num_tokens/bs) blocks popped from
 * the end of the free list, in logical order ([111cn] §3.3 allocate).  blocks_out
 * (nullable) receives them.  ALREADY_EXISTS, OUT_OF_BLOCKS, INVALID_ARGUMENT. */
PKV_API pkv_status pkv_seq_allocate(pkv_block_pool* pool, int64_t seq, int32_t num_tokens,
                            int32_t* blocks_out);

/* Appends n (>= 0) tokens ([111cn] §3.3 append_token, repeated): a token whose sequence
 * holds a multiple of bs tokens (its last block is full, or it has none) takes a fresh
 * block; otherwise it goes to the end of the last block.  If that last block is shared
 * (ref > 1) and not full it is first replaced by a fresh private block (copy-on-write,
 * [gtnt] §2.2): *num_cow_out = 1 and cow_out = {src, dst}; the caller must copy the
 * block's bytes src -> dst in both pools before writing the new rows.  slots_out
 * (nullable, n entries) receives each new token's slot.  NOT_FOUND, OUT_OF_BLOCKS. */
PKV_API pkv_status pkv_seq_extend(pkv_block_pool* pool, int64_t seq, int32_t n, int64_t* slots_out,
                          int32_t* cow_out, int32_t* num_cow_out);

/* child shares every block of parent (each ref + 1) and its token count ([gtnt] §2.1-2.2,
 * [yunthe] prefix sharing).  NOT_FOUND, ALREADY_EXISTS. */
PKV_API pkv_status pkv_seq_fork(pkv_block_pool* pool, int64_t parent, int64_t child);

/* Drops the sequence: in table order each block's ref - 1, pushed onto the end of the free
 * list when it reaches 0 (blocks return to the pool when a request ends, [yunthe]). */
PKV_API pkv_status pkv_seq_free(pkv_block_pool* pool, int64_t seq);

/* Token count of seq, or -1 if unknown. */
PKV_API int64_t pkv_seq_context_len(const pkv_block_pool* pool, int64_t seq);

/* Finds groups of batch entries whose contexts start with the same physical blocks, for
 * pkv_paged_attn_decode_prefix.  Entries (seqs[0..n-1], batch positions 0..n-1) are bucketed by
 * their first block; a bucket of two or more entries shares the leading table entries common to
 * all its members, counting only blocks every member fills completely; its prefix is that many
 * tokens rounded down to a multiple of 16.  A bucket whose prefix is below max(16,
 * min_prefix_tokens) is not a group.  Groups are listed in order of their first member, members
 * in batch order.
 *   seq_prefix_out     int32 [n]: the entry's group prefix in tokens, or 0
 *   group_offsets_out  int32 [n + 1]: group i is group_members_out[offsets[i] .. offsets[i+1])
 *   group_members_out  int32 [n]: batch positions
 *   num_groups_out, max_prefix_out: number of groups, longest prefix (0 if none)
 * Errors: INVALID_ARGUMENT (null pool or output, n < 0, min_prefix_tokens < 0), NOT_FOUND. */
PKV_API pkv_status pkv_pool_prefix_groups(const pkv_block_pool* pool, const int64_t* seqs, int32_t n,
                                  int32_t min_prefix_tokens, int32_t* seq_prefix_out,
                                  int32_t* group_offsets_out, int32_t* group_members_out,
                                  int32_t* num_groups_out, int32_t* max_prefix_out);

/* Moves whole sequences from pool `src` to pool `dst` (for example from the device pool to a
 * pool in pinned host memory and back): the swap space of [yunthe] section "生产部署注意事项",
 * where some requests' KV cache goes out to host memory when device memory runs short and
 * comes back later.  Host bookkeeping only; the bytes move with pkv_swap_blocks.
 *
 * The distinct blocks of the listed sequences (first use first: sequences in the given order,
 * each table in logical order) each take one fresh block of dst, popped from the end of its
 * free list, which inherits the block's reference count; (src block, dst block) goes to
 * pairs_out in that order.  The sequences' tables are rewritten through this map and the
 * sequences leave src exactly as pkv_seq_free would leave it (blocks whose count reaches zero
 * are pushed onto src's free list in walk order).  Blocks shared only among the moving
 * sequences stay shared in dst; a block also used by a sequence that does not move is refused.
 *
 *   seqs         n distinct sequence ids of src, none present in dst (n >= 0)
 *   pairs_out    int32 [capacity][2]; receives num_pairs_out pairs (<= the total number of
 *                blocks in the listed tables)
 * Copy the pairs' blocks (src pools -> dst pools) before any later write into src's freed
 * blocks, e.g. by enqueuing pkv_swap_blocks right away on the stream that writes the pools.
 * Errors (nothing changes): INVALID_ARGUMENT (null pool, same pool, different block sizes,
 * n < 0, a sequence listed twice, pairs_out too small), NOT_FOUND (sequence not in src),
 * ALREADY_EXISTS (sequence already in dst), UNSUPPORTED (a block shared with a sequence that
 * stays), OUT_OF_BLOCKS (dst has too few free blocks). */
PKV_API pkv_status pkv_pool_move_seqs(pkv_block_pool* src, pkv_block_pool* dst, const int64_t* seqs,
                              int32_t n, int32_t* pairs_out, int32_t capacity,
                              int32_t* num_pairs_out);

/* Block tables of seqs[0..n) as rows of tables_out[n][max_blocks_per_seq] (padded with
 * -1) and their context lengths in context_lens_out[n] (both host, nullable each): the
 * per-sequence map from logical to physical blocks that keeps the logical token order
 * ([111cn] §3.2), in the int32 [num_seqs][max_blocks_per_seq] form the decode kernels take
 * (the block_tables argument of the kernel in [gtnt] §6.2).
 * NOT_FOUND, INVALID_ARGUMENT (a table longer than max_blocks_per_seq). */
PKV_API pkv_status pkv_pool_block_tables(const pkv_block_pool* pool, const int64_t* seqs, int32_t n,
                                 int32_t max_blocks_per_seq, int32_t* tables_out,
                                 int32_t* context_lens_out);

#ifdef __cplusplus
}  /* extern "C" */
#endif

#endif /* PAGEDKV_H */
