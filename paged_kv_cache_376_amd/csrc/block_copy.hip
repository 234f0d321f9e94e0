// Whole-block copies between pools of one block shape.
//
// Copy-on-write inside a pool: when a sequence is about to write into a block it shares with
// others, it gets a private copy first (the gtnt.cn page "vLLM推理加速框架：PagedAttention
// 与连续批处理技术解析" §2.2, with the per-block reference count of §2.1).  The host pool
// decides which blocks (pkv_seq_extend reports the (source, destination) pairs); this file
// moves the bytes, for every pair of a step in one launch.
//
// Swap between a device pool and a pool in pinned host memory: the same copy with the two
// sides in different pools (device -> host to swap a sequence out, host -> device to bring it
// back).  Pinned host memory is addressable from the GPU, so one kernel moves all blocks of a
// call over the bus instead of one copy command per block.
//
// In the layout [num_blocks][block_size][Hkv][D] a block is one contiguous run of
// block_size*Hkv*D*e bytes in each pool, so a copy is a flat 16-byte-vector copy of that run
// in the K pool and in the V pool.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "pkv_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;                        // 16-byte vectors per thread and pool per step
constexpr int kStepVecs = kThreads * kUnroll;     // vectors one work-group moves per pool per step
constexpr int kMaxPairGroups = 65535;             // grid.y limit: work-groups stride over pairs

// grid (steps per block, pair groups): work-group (x, y) copies step x of every pair
// y, y + gridDim.y, ...  Pairs whose ids fall outside their pools, or that copy a block onto
// itself within one pool, are skipped.
__global__ __launch_bounds__(kThreads) void copy_blocks_kernel(uint4* __restrict__ dk, uint4* __restrict__ dv,
                                                               int32_t dst_blocks, const uint4* sk, const uint4* sv,
                                                               int32_t src_blocks, int64_t block_vecs,
                                                               const int32_t* __restrict__ pairs, int32_t num_pairs,
                                                               int same_pool) {
  for (int32_t i = blockIdx.y; i < num_pairs; i += gridDim.y) {
    const int32_t src = pairs[2 * static_cast<int64_t>(i)], dst = pairs[2 * static_cast<int64_t>(i) + 1];
    if (src < 0 || src >= src_blocks || dst < 0 || dst >= dst_blocks || (same_pool && src == dst)) continue;
    const uint4* ks = sk + src * block_vecs;
    const uint4* vs = sv + src * block_vecs;
    uint4* kd = dk + dst * block_vecs;
    uint4* vd = dv + dst * block_vecs;
    for (int64_t v0 = static_cast<int64_t>(blockIdx.x) * kStepVecs; v0 < block_vecs;
         v0 += static_cast<int64_t>(gridDim.x) * kStepVecs) {
      if (v0 + kStepVecs <= block_vecs) {  // whole step: all loads in flight, then all stores
        uint4 a[kUnroll], b[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          a[u] = ks[v0 + u * kThreads + threadIdx.x];
          b[u] = vs[v0 + u * kThreads + threadIdx.x];
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          kd[v0 + u * kThreads + threadIdx.x] = a[u];
          vd[v0 + u * kThreads + threadIdx.x] = b[u];
        }
      } else {  // tail of a block whose size is not a multiple of a step
        for (int64_t v = v0 + threadIdx.x; v < block_vecs; v += kThreads) {
          kd[v] = ks[v];
          vd[v] = vs[v];
        }
      }
    }
  }
}

// Checks a block-shape descriptor (its num_blocks is not looked at) and sets the bytes of one
// block in one pool.
pkv_status block_bytes_of(const pkv_cache_desc* cache, int64_t* bytes) {
  if (!cache) return pkv::fail(PKV_ERR_INVALID_ARGUMENT, "cache descriptor is NULL");
  const int e = pkv::dtype_bytes(cache->dtype);
  if (e == 0) return pkv::fail(PKV_ERR_UNSUPPORTED, "dtype %d", cache->dtype);
  if (cache->block_size <= 0 || cache->num_kv_heads <= 0 || cache->head_dim <= 0)
    return pkv::fail(PKV_ERR_INVALID_ARGUMENT, "bad block shape (bs=%d Hkv=%d D=%d)", cache->block_size,
                     cache->num_kv_heads, cache->head_dim);
  *bytes = static_cast<int64_t>(cache->block_size) * cache->num_kv_heads * cache->head_dim * e;
  if (*bytes % 16 != 0)
    return pkv::fail(PKV_ERR_UNSUPPORTED, "block of %lld bytes is not a multiple of 16", static_cast<long long>(*bytes));
  return PKV_OK;
}

// True when the GPU can address p directly: device memory, or pinned host memory mapped at
// the same address for the current device.  Pageable host memory and unknown pointers are
// refused here, before any kernel could touch them.
bool gpu_addressable(const void* p) {
  hipPointerAttribute_t a;
  if (hipPointerGetAttributes(&a, p) != hipSuccess) {
    (void)hipGetLastError();  // clear the runtime's sticky error of the failed query
    return false;
  }
  if (a.type == hipMemoryTypeDevice) return true;
  return a.type == hipMemoryTypeHost && a.devicePointer == p;
}

pkv_status launch_copy(void* dst_k, void* dst_v, int32_t dst_blocks, const void* src_k, const void* src_v,
                       int32_t src_blocks, int64_t block_bytes, const int32_t* pairs, int32_t num_pairs, bool same_pool,
                       void* stream) {
  const int64_t block_vecs = block_bytes / 16;
  const int64_t steps = (block_vecs + kStepVecs - 1) / kStepVecs;
  const dim3 grid(static_cast<unsigned>(steps < 65535 ? steps : 65535),
                  static_cast<unsigned>(num_pairs < kMaxPairGroups ? num_pairs : kMaxPairGroups));
  hipLaunchKernelGGL(copy_blocks_kernel, grid, dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<uint4*>(dst_k), static_cast<uint4*>(dst_v), dst_blocks,
                     static_cast<const uint4*>(src_k), static_cast<const uint4*>(src_v), src_blocks, block_vecs,
                     pairs, num_pairs, same_pool ? 1 : 0);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return pkv::fail(PKV_ERR_HIP, "block copy launch: %s", hipGetErrorString(err));
  return PKV_OK;
}

}  // namespace

extern "C" pkv_status pkv_copy_blocks(void* k_cache, void* v_cache, const pkv_cache_desc* cache,
                                      const int32_t* pairs, int32_t num_pairs, void* stream) {
  pkv::clear_error();
  int64_t bytes = 0;
  const pkv_status st = block_bytes_of(cache, &bytes);
  if (st != PKV_OK) return st;
  if (cache->num_blocks <= 0) return pkv::fail(PKV_ERR_INVALID_ARGUMENT, "num_blocks=%d", cache->num_blocks);
  if (num_pairs < 0) return pkv::fail(PKV_ERR_INVALID_ARGUMENT, "num_pairs=%d", num_pairs);
  if (num_pairs == 0) return PKV_OK;
  if (!k_cache || !v_cache || !pairs) return pkv::fail(PKV_ERR_INVALID_ARGUMENT, "NULL device pointer");
  if (!pkv::aligned16(k_cache) || !pkv::aligned16(v_cache) || (reinterpret_cast<uintptr_t>(pairs) & 3u))
    return pkv::fail(PKV_ERR_INVALID_ARGUMENT, "pools must be 16-byte aligned, pairs 4-byte aligned");
  return launch_copy(k_cache, v_cache, cache->num_blocks, k_cache, v_cache, cache->num_blocks, bytes, pairs, num_pairs,
                     true, stream);
}

extern "C" pkv_status pkv_swap_blocks(void* dst_k, void* dst_v, int32_t dst_num_blocks, const void* src_k,
                                      const void* src_v, int32_t src_num_blocks, const pkv_cache_desc* cache,
                                      const int32_t* pairs, int32_t num_pairs, void* stream) {
  pkv::clear_error();
  int64_t bytes = 0;
  const pkv_status st = block_bytes_of(cache, &bytes);
  if (st != PKV_OK) return st;
  if (dst_num_blocks <= 0 || src_num_blocks <= 0)
    return pkv::fail(PKV_ERR_INVALID_ARGUMENT, "pool sizes %d, %d", dst_num_blocks, src_num_blocks);
  if (num_pairs < 0) return pkv::fail(PKV_ERR_INVALID_ARGUMENT, "num_pairs=%d", num_pairs);
  if (num_pairs == 0) return PKV_OK;
  if (!dst_k || !dst_v || !src_k || !src_v || !pairs) return pkv::fail(PKV_ERR_INVALID_ARGUMENT, "NULL pointer");
  if (!pkv::aligned16(dst_k) || !pkv::aligned16(dst_v) || !pkv::aligned16(src_k) || !pkv::aligned16(src_v) ||
      (reinterpret_cast<uintptr_t>(pairs) & 3u))
    return pkv::fail(PKV_ERR_INVALID_ARGUMENT, "pools must be 16-byte aligned, pairs 4-byte aligned");
  if (dst_k == src_k || dst_v == src_v)
    return pkv::fail(PKV_ERR_INVALID_ARGUMENT, "source and destination are the same pool (use pkv_copy_blocks)");
  const void* ptrs[5] = {dst_k, dst_v, src_k, src_v, pairs};
  for (const void* q : ptrs)
    if (!gpu_addressable(q))
      return pkv::fail(PKV_ERR_INVALID_ARGUMENT, "pointer %p is neither device memory nor pinned host memory mapped "
                       "for this device", q);
  return launch_copy(dst_k, dst_v, dst_num_blocks, src_k, src_v, src_num_blocks, bytes, pairs, num_pairs, false,
                     stream);
}
