// KV append: copy each new token's K and V row into its pool slot.
//
// The append step of the 111cn.net page "大模型推理引擎高频优化：连续批处理、PagedAttention
// 与 KV Cache 实战拆解" §3.3 writes the new token at the end of the sequence's last block
// (or a freshly taken block); the host pool resolves that to a slot, so on the device this
// is a row scatter.  In the pool layout [num_blocks][block_size][Hkv][D] (per-block data of
// shape (block_size, heads, head_dim), gtnt.cn page "vLLM推理加速框架：PagedAttention与连续
// 批处理技术解析" §2.1) a slot's K row of Hkv*D elements is contiguous and so is the source
// row, so every token is one contiguous copy of Hkv*D*e bytes in 16-byte vectors.
//
// Launch: one work-group of 64..256 lanes per token, 16-byte loads/stores, the row walked
// with a stride of the work-group size (each lane moves K and V together so two
// independent loads are in flight).  The slot is read once per lane (same address for the
// whole group, served from cache).  Slots outside [0, num_blocks*block_size) are skipped
// before any pool address is formed.
#include <hip/hip_runtime.h>

#include "pkv_internal.h"

namespace {

__global__ __launch_bounds__(256) void kv_append_kernel(const uint4* __restrict__ key,
                                                        const uint4* __restrict__ value,
                                                        uint4* __restrict__ k_cache,
                                                        uint4* __restrict__ v_cache,
                                                        const int64_t* __restrict__ slot_mapping,
                                                        int64_t num_slots, int32_t row_vecs) {
  const int64_t tok = blockIdx.x;
  const uint4* ks = key + tok * row_vecs;
  const uint4* vs = value + tok * row_vecs;
  // the row's first piece is loaded together with its slot (they do not depend on each other),
  // so that a short row costs one round trip
  const int32_t i0 = threadIdx.x;
  uint4 a = make_uint4(0u, 0u, 0u, 0u), b = a;
  if (i0 < row_vecs) {
    a = ks[i0];
    b = vs[i0];
  }
  const int64_t slot = slot_mapping[tok];
  if (slot < 0 || slot >= num_slots) return;
  uint4* kd = k_cache + slot * row_vecs;
  uint4* vd = v_cache + slot * row_vecs;
  if (i0 < row_vecs) {
    kd[i0] = a;
    vd[i0] = b;
  }
  for (int32_t i = i0 + blockDim.x; i < row_vecs; i += blockDim.x) {
    const uint4 c = ks[i];
    const uint4 d = vs[i];
    kd[i] = c;
    vd[i] = d;
  }
}

}  // namespace

extern "C" pkv_status pkv_kv_cache_append(const void* key, const void* value, void* k_cache,
                                          void* v_cache, const pkv_cache_desc* cache,
                                          const int64_t* slot_mapping, int32_t num_tokens,
                                          void* stream) {
  pkv::clear_error();
  if (!cache) return pkv::fail(PKV_ERR_INVALID_ARGUMENT, "cache descriptor is NULL");
  if (num_tokens < 0) return pkv::fail(PKV_ERR_INVALID_ARGUMENT, "num_tokens=%d", num_tokens);
  const int e = pkv::dtype_bytes(cache->dtype);
  if (e == 0) return pkv::fail(PKV_ERR_UNSUPPORTED, "dtype %d", cache->dtype);
  if (cache->num_blocks <= 0 || cache->num_kv_heads <= 0 || cache->head_dim <= 0 ||
      cache->block_size <= 0)
    return pkv::fail(PKV_ERR_INVALID_ARGUMENT, "bad cache descriptor (NB=%d bs=%d Hkv=%d D=%d)",
                     cache->num_blocks, cache->block_size, cache->num_kv_heads, cache->head_dim);
  if (cache->head_dim != 64 && cache->head_dim != 128)
    return pkv::fail(PKV_ERR_UNSUPPORTED, "head_dim %d (implemented: 64, 128)", cache->head_dim);
  if (num_tokens == 0) return PKV_OK;
  if (!key || !value || !k_cache || !v_cache || !slot_mapping)
    return pkv::fail(PKV_ERR_INVALID_ARGUMENT, "NULL device pointer");
  if (!pkv::aligned16(key) || !pkv::aligned16(value) || !pkv::aligned16(k_cache) ||
      !pkv::aligned16(v_cache) || (reinterpret_cast<uintptr_t>(slot_mapping) & 7u))
    return pkv::fail(PKV_ERR_INVALID_ARGUMENT, "device pointers must be 16-byte aligned");
  const int64_t row_bytes = static_cast<int64_t>(cache->num_kv_heads) * cache->head_dim * e;
  if (row_bytes % 16 != 0 || row_bytes / 16 > INT32_MAX)
    return pkv::fail(PKV_ERR_UNSUPPORTED, "row of %lld bytes", (long long)row_bytes);
  const int32_t row_vecs = static_cast<int32_t>(row_bytes / 16);
  const int64_t num_slots = static_cast<int64_t>(cache->num_blocks) * cache->block_size;
  int threads = row_vecs >= 256 ? 256 : ((row_vecs + 63) / 64) * 64;
  hipLaunchKernelGGL(kv_append_kernel, dim3(num_tokens), dim3(threads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(key),
                     static_cast<const uint4*>(value), static_cast<uint4*>(k_cache),
                     static_cast<uint4*>(v_cache), slot_mapping, num_slots, row_vecs);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess)
    return pkv::fail(PKV_ERR_HIP, "kv_append launch: %s", hipGetErrorString(err));
  return PKV_OK;
}
