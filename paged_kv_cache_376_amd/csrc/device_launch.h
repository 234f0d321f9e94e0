// Internal launchers shared between the device translation units (not installed).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "pkv_internal.h"

namespace pkv {

// Writes each sequence's new K/V row (row s of key/value) to the slot of the sequence's last
// token, found through the block table (kv_append.hip).  Arguments already validated.
hipError_t launch_append_last(const void* key, const void* value, void* k_cache, void* v_cache,
                              const pkv_cache_desc* cache, const int32_t* block_tables,
                              int32_t max_blocks_per_seq, const int32_t* context_lens,
                              int32_t max_context_len, int32_t num_seqs, hipStream_t stream);

}  // namespace pkv
