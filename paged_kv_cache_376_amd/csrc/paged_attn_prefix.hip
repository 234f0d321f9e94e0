// Prefix-shared decode: the finalize pass (the prefix pass runs inside the even split's launch,
// see prefix_body.h).
#include <hip/hip_runtime.h>

#include <cmath>

#include "dtypes.h"
#include "pkv_internal.h"
#include "prefix.h"
#include "tile_common.h"

namespace pkv {
namespace sk {
namespace {

// Final result of every sequence, one work-group per (sequence, KV head), each thread 4
// consecutive columns of one query row:
//   * its suffix part: when the even split kept the suffix inside one of its ranges, the
//     normalised result and log2-sum-exp it wrote; otherwise the records of the ranges that
//     cut it, in range order (the first range's record of a sequence running past it, then the
//     later ranges' records of a sequence that began before them), folded as unnormalised
//     (m, l, acc);
//   * then its group's prefix partials (m_c, l_c, acc_c) in chunk order;
// each fold being the log-sum-exp rule  M' = max(M, m),  num' = num 2^(M-M') + acc 2^(m-M'),
// den' = den 2^(M-M') + l 2^(m-M'), and out = num / den.  The suffix's range bounds, its
// result and the prefix partials are loaded together; only a cut suffix's records need a second
// round of loads.  Fixed order: deterministic.
// With a fused append, the work-group also writes its sequence's new K and V rows of its KV
// head to the slot of the last token (position context_len - 1 through the block table; a
// length of 0 or a block id outside the pool writes nothing), as the plain decode's merge
// kernel does.  The launch before this one took that token from the new rows, not the pool.
template <typename T, int D>
__global__ __launch_bounds__(256) void finalize_kernel(PrefixParams pp) {
  using raw = typename T::raw;
  if (pp.new_key != nullptr) {
    constexpr int CPR = D * static_cast<int>(sizeof(raw)) / 16;  // 16-byte chunks per row
    const int s = blockIdx.x / pp.num_kv_heads, g = blockIdx.x % pp.num_kv_heads;
    if (threadIdx.x < CPR) {
      const int L0 = pp.context_lens[s];
      const int L = L0 < 0 ? 0 : (L0 > pp.max_context_len ? pp.max_context_len : L0);
      if (L > 0) {
        const int phys = pp.block_tables[static_cast<int64_t>(s) * pp.max_blocks_per_seq + (L - 1) / pp.block_size];
        if (phys >= 0 && phys < pp.num_blocks) {
          const int64_t row_bytes = static_cast<int64_t>(D) * sizeof(raw);
          const int ch = 16 * static_cast<int>(threadIdx.x);
          const int64_t src = (static_cast<int64_t>(s) * pp.num_kv_heads + g) * row_bytes + ch;
          const int64_t dst =
              ((static_cast<int64_t>(phys) * pp.block_size + (L - 1) % pp.block_size) * pp.num_kv_heads + g) * row_bytes + ch;
          const u32x4 kr = *reinterpret_cast<const u32x4*>(static_cast<const unsigned char*>(pp.new_key) + src);
          const u32x4 vr = *reinterpret_cast<const u32x4*>(static_cast<const unsigned char*>(pp.new_value) + src);
          *reinterpret_cast<u32x4*>(static_cast<unsigned char*>(pp.k_cache) + dst) = kr;
          *reinterpret_cast<u32x4*>(static_cast<unsigned char*>(pp.v_cache) + dst) = vr;
        }
      }
    }
  }
  const int s = blockIdx.x / pp.num_kv_heads, g = blockIdx.x % pp.num_kv_heads;
  const int G = pp.group, Hkv = pp.num_kv_heads, B = pp.num_seqs;
  const int c0 = pp.cu[s], c1 = pp.cu[s + 1], ntiles = pp.cu[B], R = pp.cu[B + 1];
  // chunks of this sequence's prefix, never more than the workspace holds
  const int nch = min(pp.chunks, (max(pp.seq_prefix[s], 0) / kTile + kPrefixChunkTiles - 1) / kPrefixChunkTiles);
  for (int idx = threadIdx.x; idx < G * (D / 4); idx += 256) {
    const int hr = idx / (D / 4), col = 4 * (idx % (D / 4));
    const int h = g * G + hr;
    const int64_t row = static_cast<int64_t>(s) * pp.num_q_heads + h;
    f32x4 num = *reinterpret_cast<const f32x4*>(pp.part_out + row * D + col);
    const float lse = pp.part_lse[row];
    float mc[4] = {0.f, 0.f, 0.f, 0.f}, lc[4] = {0.f, 0.f, 0.f, 0.f};
    f32x4 ac[4] = {};
    if (nch > 0) {  // the first four prefix chunks go out with the rest (uniform per work-group)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t rec = row * pp.chunks + min(u, nch - 1);
        mc[u] = pp.pre_ml[rec * 2];
        lc[u] = pp.pre_ml[rec * 2 + 1];
        ac[u] = *reinterpret_cast<const f32x4*>(pp.pre_acc + rec * D + col);
      }
    }
    const int ra = range_of(c0, ntiles, R), rb = range_of(c1 - 1, ntiles, R);
    float Mx, den;
    if (ra == rb) {  // the even split finished the suffix itself
      Mx = lse;
      den = lse == -INFINITY ? 0.f : 1.f;
    } else {  // records (ra, slot 1), (ra + 1 .. rb, slot 0), four at a time
      Mx = kNegBig;
      den = 0.f;
      num = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int r0 = ra; r0 <= rb; r0 += 4) {
        float mr[4], lr[4];
        f32x4 xr[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int r = min(r0 + u, rb);
          const int64_t rec = (static_cast<int64_t>(r) * Hkv + g) * 2 + (r == ra ? 1 : 0);
          mr[u] = pp.rec_ml[rec * 32 + hr * 2];
          lr[u] = pp.rec_ml[rec * 32 + hr * 2 + 1];
          xr[u] = *reinterpret_cast<const f32x4*>(pp.rec_acc + rec * (16 * D) + hr * D + col);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (r0 + u > rb) break;
          const float mn = fmaxf(Mx, mr[u]);
          const float f0 = __builtin_amdgcn_exp2f(Mx - mn), f1 = __builtin_amdgcn_exp2f(mr[u] - mn);
          num = num * f0 + xr[u] * f1;
          den = den * f0 + lr[u] * f1;
          Mx = mn;
        }
      }
    }
    for (int c = 0; c < nch; c += 4) {
      if (c > 0) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int64_t rec = row * pp.chunks + min(c + u, nch - 1);
          mc[u] = pp.pre_ml[rec * 2];
          lc[u] = pp.pre_ml[rec * 2 + 1];
          ac[u] = *reinterpret_cast<const f32x4*>(pp.pre_acc + rec * D + col);
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (c + u >= nch) break;
        const float mn = fmaxf(Mx, mc[u]);
        const float f0 = den > 0.f ? __builtin_amdgcn_exp2f(Mx - mn) : 0.f;
        const float f1 = __builtin_amdgcn_exp2f(mc[u] - mn);
        num = num * f0 + ac[u] * f1;
        den = den * f0 + lc[u] * f1;
        Mx = mn;
      }
    }
    num = num * (den > 0.f ? 1.f / den : 0.f);
    store4<T>(static_cast<raw*>(pp.out) + row * D + col, num);
  }
}

}  // namespace

hipError_t finalize_launch(const PrefixParams& pp, int32_t dtype, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(pp.num_seqs) * pp.num_kv_heads);
  const int D = pp.head_dim;
  if (dtype == PKV_BF16) {
    if (D == 64) hipLaunchKernelGGL((finalize_kernel<BF16, 64>), grid, dim3(256), 0, stream, pp);
    else hipLaunchKernelGGL((finalize_kernel<BF16, 128>), grid, dim3(256), 0, stream, pp);
  } else {
    if (D == 64) hipLaunchKernelGGL((finalize_kernel<F16, 64>), grid, dim3(256), 0, stream, pp);
    else hipLaunchKernelGGL((finalize_kernel<F16, 128>), grid, dim3(256), 0, stream, pp);
  }
  return hipGetLastError();
}

}  // namespace sk
}  // namespace pkv
