// Paged decode attention for gfx950.
//
// What is computed: for every sequence s and query head h, single-query scaled dot-product
// attention over the sequence's context, whose K/V rows sit in fixed 16-token blocks spread
// through a physical pool and are found through the sequence's block table (yunthe.com page
// "大模型推理显存优化实战：PagedAttention机制原理与vLLM连续批处理配置", section
// "PagedAttention分页注意力机制原理"; block table and 16-token blocks from the 111cn.net page
// "大模型推理引擎高频优化：连续批处理、PagedAttention 与 KV Cache 实战拆解" §3.2; per-block
// layout (block_size, heads, head_dim) from the gtnt.cn page "vLLM推理加速框架：
// PagedAttention与连续批处理技术解析" §2.1, whose §2.2 also has the kernel work block by
// block).  Query head h reads KV head h / G, G = Hq / Hkv.
//
// This file holds the fixed-partition path (f32 pools, or an explicit partition_size; 16-token
// blocks) and the entry points; f16/bf16 decodes with partition_size 0 go to the even split of
// paged_attn_sk.hip.
//
// Structure (one decode = phase 1, plus phase 2 only when a sequence is split):
//   phase 1  grid (Hkv, B, P): one work-group of 4 wave64s per (KV head, sequence,
//            partition of `part_blocks` blocks).  Wave w streams blocks w, w+4, ... of the
//            partition with an online softmax (running max m, sum l, unnormalised acc, in
//            the log2 domain: logits are pre-multiplied by scale*log2(e) and exp2 is used).
//            The 4 waves are merged through LDS at the end.  A sequence with one partition
//            is finished here; otherwise (m, l, acc) go to the fp32 workspace.
//   phase 2  grid (Hq, B): merges a split sequence's partitions in partition order,
//            M = max m_p, out = sum_p 2^(m_p-M) acc_p / sum_p 2^(m_p-M) l_p.
// Two phase-1 variants:
//   * VALU (any dtype, G <= 2): 4 lanes per token, each lane holds a quarter of the row;
//     the dot product is finished with two DPP quad exchanges and every lane keeps the
//     softmax state of its token slot, so nothing crosses lanes inside the block loop.
//   * MFMA (f16/bf16, 2 < G <= 16): the G query heads of a KV head are padded to 16 and
//     the block is one 16x16 tile: S^T = K * Q^T with v_mfma_f32_16x16x32 (K read straight
//     from HBM into the A operand), then O^T += V^T * P^T with v_mfma_f32_16x16x16, V^T
//     gathered from a per-wave LDS copy of the V tile.  P leaves the QK accumulator in
//     exactly the B-operand layout the PV product needs.
// Masking is by select (never multiply): slots past the context may hold anything,
// including NaN, and block-table entries past ceil(ctx/16) are never read.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <mutex>
#include <type_traits>

#include "dtypes.h"
#include "pkv_internal.h"
#include "prefix.h"
#include "stream_k.h"

namespace pkv {
namespace {

constexpr int kBlock = 16;        // tokens per block (the pages' default)
constexpr int kWaves = 4;         // waves per work-group
constexpr int kThreads = 64 * kWaves;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1.0e30f;  // finite start value for the running max

struct Params {
  void* out;
  const void* q;
  void* k_cache;  // written only with a fused append (new_key != NULL): the new rows
  void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const void* new_key;    // [B][Hkv][D] or NULL: with a fused append, each sequence's last token
  const void* new_value;  // comes from here (write_new_row puts it in its slot)
  float* ws_acc;  // [B][Hq][P][D]
  float* ws_ml;   // [B][Hq][P][2]  (m, l)
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t max_blocks_per_seq;
  int32_t max_context_len;
  int32_t num_blocks;
  int32_t part_blocks;
  int32_t num_parts;
  float scale_log2e;
};

__device__ __forceinline__ float dpp_xor1(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ float dpp_xor2(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));
}

// Context length of sequence s, clamped so no table entry past max_blocks_per_seq is read.
__device__ __forceinline__ int clamped_ctx(const Params& p, int s) {
  int ctx = p.context_lens[s];
  ctx = ctx < 0 ? 0 : ctx;
  return ctx > p.max_context_len ? p.max_context_len : ctx;
}

// Fused append: the work-group of a sequence's last partition writes the new K and V rows of
// its KV head to the slot of the sequence's last token (position ctx - 1 through the block
// table; an empty context or a block id outside the pool writes nothing).  The loads of that
// block take the token's row from new_key / new_value instead of the slot, so nothing in the
// launch reads what this writes.
template <typename T, int D>
__device__ __forceinline__ void write_new_row(const Params& p, int s, int g, int ctx) {
  constexpr int CPR = D * T::kBytes / 16;  // 16-byte chunks per row
  if (ctx <= 0 || static_cast<int>(threadIdx.x) >= 2 * CPR) return;
  const int phys = p.block_tables[static_cast<int64_t>(s) * p.max_blocks_per_seq + (ctx - 1) / kBlock];
  if (phys < 0 || phys >= p.num_blocks) return;
  const int which = threadIdx.x / CPR, ch = threadIdx.x % CPR;
  const int64_t src = (static_cast<int64_t>(s) * p.num_kv_heads + g) * CPR + ch;
  const int64_t dst =
      ((static_cast<int64_t>(phys) * kBlock + (ctx - 1) % kBlock) * p.num_kv_heads + g) * CPR + ch;
  const u32x4 x = static_cast<const u32x4*>(which ? p.new_value : p.new_key)[src];
  static_cast<u32x4*>(which ? p.v_cache : p.k_cache)[dst] = x;
}

__device__ __forceinline__ int num_parts_of(int ctx, int part_blocks) {
  const int nblk = (ctx + kBlock - 1) / kBlock;
  const int n = (nblk + part_blocks - 1) / part_blocks;
  return n < 1 ? 1 : n;
}

// Writes the merged result of one (sequence, head) for this partition: the final output
// when the sequence has a single partition, else the partial (m, l, acc) for phase 2.
template <typename T>
__device__ __forceinline__ void store_result(const Params& p, int s, int h, int part, int nparts,
                                             int d, float acc, float m, float l, int D) {
  if (nparts == 1) {
    using raw = typename T::raw;
    raw* out = static_cast<raw*>(p.out) + (static_cast<int64_t>(s) * p.num_q_heads + h) * D;
    out[d] = to_raw(T{}, l > 0.f ? acc / l : 0.f);
  } else {
    const int64_t row = (static_cast<int64_t>(s) * p.num_q_heads + h) * p.num_parts + part;
    p.ws_acc[row * D + d] = acc;
    if (d == 0) {
      p.ws_ml[row * 2] = m;
      p.ws_ml[row * 2 + 1] = l;
    }
  }
}

// ------------------------------------------------------------------------------------
// Phase 1, VALU variant.
// ------------------------------------------------------------------------------------
template <typename T, int D, int G>
__global__ __launch_bounds__(kThreads) void decode_valu_kernel(Params p) {
  using raw = typename T::raw;
  constexpr int E = kVecElems<T>;                 // elements per 16-byte vector
  constexpr int ROW_VECS = D * T::kBytes / 16;    // vectors per token row (one head)
  constexpr int VPL = ROW_VECS / 4;               // vectors per lane
  constexpr int EPL = VPL * E;                    // elements per lane
  static_assert(ROW_VECS % 4 == 0, "row must split over 4 lanes");

  const int g = blockIdx.x, s = blockIdx.y, part = blockIdx.z;
  const int ctx = clamped_ctx(p, s);
  const int nblk = (ctx + kBlock - 1) / kBlock;
  const int nparts = num_parts_of(ctx, p.part_blocks);
  if (part >= nparts) return;
  const int b_begin = part * p.part_blocks;
  const int b_end = min(nblk, b_begin + p.part_blocks);
  const bool append = p.new_key != nullptr;
  if (append && part == nparts - 1) write_new_row<T, D>(p, s, g, ctx);

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int tok = lane >> 2, quad = lane & 3;
  const int Hkv = p.num_kv_heads;
  const int64_t new_row = (static_cast<int64_t>(s) * Hkv + g) * D;  // this head's new row (fused append)

  // Query rows of the G heads, pre-scaled into the log2 domain.  Lane element (c, e) is
  // d = (quad + 4c) * E + e -- the same split the K/V rows use below.
  float qf[G][EPL];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const int h = g * G + j;
    const u32x4* qv = reinterpret_cast<const u32x4*>(static_cast<const raw*>(p.q) +
                                                     (static_cast<int64_t>(s) * p.num_q_heads + h) * D);
#pragma unroll
    for (int c = 0; c < VPL; ++c) {
      unpack(T{}, qv[quad + 4 * c], &qf[j][c * E]);
#pragma unroll
      for (int e = 0; e < E; ++e) qf[j][c * E + e] *= p.scale_log2e;
    }
  }

  float m[G], l[G], acc[G][EPL];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    m[j] = kNegBig;
    l[j] = 0.f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) acc[j][i] = 0.f;
  }

  const int32_t* bt = p.block_tables + static_cast<int64_t>(s) * p.max_blocks_per_seq;
  const raw* kbase = static_cast<const raw*>(p.k_cache);
  const raw* vbase = static_cast<const raw*>(p.v_cache);
  const int64_t tok_stride = static_cast<int64_t>(Hkv) * D;

  // Software pipeline: the next block's rows are in flight while this one is consumed.
  u32x4 kc[VPL], vc[VPL], kn[VPL], vn[VPL];
  bool have_cur = false;
  int b = b_begin + wave;
  auto load = [&](int blk, u32x4* kr, u32x4* vr) -> bool {
    const int phys = bt[blk];
    if (phys < 0 || phys >= p.num_blocks) return false;
    const int64_t off = (static_cast<int64_t>(phys) * kBlock + tok) * tok_stride +
                        static_cast<int64_t>(g) * D;
    // with a fused append, the lanes of the last token's row read it from the input
    const bool mine = append && blk == nblk - 1 && tok == (ctx - 1) % kBlock;
    const u32x4* kp = reinterpret_cast<const u32x4*>(mine ? static_cast<const raw*>(p.new_key) + new_row : kbase + off);
    const u32x4* vp = reinterpret_cast<const u32x4*>(mine ? static_cast<const raw*>(p.new_value) + new_row : vbase + off);
#pragma unroll
    for (int c = 0; c < VPL; ++c) {
      kr[c] = kp[quad + 4 * c];
      vr[c] = vp[quad + 4 * c];
    }
    return true;
  };
  if (b < b_end) have_cur = load(b, kc, vc);

  for (; b < b_end; b += kWaves) {
    const int bn = b + kWaves;
    bool have_next = false;
    if (bn < b_end) have_next = load(bn, kn, vn);
    if (have_cur) {
      const bool valid = (b * kBlock + tok) < ctx;
      float kf[EPL], vf[EPL];
#pragma unroll
      for (int c = 0; c < VPL; ++c) {
        unpack(T{}, kc[c], &kf[c * E]);
        unpack(T{}, vc[c], &vf[c * E]);
      }
#pragma unroll
      for (int i = 0; i < EPL; ++i) vf[i] = valid ? vf[i] : 0.f;
#pragma unroll
      for (int j = 0; j < G; ++j) {
        float dot = 0.f;
#pragma unroll
        for (int i = 0; i < EPL; ++i) dot = fmaf(qf[j][i], kf[i], dot);
        dot += dpp_xor1(dot);
        dot += dpp_xor2(dot);
        const float sj = valid ? dot : -INFINITY;
        const float mn = fmaxf(m[j], sj);
        const float alpha = exp2f(m[j] - mn);
        const float pr = exp2f(sj - mn);
        l[j] = fmaf(l[j], alpha, pr);
#pragma unroll
        for (int i = 0; i < EPL; ++i) acc[j][i] = fmaf(pr, vf[i], acc[j][i] * alpha);
        m[j] = mn;
      }
    }
#pragma unroll
    for (int c = 0; c < VPL; ++c) {
      kc[c] = kn[c];
      vc[c] = vn[c];
    }
    have_cur = have_next;
  }

  // Merge the 64 token slots (4 waves x 16) of the work-group: common max, then sums.
  __shared__ float red[kWaves * 16][D + 4];
  __shared__ float red_l[kWaves * 16];
  __shared__ float wmax[kWaves];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    float mw = m[j];
    mw = fmaxf(mw, __shfl_xor(mw, 4));
    mw = fmaxf(mw, __shfl_xor(mw, 8));
    mw = fmaxf(mw, __shfl_xor(mw, 16));
    mw = fmaxf(mw, __shfl_xor(mw, 32));
    if (lane == 0) wmax[wave] = mw;
    __syncthreads();
    float M = wmax[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, wmax[w]);
    const float f = exp2f(m[j] - M);
    const int row = wave * 16 + tok;
#pragma unroll
    for (int c = 0; c < VPL; ++c)
#pragma unroll
      for (int e = 0; e < E; ++e) red[row][(quad + 4 * c) * E + e] = acc[j][c * E + e] * f;
    if (quad == 0) red_l[row] = l[j] * f;
    __syncthreads();
    for (int d = threadIdx.x; d < D; d += kThreads) {
      float a = 0.f, lsum = 0.f;
      for (int r = 0; r < kWaves * 16; ++r) {
        a += red[r][d];
        lsum += red_l[r];
      }
      store_result<T>(p, s, g * G + j, part, nparts, d, a, M, lsum, D);
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------------------------
// Phase 1, MFMA variant (f16 / bf16, G <= 16).
// ------------------------------------------------------------------------------------
template <typename T> struct Mfma;
template <> struct Mfma<BF16> {
  using v8 = bf16x8;
  using v4 = i16x4;
  __device__ static f32x4 qk(v8 a, v8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static f32x4 pv(v4 a, v4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
  }
  __device__ static short pack(float x) { return __builtin_bit_cast(short, static_cast<__bf16>(x)); }
  __device__ static float unpack1(short x) {
    return __uint_as_float(static_cast<uint32_t>(static_cast<uint16_t>(x)) << 16);
  }
};
template <> struct Mfma<F16> {
  using v8 = f16x8;
  using v4 = f16x4;
  __device__ static f32x4 qk(v8 a, v8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  __device__ static f32x4 pv(v4 a, v4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
  }
  __device__ static short pack(float x) { return __builtin_bit_cast(short, static_cast<_Float16>(x)); }
  __device__ static float unpack1(short x) {
    return static_cast<float>(__builtin_bit_cast(_Float16, x));
  }
};

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void decode_mfma_kernel(Params p) {
  using M = Mfma<T>;
  using v8 = typename M::v8;
  using v4 = typename M::v4;
  constexpr int KC = D / 32;            // QK k-chunks of 32 (one 16-byte piece per lane)
  constexpr int NC = D / 16;            // PV output chunks of 16 columns of d
  constexpr int ROW_BYTES = D * 2;
  constexpr int PITCH = ROW_BYTES + 8;  // LDS row pitch of the V tile (bank spread)
  constexpr int VPL = D / 32;           // 16-byte V pieces per lane for the LDS fill

  const int g = blockIdx.x, s = blockIdx.y, part = blockIdx.z;
  const int G = p.num_q_heads / p.num_kv_heads;
  const int ctx = clamped_ctx(p, s);
  const int nblk = (ctx + kBlock - 1) / kBlock;
  const int nparts = num_parts_of(ctx, p.part_blocks);
  if (part >= nparts) return;
  const int b_begin = part * p.part_blocks;
  const int b_end = min(nblk, b_begin + p.part_blocks);
  const bool append = p.new_key != nullptr;
  if (append && part == nparts - 1) write_new_row<T, D>(p, s, g, ctx);

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r16 = lane & 15;  // MFMA row/column index of this lane
  const int grp = lane >> 4;  // MFMA k-group of this lane (0..3)
  const int Hkv = p.num_kv_heads;

  // LDS: per-wave V tiles during the loop, reused for the cross-wave merge afterwards.
  constexpr int kTileBytes = kBlock * PITCH;
  constexpr int kMergeBytes = kWaves * (D * 17 + 2 * 16) * 4;
  constexpr int kLdsBytes = (kWaves * kTileBytes > kMergeBytes) ? kWaves * kTileBytes : kMergeBytes;
  __shared__ __attribute__((aligned(16))) unsigned char lds[kLdsBytes];
  unsigned char* vtile = lds + wave * kTileBytes;

  // Q^T as the B operand of S^T = K Q^T: lane holds head r16, pieces grp + 4c of d.
  v8 qb[KC];
  {
    const bool live = r16 < G;
    const int h = g * G + (live ? r16 : 0);
    const u32x4* qv = reinterpret_cast<const u32x4*>(static_cast<const typename T::raw*>(p.q) +
                                                     (static_cast<int64_t>(s) * p.num_q_heads + h) * D);
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      u32x4 w = qv[grp + 4 * c];
      if (!live) w = u32x4{0u, 0u, 0u, 0u};
      qb[c] = __builtin_bit_cast(v8, w);
    }
  }

  float m_run = kNegBig;  // running max for head r16 (same in all 4 k-groups)
  float l_run = 0.f;      // this lane's share of the running sum for head r16
  f32x4 acc[NC];          // O^T: lane holds d = 16n + 4*grp + i, head r16
#pragma unroll
  for (int n = 0; n < NC; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int32_t* bt = p.block_tables + static_cast<int64_t>(s) * p.max_blocks_per_seq;
  const unsigned char* kbase = static_cast<const unsigned char*>(p.k_cache);
  const unsigned char* vbase = static_cast<const unsigned char*>(p.v_cache);
  const int64_t tok_bytes = static_cast<int64_t>(Hkv) * ROW_BYTES;

  // Lane roles for the loads: K as the A operand (token r16, piece grp + 4c); V for the LDS
  // fill (token lane>>2, pieces (lane&3) + 4c).
  const int vt = lane >> 2, vq = lane & 3;

  u32x4 kc[KC], vc[VPL], kn[KC], vn[VPL];
  auto load = [&](int blk, u32x4* kr, u32x4* vr) -> bool {
    const int phys = bt[blk];
    if (phys < 0 || phys >= p.num_blocks) return false;
    const int64_t blk_off = static_cast<int64_t>(phys) * kBlock * tok_bytes + static_cast<int64_t>(g) * ROW_BYTES;
    // with a fused append, the lanes of the last token's row read it from the input
    const bool last = append && blk == nblk - 1;
    const int lt = (ctx - 1) % kBlock;
    const int64_t new_off = (static_cast<int64_t>(s) * Hkv + g) * ROW_BYTES;
    const u32x4* kp = reinterpret_cast<const u32x4*>(
        last && r16 == lt ? static_cast<const unsigned char*>(p.new_key) + new_off : kbase + blk_off + r16 * tok_bytes);
    const u32x4* vp = reinterpret_cast<const u32x4*>(
        last && vt == lt ? static_cast<const unsigned char*>(p.new_value) + new_off : vbase + blk_off + vt * tok_bytes);
#pragma unroll
    for (int c = 0; c < KC; ++c) kr[c] = kp[grp + 4 * c];
#pragma unroll
    for (int c = 0; c < VPL; ++c) vr[c] = vp[vq + 4 * c];
    return true;
  };

  int b = b_begin + wave;
  bool have_cur = false;
  if (b < b_end) have_cur = load(b, kc, vc);

  for (; b < b_end; b += kWaves) {
    const int bn = b + kWaves;
    bool have_next = false;
    if (bn < b_end) have_next = load(bn, kn, vn);
    if (have_cur) {
      // V tile -> LDS (row-major, padded pitch), 8-byte stores.
#pragma unroll
      for (int c = 0; c < VPL; ++c) {
        uint2* dst = reinterpret_cast<uint2*>(vtile + vt * PITCH + (vq + 4 * c) * 16);
        dst[0] = make_uint2(vc[c][0], vc[c][1]);
        dst[1] = make_uint2(vc[c][2], vc[c][3]);
      }
      // S^T[token][head] = sum_d K[token][d] Q[head][d]
      f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < KC; ++c) sacc = M::qk(__builtin_bit_cast(v8, kc[c]), qb[c], sacc);
      // lane holds tokens 4*grp + i of head r16
      const int t0 = b * kBlock + 4 * grp;
      float sv[4];
      float mx = kNegBig;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sv[i] = (t0 + i < ctx) ? sacc[i] * p.scale_log2e : -INFINITY;
        mx = fmaxf(mx, sv[i]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mn = fmaxf(m_run, mx);
      const float alpha = exp2f(m_run - mn);
      m_run = mn;
      i16x4 pbits;
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const short ps = M::pack(exp2f(sv[i] - mn));
        pbits[i] = ps;
        psum += M::unpack1(ps);  // the sum uses exactly the rounded weights PV uses
      }
      const v4 pb = __builtin_bit_cast(v4, pbits);
      l_run = fmaf(l_run, alpha, psum);
#pragma unroll
      for (int n = 0; n < NC; ++n) acc[n] *= alpha;
      // V^T as the A operand: lane holds d = 16n + r16, tokens 4*grp + i.
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const bool tail = (b * kBlock + kBlock) > ctx;
#pragma unroll
      for (int n = 0; n < NC; ++n) {
        i16x4 vbits;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const short* src = reinterpret_cast<const short*>(vtile + (4 * grp + i) * PITCH) + 16 * n + r16;
          const short x = *src;
          vbits[i] = (tail && (t0 + i >= ctx)) ? static_cast<short>(0) : x;
        }
        acc[n] = M::pv(__builtin_bit_cast(v4, vbits), pb, acc[n]);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
#pragma unroll
    for (int c = 0; c < KC; ++c) kc[c] = kn[c];
#pragma unroll
    for (int c = 0; c < VPL; ++c) vc[c] = vn[c];
    have_cur = have_next;
  }

  // Finish this wave's sum over its 4 k-groups, then merge the 4 waves through LDS.
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  __syncthreads();  // every wave is done with its V tile
  float* m_w = reinterpret_cast<float*>(lds);             // [kWaves][16]
  float* l_w = m_w + kWaves * 16;                          // [kWaves][16]
  float* a_w = l_w + kWaves * 16;                          // [kWaves][D][17]
  if (grp == 0) {
    m_w[wave * 16 + r16] = m_run;
    l_w[wave * 16 + r16] = l_run;
  }
#pragma unroll
  for (int n = 0; n < NC; ++n)
#pragma unroll
    for (int i = 0; i < 4; ++i) a_w[(wave * D + 16 * n + 4 * grp + i) * 17 + r16] = acc[n][i];
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
    const int j = idx / D, d = idx - j * D;
    float Mx = m_w[j];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) Mx = fmaxf(Mx, m_w[w * 16 + j]);
    float a = 0.f, lsum = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = exp2f(m_w[w * 16 + j] - Mx);
      a = fmaf(a_w[(w * D + d) * 17 + j], f, a);
      lsum = fmaf(l_w[w * 16 + j], f, lsum);
    }
    store_result<T>(p, s, g * G + j, part, nparts, d, a, Mx, lsum, D);
  }
}

// ------------------------------------------------------------------------------------
// Phase 2: merge the partitions of split sequences (fixed order, deterministic).
// ------------------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(D) void reduce_kernel(Params p) {
  const int h = blockIdx.x, s = blockIdx.y, d = threadIdx.x;
  const int ctx = clamped_ctx(p, s);
  const int nparts = num_parts_of(ctx, p.part_blocks);
  if (nparts <= 1) return;
  const int64_t row0 = (static_cast<int64_t>(s) * p.num_q_heads + h) * p.num_parts;
  const float* ml = p.ws_ml + row0 * 2;
  float Mx = kNegBig;
  for (int i = 0; i < nparts; ++i) Mx = fmaxf(Mx, ml[2 * i]);
  float a = 0.f, lsum = 0.f;
  for (int i = 0; i < nparts; ++i) {
    const float f = exp2f(ml[2 * i] - Mx);
    a = fmaf(p.ws_acc[(row0 + i) * D + d], f, a);
    lsum = fmaf(ml[2 * i + 1], f, lsum);
  }
  using raw = typename T::raw;
  raw* out = static_cast<raw*>(p.out) + (static_cast<int64_t>(s) * p.num_q_heads + h) * D;
  out[d] = to_raw(T{}, lsum > 0.f ? a / lsum : 0.f);
}

// ------------------------------------------------------------------------------------
// Host side: partition planning and dispatch.
// ------------------------------------------------------------------------------------
constexpr int kAutoPartition = 512;  // tokens per partition when splitting automatically

// Resolved partition size in tokens (a multiple of 16), or 0 for invalid arguments.
int32_t resolve_partition(int32_t max_context_len, int32_t partition_size) {
  if (max_context_len < 0) return 0;
  const int32_t whole = max_context_len <= 0 ? kBlock : ((max_context_len + kBlock - 1) / kBlock) * kBlock;
  if (partition_size == -1) return whole;
  if (partition_size == 0) return max_context_len > kAutoPartition ? kAutoPartition : whole;
  if (partition_size < 0 || partition_size % kBlock != 0) return 0;
  return partition_size;
}

int32_t parts_for(int32_t max_context_len, int32_t part) {
  const int32_t n = (max_context_len + part - 1) / part;
  return n < 1 ? 1 : n;
}

template <typename T, int D>
hipError_t launch_typed(const Params& p, int G, hipStream_t stream) {
  const dim3 grid(p.num_kv_heads, p.num_seqs, p.num_parts);
  const dim3 block(kThreads);
  if (G == 1) {
    hipLaunchKernelGGL((decode_valu_kernel<T, D, 1>), grid, block, 0, stream, p);
  } else if (G == 2) {
    hipLaunchKernelGGL((decode_valu_kernel<T, D, 2>), grid, block, 0, stream, p);
  } else {
    if constexpr (std::is_same<T, F32>::value) {
      return hipErrorInvalidValue;  // rejected on the host before this point
    } else {
      hipLaunchKernelGGL((decode_mfma_kernel<T, D>), grid, block, 0, stream, p);
    }
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || p.num_parts == 1) return err;
  hipLaunchKernelGGL((reduce_kernel<T, D>), dim3(p.num_q_heads, p.num_seqs), dim3(D), 0, stream, p);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_dtype(const Params& p, int D, int G, hipStream_t stream) {
  return D == 64 ? launch_typed<T, 64>(p, G, stream) : launch_typed<T, 128>(p, G, stream);
}

}  // namespace
}  // namespace pkv

using namespace pkv;

namespace {
// Poll count of the merge kernel's bounded LDS waits (pkv_set_merge_spin_limit).
std::atomic<int32_t> g_merge_spin_limit{sk::kDefaultSpinLimit};
// The evenly split path (16-bit pools: its products run on the bf16/f16 matrix cores) serves
// partition_size 0 up to kSkMaxSeqs sequences, as long as its prefix sum and wave states fit
// one work-group's LDS (large groups at large batches do not); f32 pools, explicit partition
// sizes and the shapes that do not fit take the fixed partitions.
bool use_stream_k(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                  int32_t partition_size, int32_t dtype) {
  return partition_size == 0 && (dtype == PKV_F16 || dtype == PKV_BF16) && num_kv_heads > 0 &&
         num_q_heads % num_kv_heads == 0 && sk::sk_fits(num_seqs, head_dim, num_q_heads / num_kv_heads);
}
}  // namespace

extern "C" int32_t pkv_paged_attn_partition_size(int32_t num_seqs, int32_t num_q_heads,
                                                 int32_t num_kv_heads, int32_t head_dim,
                                                 int32_t max_context_len, int32_t partition_size,
                                                 int32_t dtype) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0) return 0;
  if (max_context_len < 0 || dtype_bytes(dtype) == 0) return 0;
  if (use_stream_k(num_seqs, num_q_heads, num_kv_heads, head_dim, partition_size, dtype)) return 0;
  return resolve_partition(max_context_len, partition_size);
}

extern "C" size_t pkv_paged_attn_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                                 int32_t num_kv_heads, int32_t head_dim,
                                                 int32_t max_context_len, int32_t partition_size,
                                                 int32_t dtype) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || max_context_len < 0) return 0;
  if (dtype_bytes(dtype) == 0) return 0;
  if (use_stream_k(num_seqs, num_q_heads, num_kv_heads, head_dim, partition_size, dtype))
    return num_seqs == 0 ? 0 : sk::sk_workspace_bytes(num_seqs, num_kv_heads, num_q_heads / num_kv_heads, head_dim,
                                                      max_context_len);
  const int32_t part = resolve_partition(max_context_len, partition_size);
  if (part == 0) return 0;
  const int32_t P = parts_for(max_context_len, part);
  if (P <= 1) return 0;
  // acc [B][Hq][P][D] followed by (m, l) [B][Hq][P][2], fp32
  return static_cast<size_t>(num_seqs) * num_q_heads * P * (static_cast<size_t>(head_dim) + 2) * sizeof(float);
}

namespace {

// Group description of a prefix-shared decode (pkv_paged_attn_decode_prefix).
struct PrefixArgs {
  const int32_t* seq_prefix;
  const int32_t* group_offsets;
  const int32_t* group_members;
  int32_t num_groups;
  int32_t max_prefix_tokens;
};

inline size_t align256(size_t x) { return (x + 255) / 256 * 256; }
inline int32_t prefix_chunks(int32_t max_prefix_tokens) {
  const int32_t tiles = (max_prefix_tokens + 15) / 16;
  return (tiles + sk::kPrefixChunkTiles - 1) / sk::kPrefixChunkTiles;
}
// Workspace of the prefix path beyond the even split's: suffix results and lse, prefix partials,
// the suffix tile-list prefix sum and ranges in use.
size_t prefix_extra_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim, int32_t chunks) {
  const size_t rows = static_cast<size_t>(num_seqs) * num_q_heads;
  return align256(rows * head_dim * 4) + align256(rows * 4) + align256(rows * chunks * head_dim * 4) +
         align256(rows * chunks * 8) + align256((static_cast<size_t>(num_seqs) + 2) * 4);
}

// Shared body of the decode entry points.  With new_key/new_value set, each sequence's
// last token is its new K/V row: the decode kernels read it from the input, and a later kernel
// of the same call (the merge kernel of the even split, the finalize kernel of the prefix-shared
// decode) or the last partition's work-group of the fixed-partition decode writes it to its
// slot.
pkv_status decode_impl(void* out, const void* q, const void* k_cache, const void* v_cache,
                       const pkv_cache_desc* cache, const int32_t* block_tables,
                       int32_t max_blocks_per_seq, const int32_t* context_lens,
                       int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads, float scale,
                       void* workspace, size_t workspace_bytes, int32_t partition_size, void* stream,
                       const void* new_key, const void* new_value, const PrefixArgs* pre = nullptr) {
  clear_error();
  const bool append = new_key != nullptr || new_value != nullptr;
  if (!cache) return fail(PKV_ERR_INVALID_ARGUMENT, "cache descriptor is NULL");
  const int e = dtype_bytes(cache->dtype);
  if (e == 0) return fail(PKV_ERR_UNSUPPORTED, "dtype %d", cache->dtype);
  if (cache->num_blocks <= 0 || cache->num_kv_heads <= 0 || cache->head_dim <= 0 || cache->block_size <= 0)
    return fail(PKV_ERR_INVALID_ARGUMENT, "bad cache descriptor (NB=%d bs=%d Hkv=%d D=%d)",
                cache->num_blocks, cache->block_size, cache->num_kv_heads, cache->head_dim);
  const int D = cache->head_dim;
  if (D != 64 && D != 128) return fail(PKV_ERR_UNSUPPORTED, "head_dim %d (implemented: 64, 128)", D);
  if (num_seqs < 0) return fail(PKV_ERR_INVALID_ARGUMENT, "num_seqs=%d", num_seqs);
  if (num_q_heads <= 0 || num_q_heads % cache->num_kv_heads != 0)
    return fail(PKV_ERR_INVALID_ARGUMENT, "num_q_heads %d is not a positive multiple of num_kv_heads %d",
                num_q_heads, cache->num_kv_heads);
  const int G = num_q_heads / cache->num_kv_heads;
  if (cache->dtype == PKV_F32 ? G > 2 : G > 16)
    return fail(PKV_ERR_UNSUPPORTED, "group size %d for dtype %d (f32: <= 2, f16/bf16: <= 16)", G, cache->dtype);
  const bool sk_path = use_stream_k(num_seqs, num_q_heads, cache->num_kv_heads, D, partition_size, cache->dtype);
  if (pre && !sk_path)
    return fail(PKV_ERR_UNSUPPORTED,
                "prefix-shared decode needs f16/bf16 pools and at most %d sequences whose decode state fits "
                "the LDS (%d sequences, group %d, head_dim %d do not)",
                sk::kSkMaxSeqs, num_seqs, G, D);
  if (pre && (pre->num_groups < 0 || pre->max_prefix_tokens < 0 || pre->max_prefix_tokens % 16 != 0 ||
              pre->max_prefix_tokens > max_context_len))
    return fail(PKV_ERR_INVALID_ARGUMENT, "num_groups %d, max_prefix_tokens %d (a multiple of 16, <= max_context_len)",
                pre ? pre->num_groups : 0, pre ? pre->max_prefix_tokens : 0);
  const int BS = cache->block_size;
  if (sk_path ? (BS != 8 && BS != 16 && BS != 32) : BS != kBlock)
    return fail(PKV_ERR_UNSUPPORTED, "block_size %d (implemented: 8, 16, 32 for f16/bf16 with partition_size 0; "
                "16 otherwise)", BS);
  if (max_blocks_per_seq < 0 || max_context_len < 0 ||
      static_cast<int64_t>(max_context_len) > static_cast<int64_t>(max_blocks_per_seq) * BS)
    return fail(PKV_ERR_INVALID_ARGUMENT, "max_context_len %d vs max_blocks_per_seq %d",
                max_context_len, max_blocks_per_seq);
  if (!std::isfinite(scale)) return fail(PKV_ERR_INVALID_ARGUMENT, "scale is not finite");
  const int32_t part = sk_path ? kBlock : resolve_partition(max_context_len, partition_size);
  if (part == 0) return fail(PKV_ERR_INVALID_ARGUMENT, "partition_size %d", partition_size);
  if (num_seqs == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !context_lens || (max_blocks_per_seq > 0 && !block_tables))
    return fail(PKV_ERR_INVALID_ARGUMENT, "NULL device pointer");
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) ||
      (reinterpret_cast<uintptr_t>(block_tables) & 3u) || (reinterpret_cast<uintptr_t>(context_lens) & 3u))
    return fail(PKV_ERR_INVALID_ARGUMENT, "device pointers must be 16-byte aligned");
  if (append && (!new_key || !new_value || !aligned16(new_key) || !aligned16(new_value)))
    return fail(PKV_ERR_INVALID_ARGUMENT, "new_key and new_value must both be 16-byte aligned device pointers");
  if (append && max_blocks_per_seq == 0)
    return fail(PKV_ERR_INVALID_ARGUMENT, "an append needs a block table (max_blocks_per_seq > 0)");
  if (pre && (!pre->seq_prefix || (pre->num_groups > 0 && (!pre->group_offsets || !pre->group_members))))
    return fail(PKV_ERR_INVALID_ARGUMENT, "NULL group description");
  if (sk_path) {
    const size_t sk_bytes = sk::sk_workspace_bytes(num_seqs, cache->num_kv_heads, G, D, max_context_len);
    const int32_t chunks = pre ? prefix_chunks(pre->max_prefix_tokens) : 0;
    const size_t need = pre ? align256(sk_bytes) + prefix_extra_bytes(num_seqs, num_q_heads, D, chunks) : sk_bytes;
    if (!workspace || workspace_bytes < need)
      return fail(PKV_ERR_WORKSPACE_TOO_SMALL, "need %zu bytes, got %zu", need, workspace ? workspace_bytes : 0);
    if (!aligned16(workspace)) return fail(PKV_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
    sk::SkParams sp{};  // value-initialised: no suffix offsets, results to out
    sp.out = out;
    sp.q = q;
    sp.k_cache = const_cast<void*>(k_cache);  // written only when appending (pools are then the caller's writable ones)
    sp.v_cache = const_cast<void*>(v_cache);
    sp.new_key = new_key;
    sp.new_value = new_value;
    sp.block_tables = block_tables;
    sp.context_lens = context_lens;
    sp.num_seqs = num_seqs;
    sp.num_q_heads = num_q_heads;
    sp.num_kv_heads = cache->num_kv_heads;
    sp.group = G;
    sp.head_dim = D;
    sp.max_blocks_per_seq = max_blocks_per_seq;
    sp.max_context_len = max_context_len;
    sp.num_blocks = cache->num_blocks;
    sp.block_size = BS;
    sp.ranges = sk::sk_ranges(num_seqs, cache->num_kv_heads, G, max_context_len);
    sp.scale_log2e = scale * kLog2e;
    const int64_t recs = static_cast<int64_t>(sp.ranges) * sp.num_kv_heads * 2;
    sp.ws_status = static_cast<int32_t*>(workspace);
    sp.spin_limit = g_merge_spin_limit.load(std::memory_order_relaxed);
    sp.ws_acc = reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) + sk::kStatusBytes);
    sp.ws_ml = sp.ws_acc + recs * 16 * D;
    sp.ws_desc = reinterpret_cast<int32_t*>(sp.ws_ml + recs * 32);
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (!pre) {
      const hipError_t err = sk::sk_launch(sp, cache->dtype, st);
      if (err != hipSuccess) return fail(PKV_ERR_HIP, "decode launch: %s", hipGetErrorString(err));
      return PKV_OK;
    }
    // prefix-shared: the prefix pass and the even split over the suffixes in one launch (fp32
    // partials, suffix results, records of suffixes its ranges cut), then the finalize kernel
    // writes out.
    const size_t rows = static_cast<size_t>(num_seqs) * num_q_heads;
    unsigned char* w = static_cast<unsigned char*>(workspace) + align256(sk_bytes);
    float* part_out = reinterpret_cast<float*>(w);
    w += align256(rows * D * 4);
    float* part_lse = reinterpret_cast<float*>(w);
    w += align256(rows * 4);
    float* pre_acc = reinterpret_cast<float*>(w);
    w += align256(rows * chunks * D * 4);
    float* pre_ml = reinterpret_cast<float*>(w);
    w += align256(rows * chunks * 8);
    int32_t* cu = reinterpret_cast<int32_t*>(w);
    sp.seq_start = pre->seq_prefix;
    sp.part_out = part_out;
    sp.part_lse = part_lse;
    sp.ws_cu = cu;
    sk::PrefixParams pp{};
    pp.q = q;
    pp.k_cache = const_cast<void*>(k_cache);  // written only with a fused append
    pp.v_cache = const_cast<void*>(v_cache);
    pp.block_tables = block_tables;
    pp.context_lens = context_lens;
    pp.new_key = new_key;
    pp.new_value = new_value;
    pp.max_context_len = max_context_len;
    pp.seq_prefix = pre->seq_prefix;
    pp.group_offsets = pre->group_offsets;
    pp.group_members = pre->group_members;
    pp.pre_acc = pre_acc;
    pp.pre_ml = pre_ml;
    pp.part_out = part_out;
    pp.part_lse = part_lse;
    pp.rec_acc = sp.ws_acc;
    pp.rec_ml = sp.ws_ml;
    pp.cu = cu;
    pp.out = out;
    pp.num_seqs = num_seqs;
    pp.num_q_heads = num_q_heads;
    pp.num_kv_heads = cache->num_kv_heads;
    pp.group = G;
    pp.head_dim = D;
    pp.max_blocks_per_seq = max_blocks_per_seq;
    pp.num_blocks = cache->num_blocks;
    pp.block_size = BS;
    pp.num_groups = pre->num_groups;
    pp.chunks = chunks;
    pp.scale_log2e = sp.scale_log2e;
    hipError_t err = pre->num_groups > 0 && chunks > 0 ? sk::sk_launch_prefix(sp, pp, cache->dtype, st)
                                                       : sk::sk_launch(sp, cache->dtype, st);
    if (err == hipSuccess) err = sk::finalize_launch(pp, cache->dtype, st);
    if (err != hipSuccess) return fail(PKV_ERR_HIP, "prefix decode launch: %s", hipGetErrorString(err));
    return PKV_OK;
  }
  const int32_t P = parts_for(max_context_len, part);
  if (num_seqs > 65535 || P > 65535)
    return fail(PKV_ERR_UNSUPPORTED, "grid too large (num_seqs %d, partitions %d)", num_seqs, P);
  const size_t need = pkv_paged_attn_workspace_bytes(num_seqs, num_q_heads, cache->num_kv_heads, D,
                                                     max_context_len, partition_size, cache->dtype);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(PKV_ERR_WORKSPACE_TOO_SMALL, "need %zu bytes, got %zu", need, workspace ? workspace_bytes : 0);
  if (need > 0 && !aligned16(workspace))
    return fail(PKV_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");

  Params p;
  p.out = out;
  p.q = q;
  p.k_cache = const_cast<void*>(k_cache);  // written only with a fused append
  p.v_cache = const_cast<void*>(v_cache);
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.new_key = new_key;
  p.new_value = new_value;
  p.ws_acc = static_cast<float*>(workspace);
  p.ws_ml = need > 0 ? p.ws_acc + static_cast<size_t>(num_seqs) * num_q_heads * P * D : nullptr;
  p.num_seqs = num_seqs;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = cache->num_kv_heads;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.max_context_len = max_context_len;
  p.num_blocks = cache->num_blocks;
  p.part_blocks = part / kBlock;
  p.num_parts = P;
  p.scale_log2e = scale * kLog2e;

  const hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t err;
  switch (cache->dtype) {
    case PKV_F32: err = launch_dtype<F32>(p, D, G, st); break;
    case PKV_F16: err = launch_dtype<F16>(p, D, G, st); break;
    default: err = launch_dtype<BF16>(p, D, G, st); break;
  }
  if (err != hipSuccess) return fail(PKV_ERR_HIP, "decode launch: %s", hipGetErrorString(err));
  return PKV_OK;
}

}  // namespace

extern "C" pkv_status pkv_paged_attn_decode(void* out, const void* q, const void* k_cache,
                                            const void* v_cache, const pkv_cache_desc* cache,
                                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                                            const int32_t* context_lens, int32_t max_context_len,
                                            int32_t num_seqs, int32_t num_q_heads, float scale,
                                            void* workspace, size_t workspace_bytes,
                                            int32_t partition_size, void* stream) {
  return decode_impl(out, q, k_cache, v_cache, cache, block_tables, max_blocks_per_seq, context_lens,
                     max_context_len, num_seqs, num_q_heads, scale, workspace, workspace_bytes,
                     partition_size, stream, nullptr, nullptr);
}

extern "C" pkv_status pkv_paged_attn_decode_append(void* out, const void* q, const void* new_key,
                                                   const void* new_value, void* k_cache, void* v_cache,
                                                   const pkv_cache_desc* cache,
                                                   const int32_t* block_tables, int32_t max_blocks_per_seq,
                                                   const int32_t* context_lens, int32_t max_context_len,
                                                   int32_t num_seqs, int32_t num_q_heads, float scale,
                                                   void* workspace, size_t workspace_bytes,
                                                   int32_t partition_size, void* stream) {
  if (!new_key || !new_value) {
    clear_error();
    return fail(PKV_ERR_INVALID_ARGUMENT, "new_key and new_value must not be NULL");
  }
  return decode_impl(out, q, k_cache, v_cache, cache, block_tables, max_blocks_per_seq, context_lens,
                     max_context_len, num_seqs, num_q_heads, scale, workspace, workspace_bytes,
                     partition_size, stream, new_key, new_value);
}

extern "C" size_t pkv_paged_attn_decode_prefix_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                                               int32_t num_kv_heads, int32_t head_dim,
                                                               int32_t max_context_len, int32_t max_prefix_tokens,
                                                               int32_t dtype) {
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || max_context_len < 0) return 0;
  if (max_prefix_tokens < 0 || max_prefix_tokens % 16 != 0 || max_prefix_tokens > max_context_len) return 0;
  if (!use_stream_k(num_seqs, num_q_heads, num_kv_heads, head_dim, 0, dtype)) return 0;
  return align256(sk::sk_workspace_bytes(num_seqs, num_kv_heads, num_q_heads / num_kv_heads, head_dim, max_context_len)) +
         prefix_extra_bytes(num_seqs, num_q_heads, head_dim, prefix_chunks(max_prefix_tokens));
}

extern "C" pkv_status pkv_paged_attn_decode_prefix(void* out, const void* q, const void* k_cache, const void* v_cache,
                                                   const pkv_cache_desc* cache, const int32_t* block_tables,
                                                   int32_t max_blocks_per_seq, const int32_t* context_lens,
                                                   int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads,
                                                   float scale, const int32_t* seq_prefix,
                                                   const int32_t* group_offsets, const int32_t* group_members,
                                                   int32_t num_groups, int32_t max_prefix_tokens, void* workspace,
                                                   size_t workspace_bytes, void* stream) {
  const PrefixArgs pre{seq_prefix, group_offsets, group_members, num_groups, max_prefix_tokens};
  return decode_impl(out, q, k_cache, v_cache, cache, block_tables, max_blocks_per_seq, context_lens,
                     max_context_len, num_seqs, num_q_heads, scale, workspace, workspace_bytes, 0, stream, nullptr,
                     nullptr, &pre);
}

extern "C" pkv_status pkv_paged_attn_decode_prefix_append(
    void* out, const void* q, const void* new_key, const void* new_value, void* k_cache, void* v_cache,
    const pkv_cache_desc* cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
    const int32_t* context_lens, int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads, float scale,
    const int32_t* seq_prefix, const int32_t* group_offsets, const int32_t* group_members, int32_t num_groups,
    int32_t max_prefix_tokens, void* workspace, size_t workspace_bytes, void* stream) {
  if (!new_key || !new_value) {
    clear_error();
    return fail(PKV_ERR_INVALID_ARGUMENT, "new_key and new_value must not be NULL");
  }
  const PrefixArgs pre{seq_prefix, group_offsets, group_members, num_groups, max_prefix_tokens};
  return decode_impl(out, q, k_cache, v_cache, cache, block_tables, max_blocks_per_seq, context_lens,
                     max_context_len, num_seqs, num_q_heads, scale, workspace, workspace_bytes, 0, stream, new_key,
                     new_value, &pre);
}

extern "C" int32_t pkv_set_merge_spin_limit(int32_t limit) {
  const int32_t v = limit < 0 ? sk::kDefaultSpinLimit : limit;
  return g_merge_spin_limit.exchange(v);
}

// ------------------------------------------------------------------------------------
// Allocation-free variant of pkv_paged_attn_decode_append, for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops).  Its workspace is a
// file-scope device array: one copy per GPU, kept until the process ends.  In host code the
// array's name is only a stand-in; its device address on each GPU comes from
// hipGetSymbolAddress, taken once per device with that device current, and only that address
// is handed to the kernels.
// ------------------------------------------------------------------------------------
namespace {
constexpr size_t kScratchBytes = size_t{32} << 20;  // every even-split workspace fits (at most about 17 MB)
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first call there).
pkv_status scratch_ptr(void** out) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return fail(PKV_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(err));
  if (dev < 0 || dev >= kMaxDevices) return fail(PKV_ERR_UNSUPPORTED, "device ordinal %d", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (err != hipSuccess || !ptr)
      return fail(PKV_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(err));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return PKV_OK;
}
}  // namespace

extern "C" size_t pkv_paged_attn_noalloc_scratch_bytes(void) { return kScratchBytes; }

extern "C" pkv_status pkv_paged_attn_decode_append_noalloc(void* out, const void* q, const void* new_key,
                                                           const void* new_value, void* k_cache, void* v_cache,
                                                           const pkv_cache_desc* cache,
                                                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                                                           const int32_t* context_lens, int32_t max_context_len,
                                                           int32_t num_seqs, int32_t num_q_heads, float scale,
                                                           int32_t partition_size, void* stream) {
  clear_error();
  if (!new_key || !new_value) return fail(PKV_ERR_INVALID_ARGUMENT, "new_key and new_value must not be NULL");
  if (!cache) return fail(PKV_ERR_INVALID_ARGUMENT, "cache descriptor is NULL");
  if (num_seqs == 0) return PKV_OK;
  const size_t need = pkv_paged_attn_workspace_bytes(num_seqs, num_q_heads, cache->num_kv_heads, cache->head_dim,
                                                     max_context_len, partition_size, cache->dtype);
  if (need > kScratchBytes)
    return fail(PKV_ERR_WORKSPACE_TOO_SMALL,
                "these arguments need a %zu-byte workspace; the allocation-free call has %zu bytes of scratch",
                need, kScratchBytes);
  // the workspace query returns 0 for arguments it rejects: those reach the decode's own
  // validation below without a device query
  void* ws = nullptr;
  if (need > 0) {
    const pkv_status st = scratch_ptr(&ws);
    if (st != PKV_OK) return st;
  }
  return decode_impl(out, q, k_cache, v_cache, cache, block_tables, max_blocks_per_seq, context_lens,
                     max_context_len, num_seqs, num_q_heads, scale, ws, need > 0 ? kScratchBytes : 0,
                     partition_size, stream, new_key, new_value);
}

