// Paged decode attention, grouped-query MFMA path with an even split of the work over the GPU.
//
// What is computed is the same as in paged_attn.hip: for every sequence and query head,
// single-query scaled dot-product attention over the sequence's context, whose K/V rows sit
// in fixed-size blocks (16 tokens, or 8 or 32) scattered through a pool and are found through
// the block table (the yunthe.com page "大模型推理显存优化实战：PagedAttention机制原理与vLLM
// 连续批处理配置", section "PagedAttention分页注意力机制原理"; block table and 16-token blocks:
// the 111cn.net page "大模型推理引擎高频优化：连续批处理、PagedAttention 与 KV Cache 实战拆解"
// §3.2; block layout (block_size, heads, head_dim): the gtnt.cn page "vLLM推理加速框架：
// PagedAttention与连续批处理技术解析" §2.1; 8-token blocks: its closing section).  This file only
// changes how the work is spread over the chip.
//
// Work split.  A "tile" is 16 tokens of one sequence for one KV head (one 16-token block, half
// of a 32-token block or two 8-token blocks; K and V: 2*16*D*e bytes).  For one KV head the
// tiles of all sequences form a list in sequence order (tiles 0..n-1 of sequence 0, then
// sequence 1, ...), T tiles long; a sequence with no context counts as one empty tile, so that
// its zero output is written like any other.  The list is cut into R equal contiguous ranges
// (R never exceeds T, so no range is empty).  A work-group serves one range for 4 consecutive
// KV heads, one head per wave column, so its waves read neighbouring 256-byte slices of the
// same token rows at the same time; the range is split again between 2 wave rows.  Every
// wave therefore streams the same number of tiles (+-1) whatever the length mix, and keeps
// loading across sequence boundaries.
//   * A sequence whose tiles lie inside one wave's sub-range is finished by that wave.
//   * A sequence cut only between the two sub-ranges of a work-group is merged in LDS.
//   * A sequence cut by range boundaries leaves one record (unnormalised acc, running max m,
//     sum l) per work-group that touched it; the merge kernel combines them in range order.
// Each work-group derives its range from the context lengths itself (prefix sum of tile
// counts in LDS), so no planning launch is needed.
//
// Per tile (one wave, 16 tokens, G <= 16 query heads padded to 16):
//   S^T = K * Q^T            v_mfma_f32_16x16x32_{bf16,f16}, K straight from HBM as the A operand
//   online softmax in base 2 (scale*log2(e) folded in), rescale only when some head's
//   running max grows by more than 8 (exact: the stale max only bounds P by 2^8)
//   O^T += V^T * P^T         v_mfma_f32_16x16x16, V^T read from an LDS copy of the V tile with
//                            ds_read_b64_tr_b16 (one transposing read per 16-column chunk)
// Loads use buffer resources that end at the tile's last row in use: the rows of a partly
// filled last tile past the context, and a tile whose block id lies outside the pool, read as
// zeros with no memory access, so the loads need no branches around them.  (With 8-token
// blocks a tile spans two blocks; there each lane loads through its own 64-bit address,
// masked the same way.)
#include <hip/hip_runtime.h>

#include <cmath>

#include "dtypes.h"
#include "pkv_internal.h"
#include "prefix_body.h"
#include "stream_k.h"
#include "tile_common.h"

namespace pkv {
namespace sk {
namespace {

// Work-group shape: 8 waves, HEADS KV heads side by side (their waves read neighbouring slices
// of the same token rows together) x 8 / HEADS consecutive sub-ranges of the tile list (merged
// in LDS).  HEADS is 4, or 1 for small batches: there a sequence is cut into many ranges, and
// eight sub-ranges merged in LDS leave a quarter of the records to the merge kernel.
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kLast = 1 << 8;             // tile flag: last tile of its sequence
constexpr int kFirst = 1 << 9;            // tile flag: first tile of its sequence
constexpr int kHalf = 1 << 10;            // tile flag (32-token blocks): second half of its block
__device__ __forceinline__ int clamp_ctx(int L, int maxc) { return L < 0 ? 0 : (L > maxc ? maxc : L); }


// Writes a wave's G output rows, which are contiguous in memory (row r16 < G holds columns
// 16c + 4grp .. +3 in v[c]), as 16-byte stores of consecutive lanes.  The rows are staged in
// `stage`, this wave's own LDS (at least G * (2D + 16) bytes), with a padded row pitch.
template <typename T, int D>
__device__ __forceinline__ void store_rows(typename T::raw* o, const f32x4* v, float inv, unsigned char* stage,
                                           int G, int lane) {
  constexpr int SP = 2 * D + 16;
  constexpr int CPR = D / 8;  // 16-byte chunks per row
  const int r16 = lane & 15, grp = lane >> 4;
  if (r16 < G) {
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      const f32x4 x = v[c] * inv;
      uint2 w;
      w.x = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, to_raw(T{}, x[0]))) |
            (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, to_raw(T{}, x[1]))) << 16);
      w.y = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, to_raw(T{}, x[2]))) |
            (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, to_raw(T{}, x[3]))) << 16);
      *reinterpret_cast<uint2*>(stage + r16 * SP + 32 * c + 8 * grp) = w;
    }
  }
  wave_lds_sync();
  for (int q = lane; q < G * CPR; q += 64)
    __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(stage + (q / CPR) * SP + 16 * (q % CPR)),
                                reinterpret_cast<u32x4*>(reinterpret_cast<unsigned char*>(o) + 16 * q));
  wave_lds_sync();
}

// Partial-result mode: writes row r16's result (columns 16c + 4grp .. +3 in v[c], times inv)
// as fp32, and from lane grp 0 its log2-sum-exp m + log2(l).
template <int D>
__device__ __forceinline__ void store_partial(const SkParams& p, int64_t row, const f32x4* v, float inv, float m,
                                              float l, int grp) {
  float* o = p.part_out + row * D;
#pragma unroll
  for (int c = 0; c < D / 16; ++c) __builtin_nontemporal_store(v[c] * inv, reinterpret_cast<f32x4*>(o + 16 * c + 4 * grp));
  if (grp == 0) p.part_lse[row] = l > 0.f ? m + __log2f(l) : -INFINITY;
}

// Per-lane tile entry of tile t (t < T): {block of rows 0-15 (8-token blocks: rows 0-7),
// sequence, block of rows 8-15 (8-token blocks only, else -1), ntok | flags}.  A tile is 16
// tokens of one sequence: for 16-token pool blocks one block, for 32-token blocks one half of
// a block (kHalf: the second half), for 8-token blocks two blocks.
template <int BS, bool SUFFIX>
__device__ __forceinline__ int4 tile_entry(const SkParams& p, const int* s_cu, const int* s_start, int t) {
  int a = 0, b = p.num_seqs;  // largest a with cu[a] <= t  (cu[0] = 0 <= t < cu[B] = T)
  while (b - a > 1) {
    const int m = (a + b) >> 1;
    if (s_cu[m] <= t) a = m; else b = m;
  }
  const int j = t - s_cu[a];
  const int ntiles = s_cu[a + 1] - s_cu[a];
  const int start = SUFFIX ? s_start[a] : 0;  // tokens skipped (suffix mode), a multiple of 16
  const int L = max(0, clamp_ctx(p.context_lens[a], p.max_context_len) - start);
  const int tok0 = start + j * kTile;  // first token of the tile in the sequence
  // The table entries are read whatever the length, so that these loads are in flight
  // together (indexes clamped into the row, which has max_blocks_per_seq > 0 entries whenever
  // L > 0).  The empty tile of a sequence with no context reads nothing (block id -1) and has
  // 0 tokens.
  const int64_t row = static_cast<int64_t>(a) * p.max_blocks_per_seq;
  const int last = p.max_blocks_per_seq - 1;
  int e0 = -1, e1 = -1;
  if (p.max_blocks_per_seq > 0) {
    e0 = p.block_tables[row + min(tok0 / BS, last)];
    if (BS == 8 && tok0 / BS + 1 <= last) e1 = p.block_tables[row + tok0 / BS + 1];
  }
  const int ntok = min(kTile, L - j * kTile);
  const int phys0 = L > 0 ? e0 : -1;
  const int phys1 = (BS == 8 && ntok > 8) ? e1 : -1;
  const int fl = ntok | (j == ntiles - 1 ? kLast : 0) | (j == 0 ? kFirst : 0) |
                 ((BS == 32 && ((tok0 >> 4) & 1)) ? kHalf : 0);
  return make_int4(phys0, a, phys1, fl);
}

// LDS layout of the decode kernel (dynamic): the prefix sum of block counts, then one region
// that holds the 8 waves' V tiles during the tile loop and the 8 wave states after it.  The
// kernel's static LDS (scan partials and wave flags) stays under kSkStaticLds bytes.
constexpr int kSkStaticLds = 256;
__host__ __device__ inline int sk_state_bytes(int D, int G) { return ((D / 16) * 4 * G * 16 + G * 8 + 15) / 16 * 16; }
__host__ __device__ inline int sk_cu_bytes(int B) { return ((B + 1) * 4 + 15) / 16 * 16 + (B * 4 + 15) / 16 * 16; }
__host__ __device__ inline int sk_lds_bytes(int B, int D, int G) {
  const int tiles = kWaves * kTile * sk_pitch(D);
  const int states = 2 * kWaves * sk_state_bytes(D, G);
  return sk_cu_bytes(B) + (tiles > states ? tiles : states);
}

// SUFFIX: suffix and partial-result mode (seq_start and part_out set), compiled apart so that
// the plain decode carries none of it.
// VEC: one query head per KV head (G = 1).  There the tile's products are a 16-token x D
// matrix-vector product, not a dense contraction, so they run on the vector ALUs: lane
// (r16, grp) holds token r16's columns 8 (grp + 4c) .. +7 of K, V and q, forms its part of the
// token's logit with dot2 instructions, sums the four parts over the lane groups, and
// accumulates weight x its V columns; the weights stay fp32.  At a sequence's end the 16 token
// lanes of each lane row are summed and the columns moved (through the wave's LDS tile) to the
// layout of the matrix path, which the rest of the kernel shares.
// The body of one work-group (index bid) of the decode launch, with s_dyn its dynamic LDS.
template <typename T, int D, int BS, bool SUFFIX, int HEADS, bool VEC>
__device__ __forceinline__ void decode_sk_body(const SkParams& p, int bid, unsigned char* s_dyn) {
  constexpr int kHeads = HEADS, kSplits = kWaves / HEADS;
  using M = Mma<T>;
  using raw = typename T::raw;
  constexpr int ROW = D * 2;                   // bytes of one head row
  constexpr int KC = D / 32;                   // QK k-chunks (one 16-byte piece per lane each)
  constexpr int NC = D / 16;                   // PV output chunks of 16 columns
  constexpr int PITCH = sk_pitch(D);           // V tile row pitch: the transposing reads hit distinct banks
  constexpr int TILE_LDS = kTile * PITCH;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, r16 = lane & 15, grp = lane >> 4;
  // wave = (split sw, head column hw); head groups innermost so that all heads of one range
  // are dispatched together
  const int hw = wave % kHeads, sw = wave / kHeads;
  const int hgroups = (p.num_kv_heads + kHeads - 1) / kHeads;
  const int hg = bid % hgroups;
  const int wgr = bid / hgroups;
  // With one query head per KV head and many head groups (MHA shapes), the four heads of a
  // work-group are two pairs from the two halves of the head range: pair hg from the first
  // half, and from the second half pair hg ^ 1 when the head groups are even in number (else
  // pair hg), e.g. {0, 1, 2h + 2, 2h + 3}, {2, 3, 2h, 2h + 1}, ... for h head groups.  Pairs
  // from the two halves were 2% faster on 64 x 32-head fp16 decode than four adjacent heads;
  // taking the second pair from the other parity, so that each work-group reads one 512-byte
  // slice at an even and one at an odd multiple of 512 bytes into the token row, was another
  // 0.1-1.3% on 64-256 sequences of 16 or 32 heads (per-work-group clock stamps had shown the
  // work-groups on even XCDs, which read only even slices, ending about 10 us after the rest).
  // Otherwise four adjacent heads, one contiguous 4 x D run of each token row; with two
  // head groups the second group's heads go to the even work-group indices.  Work-groups are
  // dealt to the 8 XCDs in turn, so head group = XCD parity: in the plain order the last heads
  // (the second half of each token row) land on the odd XCDs, and both of those read more
  // slowly (measured with per-work-group clock stamps); swapped, the two offset each other:
  // 256 lognormal 70B-GQA sequences 168.6 -> 165.5 us, 512 sequences 312.5 -> 307.6 us.
  const int g = (VEC && kHeads == 4 && hgroups >= 4)
                    ? (hw >> 1) * (2 * hgroups) + ((hgroups % 2 == 0 && (hw >> 1)) ? hg ^ 1 : hg) * 2 + (hw & 1)
                    : (kHeads == 4 && hgroups == 2 ? 1 - hg : hg) * kHeads + hw;
  const bool head_ok = g < p.num_kv_heads;
  const int G = p.group;
  const int B = p.num_seqs;

  int* s_cu = reinterpret_cast<int*>(s_dyn);                  // [B + 1]
  int* s_start = s_cu + ((B + 1 + 3) & ~3);                    // [B] tokens skipped per sequence
  unsigned char* s_work = s_dyn + sk_cu_bytes(B);              // V tiles, later wave states
  __shared__ int s_part[kWaves];
  __shared__ int s_flags[kWaves][5];
  static_assert(sizeof(s_part) + sizeof(s_flags) <= kSkStaticLds, "static LDS of the decode kernel");

  // ---- prefix sum of tile counts (every work-group derives the same list)
  const int per = (B + kThreads - 1) / kThreads;
  const int lo = min(B, tid * per), hi = min(B, lo + per);
  int run = 0;
  for (int s = lo; s < hi; ++s) {
    const int L = clamp_ctx(p.context_lens[s], p.max_context_len);
    // suffix mode: the skipped tokens, kept inside [0, L] and on a tile boundary whatever the
    // caller passed, so that every table index below stays inside the sequence's row
    const int st = SUFFIX ? (min(max(p.seq_start[s], 0), L) & ~(kTile - 1)) : 0;
    run += max(1, (max(0, L - st) + kTile - 1) / kTile);
    s_cu[s + 1] = run;
    if (SUFFIX) s_start[s] = st;
  }
  // exclusive offset of this thread's sequences: a scan within the wave, then over the waves
  int incl = run;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) s_part[wave] = incl;
  __syncthreads();
  int base = incl - run;
  for (int w = 0; w < wave; ++w) base += s_part[w];
  for (int s = lo; s < hi; ++s) s_cu[s + 1] += base;
  if (tid == 0) s_cu[0] = 0;
  __syncthreads();
  const int ntiles = s_cu[B];
  const int R = min(p.ranges, ntiles);  // ranges in use: none of them is empty
  if (SUFFIX && bid == 0) {
    // the prefix-shared decode's finalize kernel finds each sequence's ranges from these
    for (int i = tid; i <= B; i += kThreads) p.ws_cu[i] = s_cu[i];
    if (tid == 0) p.ws_cu[B + 1] = R;
  }
  if (bid == 0 && tid == 0) p.ws_status[0] = kStatusOk;  // the merge kernel runs after this launch
  if (hg == 0 && tid == 0) {
    // the merge kernel's work list: the sequence cut at this range's start, if this is the
    // first range boundary inside it, with the ranges that hold its first and last tiles
    int4 d = make_int4(-1, 0, 0, 0);
    if (wgr > 0 && wgr < R) {
      const int T0 = static_cast<int>(static_cast<int64_t>(wgr) * ntiles / R);
      int a = 0, b = B;  // largest a with s_cu[a] <= T0
      while (b - a > 1) {
        const int m = (a + b) >> 1;
        if (s_cu[m] <= T0) a = m; else b = m;
      }
      const int ra = range_of(s_cu[a], ntiles, R);
      if (s_cu[a] < T0 && ra == wgr - 1) d = make_int4(a, ra, range_of(s_cu[a + 1] - 1, ntiles, R), 0);
    }
    *reinterpret_cast<int4*>(p.ws_desc + 4 * wgr) = d;
  }
  if (wgr >= R) return;  // more work-groups than tiles
  // this work-group's range of the head's tile list, and this wave's sub-range of it
  const int T0 = static_cast<int>(static_cast<int64_t>(wgr) * ntiles / R);
  const int T1 = static_cast<int>(static_cast<int64_t>(wgr + 1) * ntiles / R);
  const int t0 = T0 + static_cast<int>(static_cast<int64_t>(T1 - T0) * sw / kSplits);
  const int t1 = T0 + static_cast<int>(static_cast<int64_t>(T1 - T0) * (sw + 1) / kSplits);
  const int n = head_ok ? t1 - t0 : 0;

  // Writes a record of this work-group's range for KV head g (rows r16 < G): slot 0 holds a
  // sequence that began before the range, slot 1 one that began inside it and runs past it.
  auto store_record = [&](int slot, float rm, float rl, const f32x4* ra) {
    const int64_t rec = (static_cast<int64_t>(wgr) * p.num_kv_heads + g) * 2 + slot;
    float* pa = p.ws_acc + rec * (16 * D) + r16 * D;
#pragma unroll
    for (int c = 0; c < NC; ++c) __builtin_nontemporal_store(ra[c], reinterpret_cast<f32x4*>(pa + 16 * c + 4 * grp));
    if (grp == 0) {
      __builtin_nontemporal_store(rm, p.ws_ml + rec * 32 + r16 * 2);
      __builtin_nontemporal_store(rl, p.ws_ml + rec * 32 + r16 * 2 + 1);
    }
  };

  // state of the segment that began before this wave (A) and of the one that runs past its end (Z)
  bool hasA = false, a_through = false, hasZ = false;
  int sA = -1, sZ = -1;
  float mA = kNegBig, lA = 0.f, lZ = 0.f;
  f32x4 accA[NC];
  float m_run = kNegBig, l_run = 0.f;
  f32x4 acc[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) { accA[c] = f32x4{0.f, 0.f, 0.f, 0.f}; acc[c] = accA[c]; }

  if (n > 0) {
    // tile entries: lane i of ent holds tile t0 + kb + i, ent2 the next 64
    int kb = 0;
    int4 ent = lane < n ? tile_entry<BS, SUFFIX>(p, s_cu, s_start, t0 + lane) : make_int4(0, 0, 0, 0);
    int4 ent2;  // read once the first tile's loads are out

    const int64_t tok_bytes = static_cast<int64_t>(p.num_kv_heads) * ROW;  // one token row, all heads
    const int64_t block_bytes = BS * tok_bytes;
    const int voff = r16 * static_cast<int>(tok_bytes) + g * ROW + grp * 16;
    unsigned char* kbase = static_cast<unsigned char*>(p.k_cache);
    unsigned char* vbase = static_cast<unsigned char*>(p.v_cache);
    unsigned char* vt = s_work + wave * TILE_LDS;
    const bool append = p.new_key != nullptr;

    u32x4 kbuf[KC], vbuf[KC], qbuf[KC], nk[KC], nv[KC];
    int last_s = -1;
    // Issues the loads of tile kk (a zero-length load when kk is past the range or its block
    // id is outside the pool).  A tile that opens a sequence also brings that sequence's
    // query; with a fused append, the last tile of a sequence also brings its new K/V row.
    // The buffer resource starts at the tile's first row: rows r16 are read at r16 * tok_bytes.
    // With 8-token blocks rows 8-15 come from a second block (nrec1: the bytes of rows 0-15
    // counted from 8 rows before that block).
    auto issue = [&](int kk) {
      int phys = 0, nrec = 0, phys1 = 0, nrec1 = 0, half = 0;
      if (kk < n) {
        const int i = kk - kb;
        phys = i < 64 ? lane_val(ent.x, i) : lane_val(ent2.x, i - 64);
        if (BS == 8) phys1 = i < 64 ? lane_val(ent.z, i) : lane_val(ent2.z, i - 64);
        const int s = i < 64 ? lane_val(ent.y, i) : lane_val(ent2.y, i - 64);
        const int fl = i < 64 ? lane_val(ent.w, i) : lane_val(ent2.w, i - 64);
        if (s != last_s) {
          last_s = s;
          const int h = g * G + (r16 < G ? r16 : 0);
          const u32x4* qv = reinterpret_cast<const u32x4*>(static_cast<const raw*>(p.q) +
                                                           (static_cast<int64_t>(s) * p.num_q_heads + h) * D);
#pragma unroll
          for (int c = 0; c < KC; ++c) qbuf[c] = qv[grp + 4 * c];
        }
        if (append && (fl & kLast)) {
          const int64_t row = (static_cast<int64_t>(s) * p.num_kv_heads + g) * D;
          const u32x4* kn = reinterpret_cast<const u32x4*>(static_cast<const raw*>(p.new_key) + row);
          const u32x4* vn = reinterpret_cast<const u32x4*>(static_cast<const raw*>(p.new_value) + row);
#pragma unroll
          for (int c = 0; c < KC; ++c) { nk[c] = kn[grp + 4 * c]; nv[c] = vn[grp + 4 * c]; }
        }
        // Rows the tile takes from the pool: its tokens, less the new token of a fused append
        // (that row comes from the input).  The resource ends after them, so the rows of a
        // partly filled last tile past the context read as zeros and fetch nothing.
        const int rows = max(0, (fl & 0xff) - ((append && (fl & kLast)) ? 1 : 0));
        nrec = (phys >= 0 && phys < p.num_blocks) ? static_cast<int>(min(rows, BS == 8 ? 8 : kTile) * tok_bytes) : 0;
        phys = (phys >= 0 && phys < p.num_blocks) ? phys : 0;
        if (BS == 32) half = (fl & kHalf) ? 1 : 0;
        if (BS == 8) {
          nrec1 = (phys1 >= 0 && phys1 < p.num_blocks) ? static_cast<int>(rows * tok_bytes) : 0;
          phys1 = nrec1 ? phys1 : 0;
        }
      }
      if constexpr (BS == 8) {
        // Rows 0-7 come from block phys and rows 8-15 from block phys1, so the two halves of
        // the wave would need different buffer resources.  Per-lane 64-bit addresses (global
        // loads) avoid that; a lane whose row is past the rows in use, or whose block id lies
        // outside the pool, loads nothing and keeps zeros.
        const bool lo = r16 < 8;
        const bool ok = r16 * tok_bytes < (lo ? nrec : nrec1);
        const int64_t a = (lo ? phys : phys1) * block_bytes + (r16 & 7) * tok_bytes + g * ROW + grp * 16;
#pragma unroll
        for (int c = 0; c < KC; ++c)
          kbuf[c] = ok ? *reinterpret_cast<const u32x4*>(kbase + a + c * 64) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int c = 0; c < KC; ++c)
          vbuf[c] = ok ? *reinterpret_cast<const u32x4*>(vbase + a + c * 64) : u32x4{0u, 0u, 0u, 0u};
      } else {
        const int64_t off = phys * block_bytes + half * kTile * tok_bytes;
        const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(kbase + off, 0, nrec, kRsrcWord3);
        const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(vbase + off, 0, nrec, kRsrcWord3);
#pragma unroll
        for (int c = 0; c < KC; ++c) kbuf[c] = __builtin_amdgcn_raw_buffer_load_b128(rk, voff + c * 64, 0, 0);
#pragma unroll
        for (int c = 0; c < KC; ++c) vbuf[c] = __builtin_amdgcn_raw_buffer_load_b128(rv, voff + c * 64, 0, 0);
      }
    };
    issue(0);
    ent2 = lane + 64 < n ? tile_entry<BS, SUFFIX>(p, s_cu, s_start, t0 + 64 + lane) : make_int4(0, 0, 0, 0);

    int cur_s = -1, seg_k0 = 0;
    bool seg_first = false;  // the current segment starts at its sequence's first tile
    typename M::v8 qb[KC];
    // transposing read of PV chunk c: row 4*grp + (r16 >> 2), columns 16c + 4*(r16 & 3) .. +3
    const int tr_base = (4 * grp + (r16 >> 2)) * PITCH + 8 * (r16 & 3);

    for (int k = 0; k < n; ++k) {
      if (k - kb == 64) {  // slide the entry window
        kb += 64;
        ent = ent2;
        ent2 = kb + 64 + lane < n ? tile_entry<BS, SUFFIX>(p, s_cu, s_start, t0 + kb + 64 + lane) : make_int4(0, 0, 0, 0);
      }
      const int i = k - kb;
      const int s = lane_val(ent.y, i), fl = lane_val(ent.w, i);
      const int ntok = fl & 0xff;
      if (s != cur_s) {  // this tile opens a segment
        cur_s = s;
        seg_first = (fl & kFirst) != 0;
        seg_k0 = k;
#pragma unroll
        for (int c = 0; c < KC; ++c)
          qb[c] = __builtin_bit_cast(typename M::v8, (VEC || r16 < G) ? qbuf[c] : u32x4{0u, 0u, 0u, 0u});
        m_run = kNegBig;
        l_run = 0.f;
#pragma unroll
        for (int c = 0; c < NC; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      if (append && (fl & kLast)) {
        // the sequence's new token is its last one (row ntok - 1 of this block): use the new
        // row (the merge kernel writes it to its pool slot)
        const bool mine = r16 == ntok - 1;
#pragma unroll
        for (int c = 0; c < KC; ++c) {
          kbuf[c] = mine ? nk[c] : kbuf[c];
          vbuf[c] = mine ? nv[c] : vbuf[c];
        }
      }
      if constexpr (VEC) {
        // token r16's logit: this lane's 8 (D / 32) columns, then the sum over the lane groups
        float dot = 0.f;
#pragma unroll
        for (int c = 0; c < KC; ++c) dot = dot8(T{}, kbuf[c], __builtin_bit_cast(u32x4, qb[c]), dot);
        // this tile's V stays in registers; the next tile's loads go out now
        u32x4 vcur[KC];
#pragma unroll
        for (int c = 0; c < KC; ++c) vcur[c] = vbuf[c];
        if (k + 1 < n) issue(k + 1);
        dot = swap32_sum(swap16_sum(dot));
        const float sv = r16 < ntok ? dot * p.scale_log2e : -INFINITY;
        const float mx = row16_max(sv);  // the tile's maximum (the same in every lane row)
        if (__builtin_amdgcn_ballot_w64(mx > m_run + kTau) != 0) {
          const float mn = fmaxf(m_run, mx);
          const float alpha = __builtin_amdgcn_exp2f(m_run - mn);
          l_run *= alpha;
#pragma unroll
          for (int c = 0; c < NC; ++c) acc[c] *= alpha;
          m_run = mn;
        }
        const float pw = __builtin_amdgcn_exp2f(sv - m_run);  // 0 for rows past the context
        l_run += pw;
#pragma unroll
        for (int c = 0; c < KC; ++c) {
          float vf[8];
          unpack(T{}, vcur[c], vf);
          acc[2 * c] += pw * f32x4{vf[0], vf[1], vf[2], vf[3]};
          acc[2 * c + 1] += pw * f32x4{vf[4], vf[5], vf[6], vf[7]};
        }
      } else {
        // V tile -> LDS (row = token r16), then S^T = K Q^T
#pragma unroll
        for (int c = 0; c < KC; ++c) *reinterpret_cast<u32x4*>(vt + r16 * PITCH + (grp + 4 * c) * 16) = vbuf[c];
        f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < KC; ++c) sacc = M::qk(__builtin_bit_cast(typename M::v8, kbuf[c]), qb[c], sacc);
        // this tile's registers are consumed: the next tile's loads go out now (none after the
        // last tile, so that nothing is left in flight when the results are written)
        if (k + 1 < n) issue(k + 1);

        // online softmax: lane holds tokens 4*grp + e of head r16
        float sv[4], mx = kNegBig;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sv[e] = (4 * grp + e < ntok) ? sacc[e] * p.scale_log2e : -INFINITY;
          mx = fmaxf(mx, sv[e]);
        }
        mx = swap32_max(swap16_max(mx));
        if (__builtin_amdgcn_ballot_w64(mx > m_run + kTau) != 0) {
          const float mn = fmaxf(m_run, mx);
          const float alpha = __builtin_amdgcn_exp2f(m_run - mn);
          l_run *= alpha;
#pragma unroll
          for (int c = 0; c < NC; ++c) acc[c] *= alpha;
          m_run = mn;
        }
        i16x4_t pbits;
        float psum = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const short pe = M::pack(__builtin_amdgcn_exp2f(sv[e] - m_run));
          pbits[e] = pe;
          psum += M::unpack(pe);  // the sum uses exactly the rounded weights of the PV product
        }
        l_run += psum;
        wave_lds_sync();
        if (ntok < kTile) {  // last tile of a sequence: rows past the context may hold anything
#pragma unroll
          for (int c = 0; c < NC; ++c) {
            i16x4_t vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vt + tr_base + 32 * c));
#pragma unroll
            for (int e = 0; e < 4; ++e) vb[e] = (4 * grp + e < ntok) ? vb[e] : static_cast<short>(0);
            acc[c] = M::pv(vb, pbits, acc[c]);
          }
        } else {
#pragma unroll
          for (int c = 0; c < NC; ++c) {
            const i16x4_t vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vt + tr_base + 32 * c));
            acc[c] = M::pv(vb, pbits, acc[c]);
          }
        }
        wave_lds_sync();
      }

      bool seg_end = (k == n - 1);
      if (!seg_end) {
        const int i2 = k + 1 - kb;
        seg_end = (i2 < 64 ? lane_val(ent.y, i2) : lane_val(ent2.y, i2 - 64)) != s;
      }
      if (!seg_end) continue;
      if constexpr (VEC) {
        // sum the 16 token lanes of each lane row, then move row 0's columns to the matrix
        // layout (lane (r16, grp): columns 16c + 4grp .. +3 in acc[c]) through this wave's tile
        l_run = row16_sum(l_run);
        l_run = grp == 0 ? l_run : 0.f;
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[c][e] = row16_sum(acc[c][e]);
        float* cols = reinterpret_cast<float*>(vt);
        if (r16 == 0) {
#pragma unroll
          for (int c = 0; c < NC; ++c) *reinterpret_cast<f32x4*>(cols + 8 * (grp + 4 * (c >> 1)) + 4 * (c & 1)) = acc[c];
        }
        wave_lds_sync();
#pragma unroll
        for (int c = 0; c < NC; ++c) acc[c] = *reinterpret_cast<const f32x4*>(cols + 16 * c + 4 * grp);
        wave_lds_sync();
      }
      const float lsum = swap32_sum(swap16_sum(l_run));
      if (seg_first && (fl & kLast)) {  // the whole sequence lies in this wave's sub-range
        const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
        if constexpr (SUFFIX) {
          if (r16 < G) store_partial<D>(p, static_cast<int64_t>(s) * p.num_q_heads + g * G + r16, acc, inv, m_run, lsum, grp);
        } else {
          store_rows<T, D>(static_cast<raw*>(p.out) + (static_cast<int64_t>(s) * p.num_q_heads + g * G) * D, acc, inv,
                           vt, G, lane);
        }
      } else if (seg_k0 == 0 && !seg_first) {  // began in an earlier sub-range (A)
        hasA = true;
        a_through = !(fl & kLast);
        sA = s;
        mA = m_run;
        lA = lsum;
#pragma unroll
        for (int c = 0; c < NC; ++c) accA[c] = acc[c];
      } else {  // runs past this sub-range (Z): it is the last segment, acc stays as it is
        hasZ = true;
        sZ = s;
        lZ = lsum;
      }
      cur_s = -1;
    }
  }

  // Records that no other wave of the work-group joins go out now rather than after its
  // barriers (none inside the tile loop: there a store would hold up the next tile's loads, as
  // loads and stores share one counter): a sequence that began before the range and ends in
  // its first sub-range (slot 0), one that began in its last sub-range and runs past it (slot 1).
  if (sw == 0 && hasA && !a_through) {
    if (head_ok && r16 < G) store_record(0, mA, lA, accA);
    hasA = false;
  }
  if (sw == kSplits - 1 && hasZ) {
    if (head_ok && r16 < G) store_record(1, m_run, lZ, acc);
    hasZ = false;
  }

  // ---- merge what crosses the sub-ranges of this work-group; hand the rest to the merge kernel
  __syncthreads();  // every wave is done with its V tile: the region now holds wave states
  const int sb = sk_state_bytes(D, G);
  auto st_acc = [&](int w, int slot) { return reinterpret_cast<f32x4*>(s_work + (w * 2 + slot) * sb); };
  auto st_ml = [&](int w, int slot) { return reinterpret_cast<float2*>(s_work + (w * 2 + slot) * sb + NC * 4 * G * 16); };
  if (r16 < G) {
    if (hasA) {
#pragma unroll
      for (int c = 0; c < NC; ++c) st_acc(wave, 0)[(c * 4 + grp) * G + r16] = accA[c];
      if (grp == 0) st_ml(wave, 0)[r16] = make_float2(mA, lA);
    }
    if (hasZ) {
#pragma unroll
      for (int c = 0; c < NC; ++c) st_acc(wave, 1)[(c * 4 + grp) * G + r16] = acc[c];
      if (grp == 0) st_ml(wave, 1)[r16] = make_float2(m_run, lZ);
    }
  }
  if (lane == 0) {
    s_flags[wave][0] = hasA;
    s_flags[wave][1] = a_through;
    s_flags[wave][2] = hasZ;
    s_flags[wave][3] = sA;
    s_flags[wave][4] = sZ;
  }
  __syncthreads();
  if (sw != 0 || !head_ok || r16 >= G) return;
  // Walk the sub-ranges of head column hw in order.  A chain is a sequence cut by sub-range boundaries; it is
  // finished here when it starts and ends inside the work-group, and otherwise leaves one
  // record: slot 0 if it began before this work-group's range, slot 1 if it only runs past it.
  // A sequence that lies in the first sub-range alone and began before the range, or in the
  // last sub-range alone and runs past it, left its record from its own wave already.
  bool open = false, before = false;
  float cm = kNegBig, cl = 0.f;
  f32x4 ca[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) ca[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto absorb = [&](int w, int slot) {
    const float2 ml = st_ml(w, slot)[r16];
    const float mn = fmaxf(cm, ml.x);
    const float f0 = __builtin_amdgcn_exp2f(cm - mn), f1 = __builtin_amdgcn_exp2f(ml.x - mn);
    cl = cl * f0 + ml.y * f1;
#pragma unroll
    for (int c = 0; c < NC; ++c) ca[c] = ca[c] * f0 + st_acc(w, slot)[(c * 4 + grp) * G + r16] * f1;
    cm = mn;
  };
  auto restart = [&]() {
    cm = kNegBig;
    cl = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c) ca[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  };
  auto record = [&](int slot) { store_record(slot, cm, cl, ca); };
  for (int sp = 0; sp < kSplits; ++sp) {
    const int w = sp * kHeads + hw;
    if (s_flags[w][0]) {
      if (!open) {  // no earlier sub-range of this work-group holds it: it began before the range
        open = true;
        before = true;
        restart();
      }
      absorb(w, 0);
      if (!s_flags[w][1]) {  // ends inside sub-range sp
        if (before) {
          record(0);
        } else {
          const float inv = cl > 0.f ? 1.f / cl : 0.f;
          const int64_t orow = static_cast<int64_t>(s_flags[w][3]) * p.num_q_heads + g * G + r16;
          if constexpr (SUFFIX) {
            store_partial<D>(p, orow, ca, inv, cm, cl, grp);
          } else {
            raw* o = static_cast<raw*>(p.out) + orow * D;
#pragma unroll
            for (int c = 0; c < NC; ++c) store4<T>(o + 16 * c + 4 * grp, ca[c] * inv);
          }
        }
        open = false;
      }
    }
    if (s_flags[w][2]) {
      open = true;
      before = false;
      restart();
      absorb(w, 1);
    }
  }
  if (open) record(before ? 0 : 1);
}

template <typename T, int D, int BS, bool SUFFIX, int HEADS, bool VEC>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void decode_sk_kernel(SkParams p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char s_dyn[];
  decode_sk_body<T, D, BS, SUFFIX, HEADS, VEC>(p, blockIdx.x, s_dyn);
}

// The prefix-shared decode's prefix pass and suffix pass in one launch: each work-group first
// takes its units of the prefix pass (units blockIdx.x, + gridDim.x, ...), then its range of the
// even split over the suffixes.  Both passes fill the GPU; running them back to back inside
// each work-group saves a launch boundary, and work-groups that finish their prefix units early
// start streaming suffix tiles while the others still read prefix tiles.
template <typename T, int D, int BS, int HEADS, bool VEC>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void prefix_suffix_kernel(SkParams p, PrefixParams pp) {
  extern __shared__ __attribute__((aligned(16))) unsigned char s_dyn[];
  const int units = pp.num_groups * pp.chunks * pp.num_kv_heads;
  for (int u = blockIdx.x; u < units; u += gridDim.x) {
    prefix_unit<T, D, BS>(pp, u, s_dyn);
    __syncthreads();  // the next unit, or the even split, reuses the LDS
  }
  decode_sk_body<T, D, BS, true, HEADS, VEC>(p, blockIdx.x, s_dyn);
}

// Merge of the sequences cut by range boundaries, and the pool writes of a fused append.
//
// One work-group of 8 waves per (range r, group of 4 KV heads).  The range's descriptor names
// the sequence whose first cut lies at the range's start (or none).  Such a sequence has its
// first tile in range r - 1 and spans ranges r - 1 .. rb, so its first two records (range
// r - 1, slot 1; range r, slot 0) are loaded before the descriptor arrives.  Two waves serve
// each KV head of the group: after that first pair (wave row 0), the records of ranges
// r + 1 + 4k .. r + 4 + 4k go to wave row k % 2, four loads in flight (with at most 8 query
// heads per KV head a load carries two records, one per half of the wave, so a row takes
// eight ranges per round); wave row 0 then adds row 1's result and writes the output.  The
// order is fixed: deterministic.
//
// With a fused append the decode kernel took each sequence's new K/V row from new_key /
// new_value; wave row 1 of this kernel writes those rows to their pool slots (position
// context_len - 1, found through the block table), work-group r taking sequences r,
// r + ranges, ...  Wave row 0 waits for row 1's partial result on an LDS flag rather than a
// work-group barrier, so the append does not hold up the merge.
constexpr int kMergeThreads = 512;
// LDS of the merge kernel: for each head column, the partial results of wave rows 1 .. rows-1.
__host__ __device__ inline int merge_lds_bytes(int D, int heads) {
  return heads * (kWaves / heads - 1) * ((D / 16) * 64 * 16 + 64 * 8);
}

// Folds U records (loaded into x / ml; u valid when u < nvalid) into the running (m, l, a).
template <int U, int NC>
__device__ __forceinline__ void fold_records(float& m, float& l, f32x4* a, const float2* ml, f32x4 (*x)[NC], int nvalid) {
  float mn = m;
#pragma unroll
  for (int u = 0; u < U; ++u) mn = u < nvalid ? fmaxf(mn, ml[u].x) : mn;
  const float f0 = __builtin_amdgcn_exp2f(m - mn);
  l *= f0;
#pragma unroll
  for (int q = 0; q < NC; ++q) a[q] *= f0;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const float f = u < nvalid ? __builtin_amdgcn_exp2f(ml[u].x - mn) : 0.f;
    l = fmaf(ml[u].y, f, l);
#pragma unroll
    for (int q = 0; q < NC; ++q) a[q] += x[u][q] * f;
  }
  m = mn;
}

template <typename T, int D, int HEADS>
__global__ __launch_bounds__(kMergeThreads) void merge_sk_kernel(SkParams p) {
  constexpr int kHeads = HEADS, kRows = kWaves / HEADS;  // wave rows per KV head
  using raw = typename T::raw;
  constexpr int NC = D / 16;
  constexpr int U = 4;  // records in flight per wave after the first pair
  const int hgroups = (p.num_kv_heads + kHeads - 1) / kHeads;
  const int r = blockIdx.x / hgroups, hg = blockIdx.x % hgroups;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, r16 = lane & 15,
            grp = lane >> 4;
  const int hw = wave % kHeads, pw = wave / kHeads;
  const int g = hg * kHeads + hw;
  const bool live = g < p.num_kv_heads;
  const int G = p.group;
  const int hr = r16 < G ? r16 : 0;  // rows past the group repeat row 0 (never stored)
  auto rec_of = [&](int c, int slot) { return (static_cast<int64_t>(c) * p.num_kv_heads + g) * 2 + slot; };
  auto load_rec = [&](int64_t rec, float2& ml, f32x4* x) {
    ml = *reinterpret_cast<const float2*>(p.ws_ml + rec * 32 + hr * 2);
#pragma unroll
    for (int q = 0; q < NC; ++q) x[q] = *reinterpret_cast<const f32x4*>(p.ws_acc + rec * (16 * D) + hr * D + 16 * q + 4 * grp);
  };
  // The same through buffer resources: a record that is not needed (valid false) is a
  // zero-length load, which touches no memory, so a batch never loads one record twice.
  auto load_rec_if = [&](int64_t rec, bool valid, float2& ml, f32x4* x) {
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(p.ws_acc) + rec * (16 * D), 0, valid ? 16 * D * 4 : 0, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rm = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(p.ws_ml) + rec * 32, 0, valid ? 32 * 4 : 0, kRsrcWord3);
    ml = __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(rm, hr * 8, 0, 0));
#pragma unroll
    for (int q = 0; q < NC; ++q)
      x[q] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, (hr * D + 16 * q + 4 * grp) * 4, 0, 0));
  };
  extern __shared__ __attribute__((aligned(16))) unsigned char s_merge[];
  // partial result of wave row j >= 1 of head column hw
  auto slot = [&](int j) { return s_merge + (hw * (kRows - 1) + j - 1) * (NC * 64 * 16 + 64 * 8); };
  auto s_a = [&](int j) { return reinterpret_cast<f32x4*>(slot(j)); };
  auto s_ml = [&](int j) { return reinterpret_cast<float2*>(slot(j) + NC * 64 * 16); };
  __shared__ int s_ready[kWaves];  // wave row pw of head column hw has left its partial result

  const int4 dl = *reinterpret_cast<const int4*>(p.ws_desc + 4 * r);
  // the descriptor is the same for every lane: keep it in scalar registers, so that the record
  // loads below take wave-uniform buffer resources
  const int4 d = make_int4(__builtin_amdgcn_readfirstlane(dl.x), __builtin_amdgcn_readfirstlane(dl.y),
                           __builtin_amdgcn_readfirstlane(dl.z), 0);
  float2 ml0[2];
  f32x4 x0[2][NC];
  const bool first = pw == 0 && live && r > 0;
  if (first) {
    load_rec(rec_of(r - 1, 1), ml0[0], x0[0]);
    load_rec(rec_of(r, 0), ml0[1], x0[1]);
  }
  if (tid < kWaves) s_ready[tid] = 0;
  __syncthreads();

  if (d.x >= 0) {  // uniform over the work-group
    const int s = d.x, rb = d.z;  // d.y == r - 1
    float m = kNegBig, l = 0.f;
    f32x4 a[NC];
#pragma unroll
    for (int q = 0; q < NC; ++q) a[q] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (first) fold_records<2, NC>(m, l, a, ml0, x0, 2);
    if (G <= 8) {
      // Two records per load: a record holds G <= 8 rows, so lanes r16 < 8 take ranges
      // c0 .. c0+3 and lanes r16 >= 8 ranges c0+4 .. c0+7, each lane the row r16 & 7 of its
      // record, and one round of four loads folds eight ranges (a sequence spanning up to 17
      // ranges needs one round per wave row).  The two halves fold apart (the second starts
      // empty) and are combined at the end, first half first: a fixed order.
      const int half = r16 >> 3, row = r16 & 7, hr8 = row < G ? row : 0;
      if (half) {
        m = kNegBig;
        l = 0.f;
#pragma unroll
        for (int q = 0; q < NC; ++q) a[q] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      for (int c0 = r + 1 + 2 * U * pw; live && c0 <= rb; c0 += 2 * U * kRows) {
        const int cb = c0 + U * half;  // this half's first range
        float2 ml[U];
        f32x4 x[U][NC];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const bool ok = cb + u <= rb;  // a record past rb is not loaded
          const int64_t rec = rec_of(ok ? cb + u : r, 0);
          ml[u] = ok ? *reinterpret_cast<const float2*>(p.ws_ml + rec * 32 + hr8 * 2) : make_float2(kNegBig, 0.f);
#pragma unroll
          for (int q = 0; q < NC; ++q)
            x[u][q] = ok ? *reinterpret_cast<const f32x4*>(p.ws_acc + rec * (16 * D) + hr8 * D + 16 * q + 4 * grp)
                         : f32x4{0.f, 0.f, 0.f, 0.f};
        }
        __builtin_amdgcn_sched_barrier(0);  // every load above is issued before the first use
        fold_records<U, NC>(m, l, a, ml, x, min(U, max(0, rb - cb + 1)));
      }
      // the second half's result (same row, lane ^ 8) folded into the first half's
      float2 mlo[1] = {make_float2(__shfl_xor(m, 8, 64), __shfl_xor(l, 8, 64))};
      f32x4 xo[1][NC];
#pragma unroll
      for (int q = 0; q < NC; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) xo[0][q][e] = __shfl_xor(a[q][e], 8, 64);
      if (!half) fold_records<1, NC>(m, l, a, mlo, xo, 1);
    } else {
      for (int c0 = r + 1 + U * pw; live && c0 <= rb; c0 += U * kRows) {
        float2 ml[U];
        f32x4 x[U][NC];
#pragma unroll
        for (int u = 0; u < U; ++u) load_rec_if(rec_of(c0 + u <= rb ? c0 + u : c0, 0), c0 + u <= rb, ml[u], x[u]);
        __builtin_amdgcn_sched_barrier(0);  // every load above is issued before the first use
        fold_records<U, NC>(m, l, a, ml, x, rb - c0 + 1);
      }
    }
    if (pw >= 1) {  // hand the partial result to wave row 0 (no work-group barrier: the row goes on)
#pragma unroll
      for (int q = 0; q < NC; ++q) s_a(pw)[q * 64 + lane] = a[q];
      s_ml(pw)[lane] = make_float2(m, l);
      __hip_atomic_store(&s_ready[hw * kRows + pw], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    } else {
      // the other rows of the same work-group always set their flags; the cap only bounds the
      // wait, and a wait that reaches it leaves kStatusWaitGaveUp in the status word (the row's
      // partial result is then not trusted by the caller).  Results are folded in row order: a
      // fixed order.
      bool gave_up = false;
#pragma unroll 1
      for (int j = 1; j < kRows; ++j) {
        int spin = 0;
        while (spin < p.spin_limit &&
               __hip_atomic_load(&s_ready[hw * kRows + j], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) == 0) {
          __builtin_amdgcn_s_sleep(1);
          ++spin;
        }
        gave_up = gave_up || spin >= p.spin_limit;
        float2 mlj[1] = {s_ml(j)[lane]};
        f32x4 xj[1][NC];
#pragma unroll
        for (int q = 0; q < NC; ++q) xj[0][q] = s_a(j)[q * 64 + lane];
        fold_records<1, NC>(m, l, a, mlj, xj, 1);
      }
      if (gave_up && lane == 0) p.ws_status[0] = kStatusWaitGaveUp;
      if (live && r16 < G) {
        const float inv = l > 0.f ? 1.f / l : 0.f;
        const int64_t orow = static_cast<int64_t>(s) * p.num_q_heads + g * G + r16;
        if (p.part_out) {
          store_partial<D>(p, orow, a, inv, m, l, grp);
        } else {
          raw* o = static_cast<raw*>(p.out) + orow * D;
#pragma unroll
          for (int q = 0; q < NC; ++q) store4<T>(o + 16 * q + 4 * grp, a[q] * inv);
        }
      }
    }
  }

  if (p.new_key != nullptr && pw >= 1) {  // fused append (wave rows 1 ..): new rows to their slots
    constexpr int CPR = D * static_cast<int>(sizeof(raw)) / 16;  // 16-byte chunks per row
    constexpr int kRowThreads = 64 * kHeads * (kRows - 1);
    const int64_t row_bytes = static_cast<int64_t>(D) * sizeof(raw);
    const int t = tid - 64 * kHeads, ch = 16 * (t % CPR);
    const int nseq = (p.num_seqs - r + p.ranges - 1) / p.ranges;
    for (int pi = t / CPR; pi < nseq * kHeads; pi += kRowThreads / CPR) {
      const int s = r + p.ranges * (pi / kHeads), gg = hg * kHeads + pi % kHeads;
      if (gg >= p.num_kv_heads) continue;
      const int L = clamp_ctx(p.context_lens[s], p.max_context_len);
      if (L == 0) continue;
      const int phys = p.block_tables[static_cast<int64_t>(s) * p.max_blocks_per_seq + (L - 1) / p.block_size];
      if (phys < 0 || phys >= p.num_blocks) continue;
      const int64_t src = (static_cast<int64_t>(s) * p.num_kv_heads + gg) * row_bytes + ch;
      const int64_t dst = ((static_cast<int64_t>(phys) * p.block_size + (L - 1) % p.block_size) * p.num_kv_heads + gg) *
                              row_bytes + ch;
      const u32x4 kr = *reinterpret_cast<const u32x4*>(static_cast<const unsigned char*>(p.new_key) + src);
      const u32x4 vr = *reinterpret_cast<const u32x4*>(static_cast<const unsigned char*>(p.new_value) + src);
      *reinterpret_cast<u32x4*>(static_cast<unsigned char*>(p.k_cache) + dst) = kr;
      *reinterpret_cast<u32x4*>(static_cast<unsigned char*>(p.v_cache) + dst) = vr;
    }
  }
}

template <typename T, int D, int BS, int HEADS, bool VEC>
void launch_decode(const SkParams& p, dim3 grid, size_t lds, hipStream_t stream) {
  if (p.seq_start)
    hipLaunchKernelGGL((decode_sk_kernel<T, D, BS, true, HEADS, VEC>), grid, dim3(kThreads), lds, stream, p);
  else
    hipLaunchKernelGGL((decode_sk_kernel<T, D, BS, false, HEADS, VEC>), grid, dim3(kThreads), lds, stream, p);
}

template <typename T, int D, int BS, int HEADS>
hipError_t launch(const SkParams& p, hipStream_t stream) {
  const size_t lds = static_cast<size_t>(sk_lds_bytes(p.num_seqs, D, p.group));
  const int hgroups = (p.num_kv_heads + HEADS - 1) / HEADS;
  const dim3 grid(p.ranges * hgroups);
  if constexpr (HEADS == 2) {  // only with a query-head group (sk_heads): no vector-path build
    launch_decode<T, D, BS, HEADS, false>(p, grid, lds, stream);
  } else {
    if (p.group == 1) launch_decode<T, D, BS, HEADS, true>(p, grid, lds, stream);
    else launch_decode<T, D, BS, HEADS, false>(p, grid, lds, stream);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || p.ws_cu) return err;  // suffix mode: the finalize kernel merges
  hipLaunchKernelGGL((merge_sk_kernel<T, D, HEADS>), dim3(p.ranges * hgroups), dim3(kMergeThreads),
                     static_cast<size_t>(merge_lds_bytes(D, HEADS)), stream, p);
  return hipGetLastError();
}

template <typename T, int D, int BS, int HEADS>
hipError_t launch_prefix(const SkParams& p, const PrefixParams& pp, hipStream_t stream) {
  const int sk_lds = sk_lds_bytes(p.num_seqs, D, p.group), pre_lds = prefix_tile_lds_bytes(D);
  const size_t lds = static_cast<size_t>(sk_lds > pre_lds ? sk_lds : pre_lds);
  const int hgroups = (p.num_kv_heads + HEADS - 1) / HEADS;
  const dim3 grid(p.ranges * hgroups), block(kThreads);
  if constexpr (HEADS == 2) {  // only with a query-head group (sk_heads): no vector-path build
    hipLaunchKernelGGL((prefix_suffix_kernel<T, D, BS, HEADS, false>), grid, block, lds, stream, p, pp);
  } else {
    if (p.group == 1)
      hipLaunchKernelGGL((prefix_suffix_kernel<T, D, BS, HEADS, true>), grid, block, lds, stream, p, pp);
    else
      hipLaunchKernelGGL((prefix_suffix_kernel<T, D, BS, HEADS, false>), grid, block, lds, stream, p, pp);
  }
  return hipGetLastError();
}

template <typename T, int D, int BS>
hipError_t launch_prefix_heads(const SkParams& p, const PrefixParams& pp, hipStream_t stream) {
  const int h = sk_heads(p.num_seqs, p.num_kv_heads, p.group);
  return h == 1 ? launch_prefix<T, D, BS, 1>(p, pp, stream)
                : h == 2 ? launch_prefix<T, D, BS, 2>(p, pp, stream) : launch_prefix<T, D, BS, 4>(p, pp, stream);
}

template <typename T, int D>
hipError_t launch_prefix_bs(const SkParams& p, const PrefixParams& pp, hipStream_t stream) {
  if (p.block_size == 8) return launch_prefix_heads<T, D, 8>(p, pp, stream);
  if (p.block_size == 32) return launch_prefix_heads<T, D, 32>(p, pp, stream);
  return launch_prefix_heads<T, D, 16>(p, pp, stream);
}

template <typename T, int D, int BS>
hipError_t launch_heads(const SkParams& p, hipStream_t stream) {
  const int h = sk_heads(p.num_seqs, p.num_kv_heads, p.group);
  return h == 1 ? launch<T, D, BS, 1>(p, stream) : h == 2 ? launch<T, D, BS, 2>(p, stream) : launch<T, D, BS, 4>(p, stream);
}

template <typename T, int D>
hipError_t launch_bs(const SkParams& p, hipStream_t stream) {
  if (p.block_size == 8) return launch_heads<T, D, 8>(p, stream);
  if (p.block_size == 32) return launch_heads<T, D, 32>(p, stream);
  return launch_heads<T, D, 16>(p, stream);
}

}  // namespace

int32_t sk_ranges(int32_t num_seqs, int32_t num_kv_heads, int32_t group, int32_t max_context_len) {
  // About 8 waves per CU on a 256-CU part (one work-group of 8 waves per range and group of
  // sk_heads KV heads), and at least 8 tiles per range (4 per wave) in the worst case: small batches
  // spread over more of the chip (a batch of 4 x 1024 tokens, G 8: 23 us instead of 39 us at
  // 32 tiles per range) without ranges so short that merging their records dominates.
  const int64_t max_blocks = (static_cast<int64_t>(max_context_len) + kTile - 1) / kTile;
  const int64_t upper_tiles = static_cast<int64_t>(num_seqs) * max_blocks;
  const int64_t heads = sk_heads(num_seqs, num_kv_heads, group);
  const int64_t hgroups = (num_kv_heads + heads - 1) / heads;
  int64_t r = kSkTargetWaves / (hgroups * kWaves);
  if (r < 1) r = 1;
  const int64_t cap = (upper_tiles + 7) / 8;
  if (r > cap) r = cap;
  return static_cast<int32_t>(r < 1 ? 1 : r);
}

int sk_lds_bytes_host(int32_t num_seqs, int32_t head_dim, int32_t group) {
  return sk_lds_bytes(num_seqs, head_dim, group) + kSkStaticLds;
}

bool sk_fits(int32_t num_seqs, int32_t head_dim, int32_t group) {
  if (num_seqs < 0 || num_seqs > kSkMaxSeqs || group < 1 || group > 16) return false;
  if (head_dim != 64 && head_dim != 128) return false;
  // the merge kernel's LDS for the largest need among the head counts sk_heads can choose
  int merge = 0;
  for (int heads : {1, 2, 4}) merge = merge > merge_lds_bytes(head_dim, heads) ? merge : merge_lds_bytes(head_dim, heads);
  return sk_lds_bytes_host(num_seqs, head_dim, group) <= kLdsPerWorkgroup &&
         merge + static_cast<int>(kWaves * sizeof(int)) <= kLdsPerWorkgroup;
}

size_t sk_workspace_bytes(int32_t num_seqs, int32_t num_kv_heads, int32_t group, int32_t head_dim,
                          int32_t max_context_len) {
  const int64_t R = sk_ranges(num_seqs, num_kv_heads, group, max_context_len);
  const int64_t recs = R * num_kv_heads * 2;
  const size_t acc = static_cast<size_t>(recs) * 16 * head_dim * sizeof(float);
  const size_t ml = static_cast<size_t>(recs) * 32 * sizeof(float);
  const size_t desc = static_cast<size_t>(R) * 4 * sizeof(int32_t);
  return kStatusBytes + acc + ml + desc;
}

hipError_t sk_launch_prefix(SkParams p, const PrefixParams& pp, int32_t dtype, hipStream_t stream) {
  const int D = p.head_dim;
  if (dtype == PKV_BF16) return D == 64 ? launch_prefix_bs<BF16, 64>(p, pp, stream) : launch_prefix_bs<BF16, 128>(p, pp, stream);
  return D == 64 ? launch_prefix_bs<F16, 64>(p, pp, stream) : launch_prefix_bs<F16, 128>(p, pp, stream);
}

hipError_t sk_launch(SkParams p, int32_t dtype, hipStream_t stream) {
  const int D = p.head_dim;
  if (dtype == PKV_BF16) return D == 64 ? launch_bs<BF16, 64>(p, stream) : launch_bs<BF16, 128>(p, stream);
  return D == 64 ? launch_bs<F16, 64>(p, stream) : launch_bs<F16, 128>(p, stream);
}

}  // namespace sk
}  // namespace pkv
