// Device code of the prefix pass of the prefix-shared decode (included by the translation unit
// that launches it).
//
// Sequences of a group share the physical blocks of their first P tokens (prefix sharing by
// referencing the same blocks: the yunthe.com page, section "PagedAttention分页注意力机制原理";
// the 111cn.net page §3.2, one block shared by several requests).  Attention is a sum over
// tokens, so it splits exactly into the shared prefix and each sequence's own suffix, merged
// with the log-sum-exp rule.  The prefix pass reads each prefix tile once for the whole group:
// a unit of work is one KV head and up to 32 tiles of one group's prefix.  In steps of 8 tiles,
// each of the work-group's 8 waves loads one tile (K and V) into LDS, and then the waves run
// their 16 query rows (member x query head of that KV head) over the step's 8 tiles (several
// waves per row tile, each taking part of the tiles, when the group has 64 rows or fewer).  The LDS
// tiles are double-buffered (144 KiB at D 128): the next step's loads are in flight while the
// current step is computed, so one barrier per step orders the reuse.  A group with more than
// 128 rows repeats the pass for each further 128 rows.  (8 waves and 32-tile chunks measured
// faster than 4 waves and 16-tile chunks at two work-groups per CU: twice the bytes per step,
// half the partial records.)
#pragma once

#include <hip/hip_runtime.h>

#include "dtypes.h"
#include "prefix.h"
#include "tile_common.h"

namespace pkv {
namespace sk {
namespace {

constexpr int kPrefixWaves = 8;  // waves per work-group = tiles per step

// One prefix unit: 32 tiles (chunk c) of one KV head of one group's prefix, for every query
// row of the group.  s_t: LDS for the double-buffered tiles, prefix_tile_lds_bytes(D) bytes.
template <typename T, int D, int BS>
__device__ __forceinline__ void prefix_unit(const PrefixParams& pp, int unit, unsigned char* s_t) {
  constexpr int kPrefixStep = kPrefixWaves;
  using M = Mma<T>;
  using raw = typename T::raw;
  constexpr int ROW = D * 2;
  constexpr int KC = D / 32;
  constexpr int NC = D / 16;
  constexpr int PITCH = sk_pitch(D);
  constexpr int TILE_LDS = kTile * PITCH;
  const int Hkv = pp.num_kv_heads, G = pp.group;
  const int g = unit % Hkv;
  const int c = (unit / Hkv) % pp.chunks;
  const int gi = unit / (Hkv * pp.chunks);
  const int mo = pp.group_offsets[gi], nm = pp.group_offsets[gi + 1] - mo;
  // a batch position belongs to at most one group, so no member list reaches past num_seqs
  if (nm <= 0 || mo < 0 || mo + nm > pp.num_seqs) return;
  const int lead = pp.group_members[mo];
  if (lead < 0 || lead >= pp.num_seqs) return;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, r16 = lane & 15, grp = lane >> 4;
  const int k0 = c * kPrefixChunkTiles;
  // lane i < kPrefixChunkTiles: block ids of chunk tile i (from the first member's table), read
  // alongside the prefix length rather than after it; entries past the prefix are never used
  const int64_t trow = static_cast<int64_t>(lead) * pp.max_blocks_per_seq;
  int e0 = -1, e1 = -1, half = 0;
  {
    const int tok0 = (k0 + lane) * kTile;
    const int bi = tok0 / BS;
    if (lane < kPrefixChunkTiles && bi + (BS == 8 ? 1 : 0) < pp.max_blocks_per_seq) {
      e0 = pp.block_tables[trow + bi];
      if (BS == 8) e1 = pp.block_tables[trow + bi + 1];
    }
    if (BS == 32) half = (tok0 >> 4) & 1;
  }
  const int ptiles = pp.seq_prefix[lead] / kTile;
  const int nk = min(ptiles - k0, kPrefixChunkTiles);
  if (nk <= 0) return;  // uniform over the work-group
  // s_t: [2 buffers][kPrefixStep (8) tiles][K tile, V tile], rows at PITCH

  const int64_t tok_bytes = static_cast<int64_t>(Hkv) * ROW;
  const int64_t block_bytes = BS * tok_bytes;
  const int voff = r16 * static_cast<int>(tok_bytes) + g * ROW + grp * 16;
  const unsigned char* kbase = static_cast<const unsigned char*>(pp.k_cache);
  const unsigned char* vbase = static_cast<const unsigned char*>(pp.v_cache);
  const int nsteps = (nk + kPrefixStep - 1) / kPrefixStep;
  const int rows = nm * G;
  const int lds_slot = r16 * PITCH + grp * 16;  // this lane's 16 bytes of a tile row (+ 64 cc)
  const int tr_base = (4 * grp + (r16 >> 2)) * PITCH + 8 * (r16 & 3);

  u32x4 kbuf[KC], vbuf[KC];
  // Loads chunk tile kk (wave-uniform) into kbuf / vbuf; past the chunk's end a zero-length load.
  auto issue = [&](int kk) {
    int phys = 0, nrec = 0, phys1 = 0, nrec1 = 0, hf = 0;
    if (kk < nk) {
      phys = lane_val(e0, kk);
      nrec = (phys >= 0 && phys < pp.num_blocks) ? static_cast<int>((BS == 8 ? 8 : kTile) * tok_bytes) : 0;
      phys = nrec ? phys : 0;
      if (BS == 32) hf = lane_val(half, kk);
      if (BS == 8) {
        phys1 = lane_val(e1, kk);
        nrec1 = (phys1 >= 0 && phys1 < pp.num_blocks) ? static_cast<int>(kTile * tok_bytes) : 0;
        phys1 = nrec1 ? phys1 : 0;
      }
    }
    if constexpr (BS == 8) {
      // rows 8-15 of the tile are rows 0-7 of the second 8-token block: per-lane 64-bit
      // addresses rather than a buffer resource that differs between the two halves of the wave
      // (a lane whose block id lies outside the pool loads nothing and keeps zeros)
      const bool lo = r16 < 8;
      const bool ok = r16 * tok_bytes < (lo ? nrec : nrec1);
      const int64_t a = (lo ? phys : phys1) * block_bytes + (r16 & 7) * tok_bytes + g * ROW + grp * 16;
#pragma unroll
      for (int cc = 0; cc < KC; ++cc)
        kbuf[cc] = ok ? *reinterpret_cast<const u32x4*>(kbase + a + cc * 64) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int cc = 0; cc < KC; ++cc)
        vbuf[cc] = ok ? *reinterpret_cast<const u32x4*>(vbase + a + cc * 64) : u32x4{0u, 0u, 0u, 0u};
    } else {
      const int64_t off = phys * block_bytes + hf * kTile * tok_bytes;
      const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(kbase) + off, 0, nrec, kRsrcWord3);
      const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(vbase) + off, 0, nrec, kRsrcWord3);
#pragma unroll
      for (int cc = 0; cc < KC; ++cc) kbuf[cc] = __builtin_amdgcn_raw_buffer_load_b128(rk, voff + cc * 64, 0, 0);
#pragma unroll
      for (int cc = 0; cc < KC; ++cc) vbuf[cc] = __builtin_amdgcn_raw_buffer_load_b128(rv, voff + cc * 64, 0, 0);
    }
  };
  // Writes this wave's loaded tile into LDS buffer b, tile slot `wave`.
  auto stash = [&](int b) {
    unsigned char* kt = s_t + (b * kPrefixStep + wave) * 2 * TILE_LDS;
#pragma unroll
    for (int cc = 0; cc < KC; ++cc) *reinterpret_cast<u32x4*>(kt + lds_slot + cc * 64) = kbuf[cc];
#pragma unroll
    for (int cc = 0; cc < KC; ++cc) *reinterpret_cast<u32x4*>(kt + TILE_LDS + lds_slot + cc * 64) = vbuf[cc];
  };

  // With four row tiles or fewer, S waves share a row tile and split each step's tiles between
  // them (tile t goes to part t % S); their partial results are merged at the end of the unit.
  // Every wave then computes, instead of only one per row tile, which halves (or better) the
  // chain of products and exponentials each wave runs per step.
  const int row_tiles = (rows + 15) / 16;
  const int S = row_tiles <= 1 ? 8 : row_tiles <= 2 ? 4 : row_tiles <= 4 ? 2 : 1;
  const int RTc = kPrefixWaves / S;  // row tiles per pass
  const int my_rt = wave % RTc, part = wave / RTc;
  for (int rb = 0; rb * 16 * RTc < rows; ++rb) {
    if (rb > 0) __syncthreads();  // the previous pass's last step is read from buffer 0 or 1
    // row r16 of this wave's row tile: member r / G, query head g * G + r % G
    const int rt0 = (rb * RTc + my_rt) * 16;
    const bool has_rows = rt0 < rows;  // wave-uniform
    const int r = rt0 + r16;
    int seq = pp.group_members[mo + (r < rows ? r / G : 0)];
    const bool valid = r < rows && seq >= 0 && seq < pp.num_seqs;  // rows of invalid members are skipped
    seq = valid ? seq : lead;
    const int qh = g * G + (valid ? r % G : 0);
    const u32x4* qv = reinterpret_cast<const u32x4*>(static_cast<const raw*>(pp.q) +
                                                     (static_cast<int64_t>(seq) * pp.num_q_heads + qh) * D);
    typename M::v8 qb[KC];
#pragma unroll
    for (int cc = 0; cc < KC; ++cc) qb[cc] = __builtin_bit_cast(typename M::v8, valid ? qv[grp + 4 * cc] : u32x4{0u, 0u, 0u, 0u});
    float m_run = kNegBig, l_run = 0.f;
    f32x4 acc[NC];
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) acc[cc] = f32x4{0.f, 0.f, 0.f, 0.f};
    issue(wave);
    for (int j = 0; j < nsteps; ++j) {
      stash(j & 1);
      __syncthreads();
      issue((j + 1) * kPrefixStep + wave);
      if (!has_rows) continue;
      const int nt = min(kPrefixStep, nk - j * kPrefixStep);
      for (int t = part; t < nt; t += S) {
        // every prefix tile is full (16 tokens): no masking
        const unsigned char* kt = s_t + ((j & 1) * kPrefixStep + t) * 2 * TILE_LDS;
        const unsigned char* vt = kt + TILE_LDS;
        f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int cc = 0; cc < KC; ++cc)
          sacc = M::qk(__builtin_bit_cast(typename M::v8, *reinterpret_cast<const u32x4*>(kt + lds_slot + cc * 64)), qb[cc], sacc);
        float sv[4], mx = kNegBig;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sv[e] = sacc[e] * pp.scale_log2e;
          mx = fmaxf(mx, sv[e]);
        }
        mx = swap32_max(swap16_max(mx));
        if (__builtin_amdgcn_ballot_w64(mx > m_run + kTau) != 0) {
          const float mn = fmaxf(m_run, mx);
          const float alpha = __builtin_amdgcn_exp2f(m_run - mn);
          l_run *= alpha;
#pragma unroll
          for (int cc = 0; cc < NC; ++cc) acc[cc] *= alpha;
          m_run = mn;
        }
        i16x4_t pbits;
        float psum = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const short pe = M::pack(__builtin_amdgcn_exp2f(sv[e] - m_run));
          pbits[e] = pe;
          psum += M::unpack(pe);
        }
        l_run += psum;
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) {
          const i16x4_t vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vt + tr_base + 32 * cc));
          acc[cc] = M::pv(vb, pbits, acc[cc]);
        }
      }
    }
    if (S > 1) {
      // parts 1..S-1 leave (m, l, acc) in LDS slot (part - 1) * RTc + my_rt, lane-major
      // (the tile buffers are free once every wave has passed this barrier); part 0 folds them
      constexpr int SLOT = 64 * (NC * 16 + 16);
      __syncthreads();
      if (has_rows && part > 0) {
        unsigned char* sl = s_t + ((part - 1) * RTc + my_rt) * SLOT;
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) *reinterpret_cast<f32x4*>(sl + (cc * 64 + lane) * 16) = acc[cc];
        *reinterpret_cast<f32x4*>(sl + (NC * 64 + lane) * 16) = f32x4{m_run, l_run, 0.f, 0.f};
      }
      __syncthreads();
      if (has_rows && part == 0) {
        for (int q = 1; q < S; ++q) {
          const unsigned char* sl = s_t + ((q - 1) * RTc + my_rt) * SLOT;
          const f32x4 ml = *reinterpret_cast<const f32x4*>(sl + (NC * 64 + lane) * 16);
          const float mn = fmaxf(m_run, ml[0]);
          const float a0 = __builtin_amdgcn_exp2f(m_run - mn), a1 = __builtin_amdgcn_exp2f(ml[0] - mn);
          l_run = l_run * a0 + ml[1] * a1;
#pragma unroll
          for (int cc = 0; cc < NC; ++cc) acc[cc] = acc[cc] * a0 + *reinterpret_cast<const f32x4*>(sl + (cc * 64 + lane) * 16) * a1;
          m_run = mn;
        }
      }
      if (part > 0) continue;  // uniform: one pass when S > 1
    }
    const float lsum = swap32_sum(swap16_sum(l_run));
    if (valid) {
      const int64_t rec = (static_cast<int64_t>(seq) * pp.num_q_heads + qh) * pp.chunks + c;
      float* pa = pp.pre_acc + rec * D;
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) __builtin_nontemporal_store(acc[cc], reinterpret_cast<f32x4*>(pa + 16 * cc + 4 * grp));
      if (grp == 0) {
        __builtin_nontemporal_store(m_run, pp.pre_ml + rec * 2);
        __builtin_nontemporal_store(lsum, pp.pre_ml + rec * 2 + 1);
      }
    }
  }
}

// LDS bytes of one work-group's prefix tiles.  At the end of a unit the same LDS holds the
// partial results of the waves that share a row tile (at most 7 slots of 64 x (D / 16 + 1) x 16
// bytes).
__host__ __device__ constexpr int prefix_tile_lds_bytes(int D) { return 2 * kPrefixWaves * 2 * kTile * sk_pitch(D); }
static_assert(7 * 64 * (128 / 16 + 1) * 16 <= prefix_tile_lds_bytes(128), "prefix merge slots, D 128");
static_assert(7 * 64 * (64 / 16 + 1) * 16 <= prefix_tile_lds_bytes(64), "prefix merge slots, D 64");

}  // namespace
}  // namespace sk
}  // namespace pkv
