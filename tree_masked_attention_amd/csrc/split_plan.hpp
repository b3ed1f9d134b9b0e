// Work units of the split-KV verification launch, decoded on the device.
//
// A unit is (sequence s, kv head g, key split, row block mb): rows
// mb * rows_per_wg .. of the pair (s, g) over keys [split * chunk,
// min(T_s, (split + 1) * chunk)), T_s = P_s + B_s.  Units are numbered
// sequence by sequence, then kv head, then split, with the row blocks of
// one (s, g, split) adjacent (they read the same K/V; the launch's
// XCD-aware numbering keeps adjacent units in one L2).
//
// Balanced plans (the default) size the key splits from the sequences'
// actual lengths, which only the device knows: one chunk for all
// sequences, the shortest multiple of the 64-key tile (between chunk_min
// and chunk_max) for which every sequence's units fit the launch's
// `parts` workgroups, so a sequence twice as long gets twice the splits,
// and row blocks are counted per sequence (ceil(G B_s / rows_per_wg)).
// Every workgroup computes the same plan from prefix_lens and tree_offsets
// with its own lanes (one lane per sequence, S <= 64).  Forced splits
// (forced_chunk > 0) and launches of more than 64 sequences use the
// host's uniform plan: that chunk and the host's row-block count for every
// sequence.
//
// Partials of a unit live in slot `unit index`: rows_per_wg rows of
// partial output, the row of pair row r at r - mb * rows_per_wg.  The
// slots of one (s, g, mb) for splits k = 0 .. nsplit-1 are slot0 + k *
// mblocks; its arrival counter is `seg`.
#pragma once

#include "common.hpp"

namespace tree_attn {

struct SplitParams {
  const int32_t* prefix_lens;
  const int32_t* tree_offsets;
  int S, N, Hkv, G;        // sequences, nodes, kv heads, q heads per kv head
  int rows_per_wg;         // 64, 128 or 256
  int max_tokens;          // cap of T_s: the page table's reach and the
                           // host bound max_prefix_len + max_nodes
  int max_nodes;           // cap of B_s (host bound)
  int parts;               // units the launch has workgroups for
  int chunk_min, chunk_max;  // bounds of a balanced chunk, keys
  int uniform_chunk;       // > 0: the host's uniform plan with this chunk
  int uniform_splits;      //      and this many splits,
  int uniform_mblocks;     //      this many row blocks per sequence
};

struct Unit {
  int s, g, mb, split;
  int a, B, P, T;          // first node, tree size, prefix, key range
  int nsplit, chunk, mblocks;
  int slot0, seg;
  bool valid;
  bool bounds;             // a, B, P, T and nsplit are set
};

// The tree bounds and split count of a unit of the uniform plan (the
// balanced plan knows them from the decode).  Rows or keys past them mean
// the unit has no work.
__device__ __forceinline__ void load_bounds(const SplitParams& q, Unit& u) {
  if (u.bounds) return;
  u.a = clampi(q.tree_offsets[u.s], 0, q.N);
  const int b = clampi(q.tree_offsets[u.s + 1], u.a, q.N);
  u.B = min(b - u.a, q.max_nodes);
  u.P = max(q.prefix_lens[u.s], 0);
  u.T = min(u.P + u.B, q.max_tokens);
  u.nsplit = min(q.uniform_splits, (max(u.T, 1) + u.chunk - 1) / u.chunk);
  u.bounds = true;
}

// Sum over the 64 lanes of a wave, as a wave-uniform value, from VALU
// cross-lane moves (DPP) and four lane reads (no LDS-pipe round trips; the
// balanced decode takes one sum per step of its search).  quad_perm
// [1,0,3,2] and [2,3,0,1] sum each quad, row_half_mirror and row_mirror
// each row of 16 lanes; the four row sums are then added.
__device__ __forceinline__ int wave_sum_uniform(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false);
  return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) +
         __builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48);
}

// ceil(a / b) for 0 <= a < 2^24 and 1 <= b < 2^16: a float quotient (off
// by at most 2, the quotient being below 2^24), corrected exactly in
// integers.
__device__ __forceinline__ int ceil_div_small(int a, int b) {
  int q = (int)__builtin_ceilf((float)a / (float)b);
  while (q * b < a) ++q;
  while (q > 0 && (q - 1) * b >= a) --q;
  return q;
}

// Inclusive prefix sum over the lanes of a wave, from DPP moves: row_shr
// 1, 2, 4, 8 scan each row of 16 lanes, then row_bcast:15 adds the last
// lane of rows 0 and 2 to rows 1 and 3, and row_bcast:31 the last lane of
// row 1 to rows 2 and 3 (lanes a move does not reach add 0).
__device__ __forceinline__ int wave_scan_dpp(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);
  return v;
}


__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// The unit of workgroup slot L (every lane computes the same unit; the
// fields are made wave-uniform so that they live in scalar registers).
// Invalid when L is past the plan's units.
template <bool kBalanced>
__device__ __forceinline__ Unit decode_unit_lanes(const SplitParams& q,
                                                  int L);
// kBalanced: the launch may use a balanced plan (kernels instantiated for
// uniform plans only leave that code out)
template <bool kBalanced = true>
__device__ __forceinline__ Unit decode_unit(const SplitParams& q, int L) {
  Unit u = decode_unit_lanes<kBalanced>(q, L);
  auto uni = [](int x) { return __builtin_amdgcn_readfirstlane(x); };
  u.s = uni(u.s);
  u.g = uni(u.g);
  u.mb = uni(u.mb);
  u.split = uni(u.split);
  u.a = uni(u.a);
  u.B = uni(u.B);
  u.P = uni(u.P);
  u.T = uni(u.T);
  u.nsplit = uni(u.nsplit);
  u.chunk = uni(u.chunk);
  u.mblocks = uni(u.mblocks);
  u.slot0 = uni(u.slot0);
  u.seg = uni(u.seg);
  u.valid = uni(u.valid ? 1 : 0) != 0;
  u.bounds = uni(u.bounds ? 1 : 0) != 0;
  return u;
}

template <bool kBalanced>
__device__ __forceinline__ Unit decode_unit_lanes(const SplitParams& q,
                                                  int L) {
  const int lane = __lane_id();
  Unit u{};
  u.valid = false;
  if (!kBalanced || q.uniform_chunk > 0) {
    const int mbl = q.uniform_mblocks, spl = q.uniform_splits;
    const int per_seq = q.Hkv * spl * mbl;
    if (L >= q.S * per_seq) return u;
    u.s = L / per_seq;
    int r = L - u.s * per_seq;
    u.g = r / (spl * mbl);
    r -= u.g * spl * mbl;
    u.split = r / mbl;
    u.mb = r - u.split * mbl;
    u.mblocks = mbl;
    u.chunk = q.uniform_chunk;
    u.slot0 = L - u.split * mbl;
    u.seg = (u.s * q.Hkv + u.g) * mbl + u.mb;
    u.bounds = false;  // load_bounds: after the first loads are issued
    u.valid = true;
    return u;
  }
  if constexpr (!kBalanced) {
    return u;
  }
  // balanced plan: lane s holds sequence s
  int T = 0, w = 0, B = 0, a = 0, P = 0;
  if (lane < q.S) {
    a = clampi(q.tree_offsets[lane], 0, q.N);
    B = min(clampi(q.tree_offsets[lane + 1], a, q.N) - a, q.max_nodes);
    P = max(q.prefix_lens[lane], 0);
    T = min(P + B, q.max_tokens);
    w = (B > 0 && T > 0) ? q.Hkv * ceil_div(q.G * B, q.rows_per_wg) : 0;
  }
  // key range in tiles (T < 2^30, so T64 < 2^24); chunks are whole tiles
  const int T64 = (T + 63) >> 6;
  auto parts_for = [&](int chunk) -> int {
    return wave_sum_uniform(w > 0 ? w * ceil_div_small(T64, chunk >> 6) : 0);
  };
  // shortest chunk (in tiles) whose units fit the launch
  int lo = q.chunk_min >> 6, hi = q.chunk_max >> 6;
  if (parts_for(hi << 6) <= q.parts) {
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (parts_for(mid << 6) <= q.parts) hi = mid;
      else lo = mid + 1;
    }
  }
  const int chunk = hi << 6;
  const int ns = w > 0 ? ceil_div(T, chunk) : 0;
  const int parts = w * ns;
  const int incl = wave_scan_dpp(parts);
  const int segs = wave_scan_dpp(w);
  // the sequence whose units contain L
  const uint64_t hit = __ballot(lane < q.S && L < incl && L >= incl - parts);
  if (hit == 0) return u;
  const int s = __builtin_amdgcn_readfirstlane((int)__builtin_ctzll(hit));
  const int base = __builtin_amdgcn_readlane(incl - parts, s);
  const int seg_base = __builtin_amdgcn_readlane(segs - w, s);
  u.s = s;
  u.a = __builtin_amdgcn_readlane(a, s);
  u.B = __builtin_amdgcn_readlane(B, s);
  u.P = __builtin_amdgcn_readlane(P, s);
  u.T = __builtin_amdgcn_readlane(T, s);
  u.nsplit = __builtin_amdgcn_readlane(ns, s);
  u.chunk = chunk;
  u.mblocks = ceil_div(q.G * u.B, q.rows_per_wg);
  int r = L - base;
  const int per_g = u.nsplit * u.mblocks;
  u.g = r / per_g;
  r -= u.g * per_g;
  u.split = r / u.mblocks;
  u.mb = r - u.split * u.mblocks;
  u.slot0 = L - u.split * u.mblocks;
  u.seg = seg_base + u.g * u.mblocks + u.mb;
  u.valid = true;
  u.bounds = true;
  return u;
}

}  // namespace tree_attn
