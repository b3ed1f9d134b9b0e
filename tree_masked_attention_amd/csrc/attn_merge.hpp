// Log-sum-exp merge of split-KV partials.
//
// Each split c of a row's key range left an unnormalised output O_c, its
// running max m_c (log2 units) and running sum l_c.  With
// m* = max_c m_c and w_c = 2^(m_c - m*):
//     out = sum_c w_c O_c / sum_c w_c l_c,
//     lse = ln2 * (m* + log2 sum_c w_c l_c).
// A split in which the row saw no allowed key has m_c = -inf, l_c = 0 and
// contributes nothing.  One wave per (node, head) row; each lane owns two
// of the 128 output columns.
#pragma once

#include "common.hpp"

namespace tree_attn {

struct MergeParams {
  const int32_t* prefix_lens;
  const int32_t* tree_offsets;
  const float* part_o;
  const float* part_ml;
  __bf16* out;
  float* lse;
  int S, N, Hq, splits, chunk, max_tokens;
};

constexpr int kMergeWaves = 4;

__global__ __launch_bounds__(kMergeWaves * 64) void attn_merge_kernel(
    MergeParams p) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = blockIdx.x * kMergeWaves + wave;
  const int NH = p.N * p.Hq;
  if (row >= NH) return;
  const int node = row / p.Hq;

  // sequence owning this node: last s with tree_offsets[s] <= node
  int lo = 0, hi = p.S - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p.tree_offsets[mid] <= node) lo = mid; else hi = mid - 1;
  }
  const int a = clampi(p.tree_offsets[lo], 0, p.N);
  const int b = clampi(p.tree_offsets[lo + 1], a, p.N);
  const int P = max(p.prefix_lens[lo], 0);
  const int T = min(P + (b - a), p.max_tokens);
  const int nsplit = min(p.splits, (T + p.chunk - 1) / p.chunk);

  float mstar = -INFINITY;
  for (int c = 0; c < nsplit; ++c) {
    mstar = fmaxf(mstar, p.part_ml[((size_t)c * NH + row) * 2]);
  }
  const float mref = (mstar == -INFINITY) ? 0.f : mstar;
  float lsum = 0.f;
  f32x2 acc = {0.f, 0.f};
  for (int c = 0; c < nsplit; ++c) {
    const size_t prow = (size_t)c * NH + row;
    const f32x2 ml = *reinterpret_cast<const f32x2*>(p.part_ml + prow * 2);
    const float w = fast_exp2(ml[0] - mref);
    lsum += w * ml[1];
    const f32x2 oc =
        *reinterpret_cast<const f32x2*>(p.part_o + prow * kHeadDim + lane * 2);
    acc[0] += w * oc[0];
    acc[1] += w * oc[1];
  }
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  bf16x2 r2 = {(__bf16)(acc[0] * inv), (__bf16)(acc[1] * inv)};
  *reinterpret_cast<bf16x2*>(p.out + (size_t)row * kHeadDim + lane * 2) = r2;
  if (lane == 0) {
    p.lse[row] = lsum > 0.f ? (mstar + log2f(lsum)) * kLn2 : -INFINITY;
  }
}

}  // namespace tree_attn
