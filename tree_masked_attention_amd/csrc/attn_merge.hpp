// Log-sum-exp merge of split-KV partials.
//
// Each split c of a row's key range left its output normalised by its own
// row sum, O'_c = O_c / l_c (fp16), its running max m_c (log2 units) and
// its row sum l_c.  With m* = max_c m_c and w_c = 2^(m_c - m*) l_c:
//     out = sum_c w_c O'_c / sum_c w_c,
//     lse = ln2 * (m* + log2 sum_c w_c).
// A split in which the row saw no allowed key has m_c = -inf, l_c = 0 and
// contributes nothing.  The sums are accumulated with a running maximum,
// which gives the same values up to rounding order.
#pragma once

#include "common.hpp"

namespace tree_attn {

struct MergeParams {
  const int32_t* prefix_lens;
  const int32_t* tree_offsets;
  const _Float16* part_o;
  const float* part_ml;
  __bf16* out;
  float* lse;
  int S, N, Hq, Hkv, G, splits, chunk, max_tokens;
  int mblocks, rows_per_block;  // row blocks of the attention launch
};

constexpr int kMergeWaves = 4;
constexpr int kMergeRows = 8;    // rows per wave: 4 per lane half
constexpr int kMergeSplits = 4;  // splits whose loads are issued together
constexpr int kMergeRowsPerWG = kMergeWaves * kMergeRows;

// Workgroups are laid out like the attention launch: (sequence, kv head,
// row block), each row block cut into pieces of kMergeRowsPerWG rows, so
// the sequence of every row is known from the workgroup id.  A wave merges
// kMergeRows rows, each lane half one row at a time with four columns per
// lane (8-byte loads, a whole 256-byte row per half-wave instruction); the
// loads of kMergeSplits splits of all its rows are issued before any is
// used, and the sums run with a running maximum.
__global__ __launch_bounds__(kMergeWaves * 64) void attn_merge_kernel(
    MergeParams p) {
  constexpr int RL = kMergeRows / 2;  // rows per lane
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int half = lane >> 5, c4 = (lane & 31) * 4;
  const int pieces = p.rows_per_block / kMergeRowsPerWG;
  int L = blockIdx.x / pieces;
  const int piece = blockIdx.x - L * pieces;
  const int mb = L % p.mblocks;
  L /= p.mblocks;
  const int g = L % p.Hkv;
  const int s = L / p.Hkv;
  const int a = clampi(p.tree_offsets[s], 0, p.N);
  const int b = clampi(p.tree_offsets[s + 1], a, p.N);
  const int rows = p.G * (b - a);
  const int r0 = mb * p.rows_per_block + piece * kMergeRowsPerWG +
                 wave * kMergeRows;
  if (r0 >= rows) return;
  const int P = max(p.prefix_lens[s], 0);
  const int T = min(P + (b - a), p.max_tokens);
  const int nsplit = min(p.splits, (T + p.chunk - 1) / p.chunk);
  const size_t NH = (size_t)p.N * p.Hq;

  size_t qrow[RL];
  float m_run[RL], l_run[RL];
  f32x4 acc[RL];
#pragma unroll
  for (int k = 0; k < RL; ++k) {
    const int r = min(r0 + 2 * k + half, rows - 1);
    qrow[k] = (size_t)(a + r / p.G) * p.Hq + g * p.G + r % p.G;
    m_run[k] = -INFINITY;
    l_run[k] = 0.f;
    acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  for (int c0 = 0; c0 < nsplit; c0 += kMergeSplits) {
    f32x2 ml[RL][kMergeSplits];
    f16x4 oc[RL][kMergeSplits];
#pragma unroll
    for (int k = 0; k < RL; ++k) {
#pragma unroll
      for (int u = 0; u < kMergeSplits; ++u) {
        const int c = min(c0 + u, nsplit - 1);  // in range; unused if past
        const size_t prow = (size_t)c * NH + qrow[k];
        ml[k][u] = *reinterpret_cast<const f32x2*>(p.part_ml + prow * 2);
        oc[k][u] = *reinterpret_cast<const f16x4*>(p.part_o + prow * kHeadDim +
                                                   c4);
      }
    }
#pragma unroll
    for (int u = 0; u < kMergeSplits; ++u) {
      if (c0 + u >= nsplit) break;
#pragma unroll
      for (int k = 0; k < RL; ++k) {
        const float m_new = fmaxf(m_run[k], ml[k][u][0]);
        if (m_new == -INFINITY) continue;  // no key seen yet
        const float s_old = fast_exp2(m_run[k] - m_new);
        const float w = fast_exp2(ml[k][u][0] - m_new) * ml[k][u][1];
        l_run[k] = l_run[k] * s_old + w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[k][e] = acc[k][e] * s_old + w * (float)oc[k][u][e];
        }
        m_run[k] = m_new;
      }
    }
  }
#pragma unroll
  for (int k = 0; k < RL; ++k) {
    if (r0 + 2 * k + half >= rows) continue;
    const float inv = l_run[k] > 0.f ? 1.f / l_run[k] : 0.f;
    bf16x4 r4;
#pragma unroll
    for (int e = 0; e < 4; ++e) r4[e] = (__bf16)(acc[k][e] * inv);
    *reinterpret_cast<bf16x4*>(p.out + qrow[k] * kHeadDim + c4) = r4;
    if ((lane & 31) == 0) {
      p.lse[qrow[k]] =
          l_run[k] > 0.f ? (m_run[k] + log2f(l_run[k])) * kLn2 : -INFINITY;
    }
  }
}

}  // namespace tree_attn
