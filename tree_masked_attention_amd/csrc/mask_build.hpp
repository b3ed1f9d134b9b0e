// Ancestor-or-self bitmasks of draft trees.
//
// Rule implemented: a tree node attends to its ancestors (JETFLOW,
// gist.science 2606.18394, section 2 "Arquitectura Central", tree-causal
// attention mask), the root-to-node path including the node itself.
// Nodes come in topological order (parent[i] < i), so every ancestor of i
// has a smaller index.
//
// One workgroup per sequence, one thread per node, one wave per chunk of 64
// consecutive nodes (chunk c = nodes 64c .. 64c+63, mask word c).
//  1. Inside a wave, pointer jumping over the in-chunk part of each path,
//     with cross-lane reads (ds_bpermute) and no barrier: node i keeps
//     loc_i (its ancestor-or-self bits inside its own chunk), J_i (an
//     in-chunk ancestor not yet merged, or -1) and E_i (its nearest ancestor
//     in an earlier chunk, or -1; final once J_i = -1).  A round sets
//     loc_i |= loc_{J_i}, E_i = E_{J_i}, J_i = J_{J_i}; six rounds cover 64.
//  2. loc and E of every node go to LDS (one barrier).  Word w of node i's
//     mask is then loc_i for w = c, zero for w > c, and for w < c the loc of
//     the node where the chain E_i, E_{E_i}, ... passes through chunk w
//     (each step of that chain lands in a strictly earlier chunk), or zero.
#pragma once

#include "common.hpp"

namespace tree_attn {

constexpr int kMaskThreads = 1024;  // = largest supported tree
constexpr int kMaskMaxWords = 16;

__device__ __forceinline__ int lane_read(int v, int src_lane) {
  return __builtin_amdgcn_ds_bpermute(src_lane << 2, v);
}

__global__ __launch_bounds__(kMaskThreads) void build_mask_kernel(
    const int32_t* __restrict__ parents, const int32_t* __restrict__ offsets,
    int num_seqs, int total_nodes, int max_nodes, int W,
    uint64_t* __restrict__ masks, int32_t* __restrict__ bad_node) {
  __shared__ uint64_t loc_lds[kMaskThreads];
  __shared__ int ext_lds[kMaskThreads];
  __shared__ int first_bad;

  const int s = blockIdx.x;
  const int i = threadIdx.x;
  const int a = clampi(offsets[s], 0, total_nodes);
  const int b = clampi(offsets[s + 1], a, total_nodes);
  const int cap = min(max_nodes, 64 * W);
  const int B = min(b - a, cap);  // nodes handled; the rest are flagged
  if (i == 0) first_bad = (b - a > cap) ? cap : 0x7fffffff;
  __syncthreads();

  const int lane = i & 63;
  const int c0 = i & ~63;  // first node of this wave's chunk
  const bool mine = i < B;
  int p = -1;
  if (mine) {
    p = parents[a + i];
    if (!(p >= -1 && p < i)) {  // not topological: report, treat as a root
      atomicMin(&first_bad, i);
      p = -1;
    }
  }

  // 1. in-chunk pointer jumping
  uint64_t loc = mine ? (1ull << lane) : 0ull;
  int J = (p >= c0) ? p - c0 : -1;
  int E = (p >= 0 && p < c0) ? p : -1;
  for (int r = 0; r < 6 && __any(J >= 0); ++r) {
    const int src = J >= 0 ? J : lane;
    const unsigned lo = (unsigned)lane_read((int)(unsigned)loc, src);
    const unsigned hi = (unsigned)lane_read((int)(unsigned)(loc >> 32), src);
    const int J2 = lane_read(J, src);
    const int E2 = lane_read(E, src);
    if (J >= 0) {
      loc |= ((uint64_t)hi << 32) | lo;
      E = E2;
      J = J2;
    }
  }
  loc_lds[i] = loc;
  ext_lds[i] = E;
  __syncthreads();

  // 2. words of the row, highest first, following the chain of exits
  if (mine) {
    const int c = i >> 6;
    uint64_t* row = masks + (size_t)(a + i) * W;
    int e = E;
    for (int w = W - 1; w >= 0; --w) {
      uint64_t v = 0;
      if (w == c) {
        v = loc;
      } else if (w < c && e >= 0 && (e >> 6) == w) {
        v = loc_lds[e];
        e = ext_lds[e];
      }
      row[w] = v;
    }
  }
  // rows past the handled part of an oversized tree are zeroed
  for (int e = B * W + i; e < (b - a) * W; e += blockDim.x) {
    masks[(size_t)a * W + e] = 0;
  }
  __syncthreads();
  if (i == 0) bad_node[s] = (first_bad == 0x7fffffff) ? -1 : a + first_bad;
}

}  // namespace tree_attn
