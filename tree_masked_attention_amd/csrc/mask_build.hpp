// Ancestor-or-self bitmasks of draft trees by pointer jumping.
//
// Rule implemented: a tree node attends to its ancestors (JETFLOW,
// gist.science 2606.18394, section 2 "Arquitectura Central", tree-causal
// attention mask), the root-to-node path including the node itself.
//
// One workgroup per sequence, one thread per node.  Instead of walking each
// node's path (up to B dependent steps), node i keeps its set A_i (W words,
// in registers) and a jump pointer J_i.  Initially A_i = {i} and
// J_i = parent(i).  A round publishes every (A_i, J_i) to LDS and then sets
//     A_i <- A_i | A_{J_i}        J_i <- J_{J_i}
// so after r rounds A_i holds the ancestors within distance < 2^r and J_i
// is the ancestor at distance 2^r (or -1).  At most ceil(log2 B) rounds
// are needed; the loop stops as soon as every jump pointer is -1.
// Ancestors of i have indices <= i, so only words 0 .. i/64 can be set.
#pragma once

#include "common.hpp"

namespace tree_attn {

constexpr int kMaskThreads = 1024;  // = largest supported tree
constexpr int kMaskMaxWords = 16;

// LDS: sets [max_nodes][W] u64 followed by jump [max_nodes] int32.
__global__ __launch_bounds__(kMaskThreads) void build_mask_kernel(
    const int32_t* __restrict__ parents, const int32_t* __restrict__ offsets,
    int num_seqs, int total_nodes, int max_nodes, int W,
    uint64_t* __restrict__ masks, int32_t* __restrict__ bad_node) {
  extern __shared__ __align__(16) unsigned char smem[];
  uint64_t* sets = reinterpret_cast<uint64_t*>(smem);
  int* jump = reinterpret_cast<int*>(sets + (size_t)max_nodes * W);
  __shared__ int first_bad;

  const int s = blockIdx.x;
  const int i = threadIdx.x;
  const int a = clampi(offsets[s], 0, total_nodes);
  const int b = clampi(offsets[s + 1], a, total_nodes);
  const int cap = min(max_nodes, 64 * W);
  const int B = min(b - a, cap);  // nodes handled; the rest are flagged
  if (i == 0) first_bad = (b - a > cap) ? cap : 0x7fffffff;
  __syncthreads();

  const bool mine = i < B;
  uint64_t my[kMaskMaxWords];
  int jp = -1;
  if (mine) {
    const int p = parents[a + i];
    const bool ok = (p >= -1) && (p < i);
    if (!ok) atomicMin(&first_bad, i);
    jp = ok ? p : -1;
  }
#pragma unroll
  for (int w = 0; w < kMaskMaxWords; ++w) {
    my[w] = (mine && w == (i >> 6)) ? (uint64_t(1) << (i & 63)) : uint64_t(0);
  }

  for (int round = 0; round < 11; ++round) {
    if (mine) {
#pragma unroll
      for (int w = 0; w < kMaskMaxWords; ++w) {
        if (w < W && w <= (i >> 6)) sets[i * W + w] = my[w];
      }
      jump[i] = jp;
    }
    // barrier that also tells every thread whether any pointer is left
    if (!__syncthreads_or(jp >= 0)) break;
    if (jp >= 0) {
#pragma unroll
      for (int w = 0; w < kMaskMaxWords; ++w) {
        if (w < W && w <= (jp >> 6)) my[w] |= sets[jp * W + w];
      }
      jp = jump[jp];
    }
    __syncthreads();
  }

  if (mine) {
#pragma unroll
    for (int w = 0; w < kMaskMaxWords; ++w) {
      if (w < W) masks[(size_t)(a + i) * W + w] = my[w];
    }
  }
  // rows past the handled part of an oversized tree are zeroed
  for (int e = B * W + i; e < (b - a) * W; e += kMaskThreads) {
    masks[(size_t)a * W + e] = 0;
  }
  __syncthreads();
  if (i == 0) bad_node[s] = (first_bad == 0x7fffffff) ? -1 : a + first_bad;
}

}  // namespace tree_attn
