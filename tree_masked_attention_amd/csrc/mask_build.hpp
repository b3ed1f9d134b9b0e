// Ancestor-or-self bitmasks of draft trees by pointer jumping in LDS.
//
// Rule implemented: a tree node attends to its ancestors (JETFLOW,
// gist.science 2606.18394, section 2 "Arquitectura Central", tree-causal
// attention mask), the root-to-node path including the node itself.
//
// One workgroup per sequence.  Instead of walking each node's path (up to
// B dependent steps), every node i keeps a set A_i and a jump pointer J_i.
// Initially A_i = {i} and J_i = parent(i).  A round replaces
//     A_i <- A_i  |  A_{J_i}        J_i <- J_{J_i}
// so after r rounds A_i holds the ancestors within distance < 2^r and J_i
// is the ancestor at distance 2^r (or -1).  ceil(log2 B) rounds finish the
// job; the loop stops as soon as every jump pointer is -1.
#pragma once

#include "common.hpp"

namespace tree_attn {

constexpr int kMaskThreads = 1024;
constexpr int kMaskMaxWords = 16;
// Each thread carries at most this many (node, word) pairs through a round.
constexpr int kMaskPerThread = (1024 * kMaskMaxWords) / kMaskThreads;

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
  const int tid = threadIdx.x;
  const int a = clampi(offsets[s], 0, total_nodes);
  const int b = clampi(offsets[s + 1], a, total_nodes);
  const int cap = min(max_nodes, 64 * W);
  const int B = min(b - a, cap);  // nodes handled; the rest are flagged
  if (tid == 0) first_bad = (b - a > cap) ? cap : 0x7fffffff;
  __syncthreads();

  for (int i = tid; i < B; i += kMaskThreads) {
    int p = parents[a + i];
    bool ok = (p >= -1) && (p < i);
    if (!ok) atomicMin(&first_bad, i);
    jump[i] = ok ? p : -1;
  }
  const int pairs = B * W;
  for (int e = tid; e < pairs; e += kMaskThreads) {
    int i = e / W, w = e - i * W;
    sets[e] = (w == (i >> 6)) ? (uint64_t(1) << (i & 63)) : uint64_t(0);
  }
  __syncthreads();

  for (int round = 0; round < 11; ++round) {
    int any_jump = 0;
    uint64_t nv[kMaskPerThread];
    int nj[kMaskPerThread];
#pragma unroll
    for (int k = 0; k < kMaskPerThread; ++k) {
      int e = tid + k * kMaskThreads;
      nv[k] = 0;
      if (e < pairs) {
        int i = e / W, w = e - i * W;
        int j = jump[i];
        nv[k] = sets[e] | (j >= 0 ? sets[j * W + w] : uint64_t(0));
      }
      nj[k] = -1;
      if (e < B) {
        int j = jump[e];
        nj[k] = j >= 0 ? jump[j] : -1;
        if (nj[k] >= 0) any_jump = 1;
      }
    }
    // barrier that also tells every thread whether any pointer is left
    any_jump = __syncthreads_or(any_jump);
#pragma unroll
    for (int k = 0; k < kMaskPerThread; ++k) {
      int e = tid + k * kMaskThreads;
      if (e < pairs) sets[e] = nv[k];
      if (e < B) jump[e] = nj[k];
    }
    __syncthreads();
    if (!any_jump) break;
  }

  for (int e = tid; e < pairs; e += kMaskThreads) {
    masks[(size_t)a * W + e] = sets[e];
  }
  // rows past the handled part of an oversized tree are zeroed
  for (int e = pairs + tid; e < (b - a) * W; e += kMaskThreads) {
    masks[(size_t)a * W + e] = 0;
  }
  if (tid == 0) bad_node[s] = (first_bad == 0x7fffffff) ? -1 : a + first_bad;
}

}  // namespace tree_attn
