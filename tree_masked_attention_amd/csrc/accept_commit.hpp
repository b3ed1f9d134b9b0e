// Acceptance of the verified draft trees and commit of the accepted keys
// and values, the step that follows the verification attention.
//
// The pages give the quantities, not the kernels: decoding keeps tau
// accepted tokens of the tree per step (JETFLOW, gist.science 2606.18394,
// section 4), and the cache / state commit waits until the accepted branch
// is known (DFlash-TfM, gist.science 2607.06763, method section on
// rollback-free verification).  Acceptance here is exact match against the
// target's own choices: node i matches when its draft token equals the
// target's token after its parent (after the prefix, for a root); the
// accepted path is the longest root path whose nodes all match, the one
// ending at the smallest node index among equally long ones.
#pragma once

#include "common.hpp"

namespace tree_attn {

constexpr int kAcceptThreads = 1024;  // one thread per node, largest tree
constexpr int kAcceptMaxWords = 16;

// Bits of mask word w that stand for nodes below B.
__device__ __forceinline__ uint64_t nodes_below(int B, int w) {
  const int lim = B - 64 * w;
  return lim >= 64 ? ~0ull : (lim <= 0 ? 0ull : (1ull << lim) - 1ull);
}

// One workgroup per sequence, thread i = local node i.
//  1. Node i's match bit; one ballot per wave gives mask word i / 64 of the
//     tree's match set M.
//  2. Node i ends a fully matching path when its ancestor-or-self row has
//     no bit outside M; its depth is the row's popcount.  The largest key
//     (depth << 16 | 0xFFFF - i) over such nodes names the end node.
//  3. The end node's row, read once into LDS, is the accepted path: its
//     set bits in increasing order are root first (parent[i] < i), so a
//     path node's position is the number of row bits below it.
__global__ __launch_bounds__(kAcceptThreads) void accept_kernel(
    const int32_t* __restrict__ parents, const int32_t* __restrict__ offsets,
    const uint64_t* __restrict__ masks, int W,
    const int32_t* __restrict__ draft, const int32_t* __restrict__ target,
    const int32_t* __restrict__ root_tokens, int total_nodes, int max_nodes,
    int32_t* __restrict__ accept_len, int32_t* __restrict__ accept_nodes,
    int32_t* __restrict__ bonus) {
  __shared__ uint64_t match[kAcceptMaxWords];
  __shared__ uint64_t path[kAcceptMaxWords];
  __shared__ uint32_t best;
  const int s = blockIdx.x, i = threadIdx.x, lane = i & 63;
  const int a = clampi(offsets[s], 0, total_nodes);
  const int b = clampi(offsets[s + 1], a, total_nodes);
  const int B = min(b - a, max_nodes);  // max_nodes <= 64 * W
  const int root = root_tokens[s];

  bool m = false;
  if (i < B) {
    const int par = parents[a + i];
    if (par == -1) {
      m = draft[a + i] == root;
    } else if (par >= 0 && par < i) {
      m = draft[a + i] == target[a + par];
    }
  }
  const uint64_t ballot = __ballot(m);
  if (lane == 0) match[i >> 6] = ballot;  // blockDim.x <= 64 * W
  if (i == 0) best = 0u;
  __syncthreads();

  if (i < B) {
    bool full = true;
    int depth = 0;
    for (int w = 0; w < W; ++w) {
      const uint64_t r = masks[(size_t)(a + i) * W + w] & nodes_below(B, w);
      full = full && (r & ~match[w]) == 0ull;
      depth += __popcll(r);
    }
    if (full && depth > 0) {
      atomicMax(&best, ((uint32_t)depth << 16) | (uint32_t)(0xFFFF - i));
    }
  }
  __syncthreads();

  const uint32_t key = best;
  const int end = key ? 0xFFFF - (int)(key & 0xFFFFu) : -1;
  if (i < W) {
    path[i] = end >= 0 ? masks[(size_t)(a + end) * W + i] & nodes_below(B, i)
                       : 0ull;
  }
  __syncthreads();

  int tau = 0, rank = 0;
  for (int w = 0; w < W; ++w) {
    const int c = __popcll(path[w]);
    tau += c;
    if (w < (i >> 6)) rank += c;
  }
  int32_t* row = accept_nodes + (size_t)s * max_nodes;
  if (i < B) {
    const uint64_t word = path[i >> 6];
    const uint64_t bit = 1ull << (i & 63);
    if (word & bit) row[rank + __popcll(word & (bit - 1ull))] = i;
  }
  for (int j = tau + i; j < max_nodes; j += blockDim.x) row[j] = -1;
  if (i == 0) {
    accept_len[s] = tau;
    bonus[s] = end >= 0 ? target[a + end] : root;
  }
}

struct CommitParams {
  uint8_t* k;
  uint8_t* v;
  const int32_t* page_table;
  const int32_t* prefix_lens;
  const int32_t* accept_len;
  const int32_t* accept_nodes;
  int max_pages, num_pages, log2_page, max_nodes;
  int pieces;   // 16-byte pieces of one token row of one cache
  int slices;   // workgroups per sequence
  int token_bytes;
};

constexpr int kCommitThreads = 256;
constexpr int kCommitRows = 16;  // rows whose loads are in flight together

// Moves row P + n_j to row P + j for every accepted j with n_j != j (a row
// already in place needs no copy), in the K and the V cache.
//
// First the workgroup turns the accepted list into physical row pairs in
// LDS (-1 = nothing to copy: a row in place, or a source or destination
// outside the page table).  Then thread t of slice sl owns byte columns
// [16 q, 16 q + 16) of every token row, q = 256 sl + t counted over the K
// row then the V row, so the only aliasing between a read and a write is
// inside one thread.  Rows go in increasing j, kCommitRows at a time: every
// load of a group completes before the group's first store.  That is
// enough because accepted nodes are increasing with n_j >= j: a row a group
// writes (P + j) can only be the source of an earlier or the same group
// (n_j' = j needs j' <= j), and a later group only reads rows past every
// row written before it.
__global__ __launch_bounds__(kCommitThreads) void commit_kv_kernel(
    CommitParams p) {
  __shared__ long long src_row[kAcceptThreads];
  __shared__ long long dst_row[kAcceptThreads];
  __shared__ int first;
  const int s = blockIdx.x / p.slices;
  const int q = (blockIdx.x - s * p.slices) * kCommitThreads + threadIdx.x;
  const long long P = p.prefix_lens[s];
  const int tau = clampi(p.accept_len[s], 0, p.max_nodes);
  const int32_t* nodes = p.accept_nodes + (size_t)s * p.max_nodes;
  const int32_t* pt = p.page_table + (size_t)s * p.max_pages;
  const long long pmask = (1ll << p.log2_page) - 1;

  if (threadIdx.x == 0) first = tau;
  __syncthreads();
  for (int j = threadIdx.x; j < tau; j += kCommitThreads) {
    const int n = nodes[j];
    long long sr = -1, dr = -1;
    if (n != j && n >= 0 && n < p.max_nodes && P >= 0) {
      const long long sp = P + n, dp = P + j;
      const long long ls = sp >> p.log2_page, ld = dp >> p.log2_page;
      if (ls < p.max_pages && ld < p.max_pages) {
        const int ps = pt[ls], pd = pt[ld];
        if (ps >= 0 && ps < p.num_pages && pd >= 0 && pd < p.num_pages) {
          sr = ((long long)ps << p.log2_page) + (sp & pmask);
          dr = ((long long)pd << p.log2_page) + (dp & pmask);
          atomicMin(&first, j);
        }
      }
    }
    src_row[j] = sr;
    dst_row[j] = dr;
  }
  __syncthreads();
  if (q >= 2 * p.pieces) return;

  uint8_t* base = q < p.pieces ? p.k : p.v;
  const size_t col = (size_t)(q < p.pieces ? q : q - p.pieces) * 16;
  const size_t tb = (size_t)p.token_bytes;
  for (int j0 = first; j0 < tau; j0 += kCommitRows) {
    u32x4 buf[kCommitRows];
    long long dst[kCommitRows];
#pragma unroll
    for (int u = 0; u < kCommitRows; ++u) {
      const int j = min(j0 + u, tau - 1);
      const long long sr = j0 + u < tau ? src_row[j] : -1;
      dst[u] = j0 + u < tau ? dst_row[j] : -1;
      if (sr >= 0) {
        buf[u] = *reinterpret_cast<const u32x4*>(base + (size_t)sr * tb + col);
      }
    }
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int u = 0; u < kCommitRows; ++u) {
      if (dst[u] >= 0) {
        *reinterpret_cast<u32x4*>(base + (size_t)dst[u] * tb + col) = buf[u];
      }
    }
  }
}

}  // namespace tree_attn
