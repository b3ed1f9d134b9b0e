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

struct AcceptArgs {
  const int32_t* parents;
  const int32_t* offsets;
  const uint64_t* masks;
  const int32_t* draft;
  const int32_t* target;
  const int32_t* root_tokens;
  int32_t* accept_len;
  int32_t* accept_nodes;
  int32_t* bonus;
  int W, total_nodes, max_nodes;
};

struct AcceptShared {
  uint64_t match[kAcceptMaxWords];
  uint64_t path[kAcceptMaxWords];
  int32_t target[kAcceptThreads];
  uint32_t best;
};

// The accepted path of tree s, computed by the whole workgroup (thread i =
// local node i; blockDim.x >= the tree's node count, whole waves).  Every
// global load is issued in one round: node i's parent, draft and target
// tokens and its ancestor-or-self row (kept in registers).
//  1. Node i matches when its draft token equals the target's token after
//     its parent (read from LDS); one ballot per wave gives mask word i / 64
//     of the tree's match set M.
//  2. Node i ends a fully matching path when its row has no bit outside M;
//     its depth is the row's popcount.  The largest key
//     (depth << 16 | 0xFFFF - i) over such nodes names the end node, which
//     copies its row to LDS (sh.path).
//  3. That row is the accepted path: its set bits in increasing order are
//     root first (parent[i] < i), so a path node's position is the number
//     of row bits below it.
// Returns tau; *rank_out is node i's position on the path, or -1.  With
// write_out the accepted list (padded with -1), tau and the bonus token go
// to the outputs.
__device__ __forceinline__ int accept_tree(const AcceptArgs& p, int s,
                                           AcceptShared& sh, bool write_out,
                                           int* rank_out) {
  const int i = threadIdx.x, lane = i & 63;
  const int a = clampi(p.offsets[s], 0, p.total_nodes);
  const int b = clampi(p.offsets[s + 1], a, p.total_nodes);
  const int B = min(b - a, p.max_nodes);  // max_nodes <= 64 * W
  const int root = p.root_tokens[s];
  const int W = p.W;

  int par = -2, draft = 0;
  uint64_t row[kAcceptMaxWords];
#pragma unroll
  for (int w = 0; w < kAcceptMaxWords; ++w) row[w] = 0ull;
  if (i < B) {
    par = p.parents[a + i];
    draft = p.draft[a + i];
    sh.target[i] = p.target[a + i];
#pragma unroll
    for (int w = 0; w < kAcceptMaxWords; ++w) {
      if (w < W) row[w] = p.masks[(size_t)(a + i) * W + w] & nodes_below(B, w);
    }
  }
  if (i == 0) sh.best = 0u;
  __syncthreads();

  bool m = false;
  if (par == -1) {
    m = draft == root;
  } else if (par >= 0 && par < i) {
    m = draft == sh.target[par];
  }
  const uint64_t ballot = __ballot(m);
  if (lane == 0 && (i >> 6) < W) sh.match[i >> 6] = ballot;
  __syncthreads();

  if (i < B) {
    bool full = true;
    int depth = 0;
#pragma unroll
    for (int w = 0; w < kAcceptMaxWords; ++w) {
      if (w < W) {
        full = full && (row[w] & ~sh.match[w]) == 0ull;
        depth += __popcll(row[w]);
      }
    }
    if (full && depth > 0) {
      atomicMax(&sh.best, ((uint32_t)depth << 16) | (uint32_t)(0xFFFF - i));
    }
  }
  __syncthreads();

  const uint32_t key = sh.best;
  const int end = key ? 0xFFFF - (int)(key & 0xFFFFu) : -1;
  if (end < 0 && i < W) sh.path[i] = 0ull;
  if (i == end) {
#pragma unroll
    for (int w = 0; w < kAcceptMaxWords; ++w) {
      if (w < W) sh.path[w] = row[w];
    }
  }
  __syncthreads();

  int tau = 0, rank = 0;
  for (int w = 0; w < W; ++w) {
    const int c = __popcll(sh.path[w]);
    tau += c;
    if (w < (i >> 6)) rank += c;
  }
  *rank_out = -1;
  if (i < B) {
    const uint64_t word = sh.path[i >> 6];
    const uint64_t bit = 1ull << (i & 63);
    if (word & bit) *rank_out = rank + __popcll(word & (bit - 1ull));
  }
  if (write_out) {
    int32_t* out = p.accept_nodes + (size_t)s * p.max_nodes;
    if (*rank_out >= 0) out[*rank_out] = i;
    for (int j = tau + i; j < p.max_nodes; j += blockDim.x) out[j] = -1;
    if (i == 0) {
      p.accept_len[s] = tau;
      p.bonus[s] = end >= 0 ? sh.target[end] : root;
    }
  }
  return tau;
}

__global__ __launch_bounds__(kAcceptThreads) void accept_kernel(AcceptArgs p) {
  __shared__ AcceptShared sh;
  int rank;
  accept_tree(p, blockIdx.x, sh, true, &rank);
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

struct CommitShared {
  long long src_row[kAcceptThreads];
  long long dst_row[kAcceptThreads];
  int first;
};

// Page-table entry of logical page lp of sequence s (-1 outside the table).
__device__ __forceinline__ int page_entry(const CommitParams& p, int s,
                                          long long lp) {
  return lp < p.max_pages ? p.page_table[(size_t)s * p.max_pages + lp] : -1;
}

// Physical rows (page * page_size + slot) of the copy P + n -> P + j into
// sh (-1 for no copy: a row already in place, or a source or destination
// outside the page table); first = smallest j copied.  ps / pd are the
// page-table entries of the source and destination pages.
__device__ __forceinline__ void plan_pair(const CommitParams& p, long long P,
                                          int j, int n, int ps, int pd,
                                          CommitShared& sh) {
  long long sr = -1, dr = -1;
  if (n != j && ps >= 0 && ps < p.num_pages && pd >= 0 && pd < p.num_pages) {
    const long long pmask = (1ll << p.log2_page) - 1;
    sr = ((long long)ps << p.log2_page) + ((P + n) & pmask);
    dr = ((long long)pd << p.log2_page) + ((P + j) & pmask);
    atomicMin(&sh.first, j);
  }
  sh.src_row[j] = sr;
  sh.dst_row[j] = dr;
}

// plan_pair with the page-table entries read from memory.
__device__ __forceinline__ void plan_row(const CommitParams& p, int s,
                                         long long P, int j, int n,
                                         CommitShared& sh) {
  const bool ok = n >= 0 && n < p.max_nodes && P >= 0;
  const int ps = ok ? page_entry(p, s, (P + n) >> p.log2_page) : -1;
  const int pd = ok ? page_entry(p, s, (P + j) >> p.log2_page) : -1;
  plan_pair(p, P, j, n, ps, pd, sh);
}

// The copies planned in sh, rows first .. tau-1.  Thread t of slice sl
// owns byte columns [16 q, 16 q + 16) of every token row, q = sl *
// blockDim.x + t counted over the K row then the V row, so the only
// aliasing between a read and a write is inside one thread.  Rows go in
// increasing j, kCommitRows at a time: every load of a group completes
// before the group's first store.  That is enough because accepted nodes
// are increasing with n_j >= j: a row a group writes (P + j) can only be
// the source of an earlier or the same group (n_j' = j needs j' <= j), and
// a later group only reads rows past every row written before it.
__device__ __forceinline__ void copy_rows(const CommitParams& p, int slice,
                                          int tau, const CommitShared& sh) {
  const int q = slice * blockDim.x + threadIdx.x;
  if (q >= 2 * p.pieces) return;
  uint8_t* base = q < p.pieces ? p.k : p.v;
  const size_t col = (size_t)(q < p.pieces ? q : q - p.pieces) * 16;
  const size_t tb = (size_t)p.token_bytes;
  for (int j0 = sh.first; j0 < tau; j0 += kCommitRows) {
    u32x4 buf[kCommitRows];
    long long dst[kCommitRows];
#pragma unroll
    for (int u = 0; u < kCommitRows; ++u) {
      const int j = min(j0 + u, tau - 1);
      const long long sr = j0 + u < tau ? sh.src_row[j] : -1;
      dst[u] = j0 + u < tau ? sh.dst_row[j] : -1;
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

// Moves row P + n_j to row P + j for every accepted j with n_j != j (a row
// already in place needs no copy), in the K and the V cache, from the
// accepted lists in memory.  One workgroup per (sequence, column slice).
__global__ __launch_bounds__(kCommitThreads) void commit_kv_kernel(
    CommitParams p) {
  __shared__ CommitShared sh;
  const int s = blockIdx.x / p.slices;
  const int tau = clampi(p.accept_len[s], 0, p.max_nodes);
  const long long P = p.prefix_lens[s];
  const int32_t* nodes = p.accept_nodes + (size_t)s * p.max_nodes;
  if (threadIdx.x == 0) sh.first = tau;
  __syncthreads();
  for (int j = threadIdx.x; j < tau; j += blockDim.x) {
    plan_row(p, s, P, j, nodes[j], sh);
  }
  __syncthreads();
  copy_rows(p, blockIdx.x - s * p.slices, tau, sh);
}

// Acceptance and commit in one launch: every workgroup of sequence s
// computes the accepted path on chip (slice 0 also writes it out), plans
// the copies from it and moves its column slice.  The page-table entries of
// the tree's positions P .. P+B-1 are loaded into LDS in the same round as
// the acceptance inputs.
__global__ __launch_bounds__(kAcceptThreads) void accept_commit_kernel(
    AcceptArgs ap, CommitParams cp) {
  __shared__ AcceptShared ash;
  __shared__ CommitShared csh;
  __shared__ int pages[kAcceptThreads + 1];
  const int s = blockIdx.x / cp.slices;
  const int slice = blockIdx.x - s * cp.slices;
  const long long P = cp.prefix_lens[s];
  const int a = clampi(ap.offsets[s], 0, ap.total_nodes);
  const int B = min(clampi(ap.offsets[s + 1], a, ap.total_nodes) - a,
                    ap.max_nodes);
  // logical pages lp0 .. lp0 + npg - 1 hold the tree (npg <= B + 1)
  const long long lp0 = P >= 0 ? (P >> cp.log2_page) : 0;
  const int npg =
      B > 0 && P >= 0 ? (int)(((P + B - 1) >> cp.log2_page) - lp0 + 1) : 0;
  for (int k = threadIdx.x; k < npg; k += blockDim.x) {
    pages[k] = page_entry(cp, s, lp0 + k);
  }
  if (threadIdx.x == 0) csh.first = cp.max_nodes;
  int rank;
  const int tau = accept_tree(ap, s, ash, slice == 0, &rank);
  if (rank >= 0) {
    // node i = threadIdx.x < B sits at position P + i, its path slot at
    // P + rank with rank <= i: both pages lie in the loaded slice
    const int n = threadIdx.x;
    const bool ok = P >= 0;
    const int ps = ok ? pages[((P + n) >> cp.log2_page) - lp0] : -1;
    const int pd = ok ? pages[((P + rank) >> cp.log2_page) - lp0] : -1;
    plan_pair(cp, P, rank, n, ps, pd, csh);
  }
  __syncthreads();
  copy_rows(cp, slice, tau, csh);
}

}  // namespace tree_attn
