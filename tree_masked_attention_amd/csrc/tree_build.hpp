// Draft-tree construction by best-first expansion of cumulative draft
// log-probabilities, the step before the verification attention.
//
// The drafting head emits, for every depth d = 1 .. D, its top-K candidates
// with log-probabilities (each row non-increasing); a node's score is its
// parent's score plus its own log-probability, and best-first expansion
// builds the tree up to a budget of B nodes (JETFLOW, gist.science
// 2606.18394, section 2, bullet on tree construction).  Each step takes the
// best w candidates at once and expands them together (DFlash-TfM,
// gist.science 2607.06763, method section 2, tree construction); w = 1 is
// strict best-first.  Candidate order: higher score, then lower parent node
// index (the prefix counts as -1), then lower rank -- the order in which an
// eager heap would create them.
//
// One wave per sequence.  The eager heap is kept lazily: because every row
// is sorted, a node's children enter the tree in rank order, so each node
// (and the prefix) needs only one live candidate, its next child.  Slot
// sigma = 0 is the prefix, slot sigma = v + 1 is node v; lane l owns slots
// l, l + 64, ... and keeps, in registers (MS per lane), their live key, next
// rank and node depth and score.  An extraction takes the wave's best key
// (the fp32 score mapped to an ordered integer, reduced with DPP lane moves;
// ties to the lowest slot), appends the node, advances the slot to its
// next child and records the new node's own first child as a candidate
// that becomes live when the step's w extractions are done.  The
// log-probability rows live in LDS, and slot v + 1 keeps node v's record
// (parent, rank, depth, score) in its lane's registers until the outputs
// are written; the extractions of a tree are sequential, so the kernel is
// bound by their latency.
#pragma once

#include "common.hpp"

namespace tree_attn {

constexpr int kTreeMaxLogp = 8192;    // D * K values staged in LDS
constexpr int kTreeMaxTopK = 64;

struct TreeParams {
  const float* logp;      // [S][D][K]
  const int32_t* tokens;  // [S][D][K]
  int32_t* parents;       // [S][B]
  int32_t* out_tokens;    // [S][B]
  int32_t* depths;        // [S][B]
  float* scores;          // [S][B]
  int32_t* sizes;         // [S]
  int D, K, B, W;
};

// fp32 -> unsigned integer with the same order (0 is below every finite
// score and marks an empty slot).
__device__ __forceinline__ uint32_t ordered_key(float x) {
  const uint32_t b = __builtin_bit_cast(uint32_t, x);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float key_score(uint32_t k) {
  const uint32_t b = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __builtin_bit_cast(float, b);
}

// Wave-wide max / min through DPP operands (no LDS round trip): within
// quads, half rows and rows by mirrors, then across rows by the row-15 and
// row-31 broadcasts; lane 63 ends with the result.  Each step is one
// v_max/v_min with a DPP source (two wait states after the previous write
// of that register).
#define TREE_DPP_STEP(op, x, sel, rmask)                                  \
  asm volatile("s_nop 1\n\t" op " %0, %0, %0 " sel " row_mask:" rmask    \
               " bank_mask:0xf"                                          \
               : "+v"(x))

template <bool kMax>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t x) {
  if (kMax) {
    TREE_DPP_STEP("v_max_u32_dpp", x, "quad_perm:[1,0,3,2]", "0xf");
    TREE_DPP_STEP("v_max_u32_dpp", x, "quad_perm:[2,3,0,1]", "0xf");
    TREE_DPP_STEP("v_max_u32_dpp", x, "row_half_mirror", "0xf");
    TREE_DPP_STEP("v_max_u32_dpp", x, "row_mirror", "0xf");
    TREE_DPP_STEP("v_max_u32_dpp", x, "row_bcast:15", "0xa");
    TREE_DPP_STEP("v_max_u32_dpp", x, "row_bcast:31", "0xc");
  } else {
    TREE_DPP_STEP("v_min_u32_dpp", x, "quad_perm:[1,0,3,2]", "0xf");
    TREE_DPP_STEP("v_min_u32_dpp", x, "quad_perm:[2,3,0,1]", "0xf");
    TREE_DPP_STEP("v_min_u32_dpp", x, "row_half_mirror", "0xf");
    TREE_DPP_STEP("v_min_u32_dpp", x, "row_mirror", "0xf");
    TREE_DPP_STEP("v_min_u32_dpp", x, "row_bcast:15", "0xa");
    TREE_DPP_STEP("v_min_u32_dpp", x, "row_bcast:31", "0xc");
  }
  asm volatile("s_nop 1" ::: "memory");
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

template <int MS, bool kStrict>
__global__ __launch_bounds__(64) void build_tree_kernel(TreeParams p) {
  __shared__ float L[kTreeMaxLogp];
  const int s = blockIdx.x, lane = threadIdx.x;
  const int D = p.D, K = p.K, B = p.B;
  const float* lp = p.logp + (size_t)s * D * K;
  for (int i = lane; i < D * K; i += 64) L[i] = lp[i];
  __syncthreads();

  // this lane's slots: sigma = lane + 64 m; slot sigma > 0 also keeps the
  // record of node sigma - 1 (parent slot, rank, depth, score)
  uint32_t key[MS];   // live candidate of the slot (ordered score), 0 = none
  uint32_t pend[MS];  // candidate that becomes live at the end of the step
  int nx[MS];         // rank of the slot's live candidate
  int sdep[MS];       // depth of the slot's node (0: the prefix)
  float ssc[MS];      // score of the slot's node (0: the prefix)
  int spar[MS];       // parent node index of the slot's node
  int srank[MS];      // rank of the slot's node among its parent's children
#pragma unroll
  for (int m = 0; m < MS; ++m) {
    key[m] = 0u;
    pend[m] = 0u;
    nx[m] = 0;
    sdep[m] = 0;
    ssc[m] = 0.f;
    spar[m] = -1;
    srank[m] = 0;
  }
  if (lane == 0 && D > 0 && K > 0) key[0] = ordered_key(L[0]);  // prefix slot

  // lane-local best: highest key, lowest slot on ties (slots ascend with m)
  uint32_t bkey = 0u;
  int bslot = 0;
  auto rescan = [&]() {
    bkey = 0u;
    bslot = 0;
#pragma unroll
    for (int m = 0; m < MS; ++m) {
      const bool better = key[m] > bkey;
      bkey = better ? key[m] : bkey;
      bslot = better ? lane + 64 * m : bslot;
    }
  };
  rescan();

  // Every update below is a per-lane select on (lane, slot) rather than a
  // branch on the owning lane: the extraction is one dependent chain, and
  // on one wave a branch costs more than the selects it skips.
  const int last = max(D * K - 1, 0);
  int size = 0;
  while (size < B) {
    // a step takes min(w, B - size) candidates, fewer when the live ones
    // run out (the step's new nodes only add candidates at its end)
    const int take = kStrict ? 1 : min(p.W, B - size);
    int done = 0;
    for (; done < take; ++done) {
      const uint32_t top = wave_reduce_u32<true>(bkey);
      if (top == 0u) break;
      // lowest slot among the lanes holding the best score
      const uint64_t tied = __ballot(bkey == top);
      int sig;
      if ((tied & (tied - 1)) == 0) {
        sig = __builtin_amdgcn_readlane(bslot, __builtin_ctzll(tied));
      } else {
        sig = (int)wave_reduce_u32<false>(bkey == top ? (uint32_t)bslot
                                                      : 0xffffffffu);
      }
      sig = __builtin_amdgcn_readfirstlane(sig);
      const int owner = sig & 63, ms = sig >> 6;
      // every lane's view of its register ms: next rank, node depth and
      // score; the owner's is the extracted slot's
      int c = 0, pd = 0;
      float ps = 0.f;
#pragma unroll
      for (int m = 0; m < MS; ++m) {
        if (m == ms) {
          c = nx[m];
          pd = sdep[m];
          ps = ssc[m];
        }
      }
      // the slot's next child (row pd: its children are at depth pd + 1),
      // read by every lane at its own in-range address
      const int c1 = c + 1;
      const float l1 = L[min(__mul24(pd, K) + min(c1, K - 1), last)];
      const int cu = __builtin_amdgcn_readlane(c, owner);
      const int d = __builtin_amdgcn_readlane(pd, owner) + 1;
      const float sc = key_score(top);
      // the new node's first child (row d)
      const float l0 = L[min(d, D - 1) * K];
      const int v = size++;
      // the owner's slot advances to its next child (depth-1 scores are
      // the row values themselves)
      const uint32_t nk = c1 < K ? ordered_key(pd == 0 ? l1 : ps + l1) : 0u;
      // the new node takes slot v + 1
      const int sig2 = v + 1, m2 = sig2 >> 6;
      const bool own = lane == owner, mine = lane == (sig2 & 63);
      const uint32_t pk = d < D ? ordered_key(sc + l0) : 0u;
#pragma unroll
      for (int m = 0; m < MS; ++m) {
        const bool adv = own && m == ms;
        key[m] = adv ? nk : key[m];
        nx[m] = adv ? c1 : nx[m];
        const bool put = mine && m == m2;
        sdep[m] = put ? d : sdep[m];
        ssc[m] = put ? sc : ssc[m];
        spar[m] = put ? sig - 1 : spar[m];
        srank[m] = put ? cu : srank[m];
        nx[m] = put ? 0 : nx[m];
        if (kStrict) {
          key[m] = put ? pk : key[m];  // the step ends with this extraction
        } else {
          pend[m] = put ? pk : pend[m];
        }
      }
      rescan();
    }
    if (!kStrict) {
      // end of the step: the new nodes' first children become candidates
#pragma unroll
      for (int m = 0; m < MS; ++m) {
        key[m] = pend[m] != 0u ? pend[m] : key[m];
        pend[m] = 0u;
      }
      rescan();
    }
    if (done == 0) break;  // nothing was live: the tree is complete
  }

  // outputs from the slot records (node v is slot v + 1), padded past the
  // tree's size
  const size_t o = (size_t)s * B;
#pragma unroll
  for (int m = 0; m < MS; ++m) {
    const int v = lane + 64 * m - 1;
    if (v >= 0 && v < B) {
      if (v < size) {
        const int d = sdep[m];
        p.parents[o + v] = spar[m];
        p.out_tokens[o + v] =
            p.tokens[((size_t)s * D + (d - 1)) * K + srank[m]];
        p.depths[o + v] = d;
        p.scores[o + v] = ssc[m];
      } else {
        p.parents[o + v] = -1;
        p.out_tokens[o + v] = -1;
        p.depths[o + v] = 0;
        p.scores[o + v] = 0.f;
      }
    }
  }
  if (lane == 0) p.sizes[s] = size;
}

}  // namespace tree_attn
