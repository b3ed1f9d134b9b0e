// Log-sum-exp merge of split-KV partials.
//
// Each split c of a row's key range leaves its output normalised by its
// own row sum, O'_c = O_c / l_c, stored in fp16 as 2^-e_c O'_c with the
// row's scale exponent e_c (f16_row_exp in common.hpp: 0 unless the row
// reaches 2^15), and two 32-bit words: its log-sum-exp in log2 units,
// L_c = m_c + log2 l_c (m_c its running max, scores in log2 units), and
// e_c.  With L* = max_c L_c and w_c = 2^(L_c - L*):
//     out = sum_c w_c 2^e_c (2^-e_c O'_c) / sum_c w_c,
//     lse = ln2 * (L* + log2 sum_c w_c).
// A split in which the row saw no allowed key has L_c = -inf and
// contributes nothing.  The sums are accumulated with a running maximum,
// which gives the same values up to rounding order.
//
// Two users: attn_merge_kernel (a launch of its own after the attention
// kernel) and merge_rows_wg, which the attention kernel's last split
// workgroup of a row block runs in its epilogue.  Both take every element
// through merge_weights and the same multiply-adds, splits in index
// order, so they produce identical bits.
#pragma once

#include "common.hpp"
#include "split_plan.hpp"

namespace tree_attn {

// The workspace of a split launch starts with this many 32-bit arrival
// counters, one per (sequence, kv head, row block), then the partials.
constexpr int kMergeCounters = 16384;
constexpr size_t kCounterBytes = (size_t)kMergeCounters * 4;

// Split statistics word pair: (L_c, e_c) as (fp32, int32 bits).
__device__ __forceinline__ uint64_t pack_split_stats(float lse2, int e) {
  return (uint64_t)__float_as_uint(lse2) | ((uint64_t)(unsigned)e << 32);
}

// L_c of a split from its running max and row sum (-inf when empty).
__device__ __forceinline__ float split_lse2(float m, float l) {
  return l > 0.f ? m + log2f(l) : -INFINITY;
}

// Folds split c's (L_c, e_c) into a row's running (max, sum of weights);
// returns false when no split so far saw an allowed key (the row's sums
// stay zero), else the factors for acc <- acc * s_old + w * stored_c
// (merge_acc), where w = w_c 2^e_c undoes the partial's scale.
__device__ __forceinline__ bool merge_weights(float& m_run, float& l_run,
                                              f32x2 ml, float& s_old,
                                              float& w) {
  const float m_new = fmaxf(m_run, ml[0]);
  if (m_new == -INFINITY) return false;
  s_old = fast_exp2(m_run - m_new);
  const float wc = fast_exp2(ml[0] - m_new);
  l_run = __builtin_fmaf(l_run, s_old, wc);
  w = ldexp2(wc, __float_as_int(ml[1]));
  m_run = m_new;
  return true;
}

// Where the partials of one row block's splits live: split k's row r of
// the pair is row (slot0 + k * stride) * rows_per_wg + r - r0 of the
// partial arrays (the unit slots of split_plan.hpp).
struct PartSlots {
  int slot0, stride, rows_per_wg, r0;
  __device__ __forceinline__ size_t row(int k, int r) const {
    return (size_t)(slot0 + k * stride) * rows_per_wg + (r - r0);
  }
};

// One output element's running sum (an explicit fma, so that no compiler
// contraction choice can make the two merge paths differ).
__device__ __forceinline__ float merge_acc(float acc, float s_old, float w,
                                          float o) {
  return __builtin_fmaf(w, o, acc * s_old);
}

__device__ __forceinline__ float merge_inv(float l_run) {
  return l_run > 0.f ? 1.f / l_run : 0.f;
}

__device__ __forceinline__ float merge_lse(float m_run, float l_run) {
  return l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
}

struct MergeParams {
  const _Float16* part_o;
  const float* part_ml;
  __bf16* out;
  float* lse;
  int Hq, G;
  SplitParams plan;  // the attention launch's units
};

constexpr int kMergeWaves = 4;
constexpr int kMergeRows = 8;    // rows per wave: 4 per lane half
constexpr int kMergeSplits = 4;  // splits whose loads are issued together
constexpr int kMergeRowsPerWG = kMergeWaves * kMergeRows;

// Workgroups follow the attention launch's units, each unit's rows cut
// into pieces of kMergeRowsPerWG rows; the workgroups of a row block's
// split-0 unit merge it (the others have nothing to do).  A wave merges
// kMergeRows rows, D/4 lanes per row (one row per half-wave for D = 128,
// per quarter-wave for D = 64) with four columns per lane (8-byte loads,
// a whole row per instruction); the loads of kMergeSplits splits of all
// its rows are issued before any is used, and the sums run with a running
// maximum.
template <int D = kHeadDim>
__global__ __launch_bounds__(kMergeWaves * 64) void attn_merge_kernel(
    MergeParams p) {
  constexpr int LPR = D / 4;          // lanes per row
  constexpr int RPP = 64 / LPR;       // rows per pass of the wave
  constexpr int RL = kMergeRows / RPP;  // rows per lane
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int half = lane / LPR, c4 = (lane % LPR) * 4;
  const int pieces = p.plan.rows_per_wg / kMergeRowsPerWG;
  const int L = blockIdx.x / pieces;
  const int piece = blockIdx.x - L * pieces;
  if (L >= p.plan.parts) return;
  Unit un = decode_unit(p.plan, L);
  if (!un.valid || un.split != 0) return;
  load_bounds(p.plan, un);
  if (un.nsplit == 1) return;
  const int rows = p.G * un.B;
  const int rb = un.mb * p.plan.rows_per_wg;
  const int r0 = rb + piece * kMergeRowsPerWG + wave * kMergeRows;
  if (r0 >= rows) return;
  const int nsplit = un.nsplit;
  const PartSlots slots{un.slot0, un.mblocks, p.plan.rows_per_wg, rb};

  size_t qrow[RL];
  int rr[RL];
  float m_run[RL], l_run[RL];
  f32x4 acc[RL];
#pragma unroll
  for (int k = 0; k < RL; ++k) {
    rr[k] = min(r0 + RPP * k + half, rows - 1);
    qrow[k] = (size_t)(un.a + rr[k] / p.G) * p.Hq + un.g * p.G + rr[k] % p.G;
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
        if (c0 + u >= nsplit) break;  // (uniform over the workgroup)
        const int c = c0 + u;
        const size_t prow = slots.row(c, rr[k]);
        ml[k][u] = *reinterpret_cast<const f32x2*>(p.part_ml + prow * 2);
        oc[k][u] = *reinterpret_cast<const f16x4*>(p.part_o + prow * D + c4);
      }
    }
#pragma unroll
    for (int u = 0; u < kMergeSplits; ++u) {
      if (c0 + u >= nsplit) break;
#pragma unroll
      for (int k = 0; k < RL; ++k) {
        float s_old, w;
        if (!merge_weights(m_run[k], l_run[k], ml[k][u], s_old, w)) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[k][e] = merge_acc(acc[k][e], s_old, w, (float)oc[k][u][e]);
        }
      }
    }
  }
#pragma unroll
  for (int k = 0; k < RL; ++k) {
    if (r0 + RPP * k + half >= rows) continue;
    const float inv = merge_inv(l_run[k]);
    bf16x4 r4;
#pragma unroll
    for (int e = 0; e < 4; ++e) r4[e] = (__bf16)(acc[k][e] * inv);
    *reinterpret_cast<bf16x4*>(p.out + qrow[k] * D + c4) = r4;
    if (c4 == 0) p.lse[qrow[k]] = merge_lse(m_run[k], l_run[k]);
  }
}

// Merges rows [r_lo, r_hi) of the (sequence, kv head g) pair whose tree
// starts at node a, over its nsplit splits (partials at slots), with the
// NT threads of a workgroup (head dim D, rows of D fp16 partials): thread
// t takes the
// 16-byte column chunk t % (D/8) of rows r_lo + t / (D/8) + k * NT / (D/8);
// the loads of RT rows and 16 / RT splits are issued before any is used
// (RT = 8 lets a 512-thread workgroup take 256 rows in one pass, whose
// loads then cover two splits at a time), and only those of splits that
// exist.  kCoherent: the partials are read with device-coherent loads
// (written by other workgroups of the running launch).
template <int NT, int D, bool kCoherent, int RT = 4>
__device__ __forceinline__ void merge_rows_wg(
    const _Float16* part_o, const float* part_ml, __bf16* out, float* lse,
    int Hq, int G, int g, int a, int r_lo, int r_hi, int nsplit,
    const PartSlots& slots, int tid) {
  constexpr int CH = D / 8;                  // 16-byte chunks per row
  constexpr int RS = NT / CH;                // rows per pass of the group
  constexpr int KS = 16 / RT;                // splits per round of loads
  static_assert(RT * KS == 16, "merge batch");
  static_assert(NT % CH == 0, "merge layout");
  typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
  const int ch = tid % CH, rsub = tid / CH;
  for (int rb = r_lo; rb < r_hi; rb += RS * RT) {
    size_t qrow[RT];
    int rr[RT];
    float m_run[RT], l_run[RT], acc[RT][8];
#pragma unroll
    for (int k = 0; k < RT; ++k) {
      const int r = min(rb + rsub + k * RS, r_hi - 1);
      rr[k] = r;
      qrow[k] = (size_t)(a + r / G) * Hq + g * G + r % G;
      m_run[k] = -INFINITY;
      l_run[k] = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[k][e] = 0.f;
    }
    for (int c0 = 0; c0 < nsplit; c0 += KS) {
      f32x2 ml[RT][KS];
      f16x8 oc[RT][KS];
#pragma unroll
      for (int k = 0; k < RT; ++k) {
#pragma unroll
        for (int u = 0; u < KS; ++u) {
          if (c0 + u >= nsplit) break;  // (uniform over the workgroup)
          const int c = c0 + u;
          const size_t prow = slots.row(c, rr[k]);
          const _Float16* po = part_o + prow * D + ch * 8;
          if (kCoherent) {
            const uint64_t m2 = load_coherent8(part_ml + prow * 2);
            const uint64_t o0 = load_coherent8(po);
            const uint64_t o1 = load_coherent8(po + 4);
            ml[k][u] = f32x2{__uint_as_float((unsigned)m2),
                             __uint_as_float((unsigned)(m2 >> 32))};
            oc[k][u] = __builtin_bit_cast(f16x8, u64x2{o0, o1});
          } else {
            ml[k][u] = *reinterpret_cast<const f32x2*>(part_ml + prow * 2);
            oc[k][u] = *reinterpret_cast<const f16x8*>(po);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < KS; ++u) {
        if (c0 + u >= nsplit) break;
#pragma unroll
        for (int k = 0; k < RT; ++k) {
          float s_old, w;
          if (!merge_weights(m_run[k], l_run[k], ml[k][u], s_old, w)) continue;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            acc[k][e] = merge_acc(acc[k][e], s_old, w, (float)oc[k][u][e]);
          }
        }
      }
    }
#pragma unroll
    for (int k = 0; k < RT; ++k) {
      if (rb + rsub + k * RS >= r_hi) continue;
      const float inv = merge_inv(l_run[k]);
      bf16x8 r8;
#pragma unroll
      for (int e = 0; e < 8; ++e) r8[e] = (__bf16)(acc[k][e] * inv);
      *reinterpret_cast<bf16x8*>(out + qrow[k] * D + ch * 8) = r8;
      if (ch == 0) lse[qrow[k]] = merge_lse(m_run[k], l_run[k]);
    }
  }
}

// Epilogue of a split workgroup when the launch merges its own partials.
// Every workgroup of a row block that reaches its epilogue (nsplit of
// them) has stored its partials with device-coherent stores (the reader
// may run on another XCD, whose L2 does not see this one's lines); each
// waits for them to complete and counts itself in by a wrapping atomic
// increment at device scope on the block's counter ctr.  The one that sees
// the count reach nsplit - 1 is the last, resets the counter to zero by
// the same increment (so that the next call finds it at zero) and merges
// rows [r_lo, r_hi), reading the partials with device-coherent loads.
// This is the release/acquire pattern with the cache-wide writeback and
// invalidate left out, which only plain (non-coherent) accesses need.  No
// workgroup waits for another.  flag_lds: one int of LDS that no wave uses
// any more.
template <int NT, int D, int RT = 4>
__device__ __forceinline__ void merge_if_last_rows(
    unsigned* ctr, int nsplit, const _Float16* part_o, const float* part_ml,
    __bf16* out, float* lse, int Hq, int G, int g, int a, int r_lo,
    int r_hi, const PartSlots& slots, int tid, int* flag_lds) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // own partials complete
  __syncthreads();
  if (tid == 0) {
    const unsigned old = __builtin_amdgcn_atomic_inc32(
        ctr, (unsigned)(nsplit - 1), __ATOMIC_RELAXED, "agent");
    *flag_lds = old == (unsigned)(nsplit - 1) ? 1 : 0;
  }
  __syncthreads();
  if (*flag_lds == 0) return;
  // issued after the barrier, i.e. after the count was seen complete
  merge_rows_wg<NT, D, true, RT>(part_o, part_ml, out, lse, Hq, G, g, a, r_lo,
                             r_hi, nsplit, slots, tid);
}

}  // namespace tree_attn
