// Tree verification of Gated DeltaNet layers, and the deferred state commit
// (DFlash-TfM, gist.science 2607.06763, method section 3: the tree is
// sorted topologically, verification solves a masked triangular system
// (I + X) U = beta V over ancestor relations, and the recurrent state is
// committed only once the accepted branch is known).
//
// What is computed.  Per head, a GDN layer carries a state S (d_k x d_v)
// updated token by token as S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} +
// beta_t k_t v_t^T.  In a draft tree, node i's state is that recurrence run
// along its root-to-node path from the committed state S0, and its output
// is o_i = S_i^T q_i.  Writing S_i = alpha_i S_parent + k_i u_i^T, with
// G_i the sum of log-decays g along the path (alpha = e^g) and gamma_i =
// e^{G_i}, the update vectors u satisfy, over the ancestors j of i,
//   u_i + sum_{j strict anc i} beta_i e^{G_i - G_j} (k_i . k_j) u_j
//       = beta_i (v_i - gamma_i S0^T k_i),
// i.e. (I + X) U = R, X strictly lower triangular in topological order,
// and
//   o_i = gamma_i S0^T q_i + sum_{j anc-or-self i} e^{G_i - G_j}(q_i . k_j) u_j
//       = gamma_i (Q S0)_i + (Y U)_i.
// The commit of an accepted path p_1 .. p_n runs S <- alpha S + k u^T
// along it: S_n = gamma_n S0 + sum_j e^{G_n - G_{p_j}} k_{p_j} u_{p_j}^T.
//
// Verify kernel: one workgroup of four waves per (sequence, head), trees of
// at most 128 nodes, d_k = d_v = 128.  Wave w owns value columns
// 32w .. 32w+31 of U and O, so the triangular solve needs no exchange
// between waves: the columns of U are independent.  Everything with a
// contraction runs on the bf16 matrix cores (v_mfma_f32_32x32x16_bf16).
// q, k and v are bf16 already, so K S0, the Gram matrices K K^T and Q K^T
// are exact products; an fp32 operand x (S0, X, Y, T, U) is split into two
// bf16 parts hi = bf16(x), lo = bf16(x - hi) and a product takes the terms
// hi*hi + hi*lo + lo*hi (S0 against bf16 K and Q: two terms), which keeps
// about 16 mantissa bits -- the bf16x3 scheme of Henry, Tang and Heinecke,
// "Leveraging the bfloat16 Artificial Intelligence Datatype For
// Higher-Precision Computations" (ARITH 2019).
//
// Phases (barriers between them):
//  1. K and Q rows (bf16) to LDS; per node the mask words, g and beta; the
//     wave's 128 x 32 slice of S0 straight from global memory into B
//     operand registers (split).
//  2. G_i from the ancestor bitmask (the masks the attention path uses).
//  3. K S0 and Q S0 for the wave's columns (accumulators stay in
//     registers), and the lower-triangular 32 x 32 tiles of K K^T and
//     Q K^T, four waves sharing the tiles; a tile is computed transposed
//     (K_J times the row block's K or Q) so that a lane ends up holding
//     runs of 4 consecutive columns of one row of X or Y.
//  4. X (negated) and Y, masked and decayed, written over K / Q in LDS as
//     bf16 hi / lo rows; the diagonal 32 x 32 blocks of X also in fp32.
//  5. T_J = (I + X_JJ)^{-1} of every diagonal block by forward substitution
//     (one wave per block, one column per lane), written over X_JJ.
//  6. Per wave: R = beta (V - gamma K S0); blocked forward substitution
//     U_J = T_J (R_J - sum_{I<J} X_JI U_I); O_J = gamma (Q S0)_J +
//     sum_{I<=J} Y_JI U_I; stores of O (bf16) and U (fp32).
// U never leaves registers between the solve and the output stage: a
// 32 x 32 accumulator tile held by a lane pair as runs of 4 rows is used
// directly as the B operand of the next product, with the A operand's
// columns read from LDS in the same permuted order (the reduction order of
// an MFMA is free, so permuting k in both operands gives the same sum).
#pragma once

#include "common.hpp"

namespace tree_attn {

constexpr int kGdnMaxNodes = 128;
constexpr int kGdnThreads = 256;
constexpr int kGdnKPitch = 272;  // bytes per staged K / Q row (256 + 16)
constexpr int kGdnXPitch = 264;  // bytes per split X / Y row (256 + 8)
constexpr int kGdnKOff = 0;
constexpr int kGdnQOff = kGdnMaxNodes * kGdnKPitch;
// phase 4 regions, written over the K / Q rows once those are consumed
constexpr int kGdnMat = kGdnMaxNodes * kGdnXPitch;
constexpr int kGdnXhi = 0, kGdnXlo = kGdnMat, kGdnYhi = 2 * kGdnMat,
              kGdnYlo = 3 * kGdnMat;
constexpr int kGdnLOff = 4 * kGdnMat;       // fp32 diagonal blocks of X
constexpr int kGdnLdsBytes = kGdnLOff + 4 * 32 * 32 * 4;
static_assert(2 * kGdnQOff <= kGdnLOff, "K / Q staging must fit");

struct GdnParams {
  const __bf16* q;              // [N][H][128]
  const __bf16* k;              // [N][H][128]
  const __bf16* v;              // [N][H][128]
  const float* g;               // [N][H]  log-decay
  const float* beta;            // [N][H]
  const float* state;           // [S][H][128 (k)][128 (v)]  S0
  const int32_t* tree_offsets;  // [S + 1]
  const uint64_t* masks;        // [N][W]
  __bf16* out;                  // [N][H][128]
  float* u;                     // [N][H][128]
  int H, W;
};

typedef __attribute__((address_space(3))) u32x4 gdn_lds_u32x4;
typedef __attribute__((address_space(3))) u32x2 gdn_lds_u32x2;
typedef __attribute__((address_space(3))) f32x4 gdn_lds_f32x4;
typedef __attribute__((address_space(3))) __bf16 gdn_lds_bf16;

__device__ __forceinline__ bf16x8 gdn_read16(unsigned addr) {
  return __builtin_bit_cast(bf16x8, *(const gdn_lds_u32x4*)(size_t)addr);
}

// A operand of a product whose B operand is an accumulator tile: columns
// cb + 4 half .. +3 and cb + 8 + 4 half .. +3 of row `row`.
__device__ __forceinline__ bf16x8 gdn_read_perm(unsigned arr, int row, int cb,
                                                int half) {
  const unsigned a = arr + row * kGdnXPitch + (cb + 4 * half) * 2;
  const u32x2 x = *(const gdn_lds_u32x2*)(size_t)a;
  const u32x2 y = *(const gdn_lds_u32x2*)(size_t)(a + 16);
  const u32x4 r = {x.x, x.y, y.x, y.y};
  return __builtin_bit_cast(bf16x8, r);
}

__device__ __forceinline__ void gdn_split(float x, __bf16& hi, __bf16& lo) {
  hi = (__bf16)x;
  lo = (__bf16)(x - (float)hi);
}

// B operand (k-step s2 of a 32-row product) from an accumulator tile:
// registers 8 s2 .. 8 s2 + 7, split into hi and lo parts.
template <int S2>
__device__ __forceinline__ void gdn_split_tile(const f32x16& c, bf16x8& hi,
                                               bf16x8& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    __bf16 a, b;
    gdn_split(c[8 * S2 + e], a, b);
    hi[e] = a;
    lo[e] = b;
  }
}

// acc += A * B with both operands split (three bf16 products).
__device__ __forceinline__ f32x16 gdn_mfma3(bf16x8 ah, bf16x8 al, bf16x8 bh,
                                            bf16x8 bl, f32x16 acc) {
  acc = mfma32x32x16(ah, bh, acc);
  acc = mfma32x32x16(ah, bl, acc);
  acc = mfma32x32x16(al, bh, acc);
  return acc;
}

__global__ __launch_bounds__(kGdnThreads, 1) void gdn_verify_kernel(
    GdnParams p) {
  __shared__ __align__(16) unsigned char lds[kGdnLdsBytes];
  __shared__ uint64_t mk[kGdnMaxNodes][2];
  __shared__ float gl[kGdnMaxNodes];   // g
  __shared__ float Gc[kGdnMaxNodes];   // G (sum of g over the root path)
  __shared__ float gam[kGdnMaxNodes];  // e^G
  __shared__ float bl[kGdnMaxNodes];   // beta

  const int H = p.H;
  const int s = blockIdx.x / H, h = blockIdx.x - s * H;
  const int n0 = p.tree_offsets[s];
  const int B = p.tree_offsets[s + 1] - n0;
  // trees beyond the supported size are rejected on the host through
  // max_nodes; a tree that breaks that bound is skipped, never overrun
  if (B <= 0 || B > kGdnMaxNodes) return;
  const int NT = (B + 31) >> 5, Bp = NT * 32;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int col = lane & 31, half = lane >> 5;
  const unsigned base =
      (unsigned)(size_t)(__attribute__((address_space(3))) unsigned char*)lds;

  // ---- 1. staging
  for (int x = tid; x < Bp * 16; x += kGdnThreads) {
    const int i = x >> 4, c = x & 15;
    u32x4 kv = {0u, 0u, 0u, 0u}, qv = {0u, 0u, 0u, 0u};
    if (i < B) {
      const size_t off = ((size_t)(n0 + i) * H + h) * kHeadDim + c * 8;
      kv = *reinterpret_cast<const u32x4*>(p.k + off);
      qv = *reinterpret_cast<const u32x4*>(p.q + off);
    }
    *(gdn_lds_u32x4*)(size_t)(base + kGdnKOff + i * kGdnKPitch + c * 16) = kv;
    *(gdn_lds_u32x4*)(size_t)(base + kGdnQOff + i * kGdnKPitch + c * 16) = qv;
  }
  if (tid < Bp) {
    const int i = tid;
    uint64_t m0 = 0, m1 = 0;
    float gv = 0.f, bv = 0.f;
    if (i < B) {
      const uint64_t* mrow = p.masks + (size_t)(n0 + i) * p.W;
      m0 = mrow[0];
      if (B > 64 && p.W > 1) m1 = mrow[1];
      gv = p.g[(size_t)(n0 + i) * H + h];
      bv = p.beta[(size_t)(n0 + i) * H + h];
    }
    mk[i][0] = m0;
    mk[i][1] = m1;
    gl[i] = gv;
    bl[i] = bv;
  }
  // S0 columns 32 w + col, rows 16 ks + 8 half + e: B operands of K S0
  bf16x8 shi[8], slo[8];
  {
    const float* st = p.state + ((size_t)s * H + h) * kHeadDim * kHeadDim +
                      32 * w + col;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        __bf16 a, b;
        gdn_split(st[(size_t)(16 * ks + 8 * half + e) * kHeadDim], a, b);
        shi[ks][e] = a;
        slo[ks][e] = b;
      }
    }
  }
  __syncthreads();

  // ---- 2. G_i over the ancestor-or-self bits, in increasing node order
  if (tid < Bp) {
    float G = 0.f;
    if (tid < B) {
#pragma unroll
      for (int wd = 0; wd < 2; ++wd) {
        uint64_t m = mk[tid][wd];
        while (m) {
          G += gl[wd * 64 + __builtin_ctzll(m)];
          m &= m - 1;
        }
      }
    }
    Gc[tid] = G;
    gam[tid] = fast_exp2(G * kLog2e);
  }
  __syncthreads();

  // ---- 3a. K S0 and Q S0 for this wave's 32 columns
  f32x16 ks[4], qs[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    ks[t] = f32x16{};
    qs[t] = f32x16{};
    if (t < NT) {
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const unsigned ra = (t * 32 + col) * kGdnKPitch + (2 * kk + half) * 16;
        const bf16x8 ak = gdn_read16(base + kGdnKOff + ra);
        const bf16x8 aq = gdn_read16(base + kGdnQOff + ra);
        ks[t] = mfma32x32x16(ak, shi[kk], ks[t]);
        ks[t] = mfma32x32x16(ak, slo[kk], ks[t]);
        qs[t] = mfma32x32x16(aq, shi[kk], qs[t]);
        qs[t] = mfma32x32x16(aq, slo[kk], qs[t]);
      }
    }
  }

  // ---- 3b. Gram tiles: tile n < T1 is X tile (I, J) of the lower
  // triangle in row order, tile T1 + n the Y tile; wave w takes w, w+4, ..
  const int T1 = NT * (NT + 1) / 2;
  f32x16 gt[5];
  int tI[5], tJ[5];
#pragma unroll
  for (int m = 0; m < 5; ++m) {
    const int n = w + 4 * m;
    gt[m] = f32x16{};
    tI[m] = -1;
    tJ[m] = 0;
    if (n < 2 * T1) {
      const bool isx = n < T1;
      int idx = isx ? n : n - T1, I = 0;
      while (idx > I) {
        idx -= I + 1;
        ++I;
      }
      const int J = idx;
      tI[m] = I;
      tJ[m] = J;
      const unsigned src = base + (isx ? kGdnKOff : kGdnQOff);
      f32x16 acc = f32x16{};
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const unsigned off = (2 * kk + half) * 16;
        const bf16x8 a =
            gdn_read16(base + kGdnKOff + (J * 32 + col) * kGdnKPitch + off);
        const bf16x8 b = gdn_read16(src + (I * 32 + col) * kGdnKPitch + off);
        acc = mfma32x32x16(a, b, acc);
      }
      // lane: row i of X / Y, columns J*32 + 8 (r/4) + 4 half + r%4
      const int i = I * 32 + col;
      const float Gi = Gc[i], bi = bl[i];
      const uint32_t mw = (uint32_t)(mk[i][J >> 1] >> ((J & 1) * 32));
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int jl = 8 * (r >> 2) + 4 * half + (r & 3);
        const int j = J * 32 + jl;
        const bool anc = ((mw >> jl) & 1u) && (!isx || j != i);
        const float e = fast_exp2((Gi - Gc[j]) * kLog2e);
        gt[m][r] = anc ? (isx ? bi * e * acc[r] : e * acc[r]) : 0.f;
      }
      if (!isx) tI[m] += 8;  // marks a Y tile (I + 8)
    }
  }
  __syncthreads();  // K / Q rows consumed

  // ---- 4. X (negated) / Y split into LDS; diagonal X blocks in fp32
#pragma unroll
  for (int m = 0; m < 5; ++m) {
    if (tI[m] >= 0) {
      const bool isx = tI[m] < 8;
      const int I = isx ? tI[m] : tI[m] - 8, J = tJ[m];
      const int row = I * 32 + col;
      const unsigned hi_arr = base + (isx ? kGdnXhi : kGdnYhi);
      const unsigned lo_arr = base + (isx ? kGdnXlo : kGdnYlo);
#pragma unroll
      for (int mm = 0; mm < 4; ++mm) {
        bf16x4 hv, lv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x = isx ? -gt[m][4 * mm + e] : gt[m][4 * mm + e];
          __bf16 a, b;
          gdn_split(x, a, b);
          hv[e] = a;
          lv[e] = b;
        }
        const unsigned off = row * kGdnXPitch + (J * 32 + 8 * mm + 4 * half) * 2;
        *(gdn_lds_u32x2*)(size_t)(hi_arr + off) = __builtin_bit_cast(u32x2, hv);
        *(gdn_lds_u32x2*)(size_t)(lo_arr + off) = __builtin_bit_cast(u32x2, lv);
        if (isx && I == J) {
          const f32x4 xv = {gt[m][4 * mm], gt[m][4 * mm + 1],
                            gt[m][4 * mm + 2], gt[m][4 * mm + 3]};
          *(gdn_lds_f32x4*)(size_t)(base + kGdnLOff + J * 4096 + col * 128 +
                                    (8 * mm + 4 * half) * 4) = xv;
        }
      }
    }
  }
  __syncthreads();

  // ---- 5. T_J = (I + X_JJ)^{-1}: lane c computes column c
  if (w < NT) {
    const int J = w, c = col;
    const unsigned Lb = base + kGdnLOff + J * 4096;
    float t[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      float acc = (i == c) ? 1.f : 0.f;
#pragma unroll
      for (int j4 = 0; j4 < (i + 3) / 4; ++j4) {
        const f32x4 L = *(const gdn_lds_f32x4*)(size_t)(Lb + i * 128 + j4 * 16);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (4 * j4 + e < i) acc -= L[e] * t[4 * j4 + e];
        }
      }
      t[i] = acc;
    }
    if (half == 0) {
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        __bf16 a, b;
        gdn_split(t[i], a, b);
        const unsigned off = (J * 32 + i) * kGdnXPitch + (J * 32 + c) * 2;
        *(gdn_lds_bf16*)(size_t)(base + kGdnXhi + off) = a;
        *(gdn_lds_bf16*)(size_t)(base + kGdnXlo + off) = b;
      }
    }
  }
  __syncthreads();

  // ---- 6. R = beta (V - gamma K S0) in place of K S0
  const size_t colg = (size_t)h * kHeadDim + 32 * w + col;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    if (t < NT) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = t * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        float vv = 0.f;
        if (row < B) vv = (float)p.v[(size_t)(n0 + row) * H * kHeadDim + colg];
        ks[t][r] = bl[row] * (vv - gam[row] * ks[t][r]);
      }
    }
  }

  // blocked forward substitution, one 32-row block at a time
  f32x16 uu[4];
  bf16x8 uh[4][2], ul[4][2];
#pragma unroll
  for (int J = 0; J < 4; ++J) {
    uu[J] = f32x16{};
    if (J < NT) {
      f32x16 acc = ks[J];
      const int row = J * 32 + col;
#pragma unroll
      for (int I = 0; I < J; ++I) {
        acc = gdn_mfma3(gdn_read_perm(base + kGdnXhi, row, I * 32, half),
                        gdn_read_perm(base + kGdnXlo, row, I * 32, half),
                        uh[I][0], ul[I][0], acc);
        acc = gdn_mfma3(gdn_read_perm(base + kGdnXhi, row, I * 32 + 16, half),
                        gdn_read_perm(base + kGdnXlo, row, I * 32 + 16, half),
                        uh[I][1], ul[I][1], acc);
      }
      bf16x8 rh0, rl0, rh1, rl1;
      gdn_split_tile<0>(acc, rh0, rl0);
      gdn_split_tile<1>(acc, rh1, rl1);
      f32x16 uj = f32x16{};
      uj = gdn_mfma3(gdn_read_perm(base + kGdnXhi, row, J * 32, half),
                     gdn_read_perm(base + kGdnXlo, row, J * 32, half), rh0,
                     rl0, uj);
      uj = gdn_mfma3(gdn_read_perm(base + kGdnXhi, row, J * 32 + 16, half),
                     gdn_read_perm(base + kGdnXlo, row, J * 32 + 16, half),
                     rh1, rl1, uj);
      uu[J] = uj;
      gdn_split_tile<0>(uj, uh[J][0], ul[J][0]);
      gdn_split_tile<1>(uj, uh[J][1], ul[J][1]);
    }
  }

  // output stage
#pragma unroll
  for (int J = 0; J < 4; ++J) {
    if (J < NT) {
      const int row = J * 32 + col;
      f32x16 acc = f32x16{};
#pragma unroll
      for (int I = 0; I <= J; ++I) {
        acc = gdn_mfma3(gdn_read_perm(base + kGdnYhi, row, I * 32, half),
                        gdn_read_perm(base + kGdnYlo, row, I * 32, half),
                        uh[I][0], ul[I][0], acc);
        acc = gdn_mfma3(gdn_read_perm(base + kGdnYhi, row, I * 32 + 16, half),
                        gdn_read_perm(base + kGdnYlo, row, I * 32 + 16, half),
                        uh[I][1], ul[I][1], acc);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rr = J * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        if (rr < B) {
          const size_t o = (size_t)(n0 + rr) * H * kHeadDim + colg;
          p.out[o] = (__bf16)(gam[rr] * qs[J][r] + acc[r]);
          p.u[o] = uu[J][r];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// State commit.  One workgroup per (sequence, head) updates S0 in place to
// S_n = gamma_n S0 + sum_j e^{G_n - G_{p_j}} k_{p_j} u_{p_j}^T over the
// accepted path p_1 .. p_n (the order tree_attn_accept writes it in).
// Thread t owns 4 consecutive columns 4 (t % 32) .. +3 of the rows
// t / 32 + 8 m; the path's k (fp32) and u (scaled by its decay to the end
// of the path) pass through LDS 32 nodes at a time.

constexpr int kGdnCommitChunk = 32;
constexpr int kGdnMaxPath = 1024;

struct GdnCommitParams {
  const __bf16* k;              // [N][H][128]
  const float* u;               // [N][H][128]
  const float* g;               // [N][H]
  const int32_t* tree_offsets;  // [S + 1]
  const int32_t* accept_len;    // [S]
  const int32_t* accept_nodes;  // [S][max_nodes]  local node indices
  float* state;                 // [S][H][128][128]
  int H, max_nodes;
};

__global__ __launch_bounds__(kGdnThreads) void gdn_commit_kernel(
    GdnCommitParams p) {
  __shared__ __align__(16) float kc[kGdnCommitChunk][kHeadDim];
  __shared__ __align__(16) float uc[kGdnCommitChunk][kHeadDim];
  __shared__ float cf[kGdnMaxPath];  // e^{G_n - G_{p_j}}
  __shared__ int nd[kGdnMaxPath];    // global node index, -1 = skipped
  __shared__ float gam_n;

  const int H = p.H;
  const int s = blockIdx.x / H, h = blockIdx.x - s * H;
  const int tid = threadIdx.x;
  const int n0 = p.tree_offsets[s];
  const int B = p.tree_offsets[s + 1] - n0;
  const int tau = min(max(p.accept_len[s], 0), min(p.max_nodes, kGdnMaxPath));
  if (tau == 0) return;  // nothing accepted: the state stays S0
  const int32_t* path = p.accept_nodes + (size_t)s * p.max_nodes;
  for (int j = tid; j < tau; j += kGdnThreads) {
    const int v = path[j];
    nd[j] = (v >= 0 && v < B) ? n0 + v : -1;
  }
  __syncthreads();
  if (tid == 0) {
    // suffix sums of g from the end of the path
    float acc = 0.f;
    for (int j = tau - 1; j >= 0; --j) {
      cf[j] = fast_exp2(acc * kLog2e);
      if (nd[j] >= 0) acc += p.g[(size_t)nd[j] * H + h];
    }
    gam_n = fast_exp2(acc * kLog2e);
  }
  const int c4 = (tid & 31) * 4, r0 = tid >> 5;
  float* st = p.state + ((size_t)s * H + h) * kHeadDim * kHeadDim;
  f32x4 acc[16];
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    acc[m] = *reinterpret_cast<const f32x4*>(st + (r0 + 8 * m) * kHeadDim + c4);
  }
  __syncthreads();
  const float gn = gam_n;
#pragma unroll
  for (int m = 0; m < 16; ++m) acc[m] *= gn;

  for (int j0 = 0; j0 < tau; j0 += kGdnCommitChunk) {
    const int nc = min(kGdnCommitChunk, tau - j0);
    for (int x = tid; x < kGdnCommitChunk * kHeadDim; x += kGdnThreads) {
      const int jj = x >> 7, e = x & 127;
      float kv = 0.f, uv = 0.f;
      if (jj < nc && nd[j0 + jj] >= 0) {
        const size_t o = ((size_t)nd[j0 + jj] * H + h) * kHeadDim + e;
        kv = (float)p.k[o];
        uv = p.u[o] * cf[j0 + jj];
      }
      kc[jj][e] = kv;
      uc[jj][e] = uv;
    }
    __syncthreads();
    for (int jj = 0; jj < nc; ++jj) {
      const f32x4 uv = *reinterpret_cast<const f32x4*>(&uc[jj][c4]);
#pragma unroll
      for (int m = 0; m < 16; ++m) acc[m] += kc[jj][r0 + 8 * m] * uv;
    }
    __syncthreads();
  }
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    *reinterpret_cast<f32x4*>(st + (r0 + 8 * m) * kHeadDim + c4) = acc[m];
  }
}

}  // namespace tree_attn
