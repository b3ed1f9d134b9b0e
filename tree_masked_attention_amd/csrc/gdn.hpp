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
//  1. Every global load of the tree issued up front: the wave's 128 x 32
//     slice of S0 into registers, K, Q and V rows through registers into
//     LDS, per node the mask words, g and beta.
//  2. G_i by pointer jumping over the parents read from the mask rows.
//  3. The diagonal 32 x 32 X blocks in fp32 (one per wave).
//  4. K S0 and Q S0 on the matrix cores, interleaved with the inversion
//     T_w = (I + X_ww)^{-1} of diagonal block w (right-looking
//     substitution, VALU); then R = beta (V - gamma K S0).
//  5. The off-diagonal X tiles and all Y tiles of the lower triangle, four
//     waves sharing them; a tile is computed transposed (K_J times the row
//     block's K or Q) so that a lane holds runs of 4 consecutive columns
//     of one row of X or Y.
//  6. -X, Y and T_w written over the staged rows as bf16 hi / lo rows.
//  7. Per wave: blocked forward substitution U_I = T_I (R_I - sum_{I'<I}
//     X_II' U_I'), right-looking; O_J = gamma (Q S0)_J + sum_{I<=J} Y_JI
//     U_I; U (fp32) and O (bf16) stored straight from registers.
// U never leaves registers between the solve and the output stage: a
// 32 x 32 accumulator tile held by a lane pair as runs of 4 rows is used
// directly as the B operand of the next product, with the A operand's
// columns read from LDS in the same permuted order (the reduction order of
// an MFMA is free, so permuting k in both operands gives the same sum).
#pragma once

#include <type_traits>

#include "common.hpp"

namespace tree_attn {

constexpr int kGdnMaxNodes = 128;
constexpr int kGdnMaxHeads = 16384;  // keeps a tree's u rows below 2^31 bytes
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
constexpr int kGdnVOff = 2 * kGdnQOff;      // V rows (256 bytes), phase 1-4
constexpr int kGdnLdsBytes = kGdnLOff + 4 * 32 * 32 * 4;
static_assert(kGdnVOff + kGdnMaxNodes * 256 <= kGdnLOff,
              "K / Q / V staging must fit below the fp32 blocks");

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

// Two values split at once (one packed conversion per part): hi and lo
// hold the bf16 pairs (x0 in the low half).
__device__ __forceinline__ void gdn_split2(float x0, float x1, uint32_t& hi,
                                           uint32_t& lo) {
  const bf16x2 h = {(__bf16)x0, (__bf16)x1};
  const uint32_t hb = __builtin_bit_cast(uint32_t, h);
  const float h0 = __builtin_bit_cast(float, hb << 16);
  const float h1 = __builtin_bit_cast(float, hb & 0xffff0000u);
  const bf16x2 l = {(__bf16)(x0 - h0), (__bf16)(x1 - h1)};
  hi = hb;
  lo = __builtin_bit_cast(uint32_t, l);
}

// B operand (k-step s2 of a 32-row product) from an accumulator tile:
// registers 8 s2 .. 8 s2 + 7, split into hi and lo parts.
template <int S2>
__device__ __forceinline__ void gdn_split_tile(const f32x16& c, bf16x8& hi,
                                               bf16x8& lo) {
  u32x4 h, l;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    uint32_t a, b;
    gdn_split2(c[8 * S2 + 2 * e], c[8 * S2 + 2 * e + 1], a, b);
    h[e] = a;
    l[e] = b;
  }
  hi = __builtin_bit_cast(bf16x8, h);
  lo = __builtin_bit_cast(bf16x8, l);
}

// acc += A * B with both operands split (three bf16 products).
__device__ __forceinline__ f32x16 gdn_mfma3(bf16x8 ah, bf16x8 al, bf16x8 bh,
                                            bf16x8 bl, f32x16 acc) {
  acc = mfma32x32x16(ah, bh, acc);
  acc = mfma32x32x16(ah, bl, acc);
  acc = mfma32x32x16(al, bh, acc);
  return acc;
}

struct GdnSmall {
  uint64_t mk[kGdnMaxNodes][2];  // ancestor-or-self words of each node
  float gl[kGdnMaxNodes];        // g
  float Gc[kGdnMaxNodes];        // G log2(e): G the sum of g over the root path
  float gam[kGdnMaxNodes];       // e^G
  float bl[kGdnMaxNodes];        // beta
};

typedef __attribute__((address_space(3))) float gdn_lds_f32;

// Highest strict ancestor (the parent) of local node i from its mask row.
__device__ __forceinline__ int gdn_parent(const GdnSmall& sm, int i) {
  uint64_t m0 = sm.mk[i][0], m1 = sm.mk[i][1];
  if (i < 64) {
    m0 &= ~(1ull << i);
  } else {
    m1 &= ~(1ull << (i - 64));
  }
  if (m1) return 127 - __builtin_clzll(m1);
  if (m0) return 63 - __builtin_clzll(m0);
  return -1;
}

__device__ __forceinline__ float gdn_bperm(int lane_src, float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_ds_bpermute(lane_src << 2,
                                          __builtin_bit_cast(int, x)));
}

__device__ __forceinline__ int gdn_bperm(int lane_src, int x) {
  return __builtin_amdgcn_ds_bpermute(lane_src << 2, x);
}

// Raw buffer resource over `bytes` bytes from p: loads past the end read 0,
// stores past the end are dropped by the hardware range check.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t gdn_rsrc(void* p,
                                                          uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, (int)bytes,
                                           0x00020000);
}

// Stores a 32 x 32 fp32 accumulator tile (lane (col, half), register r:
// row row0 + 8 (r/4) + 4 half + r%4, column col) straight from registers
// through a buffer resource whose range ends at the tree's last row, so
// rows past the tree are dropped without a test.  Each store writes two
// 32-column row segments.  With kBf16 the values are rounded to bf16.
template <bool kBf16>
__device__ __forceinline__ void gdn_store_tile(const f32x16& c,
                                               __amdgpu_buffer_rsrc_t rs,
                                               uint32_t ld_bytes, int row0,
                                               int lane) {
  const int col = lane & 31, half = lane >> 5;
  constexpr int esz = kBf16 ? 2 : 4;
  const uint32_t lo = 4 * half * ld_bytes + col * esz;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const uint32_t off = lo + (uint32_t)(row0 + 8 * (r >> 2) + (r & 3)) * ld_bytes;
    // through a scalar: a bit cast of the vector element itself reads
    // element 0 (seen with this compiler)
    const float x = c[r];
    if (kBf16) {
      const __bf16 y = (__bf16)x;
      __builtin_amdgcn_raw_buffer_store_b16(
          __builtin_bit_cast(unsigned short, y), rs, off, 0, 0);
    } else {
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, x),
                                            rs, off, 0, 0);
    }
  }
}

// Keeps a value computed where it stands: without it the optimizer sinks
// pure arithmetic past a barrier to its use and keeps the loaded operands
// alive across the barrier instead.
__device__ __forceinline__ void gdn_pin(float& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void gdn_pin(f32x16& x) {
  asm volatile("" : "+v"(x));
}

// Row col of T = (I + L)^{-1} (L strictly lower triangular, 32 x 32, row
// major at Lb in fp32), right-looking: t holds the partial sums
// t_j = [j == col] - sum_{i > j, done} t_i L_ij; step I takes t_I as final
// and subtracts t_I L_Ij from every t_j, j < I.  The FMAs of a step are
// independent of each other and row I - 2 of L is read during step I, so
// a step is bound by issue, not latency, and slot(31 - I) issues matrix-core
// work beside it.  One instantiation per step keeps every index static;
// the scheduling barrier between steps keeps the compiler from hoisting
// all reads of L to the top (and spilling them).
template <int I, class Slot>
__device__ __forceinline__ void gdn_t_step(float (&tr)[32], f32x4 (&L0)[8],
                                           f32x4 (&L1)[8], f32x4 (&L2)[8],
                                           unsigned Lb, Slot& slot) {
  // L0 holds row I, L1 row I - 1 (in flight); read row I - 2 into L2
  if constexpr (I > 2) {
#pragma unroll
    for (int j4 = 0; j4 < (I - 2 + 3) / 4; ++j4) {
      L2[j4] = *(const gdn_lds_f32x4*)(size_t)(Lb + (I - 2) * 128 + j4 * 16);
    }
  }
  slot(std::integral_constant<int, 31 - I>{});
  const float ti = tr[I];
#pragma unroll
  for (int j = 0; j < I; ++j) tr[j] -= ti * L0[j >> 2][j & 3];
  gdn_pin(tr[I]);
#pragma unroll
  for (int j4 = 0; j4 < 8; ++j4) {
    L0[j4] = L1[j4];
    L1[j4] = L2[j4];
  }
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (I > 0) gdn_t_step<I - 1>(tr, L0, L1, L2, Lb, slot);
}

// The work of one (sequence, head) whose tree has B nodes, NT = ceil(B/32).
template <int NT>
__device__ __forceinline__ void gdn_verify_tree(const GdnParams& p,
                                                unsigned base, GdnSmall& sm,
                                                int s, int h, int n0, int B) {
  constexpr int Bp = NT * 32;
  constexpr int NX = NT * (NT - 1) / 2;   // off-diagonal X tiles
  constexpr int T1 = NT * (NT + 1) / 2;   // Y tiles (lower triangle)
  constexpr int NG = (NX + T1 + 3) / 4;   // Gram tiles per wave, at most
  constexpr int kJumps = NT == 1 ? 5 : (NT == 2 ? 6 : 7);  // ceil log2 Bp
  const int H = p.H;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int col = lane & 31, half = lane >> 5;

  // ---- 1. every global load of the tree issued up front: S0 into
  // registers, K / Q / V rows through registers into LDS
  float sraw[64];  // S0 rows 16 ks + 8 half + e, column 32 w + col
  {
    const float* st = p.state + ((size_t)s * H + h) * kHeadDim * kHeadDim +
                      32 * w + col;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        sraw[8 * ks + e] = st[(size_t)(16 * ks + 8 * half + e) * kHeadDim];
      }
    }
  }
  {
    u32x4 kreg[Bp / 16], qreg[Bp / 16], vreg[Bp / 16];
#pragma unroll
    for (int m = 0; m < Bp / 16; ++m) {
      const int i = (tid >> 4) + 16 * m;
      const size_t off =
          ((size_t)(n0 + min(i, B - 1)) * H + h) * kHeadDim + (tid & 15) * 8;
      kreg[m] = *reinterpret_cast<const u32x4*>(p.k + off);
      qreg[m] = *reinterpret_cast<const u32x4*>(p.q + off);
      vreg[m] = *reinterpret_cast<const u32x4*>(p.v + off);
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
      sm.mk[i][0] = m0;
      sm.mk[i][1] = m1;
      sm.gl[i] = gv;
      sm.bl[i] = bv;
    }
#pragma unroll
    for (int m = 0; m < Bp / 16; ++m) {
      const int i = (tid >> 4) + 16 * m;
      const u32x4 z = {0u, 0u, 0u, 0u};
      const unsigned o = i * kGdnKPitch + (tid & 15) * 16;
      *(gdn_lds_u32x4*)(size_t)(base + kGdnKOff + o) = i < B ? kreg[m] : z;
      *(gdn_lds_u32x4*)(size_t)(base + kGdnQOff + o) = i < B ? qreg[m] : z;
      // rows past the tree keep finite values (clamped), beta = 0 there
      *(gdn_lds_u32x4*)(size_t)(base + kGdnVOff + i * 256 + (tid & 15) * 16) =
          vreg[m];
    }
  }
  __syncthreads();

  // ---- 2. G by pointer jumping over parents (wave 0; lane l holds nodes
  // l and l + 64): G_i += G_{P_i}, P_i <- P_{P_i}, until every P is -1
  if (w == 0) {
    int P0 = lane < Bp ? gdn_parent(sm, lane) : -1;
    int P1 = lane + 64 < Bp ? gdn_parent(sm, lane + 64) : -1;
    float G0 = lane < Bp ? sm.gl[lane] : 0.f;
    float G1 = lane + 64 < Bp ? sm.gl[lane + 64] : 0.f;
#pragma unroll
    for (int it = 0; it < kJumps; ++it) {
      const int a0 = P0 & 63, a1 = P1 & 63;
      const float g00 = gdn_bperm(a0, G0), g01 = gdn_bperm(a0, G1);
      const int p00 = gdn_bperm(a0, P0), p01 = gdn_bperm(a0, P1);
      const float g10 = gdn_bperm(a1, G0), g11 = gdn_bperm(a1, G1);
      const int p10 = gdn_bperm(a1, P0), p11 = gdn_bperm(a1, P1);
      if (P0 >= 0) {
        G0 += P0 < 64 ? g00 : g01;
        P0 = P0 < 64 ? p00 : p01;
      }
      if (P1 >= 0) {
        G1 += P1 < 64 ? g10 : g11;
        P1 = P1 < 64 ? p10 : p11;
      }
    }
    if (lane < Bp) {
      sm.Gc[lane] = G0 * kLog2e;
      sm.gam[lane] = fast_exp2(G0 * kLog2e);
    }
    if (lane + 64 < Bp) {
      sm.Gc[lane + 64] = G1 * kLog2e;
      sm.gam[lane + 64] = fast_exp2(G1 * kLog2e);
    }
  }
  __syncthreads();

  // Gram tile (I, J) of X (isx) or Y, masked and decayed.  Computed
  // transposed (K_J times the row block's K or Q), so lane (col, half)
  // holds row I*32 + col, columns J*32 + 8 (r/4) + 4 half + r%4.
  // sgn: sign applied to X (the solve reads -X); kDiag: a diagonal X tile,
  // whose own diagonal (j == i) is not an ancestor relation
  auto gram = [&](auto diag_c, bool isx, float sgn, int I, int J) {
    constexpr bool kDiag = decltype(diag_c)::value;
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
    const int i = I * 32 + col;
    const float Gi = sm.Gc[i], bl_i = sm.bl[i];
    const float bi = isx ? sgn * bl_i : 1.f;
    // this lane's 16 columns are bits 8 (r/4) + r%4 of mwh
    const uint32_t mwh =
        (uint32_t)(sm.mk[i][J >> 1] >> ((J & 1) * 32)) >> (4 * half);
    // G of the 16 columns, read unconditionally: a read under the ancestor
    // test would become a branch and a wait per element
    f32x4 Gj[4];
#pragma unroll
    for (int mm = 0; mm < 4; ++mm) {
      Gj[mm] = *reinterpret_cast<const f32x4*>(&sm.Gc[J * 32 + 8 * mm + 4 * half]);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      bool anc = (mwh >> (8 * (r >> 2) + (r & 3))) & 1u;
      if constexpr (kDiag) anc = anc && (8 * (r >> 2) + 4 * half + (r & 3) != col);
      // e^{G_i - G_j} for an ancestor, 2^{-inf} = 0 otherwise
      const float d = anc ? Gi - Gj[r >> 2][r & 3] : -__builtin_inff();
      acc[r] = fast_exp2(d) * acc[r];
    }
    if (isx) acc *= bi;
    return acc;
  };

  // ---- 3. diagonal X block w in fp32 (row major) to LDS
  if (w < NT) {
    const f32x16 d = gram(std::true_type{}, true, 1.f, w, w);
#pragma unroll
    for (int mm = 0; mm < 4; ++mm) {
      const f32x4 x4 = {d[4 * mm], d[4 * mm + 1], d[4 * mm + 2], d[4 * mm + 3]};
      *(gdn_lds_f32x4*)(size_t)(base + kGdnLOff + w * 4096 + col * 128 +
                                (8 * mm + 4 * half) * 4) = x4;
    }
  }
  __syncthreads();

  // ---- 4. K S0 and Q S0 on the matrix cores, interleaved with (VALU) row
  // col of T_w = (I + L_w)^{-1}: 32 slots of 4 products, one per step
  f32x16 ks[NT], qs[NT];
  bf16x8 shi[8], slo[8];
#pragma unroll
  for (int k8 = 0; k8 < 8; ++k8) {
    u32x4 h, l;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint32_t a, b;
      gdn_split2(sraw[8 * k8 + 2 * e], sraw[8 * k8 + 2 * e + 1], a, b);
      h[e] = a;
      l[e] = b;
    }
    shi[k8] = __builtin_bit_cast(bf16x8, h);
    slo[k8] = __builtin_bit_cast(bf16x8, l);
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    ks[t] = f32x16{};
    qs[t] = f32x16{};
  }
  // 8 NT slots of four products each.  Per k-step kk the slots take the
  // hi parts of S0 for tile pairs (0, 1), (2, 3), then the lo parts, so
  // two products into one accumulator are several MFMAs apart; a single
  // tile (NT odd) pairs with itself.  A operands are read one k-step ahead.
  constexpr int NP = (NT + 1) / 2;  // tile pairs
  bf16x8 ak[NT], aq[NT], akn[NT], aqn[NT];
  auto read_ks = [&](int kk, bf16x8 (&k_)[NT], bf16x8 (&q_)[NT]) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const unsigned ra = (t * 32 + col) * kGdnKPitch + (2 * kk + half) * 16;
      k_[t] = gdn_read16(base + kGdnKOff + ra);
      q_[t] = gdn_read16(base + kGdnQOff + ra);
    }
  };
  read_ks(0, ak, aq);
  auto slot = [&](auto sc) {
    constexpr int sl = decltype(sc)::value;
    if constexpr (sl < 16 * NP) {
      constexpr int kk = sl / (2 * NP), r = sl % (2 * NP);
      constexpr bool lo = r >= NP;
      constexpr int t0 = 2 * (r % NP), t1 = t0 + 1 < NT ? t0 + 1 : t0;
      if constexpr (r == 0 && kk + 1 < 8) read_ks(kk + 1, akn, aqn);
      const bf16x8 bs = lo ? slo[kk] : shi[kk];
      ks[t0] = mfma32x32x16(ak[t0], bs, ks[t0]);
      qs[t0] = mfma32x32x16(aq[t0], bs, qs[t0]);
      if constexpr (t1 != t0) {
        ks[t1] = mfma32x32x16(ak[t1], bs, ks[t1]);
        qs[t1] = mfma32x32x16(aq[t1], bs, qs[t1]);
      }
      if constexpr (r == 2 * NP - 1) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          ak[t] = akn[t];
          aq[t] = aqn[t];
        }
      }
    }
  };
  __builtin_amdgcn_sched_barrier(0);
  float tr[32];
  {
    // waves >= NT run it on a block no tree uses and discard the result
    const unsigned Lb = base + kGdnLOff + w * 4096;
    f32x4 L0[8], L1[8], L2[8];
#pragma unroll
    for (int j = 0; j < 32; ++j) tr[j] = (j == col) ? 1.f : 0.f;
#pragma unroll
    for (int j4 = 0; j4 < 8; ++j4) {
      L0[j4] = *(const gdn_lds_f32x4*)(size_t)(Lb + 31 * 128 + j4 * 16);
      L1[j4] = *(const gdn_lds_f32x4*)(size_t)(Lb + 30 * 128 + j4 * 16);
      L2[j4] = f32x4{};
    }
    gdn_t_step<31>(tr, L0, L1, L2, Lb, slot);
  }
  // R = beta (V - gamma K S0), in place of K S0
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = t * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
      const float vv = (float)*(const gdn_lds_bf16*)(size_t)(
          base + kGdnVOff + row * 256 + (32 * w + col) * 2);
      ks[t][r] = sm.bl[row] * (vv - sm.gam[row] * ks[t][r]);
    }
    gdn_pin(ks[t]);
  }

  // ---- 5. the other Gram tiles: off-diagonal X tiles in row order, then
  // the Y tiles of the lower triangle; wave w takes w, w + 4, ...
  // Tiles are decoded first (scalar loops) so that the products of all of
  // a wave's tiles form one block the scheduler can interleave; a wave with
  // fewer tiles repeats the last one and drops it.
  f32x16 gt[NG];
  int tI[NG], tJ[NG];
  bool tX[NG];
#pragma unroll
  for (int m = 0; m < NG; ++m) {
    const int n0t = w + 4 * m;
    const int n = min(n0t, NX + T1 - 1);
    const bool isx = n < NX;
    int I, J;
    if (isx) {
      int idx = n;
      I = 1;
      while (idx >= I) {
        idx -= I;
        ++I;
      }
      J = idx;
    } else {
      int idx = n - NX;
      I = 0;
      while (idx > I) {
        idx -= I + 1;
        ++I;
      }
      J = idx;
    }
    tX[m] = isx;
    tI[m] = n0t < NX + T1 ? I : -1;
    tJ[m] = J;
    gt[m] = f32x16{};
  }
#pragma unroll
  for (int m = 0; m < NG; ++m) {
    gt[m] = gram(std::false_type{}, tX[m], -1.f, max(tI[m], 0), tJ[m]);
  }
#pragma unroll
  for (int m = 0; m < NG; ++m) gdn_pin(gt[m]);
  __syncthreads();  // K / Q / V rows and the fp32 blocks consumed

  // ---- 6. X (negated) / Y split into LDS over the staged rows; T_w in
  // the diagonal block w of the X arrays
#pragma unroll
  for (int m = 0; m < NG; ++m) {
    if (tI[m] >= 0) {
      const bool isx = tX[m];
      const int I = tI[m], J = tJ[m];
      const int row = I * 32 + col;
      const unsigned hi_arr = base + (isx ? kGdnXhi : kGdnYhi);
      const unsigned lo_arr = base + (isx ? kGdnXlo : kGdnYlo);
#pragma unroll
      for (int mm = 0; mm < 4; ++mm) {
        u32x2 hv, lv;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          uint32_t a, b;
          gdn_split2(gt[m][4 * mm + 2 * e], gt[m][4 * mm + 2 * e + 1], a, b);
          hv[e] = a;
          lv[e] = b;
        }
        const unsigned off =
            row * kGdnXPitch + (J * 32 + 8 * mm + 4 * half) * 2;
        *(gdn_lds_u32x2*)(size_t)(hi_arr + off) = hv;
        *(gdn_lds_u32x2*)(size_t)(lo_arr + off) = lv;
      }
    }
  }
  if (w < NT && half == 0) {
    const unsigned off = (w * 32 + col) * kGdnXPitch + w * 32 * 2;
#pragma unroll
    for (int c4 = 0; c4 < 8; ++c4) {
      u32x2 hv, lv;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        uint32_t a, b;
        gdn_split2(tr[4 * c4 + 2 * e], tr[4 * c4 + 2 * e + 1], a, b);
        hv[e] = a;
        lv[e] = b;
      }
      *(gdn_lds_u32x2*)(size_t)(base + kGdnXhi + off + c4 * 8) = hv;
      *(gdn_lds_u32x2*)(size_t)(base + kGdnXlo + off + c4 * 8) = lv;
    }
  }
  __syncthreads();

  // ---- 7. blocked forward substitution, right-looking: U_I = T_I R_I,
  // then R_J -= X_JI U_I for every later block J; U is stored as soon as
  // it is known
  const uint32_t row_elems = (uint32_t)H * kHeadDim;
  const __amdgpu_buffer_rsrc_t out_rs = gdn_rsrc(
      p.out + (size_t)n0 * row_elems + (size_t)h * kHeadDim + 32 * w,
      (uint32_t)B * row_elems * 2);
  const __amdgpu_buffer_rsrc_t u_rs = gdn_rsrc(
      p.u + (size_t)n0 * row_elems + (size_t)h * kHeadDim + 32 * w,
      (uint32_t)B * row_elems * 4);
  bf16x8 uh[NT][2], ul[NT][2];
#pragma unroll
  for (int I = 0; I < NT; ++I) {
    const int row = I * 32 + col;
    bf16x8 rh0, rl0, rh1, rl1;
    gdn_split_tile<0>(ks[I], rh0, rl0);
    gdn_split_tile<1>(ks[I], rh1, rl1);
    f32x16 ua = gdn_mfma3(gdn_read_perm(base + kGdnXhi, row, I * 32, half),
                          gdn_read_perm(base + kGdnXlo, row, I * 32, half),
                          rh0, rl0, f32x16{});
    ua = gdn_mfma3(gdn_read_perm(base + kGdnXhi, row, I * 32 + 16, half),
                   gdn_read_perm(base + kGdnXlo, row, I * 32 + 16, half), rh1,
                   rl1, ua);
    gdn_split_tile<0>(ua, uh[I][0], ul[I][0]);
    gdn_split_tile<1>(ua, uh[I][1], ul[I][1]);
#pragma unroll
    for (int J = I + 1; J < NT; ++J) {
      const int rj = J * 32 + col;
      ks[J] = gdn_mfma3(gdn_read_perm(base + kGdnXhi, rj, I * 32, half),
                        gdn_read_perm(base + kGdnXlo, rj, I * 32, half),
                        uh[I][0], ul[I][0], ks[J]);
      ks[J] = gdn_mfma3(gdn_read_perm(base + kGdnXhi, rj, I * 32 + 16, half),
                        gdn_read_perm(base + kGdnXlo, rj, I * 32 + 16, half),
                        uh[I][1], ul[I][1], ks[J]);
    }
    gdn_store_tile<false>(ua, u_rs, row_elems * 4, I * 32, lane);
  }

  // ---- 8. O_J = gamma (Q S0)_J + sum_{I <= J} Y_JI U_I
#pragma unroll
  for (int J = 0; J < NT; ++J) {
    const int row = J * 32 + col;
    f32x16 o = f32x16{};
#pragma unroll
    for (int I = 0; I <= J; ++I) {
      o = gdn_mfma3(gdn_read_perm(base + kGdnYhi, row, I * 32, half),
                    gdn_read_perm(base + kGdnYlo, row, I * 32, half),
                    uh[I][0], ul[I][0], o);
      o = gdn_mfma3(gdn_read_perm(base + kGdnYhi, row, I * 32 + 16, half),
                    gdn_read_perm(base + kGdnYlo, row, I * 32 + 16, half),
                    uh[I][1], ul[I][1], o);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int rr = J * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
      o[r] += sm.gam[rr] * qs[J][r];
    }
    gdn_store_tile<true>(o, out_rs, row_elems * 2, J * 32, lane);
  }
}

__global__ __launch_bounds__(kGdnThreads, 1) void gdn_verify_kernel(
    GdnParams p) {
  __shared__ __align__(16) unsigned char lds[kGdnLdsBytes];
  __shared__ __align__(16) GdnSmall sm;
  const int H = p.H;
  const int s = blockIdx.x / H, h = blockIdx.x - s * H;
  const int n0 = p.tree_offsets[s];
  const int B = p.tree_offsets[s + 1] - n0;
  // trees beyond the supported size are rejected on the host through
  // max_nodes; a tree that breaks that bound is skipped, never overrun
  if (B <= 0 || B > kGdnMaxNodes) return;
  const unsigned base =
      (unsigned)(size_t)(__attribute__((address_space(3))) unsigned char*)lds;
  switch ((B + 31) >> 5) {
    case 1: gdn_verify_tree<1>(p, base, sm, s, h, n0, B); break;
    case 2: gdn_verify_tree<2>(p, base, sm, s, h, n0, B); break;
    case 3: gdn_verify_tree<3>(p, base, sm, s, h, n0, B); break;
    default: gdn_verify_tree<4>(p, base, sm, s, h, n0, B); break;
  }
}

// ---------------------------------------------------------------------------
// State commit.  One workgroup per (sequence, head) updates S0 in place to
// S_n = gamma_n S0 + sum_j e^{G_n - G_{p_j}} k_{p_j} u_{p_j}^T over the
// accepted path p_1 .. p_n (the order tree_attn_accept writes it in).
// Thread t owns 4 consecutive columns of 16 consecutive rows; the path's
// k (fp32) and u (scaled by its decay to the end of the path) pass through
// LDS 32 nodes at a time.

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
  // thread t owns rows 16 (t / 32) .. +15, columns 4 (t % 32) .. +3: a row
  // of the state is read and written by 32 consecutive threads (512
  // bytes); its loads go out first, beside the path's
  const int c4 = (tid & 31) * 4, r0 = (tid >> 5) * 16;
  float* st = p.state + ((size_t)s * H + h) * kHeadDim * kHeadDim;
  f32x4 acc[16];
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    acc[m] = *reinterpret_cast<const f32x4*>(st + (r0 + m) * kHeadDim + c4);
  }
  const int32_t* path = p.accept_nodes + (size_t)s * p.max_nodes;
  // the path's nodes and their log-decays, read in parallel (cf holds g
  // until the suffix sums replace it)
  for (int j = tid; j < tau; j += kGdnThreads) {
    const int v = path[j];
    const int n = (v >= 0 && v < B) ? n0 + v : -1;
    nd[j] = n;
    cf[j] = n >= 0 ? p.g[(size_t)n * H + h] : 0.f;
  }
  __syncthreads();
  // the first 32 nodes' k (bf16) and u (fp32): 32 x (16 + 32) chunks of 16
  // bytes, six per thread, issued before the decays are summed
  constexpr int kChunks = kGdnCommitChunk * 48 / kGdnThreads;
  u32x4 raw[kChunks];
  auto load_chunk = [&](int j0, int nc) {
#pragma unroll
    for (int q = 0; q < kChunks; ++q) {
      const int x = tid + kGdnThreads * q;
      const int jj = x / 48, ch = x % 48;
      raw[q] = u32x4{0u, 0u, 0u, 0u};
      if (jj < nc && nd[j0 + jj] >= 0) {
        const size_t o = ((size_t)nd[j0 + jj] * H + h) * kHeadDim;
        raw[q] = ch < 16
            ? *reinterpret_cast<const u32x4*>(p.k + o + ch * 8)
            : *reinterpret_cast<const u32x4*>(p.u + o + (ch - 16) * 4);
      }
    }
  };
  load_chunk(0, min(kGdnCommitChunk, tau));
  if (tid < 64) {
    // suffix sums of g from the end of the path (cf[j] becomes
    // e^{sum of g over the nodes after j}), 64 nodes per round: an
    // inclusive suffix scan within the wave plus the total of the rounds
    // after it
    float carry = 0.f;
    for (int base = ((tau - 1) >> 6) << 6; base >= 0; base -= 64) {
      const int j = base + tid;
      const float gj = j < tau ? cf[j] : 0.f;
      float x = gj;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const float y = __shfl_down(x, d);
        if (tid + d < 64) x += y;
      }
      if (j < tau) cf[j] = fast_exp2((carry + (x - gj)) * kLog2e);
      carry += __shfl(x, 0);
    }
    if (tid == 0) gam_n = fast_exp2(carry * kLog2e);
  }
  __syncthreads();
  const float gn = gam_n;
#pragma unroll
  for (int m = 0; m < 16; ++m) acc[m] *= gn;

  for (int j0 = 0; j0 < tau; j0 += kGdnCommitChunk) {
    const int nc = min(kGdnCommitChunk, tau - j0);
    if (j0 > 0) load_chunk(j0, nc);
#pragma unroll
    for (int q = 0; q < kChunks; ++q) {
      const int x = tid + kGdnThreads * q;
      const int jj = x / 48, ch = x % 48;
      if (ch < 16) {
        // 8 bf16 of k -> fp32
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t w32 = raw[q][e];
          kc[jj][ch * 8 + 2 * e] = __builtin_bit_cast(float, w32 << 16);
          kc[jj][ch * 8 + 2 * e + 1] =
              __builtin_bit_cast(float, w32 & 0xffff0000u);
        }
      } else {
        const float c = jj < nc ? cf[j0 + jj] : 0.f;
        f32x4 uv = __builtin_bit_cast(f32x4, raw[q]);
        *reinterpret_cast<f32x4*>(&uc[jj][(ch - 16) * 4]) = uv * c;
      }
    }
    __syncthreads();
    for (int jj = 0; jj < nc; ++jj) {
      const f32x4 uv = *reinterpret_cast<const f32x4*>(&uc[jj][c4]);
#pragma unroll
      for (int m4 = 0; m4 < 4; ++m4) {
        const f32x4 kv = *reinterpret_cast<const f32x4*>(&kc[jj][r0 + 4 * m4]);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[4 * m4 + e] += kv[e] * uv;
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    *reinterpret_cast<f32x4*>(st + (r0 + m) * kHeadDim + c4) = acc[m];
  }
}

}  // namespace tree_attn
