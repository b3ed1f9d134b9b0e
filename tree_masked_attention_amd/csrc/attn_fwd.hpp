// Split-KV tree-verification attention on the gfx950 bf16 matrix cores.
//
// Computes, for every query row (node i, q head h) of a sequence, softmax
// attention over the prefix keys plus the tree keys allowed by node i's
// ancestor bitmask (tree-causal mask of JETFLOW, gist.science 2606.18394,
// section 2 "Arquitectura Central"), over a paged KV cache (section 3,
// item 3 names a paged kernel with the tree mask staged on chip).
//
// Work decomposition.  The rows of one (sequence s, kv head g) pair are the
// G query heads of the group times the B_s nodes, packed node-major
// (row = i * G + h_in_group), so each K/V tile staged in LDS serves all G
// heads of the group.  A workgroup of NW waves owns 32*NW rows and one split
// of the key range [0, P_s + B_s).  The tree keys are the last B_s positions
// of that range, so the split that reaches them applies the bitmask on its
// tail tiles (the tree-block pass).  With one split the kernel writes the
// normalised output and the LSE; otherwise it writes (unnormalised O,
// running max, running sum) partials for the merge kernel.
//
// Matrix-core mapping (v_mfma_f32_32x32x16_bf16, D = A*B + C).  Scores are
// computed transposed, S^T = K * Q^T: the query is the MFMA column, so a
// lane holds 16 scores of ONE query and row statistics are lane-local plus
// one exchange between the two lane halves (v_permlane32_swap).  Register
// r of lane half h holds key 8*(r/4) + 4*h + r%4 of a 32-key block, i.e.
// runs of 4 consecutive keys.  O^T = V^T * P^T then takes the probabilities
// as the B operand straight from registers; its A operand (V^T, 8 keys of
// one column per lane) comes from the row-major V tile through two
// transposing LDS reads (ds_read_b64_tr_b16), each delivering the 4
// consecutive keys of one register run.
//
// Pipeline.  The split's slice of the page table is copied to LDS once.
// K/V tiles of 64 keys are double-buffered in LDS: the global loads of tile
// j+1 are issued into registers before tile j is computed and written to
// the other buffer after it, one barrier per tile.
//
// Softmax runs in base 2: scale*log2(e) is folded into the FMA that
// subtracts the running max.  The running max is only raised when a tile's
// max exceeds it by more than 8 (log2 units); otherwise the stale max is
// kept, which bounds the probabilities by 2^8 and skips the O rescale.
// The row sum accumulates the fp32 probabilities (before their rounding to
// bf16 for the PV product), which keeps the LSE accurate on short rows.
#pragma once

#include "common.hpp"

namespace tree_attn {

struct FwdParams {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const int32_t* page_table;
  const int32_t* prefix_lens;
  const int32_t* tree_offsets;
  const uint64_t* masks;
  __bf16* out;
  float* lse;
  float* part_o;   // [splits][N*Hq][128]
  float* part_ml;  // [splits][N*Hq][2]  (max in log2 units, sum)
  int max_pps, num_pages, log2_page, W;
  int max_tokens;  // min(max_pps * page_size, 2^30)
  int S, N, Hq, Hkv, G;
  int mblocks, splits, chunk;
  int units, per_xcd;  // work units; units handled per XCD slot column
  float scale_log2;
};

constexpr int kKeyTile = 64;
constexpr int kKStride = kHeadDim + 8;   // u16 per K row in LDS (272 B)
constexpr int kVStride = kHeadDim + 32;  // u16 per V row in LDS (320 B)
constexpr int kPageCache = 1024;         // page-table entries per split
constexpr float kLazyRescale = 8.f;      // log2 units

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ bf16x8 lds_bf16x8(const unsigned short* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

// Transposing LDS read: see the file comment.
__device__ __forceinline__ s16x4 lds_tr4(const unsigned short* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
}

// Value of the other lane half (lane ^ 32).
__device__ __forceinline__ float other_half(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  // r[0]: lanes 32..63 now hold lanes 0..31; r[1]: lanes 0..31 hold 32..63
  const unsigned lane = __lane_id();
  return __builtin_bit_cast(float, lane < 32 ? r[1] : r[0]);
}

template <int NW>
__global__ __launch_bounds__(NW * 64, 2) void attn_fwd_kernel(FwdParams p) {
  constexpr int kThreads = NW * 64;
  constexpr int kRowsPerWG = NW * 32;
  constexpr int kCPT = (kKeyTile * 16) / kThreads;  // 16-B chunks / thread
  __shared__ __align__(16) unsigned short k_lds[2][kKeyTile * kKStride];
  __shared__ __align__(16) unsigned short v_lds[2][kKeyTile * kVStride];
  __shared__ int pg_lds[kPageCache];

  // XCD-aware decode: consecutive work units (the row blocks of one
  // (sequence, kv head, split), which read the same K/V) go to one XCD.
  const int bid = blockIdx.x;
  int L = (bid & 7) * p.per_xcd + (bid >> 3);
  if (L >= p.units) return;
  const int mb = L % p.mblocks;
  L /= p.mblocks;
  const int split = L % p.splits;
  L /= p.splits;
  const int g = L % p.Hkv;
  const int s = L / p.Hkv;

  const int a = clampi(p.tree_offsets[s], 0, p.N);
  const int b = clampi(p.tree_offsets[s + 1], a, p.N);
  const int B = b - a;
  const int P = max(p.prefix_lens[s], 0);
  const int rows = p.G * B;
  const int r0 = mb * kRowsPerWG;
  if (r0 >= rows) return;
  const int T = min(P + B, p.max_tokens);
  const int kbeg = split * p.chunk;
  if (kbeg >= T) return;
  const int kend = min(T, kbeg + p.chunk);

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int col = lane & 31, half = lane >> 5;

  // Page-table slice of this split -> LDS.
  const int lp0 = kbeg >> p.log2_page;
  const int npg = min(((kend - 1) >> p.log2_page) - lp0 + 1, kPageCache);
  {
    const int* ptab = p.page_table + (size_t)s * p.max_pps + lp0;
    for (int i = tid; i < npg; i += kThreads) {
      pg_lds[i] = clampi(ptab[i], 0, p.num_pages - 1);
    }
  }

  const int r = r0 + wave * 32 + col;
  const bool rvalid = r < rows;
  const int node = rvalid ? r / p.G : B - 1;
  const int head = g * p.G + (rvalid ? r % p.G : 0);
  const size_t qrow = (size_t)(a + node) * p.Hq + head;

  // Q^T fragments (B operand): query `col`, d = kc*16 + half*8 + 0..7.
  bf16x8 qf[8];
  {
    const __bf16* qp = p.q + qrow * kHeadDim + half * 8;
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) {
      u32x4 raw = rvalid ? *reinterpret_cast<const u32x4*>(qp + kc * 16)
                         : u32x4{0, 0, 0, 0};
      qf[kc] = __builtin_bit_cast(bf16x8, raw);
    }
  }
  const uint64_t* mrow = p.masks + (size_t)(a + node) * p.W;
  const int pmask = (1 << p.log2_page) - 1;
  const size_t kv_head_off = (size_t)g * kHeadDim;
  const size_t tok_stride = (size_t)p.Hkv * kHeadDim;

  u32x4 kreg[kCPT], vreg[kCPT];
  auto load_tile = [&](int t0) {
#pragma unroll
    for (int k = 0; k < kCPT; ++k) {
      const int c = tid + k * kThreads;
      const int key = c >> 4, part = c & 15;
      const int pos = t0 + key;
      kreg[k] = u32x4{0, 0, 0, 0};
      vreg[k] = u32x4{0, 0, 0, 0};
      if (pos < kend) {
        const int pi = clampi((pos >> p.log2_page) - lp0, 0, kPageCache - 1);
        const size_t tok = ((size_t)pg_lds[pi] << p.log2_page) + (pos & pmask);
        const size_t off = tok * tok_stride + kv_head_off + part * 8;
        kreg[k] = *reinterpret_cast<const u32x4*>(p.k + off);
        vreg[k] = *reinterpret_cast<const u32x4*>(p.v + off);
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int k = 0; k < kCPT; ++k) {
      const int c = tid + k * kThreads;
      const int key = c >> 4, part = c & 15;
      *reinterpret_cast<u32x4*>(&k_lds[buf][key * kKStride + part * 8]) = kreg[k];
      *reinterpret_cast<u32x4*>(&v_lds[buf][key * kVStride + part * 8]) = vreg[k];
    }
  };

  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = f32x16{};
  float m_run = -INFINITY;  // log2 units, equal in both lane halves
  float l_run = 0.f;        // this lane half's share of the sum
  const float c2 = p.scale_log2;

  // per-lane constant part of the transposed V read address
  const int r16 = lane & 15;
  const int v_lane_off = (4 * half + (r16 >> 2)) * kVStride +
                         16 * ((lane >> 4) & 1) + 4 * (r16 & 3);

  const int ntiles = (kend - kbeg + kKeyTile - 1) / kKeyTile;
  __syncthreads();  // page slice visible
  load_tile(kbeg);
  store_tile(0);
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    const int t0 = kbeg + j * kKeyTile;
    const int buf = j & 1;
    if (j + 1 < ntiles) load_tile(t0 + kKeyTile);

    // ---- S^T = K Q^T : two 32-key blocks x 32 queries
    f32x16 sc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sc[kb] = f32x16{};
      const unsigned short* kp =
          &k_lds[buf][(kb * 32 + col) * kKStride + half * 8];
#pragma unroll
      for (int kc = 0; kc < 8; ++kc) {
        sc[kb] = mfma32x32x16(lds_bf16x8(kp + kc * 16), qf[kc], sc[kb]);
      }
    }

    // ---- mask: keys past the split end, tree keys not on the path
    if (t0 + kKeyTile > min(P, kend)) {
      const int nvalid = kend - t0;  // >= 1
      const int npre = P - t0;
      uint64_t allow = nvalid >= 64 ? ~0ull : ((1ull << nvalid) - 1);
      uint64_t pre = npre >= 64 ? ~0ull : (npre <= 0 ? 0ull : ((1ull << npre) - 1));
      uint64_t tree = 0;
      if (npre < 64) {
        const int j0 = t0 - P;  // tree node at tile offset 0 (may be < 0)
        if (j0 >= 0) {
          const int w0 = min(j0 >> 6, p.W - 1), sh = j0 & 63;
          tree = mrow[w0] >> sh;
          if (sh != 0 && w0 + 1 < p.W) tree |= mrow[w0 + 1] << (64 - sh);
        } else {
          tree = mrow[0] << (-j0);
        }
      }
      allow &= (pre | tree);
      allow >>= 4 * half;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          const int kk = kb * 32 + 8 * (rr >> 2) + (rr & 3);
          if (!((allow >> kk) & 1)) sc[kb][rr] = -INFINITY;
        }
      }
    }

    // ---- online softmax (base 2, lazy rescale)
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int rr = 0; rr < 16; rr += 2) {
        tmax = fmaxf(tmax, fmaxf(sc[kb][rr], sc[kb][rr + 1]));
      }
    }
    tmax = fmaxf(tmax, other_half(tmax)) * c2;
    const bool need = tmax > m_run + kLazyRescale;
    if (__any(need)) {
      const float m_new = need ? tmax : m_run;
      const float alpha = need ? fast_exp2(m_run - m_new) : 1.f;
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db) o[db] *= alpha;
    }
    const float m_ref = (m_run == -INFINITY) ? 0.f : m_run;

    bf16x8 pf[2][2];
    float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int rr = 0; rr < 16; rr += 2) {
        const float e0 = fast_exp2(fmaf(sc[kb][rr], c2, -m_ref));
        const float e1 = fast_exp2(fmaf(sc[kb][rr + 1], c2, -m_ref));
        ps0 += e0;
        ps1 += e1;
        pf[kb][rr >> 3][rr & 7] = (__bf16)e0;
        pf[kb][rr >> 3][(rr & 7) + 1] = (__bf16)e1;
      }
    }
    l_run += ps0 + ps1;

    // ---- O^T += V^T P^T
    const unsigned short* vb = &v_lds[buf][v_lane_off];
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const unsigned short* vp = vb + (kb * 32 + hf * 16) * kVStride + db * 32;
          const s16x4 lo = lds_tr4(vp);
          const s16x4 hi = lds_tr4(vp + 8 * kVStride);
          const bf16x8 vf = __builtin_bit_cast(
              bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          o[db] = mfma32x32x16(vf, pf[kb][hf], o[db]);
        }
      }
    }

    if (j + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  const float l_tot = l_run + other_half(l_run);
  if (!rvalid) return;
  if (p.splits == 1) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    __bf16* op = p.out + qrow * kHeadDim;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        bf16x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = (__bf16)(o[db][g4 * 4 + e] * inv);
        *reinterpret_cast<bf16x4*>(op + db * 32 + g4 * 8 + half * 4) = v4;
      }
    }
    if (half == 0) {
      p.lse[qrow] = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
    }
  } else {
    const size_t prow = (size_t)split * p.N * p.Hq + qrow;
    float* pp = p.part_o + prow * kHeadDim;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        f32x4 v4 = {o[db][g4 * 4 + 0], o[db][g4 * 4 + 1], o[db][g4 * 4 + 2],
                    o[db][g4 * 4 + 3]};
        *reinterpret_cast<f32x4*>(pp + db * 32 + g4 * 8 + half * 4) = v4;
      }
    }
    if (half == 0) {
      *reinterpret_cast<f32x2*>(p.part_ml + prow * 2) = f32x2{m_run, l_tot};
    }
  }
}

}  // namespace tree_attn
