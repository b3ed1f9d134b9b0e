// Tree-verification attention for the variant the tuned kernels
// (attn_fwd128h.hpp, attn_fwd8.hpp) do not cover: head dimension 64, with
// K/V pages in bf16 or in fp8 (OCP E4M3, one fp32 scale per kv head; fp8
// with head dimension 128 runs the tuned kernels).  The template also
// compiles for D = 128, which is not launched.  The operation is the same
// as theirs -- every tree
// node attends to its sequence's prefix and to its ancestors (JETFLOW,
// gist.science 2606.18394, section 2 "Arquitectura Central", bullet on the
// tree-causal mask) -- and so is the split-KV decomposition with an LSE
// merge; JETFLOW's parallel draft head uses the same mask over its own KV.
//
// Design (simpler than the tuned kernels, and written for occupancy
// instead of a deep pipeline): a workgroup of four waves owns 128 query
// rows (GQA heads packed node-major, row = node * G + head) of one
// (sequence, kv head) and one key split.  Per tile of 64 keys the threads
// load the K and V rows through the page table, convert fp8 to bf16 (exact:
// every E4M3 value is a bf16 value) and write K row-major and V transposed
// (V^T[d][key]) to LDS, 34 KB in all, so up to four workgroups share a CU
// and hide each other's latency.  Scores are computed transposed, S^T =
// K Q^T (v_mfma_f32_32x32x16_bf16; the query is the MFMA column, so a lane
// holds 16 scores of one query row), the ancestor mask is applied to the
// tree keys in registers, the online softmax runs in base 2, and
// O^T += V^T P^T takes the probabilities straight from the score registers
// as the B operand (k permuted consistently in both operands).  The fp8
// scales fold into the softmax scale (K) and the output (V).  A split
// writes its output normalised by its own row sum in fp16 (a convex
// combination of V rows, so within V's range) and (max, sum) in fp32.
#pragma once

#include "attn_merge.hpp"
#include "common.hpp"

namespace tree_attn {

constexpr int kVarRows = 128;   // query rows per workgroup (4 waves x 32)
constexpr int kVarTile = 64;    // keys per tile
constexpr int kVarDepth = 3;    // tiles in registers (in use + in flight)
constexpr float kVarLazy = 8.f; // lazy-rescale margin, log2 units
constexpr int kVarPageCache = 1040;       // page ids of a split, in LDS
constexpr int kVarMaskCache = 129 * 16;   // mask words of a workgroup's nodes
constexpr int kVarThreads = 256;

struct VarParams {
  const __bf16* q;             // [N][Hq][D]
  const unsigned char* k;      // [num_pages][page_size][Hkv][D] elements
  const unsigned char* v;
  const float* k_scale;        // [Hkv] (fp8) or null
  const float* v_scale;
  const int32_t* page_table;   // [S][max_pps]
  const int32_t* prefix_lens;  // [S]
  const int32_t* tree_offsets; // [S + 1]
  const uint64_t* masks;       // [N][W]
  __bf16* out;                 // [N][Hq][D]
  float* lse;                  // [N][Hq]
  _Float16* part_o;            // [splits][N * Hq][D]  the split's O / its l
  float* part_ml;              // [splits][N * Hq][2]  (max, log2 units; sum)
  int max_pps, num_pages, log2_page, W;
  int max_tokens;  // min(max_pps * page_size, 2^30): keys the table covers
  int S, N, Hq, Hkv, G;
  int mblocks, splits, chunk;
  float scale_log2;
};

typedef __attribute__((address_space(3))) u32x4 var_lds_u32x4;
typedef __attribute__((address_space(3))) u32x2 var_lds_u32x2;
typedef __attribute__((address_space(3))) __bf16 var_lds_bf16;
typedef short var_s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) var_s16x4 var_lds_s16x4;

// Transposing LDS read (ds_read_b64_tr_b16): four 16-bit values of four
// consecutive rows at one column for each lane.
__device__ __forceinline__ var_s16x4 var_read_tr(unsigned addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((var_lds_s16x4*)(size_t)addr);
}

__device__ __forceinline__ bf16x8 var_read16(unsigned addr) {
  return __builtin_bit_cast(bf16x8, *(const var_lds_u32x4*)(size_t)addr);
}


__device__ __forceinline__ const int32_t* table_row(const VarParams& p,
                                                   int s) {
  return p.page_table + (size_t)s * p.max_pps;
}

template <int D, bool FP8>
__global__ __launch_bounds__(kVarThreads, 2) void attn_var_kernel(VarParams p) {
  constexpr int EB = FP8 ? 1 : 2;         // bytes per cached element
  constexpr int RB = D * EB;              // bytes per cached (token, head)
  constexpr int CR = RB / 16;             // 16-byte chunks per row
  constexpr int KP = D * 2 + 16;          // K row pitch in LDS (bf16)
  constexpr int NCH = kVarTile * CR / kVarThreads;  // chunks per thread
  constexpr int DT = D / 32;              // output tiles of 32 dims
  constexpr int KS = D / 16;              // k-steps of the score product
  // V goes to LDS row-major in bf16, one 256-byte row per key (half of it
  // unused for head dim 64), 16-byte chunk c of row r at slot c ^ 4 (r & 3),
  // and the V^T operand comes from transposing reads: the tuned 128-row
  // kernel's layout and read addresses, whose dim block dt reads chunks
  // 4 dt .. 4 dt + 3 only.
  static_assert(NCH >= 1 && kVarTile * CR % kVarThreads == 0, "tile split");
  __shared__ __align__(16) unsigned char kl[kVarTile * KP];
  __shared__ __align__(16) unsigned char vl[kVarTile * 256];
  __shared__ int pg_var[kVarPageCache];
  __shared__ uint64_t mk_var[kVarMaskCache];
  const unsigned kb =
      (unsigned)(size_t)(__attribute__((address_space(3))) unsigned char*)kl;
  const unsigned vb =
      (unsigned)(size_t)(__attribute__((address_space(3))) unsigned char*)vl;

  int idx = blockIdx.x;
  const int c = idx % p.splits;
  idx /= p.splits;
  const int mb = idx % p.mblocks;
  idx /= p.mblocks;
  const int g = idx % p.Hkv;
  const int s = idx / p.Hkv;
  const int n0 = clampi(p.tree_offsets[s], 0, p.N);
  const int B = clampi(p.tree_offsets[s + 1], n0, p.N) - n0;
  const int P = max(p.prefix_lens[s], 0);
  const int rows = B * p.G;
  if (mb * kVarRows >= rows) return;
  const int T = min(P + B, p.max_tokens);
  const int k0 = c * p.chunk, k1 = min(T, k0 + p.chunk);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  // transposing-read lane offsets (the tuned kernels' V operand pattern)
  const int ty = (lane & 15) >> 2;
  const int tx = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int r = mb * kVarRows + w * 32 + col;  // this lane's query row
  const bool valid = r < rows;
  const int node = valid ? r / p.G : 0;
  const int h = g * p.G + (valid ? r % p.G : 0);
  const size_t qrow = (size_t)(n0 + node) * p.Hq + h;

  // Q^T fragments: lane (row r, half) holds dims 16 ks + 8 half .. +7
  bf16x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (valid) {
      qf[ks] = *reinterpret_cast<const bf16x8*>(p.q + qrow * D + 16 * ks +
                                                8 * half);
    } else {
      qf[ks] = bf16x8{};
    }
  }
  const float ksc = FP8 && p.k_scale ? p.k_scale[g] : 1.f;
  const float vsc = FP8 && p.v_scale ? p.v_scale[g] : 1.f;
  const float sl2 = p.scale_log2 * ksc;

  // The split's page ids and, when the split reaches the tree keys, the
  // mask rows of the workgroup's nodes go to LDS first, so that the loop's
  // lookups wait on LDS only (a global load there would have to wait for
  // every K/V load in flight before it).  The plan keeps a split's pages
  // within kVarPageCache; the rows are at most 129 nodes of at most 16
  // words.
  const int lp0 = k0 >> p.log2_page;
  const int npg =
      k0 < k1 ? min(((k1 - 1) >> p.log2_page) - lp0 + 1, kVarPageCache) : 0;
  for (int i = tid; i < npg; i += kVarThreads) {
    // a page id outside the pool is clamped into it (never read past)
    pg_var[i] = min(max(table_row(p, s)[lp0 + i], 0), p.num_pages - 1);
  }
  const int n_lo = mb * kVarRows / p.G;
  const int n_hi = (min(mb * kVarRows + kVarRows, rows) - 1) / p.G;
  const int nmw = k1 > P ? min((n_hi - n_lo + 1) * p.W, kVarMaskCache) : 0;
  for (int i = tid; i < nmw; i += kVarThreads) {
    mk_var[i] = p.masks[(size_t)(n0 + n_lo) * p.W + i];
  }
  const int mrow = (valid ? node - n_lo : 0) * p.W;
  __syncthreads();

  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16{};
  float m = -__builtin_inff(), l = 0.f;

  const int pmask = (1 << p.log2_page) - 1;
  // Staging: thread t moves 16-byte chunk ch = t % CR of NCH consecutive
  // keys kq .. kq + NCH - 1, so that its V^T writes cover NCH keys of one
  // dimension at once.  Tiles go through a ring of kVarDepth register
  // buffers: tiles t+1 .. t+kVarDepth-1 are in flight while tile t is
  // used, and the buffer of tile t is refilled with tile t+kVarDepth as soon
  // as it has been written to LDS (the loop is unrolled by the ring depth so
  // that every buffer index is a constant).
  const int ch = tid % CR, kq = (tid / CR) * NCH;
  u32x4 kc[kVarDepth][NCH], vc[kVarDepth][NCH];
  // Every load is issued unconditionally (the compiler can then count the
  // loads in flight and wait for one tile's only): keys past the split end
  // read the split's last key again (their scores are masked, so these
  // rows get probability 0), and t is at most the last tile's start.
  auto load_tile = [&](int t, u32x4 (&kd)[NCH], u32x4 (&vd)[NCH]) {
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int key = min(t + kq + j, k1 - 1);
      const int page =
          pg_var[clampi((key >> p.log2_page) - lp0, 0, kVarPageCache - 1)];
      const size_t off =
          (((size_t)page << p.log2_page) + (key & pmask)) * p.Hkv + g;
      kd[j] = *reinterpret_cast<const u32x4*>(p.k + off * RB + ch * 16);
      vd[j] = *reinterpret_cast<const u32x4*>(p.v + off * RB + ch * 16);
    }
  };
  // start of the split's last tile
  const int t_last = k0 + max((k1 - 1 - k0) / kVarTile, 0) * kVarTile;
  auto tile = [&](int t, u32x4 (&kcur)[NCH], u32x4 (&vcur)[NCH]) {
    __syncthreads();  // the previous tile's products are done
    // ---- K rows and V rows (bf16) to LDS
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int r = kq + j, sw = 4 * (r & 3);
      const unsigned vr = vb + r * 256;
      if (FP8) {
        // 16 codes = dims 16 ch .. 16 ch + 15 = bf16 chunks 2 ch, 2 ch + 1
        u32x4 k0, k1, v0, v1;
#pragma unroll
        for (int q4 = 0; q4 < 2; ++q4) {
          k0[2 * q4] = e4m3x2_to_bf16x2<false>(kcur[j][q4]);
          k0[2 * q4 + 1] = e4m3x2_to_bf16x2<true>(kcur[j][q4]);
          k1[2 * q4] = e4m3x2_to_bf16x2<false>(kcur[j][q4 + 2]);
          k1[2 * q4 + 1] = e4m3x2_to_bf16x2<true>(kcur[j][q4 + 2]);
          v0[2 * q4] = e4m3x2_to_bf16x2<false>(vcur[j][q4]);
          v0[2 * q4 + 1] = e4m3x2_to_bf16x2<true>(vcur[j][q4]);
          v1[2 * q4] = e4m3x2_to_bf16x2<false>(vcur[j][q4 + 2]);
          v1[2 * q4 + 1] = e4m3x2_to_bf16x2<true>(vcur[j][q4 + 2]);
        }
        *(var_lds_u32x4*)(size_t)(kb + r * KP + ch * 32) = k0;
        *(var_lds_u32x4*)(size_t)(kb + r * KP + ch * 32 + 16) = k1;
        *(var_lds_u32x4*)(size_t)(vr + (((2 * ch) ^ sw) << 4)) = v0;
        *(var_lds_u32x4*)(size_t)(vr + (((2 * ch + 1) ^ sw) << 4)) = v1;
      } else {
        *(var_lds_u32x4*)(size_t)(kb + r * KP + ch * 16) = kcur[j];
        *(var_lds_u32x4*)(size_t)(vr + ((ch ^ sw) << 4)) = vcur[j];
      }
    }
    __syncthreads();
    // refill: past the last tile this reloads the last tile (an L2 hit,
    // never used), which keeps the count of loads in flight the same on
    // every path through the loop
    load_tile(min(t + kVarDepth * kVarTile, t_last), kcur, vcur);

    // ---- S^T = K Q^T, two halves of 32 keys
    f32x16 sc[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      sc[kt] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 a =
            var_read16(kb + (kt * 32 + col) * KP + (2 * ks + half) * 16);
        sc[kt] = mfma32x32x16(a, qf[ks], sc[kt]);
      }
    }
    // ---- scale, mask (keys past the split; tree keys off the path)
    float mx = -__builtin_inff();
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int kbase = t + kt * 32 + 4 * half;
      // mask bits of this lane's 16 tree keys, when the half reaches them
      uint32_t bits = 0xffffffffu;
      const int j0 = kbase - P;  // tree index of the first key (may be < 0)
      if (kbase + 28 >= P) {
        bits = 0u;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          for (int e = 0; e < 4; ++e) {
            const int j = j0 + 8 * q + e;
            bool on;
            if (j < 0) {
              on = true;
            } else {
              on = j < B &&
                   ((mk_var[min(mrow + (j >> 6), kVarMaskCache - 1)] >>
                     (j & 63)) & 1u);
            }
            bits |= (on ? 1u : 0u) << (4 * q + e);
          }
        }
      }
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int key = kbase + 8 * (rr >> 2) + (rr & 3);
        const bool ok = key < k1 && ((bits >> rr) & 1u);
        const float x = ok ? sc[kt][rr] * sl2 : -__builtin_inff();
        sc[kt][rr] = x;
        mx = __builtin_fmaxf(mx, x);
      }
    }
    mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32));
    // lazy rescale: the reference max m is raised only when the tile's max
    // exceeds it by more than kVarLazy (log2 units), which bounds the
    // probabilities by 2^kVarLazy and leaves O alone on most tiles
    const bool need = mx > m + kVarLazy;
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
      const float mnew = need ? mx : m;
      const float alpha = need ? fast_exp2(m - mnew) : 1.f;
      l *= alpha;
      m = mnew;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
    }
    const float mref = m == -__builtin_inff() ? 0.f : m;
    float ps = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const float e = fast_exp2(sc[kt][rr] - mref);
        sc[kt][rr] = e;
        ps += e;
      }
    }
    ps += __shfl_xor(ps, 32);
    l += ps;
    // ---- O^T += V^T P^T
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        bf16x8 pb;
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[e] = (__bf16)sc[kt][8 * s2 + e];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const unsigned va = vb + (kt * 32 + 16 * s2 + 4 * half + ty) * 256 +
                              ((4 * (dt ^ ty) + tx) << 4) + 8 * (lane & 1);
          const var_s16x4 lo = var_read_tr(va);
          const var_s16x4 hi = var_read_tr(va + 8 * 256);
          const bf16x8 a = __builtin_bit_cast(
              bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          oacc[dt] = mfma32x32x16(a, pb, oacc[dt]);
        }
      }
    }
  };
  static_assert(kVarDepth == 3, "the loop below is unrolled by 3");
  if (k0 < k1) {
#pragma unroll
    for (int d = 0; d < kVarDepth; ++d) {
      load_tile(min(k0 + d * kVarTile, t_last), kc[d], vc[d]);
    }
    // the back edge is taken only after all three tiles of an iteration
    for (int t = k0; t < k1; t += kVarDepth * kVarTile) {
      tile(t, kc[0], vc[0]);
      if (t + kVarTile < k1) tile(t + kVarTile, kc[1], vc[1]);
      if (t + 2 * kVarTile < k1) tile(t + 2 * kVarTile, kc[2], vc[2]);
    }
  }

  // ---- epilogue: lane (row r, half) holds dims 32 dt + 8 (i/4) + 4 half +
  // i%4 of its row
  if (!valid) return;
  if (p.splits == 1) {
    const float inv = l > 0.f ? vsc / l : 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        bf16x4 o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x = oacc[dt][4 * q + e] * inv;
          o4[e] = (__bf16)x;
        }
        *reinterpret_cast<bf16x4*>(p.out + qrow * D + 32 * dt + 8 * q +
                                   4 * half) = o4;
      }
    }
    if (half == 0) {
      p.lse[qrow] = l > 0.f ? (m + __builtin_log2f(l)) * kLn2
                            : -__builtin_inff();
    }
  } else {
    const size_t rows_all = (size_t)p.N * p.Hq;
    _Float16* po = p.part_o + ((size_t)c * rows_all + qrow) * D;
    const float inv = l > 0.f ? vsc / l : 0.f;
    // fp16 scaled by 2^-ex, the row's scale exponent (f16_row_exp)
    float amax = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        amax = __builtin_elementwise_maximum(amax, __builtin_fabsf(oacc[dt][e]));
      }
    }
    const int ex = f16_row_exp(
        __builtin_elementwise_maximum(amax, other_half(amax)) * inv);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f16x4 o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          o4[e] = to_f16_sat(ldexp2(oacc[dt][4 * q + e] * inv, -ex));
        }
        *reinterpret_cast<f16x4*>(po + 32 * dt + 8 * q + 4 * half) = o4;
      }
    }
    if (half == 0) {
      float* ml = p.part_ml + ((size_t)c * rows_all + qrow) * 2;
      *reinterpret_cast<uint64_t*>(ml) = pack_split_stats(split_lse2(m, l), ex);
    }
  }
}

// LSE merge of the split partials (the identity and arithmetic of
// attn_merge.hpp: running maximum, merge_weights / merge_acc, splits in
// index order).  One thread per (row, 4 dims).
template <int D>
__global__ __launch_bounds__(256) void attn_var_merge_kernel(VarParams p) {
  const size_t rows_all = (size_t)p.N * p.Hq;
  const size_t gid = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t row = gid / (D / 4);
  const int d4 = (int)(gid % (D / 4)) * 4;
  if (row >= rows_all) return;
  float m_run = -INFINITY, l_run = 0.f;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int c = 0; c < p.splits; ++c) {
    const size_t prow = (size_t)c * rows_all + row;
    const f32x2 ml = *reinterpret_cast<const f32x2*>(p.part_ml + prow * 2);
    const f16x4 o = *reinterpret_cast<const f16x4*>(p.part_o + prow * D + d4);
    float s_old, w;
    if (!merge_weights(m_run, l_run, ml, s_old, w)) continue;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = merge_acc(acc[e], s_old, w, (float)o[e]);
  }
  const float inv = merge_inv(l_run);
  bf16x4 o4;
#pragma unroll
  for (int e = 0; e < 4; ++e) o4[e] = (__bf16)(acc[e] * inv);
  *reinterpret_cast<bf16x4*>(p.out + row * D + d4) = o4;
  if (d4 == 0) p.lse[row] = merge_lse(m_run, l_run);
}

}  // namespace tree_attn
