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
// (row = i * G + h_in_group), so every K/V tile staged in LDS serves all G
// heads of the group.  A workgroup owns kRowsPerWG rows and one split of
// the key range [0, P_s + B_s); the tree keys are the last B_s positions,
// so the split that reaches them applies the bitmask there (the
// "tree-block pass" runs as the tail tiles of the last split).  With one
// split the kernel writes the normalised output and the LSE directly;
// otherwise it writes (unnormalised O, running max, running sum) partials
// that the merge kernel combines.
//
// Matrix-core mapping (v_mfma_f32_32x32x16_bf16, D = A*B + C, A 32x16,
// B 16x32): scores are computed transposed, S^T = K * Q^T, so the query is
// the MFMA column and every lane holds 16 scores of ONE query.  Row
// statistics are then lane-local plus one exchange between the two lane
// halves.  The K rows fed to the A operand are permuted (sigma below) so
// that lane half hf holds the 16 CONSECUTIVE keys 16*hf .. 16*hf+15 of a
// 32-key block; the probabilities then feed O^T = V^T * P^T as the B
// operand straight from registers, and V^T is read from LDS with 16-byte
// loads.  Softmax runs in base 2 with scale*log2(e) folded into one
// multiply; the LSE is converted back to natural log at the end.
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
  float scale_log2;
};

constexpr int kFwdWaves = 4;
constexpr int kRowsPerWave = 32;
constexpr int kRowsPerWG = kFwdWaves * kRowsPerWave;
constexpr int kKeyTile = 64;
constexpr int kKStride = kHeadDim + 8;  // bf16 per K row in LDS (padded)
constexpr int kVStride = kKeyTile + 8;  // bf16 per V^T row in LDS (padded)

// MFMA output row m of a 32-key block holds key sigma(m); chosen so that
// lane half hf, register r (row 8*(r/4) + 4*hf + r%4) holds key 16*hf + r.
__device__ __forceinline__ int key_of_row(int m) {
  return 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3);
}

__device__ __forceinline__ bf16x8 lds_bf16x8(const unsigned short* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

__global__ __launch_bounds__(kFwdWaves * 64) void attn_fwd_kernel(FwdParams p) {
  __shared__ __align__(16) unsigned short k_lds[kKeyTile * kKStride];
  __shared__ __align__(16) unsigned short vt_lds[kHeadDim * kVStride];

  int bid = blockIdx.x;
  const int split = bid % p.splits;
  bid /= p.splits;
  const int mb = bid % p.mblocks;
  bid /= p.mblocks;
  const int g = bid % p.Hkv;
  const int s = bid / p.Hkv;

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
  const int r = r0 + wave * kRowsPerWave + col;
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
  const int* ptab = p.page_table + (size_t)s * p.max_pps;
  const int pmask = (1 << p.log2_page) - 1;

  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  for (int t0 = kbeg; t0 < kend; t0 += kKeyTile) {
    __syncthreads();
    // Stage K (row-major) and V^T (d-major) of keys t0 .. t0+63.
#pragma unroll
    for (int j = 0; j < (kKeyTile * 16) / (kFwdWaves * 64); ++j) {
      const int c = tid + j * kFwdWaves * 64;
      const int key = c >> 4, part = c & 15;
      const int pos = t0 + key;
      u32x4 kv = {0, 0, 0, 0}, vv = {0, 0, 0, 0};
      if (pos < kend) {
        const int pg = clampi(ptab[pos >> p.log2_page], 0, p.num_pages - 1);
        const size_t tok = ((size_t)pg << p.log2_page) + (pos & pmask);
        const size_t off = (tok * p.Hkv + g) * kHeadDim + part * 8;
        kv = *reinterpret_cast<const u32x4*>(p.k + off);
        vv = *reinterpret_cast<const u32x4*>(p.v + off);
      }
      *reinterpret_cast<u32x4*>(&k_lds[key * kKStride + part * 8]) = kv;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        vt_lds[(part * 8 + e) * kVStride + key] =
            (unsigned short)(vv[e >> 1] >> (16 * (e & 1)));
      }
    }
    __syncthreads();

    // S^T (two 32-key blocks x 32 queries per wave).
    f32x16 sc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sc[kb] = f32x16{};
      const unsigned short* kp =
          &k_lds[(kb * 32 + key_of_row(col)) * kKStride + half * 8];
#pragma unroll
      for (int kc = 0; kc < 8; ++kc) {
        sc[kb] = mfma32x32x16(lds_bf16x8(kp + kc * 16), qf[kc], sc[kb]);
      }
    }

    // Scale to log2 units, mask, tile max.
    const bool tree_tile = (t0 + kKeyTile > P);
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int pos = t0 + kb * 32 + half * 16 + rr;
        bool ok = pos < kend;
        if (tree_tile && ok && pos >= P) {
          const int jn = pos - P;
          const uint64_t w = mrow[min(jn >> 6, p.W - 1)];
          ok = (w >> (jn & 63)) & 1;
        }
        const float x = ok ? sc[kb][rr] * p.scale_log2 : -INFINITY;
        sc[kb][rr] = x;
        tmax = fmaxf(tmax, x);
      }
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    const float m_ref = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_ref);

    bf16x8 pf[2][2];
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const float e = fast_exp2(sc[kb][rr] - m_ref);
        psum += e;
        pf[kb][rr >> 3][rr & 7] = (__bf16)e;
      }
    }
    psum += __shfl_xor(psum, 32);
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < 4; ++db) o[db] *= alpha;

    // O^T += V^T * P^T.
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const unsigned short* vp = &vt_lds[(db * 32 + col) * kVStride + half * 16];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          o[db] = mfma32x32x16(lds_bf16x8(vp + kb * 32 + hf * 8), pf[kb][hf],
                               o[db]);
        }
      }
    }
  }

  if (!rvalid) return;
  if (p.splits == 1) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
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
      p.lse[qrow] = l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
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
      *reinterpret_cast<f32x2*>(p.part_ml + prow * 2) = f32x2{m_run, l_run};
    }
  }
}

}  // namespace tree_attn
