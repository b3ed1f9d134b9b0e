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
// Memory pipeline.  K/V tiles of 64 keys (16 KB each) flow through a
// 4-stage LDS ring (K tiles of all stages, then V tiles) filled by
// global_load_lds_dwordx4: the load unit writes
// each lane's 16 bytes straight to LDS (lane l of an instruction lands at
// M0 + 16*l), so no registers stage the data.  The loads are issued from
// inline assembly and waited for with explicit vmcnt counts, because the
// compiler would otherwise drain every such load before each barrier and
// the ring would never hold more than one tile in flight.  Tile j+3 is
// issued while tile j is consumed.  Rows are stored unpadded with an XOR
// swizzle of their 16-byte chunks (K: chunk ^ (row & 15); V: chunk ^
// 4*(row & 3)) so that the MFMA operand reads hit distinct LDS banks.  The
// split's page-table slice and the window of ancestor-mask words its tree
// keys need are copied to LDS before the ring starts, so the loop issues no
// other global loads.
//
// Compute pipeline.  Four waves per workgroup and one workgroup per CU, so
// every wave owns a SIMD and its whole register file; a wave covers QB
// blocks of 32 queries, and each K or V operand it reads from LDS feeds QB
// MFMAs.  The S^T MFMAs of tile j+1 are issued before the softmax of tile
// j, in the same basic block, so the matrix core works while the vector
// ALU exponentiates.  Softmax runs in base 2 with scale*log2(e) folded into the
// FMA that subtracts the running max; the running max is only raised when a
// tile's max exceeds it by more than 8 (log2 units), which bounds the
// probabilities by 2^8 and skips most O rescales.  The row sum accumulates
// the fp32 probabilities (before their rounding to bf16 for the PV product).
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
constexpr int kStages = 4;
constexpr int kTileBytes = kKeyTile * kHeadDim * 2;   // 16 KB per matrix
constexpr int kStageBytes = 2 * kTileBytes;           // K and V of a tile
// The ring holds the K tiles of all stages in its first half and the V
// tiles in its second, so that every operand offset of a stage fits the
// 16-bit immediate of an LDS instruction.
constexpr int kVOff = kStages * kTileBytes;
constexpr int kPageCache = 1040;                      // page ids per split
constexpr int kMaskCache = 2304;                      // mask words per WG
constexpr float kLazyRescale = 8.f;                   // log2 units

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

__device__ __forceinline__ bf16x8 lds_read16(unsigned addr) {
  return __builtin_bit_cast(bf16x8, *(const lds_u32x4*)(size_t)addr);
}

// Transposing LDS read (see the file comment).
__device__ __forceinline__ s16x4 lds_read_tr(unsigned addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(size_t)addr);
}

// 16 bytes per lane from global memory to LDS at lds_base + 16 * lane.
// The compiler does not track these loads; callers wait with wait_vmcnt.
__device__ __forceinline__ void dma16(const void* gptr, unsigned lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(lds_base), "v"(gptr) : "memory");
}

// Same, with a wave-uniform 64-bit base in SGPRs and a 32-bit per-lane
// offset (no per-lane 64-bit address arithmetic).
__device__ __forceinline__ void dma16_sbase(const void* sbase, unsigned voff,
                                            unsigned lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(lds_base), "v"(voff), "s"(sbase) : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// Value of the other lane half (lane ^ 32).
__device__ __forceinline__ float other_half(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  // r[0]: lanes 32..63 now hold lanes 0..31; r[1]: lanes 0..31 hold 32..63
  return __builtin_bit_cast(float, __lane_id() < 32 ? r[1] : r[0]);
}

// Applies the mask of one tile (keys past the split end; tree keys off the
// node's root-to-node path) to the scores of one 32-query block.
__device__ __forceinline__ void apply_tile_mask(f32x16 (&S)[2], uint64_t allow,
                                                int half) {
  allow >>= 4 * half;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const int kk = kb * 32 + 8 * (rr >> 2) + (rr & 3);
      if (!((allow >> kk) & 1)) S[kb][rr] = -INFINITY;
    }
  }
}

// QB = 32-query column blocks per wave (1 or 2).  Four waves per workgroup,
// one workgroup per CU (the LDS ring fills the CU), so each wave has a SIMD
// and its full register file to itself.
template <int QB>
__global__ __launch_bounds__(256, 1) void attn_fwd_kernel(FwdParams p) {
  constexpr int NW = 4;
  constexpr int kThreads = NW * 64;
  constexpr int kRowsPerWave = 32 * QB;
  constexpr int kRowsPerWG = NW * kRowsPerWave;
  constexpr int kOpsPerMat = 16 / NW;        // 1-KB DMA ops per wave per matrix
  constexpr int kOps = 2 * kOpsPerMat;       // per wave per tile
  __shared__ __align__(1024) unsigned char ring[2 * kVOff];
  __shared__ int pg_lds[kPageCache];
  __shared__ uint64_t mk_lds[kMaskCache];

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

  const int tid = threadIdx.x;
  // readfirstlane tells the compiler the wave index is wave-uniform
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int col = lane & 31, half = lane >> 5;

  // The prologue issues all its loads before it waits for any: the
  // split's page-table entries first (they depend only on the sequence and
  // the split), then, once the tree bounds are in, the mask words and Q.
  const int kbeg = split * p.chunk;
  const int lp0 = kbeg >> p.log2_page;
  constexpr int kPgPer = (kPageCache + kThreads - 1) / kThreads;
  int pgv[kPgPer];
  {
    // pages a split can span, within the page-table row
    const int npg_max = min(min(((p.chunk - 1) >> p.log2_page) + 2, kPageCache),
                            p.max_pps - lp0);
    const int* ptab = p.page_table + (size_t)s * p.max_pps + lp0;
#pragma unroll
    for (int k = 0; k < kPgPer; ++k) {
      const int i = tid + k * kThreads;
      pgv[k] = i < npg_max ? ptab[i] : 0;
    }
  }

  const int a = clampi(p.tree_offsets[s], 0, p.N);
  const int b = clampi(p.tree_offsets[s + 1], a, p.N);
  const int B = b - a;
  const int P = max(p.prefix_lens[s], 0);
  const int rows = p.G * B;
  const int r0 = mb * kRowsPerWG;
  if (r0 >= rows) return;
  const int T = min(P + B, p.max_tokens);
  if (kbeg >= T) return;
  const int kend = min(T, kbeg + p.chunk);
  const int ntiles = (kend - kbeg + kKeyTile - 1) / kKeyTile;
  const int npg = min(((kend - 1) >> p.log2_page) - lp0 + 1, kPageCache);

  // ---- ancestor-mask words of this workgroup's nodes for the split's
  // tree keys -> LDS (window of words wlo..whi of each node's row).  The
  // host sizes the workgroup so that nnodes * nwin <= kMaskCache.
  const int n_lo = r0 / p.G;
  const int n_hi = (min(r0 + kRowsPerWG, rows) - 1) / p.G;
  const int nnodes = n_hi - n_lo + 1;
  const bool has_tree = kend > P;
  const int wlo = has_tree ? (max(kbeg, P) - P) >> 6 : 0;
  const int whi = has_tree ? min(p.W - 1, ((kend - 1 - P) >> 6) + 1) : 0;
  const int nwin = whi - wlo + 1;
  const int nm = has_tree ? min(nnodes * nwin, kMaskCache) : 0;
  constexpr int kMkPer = (kMaskCache + kThreads - 1) / kThreads;
  uint64_t mkv[kMkPer];
  {
    // entry i = tid + k*kThreads is word w of node nn, i = nn*nwin + w;
    // stepped by kThreads without a division per entry
    const int dq = kThreads / nwin, dr = kThreads - dq * nwin;
    int nn = tid / nwin, w = tid - nn * nwin;
#pragma unroll
    for (int k = 0; k < kMkPer; ++k) {
      const int i = tid + k * kThreads;
      mkv[k] = i < nm ? p.masks[(size_t)(a + n_lo + nn) * p.W + wlo + w] : 0;
      nn += dq;
      w += dr;
      if (w >= nwin) {
        w -= nwin;
        ++nn;
      }
    }
  }

  // ---- this lane's query rows (one per column block)
  bool rvalid[QB];
  int node[QB];
  size_t qrow[QB];
  bf16x8 qf[QB][8];  // Q^T fragments (B operand): d = kc*16 + half*8 + 0..7
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int r = r0 + wave * kRowsPerWave + qb * 32 + col;
    rvalid[qb] = r < rows;
    node[qb] = rvalid[qb] ? r / p.G : n_hi;
    const int head = g * p.G + (rvalid[qb] ? r % p.G : 0);
    qrow[qb] = (size_t)(a + node[qb]) * p.Hq + head;
    const __bf16* qp = p.q + qrow[qb] * kHeadDim + half * 8;
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) {
      u32x4 raw = rvalid[qb] ? *reinterpret_cast<const u32x4*>(qp + kc * 16)
                             : u32x4{0, 0, 0, 0};
      qf[qb][kc] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  // ---- page slice and mask window -> LDS
#pragma unroll
  for (int k = 0; k < kPgPer; ++k) {
    const int i = tid + k * kThreads;
    if (i < npg) pg_lds[i] = clampi(pgv[k], 0, p.num_pages - 1);
  }
#pragma unroll
  for (int k = 0; k < kMkPer; ++k) {
    const int i = tid + k * kThreads;
    if (i < nm) mk_lds[i] = mkv[k];
  }

  // ---- LDS addresses
  const unsigned ring_base =
      (unsigned)(size_t)(__attribute__((address_space(3))) unsigned char*)ring;
  // K operand: row kb*32 + col, 16-B chunk (2*kc + half) ^ (col & 15)
  unsigned k_off[8];
#pragma unroll
  for (int kc = 0; kc < 8; ++kc) {
    k_off[kc] = col * 256 + (((2 * kc + half) ^ (col & 15)) << 4);
  }
  // V^T operand: rows kbase + 4*half + y (y = lane%16 / 4), chunk
  // 4*db + x, x = 2*((lane/16)&1) + (lane%4)/2, swizzled by 4*y.
  const int y = (lane & 15) >> 2;
  const int x = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  unsigned v_off[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    v_off[db] = kVOff + (4 * half + y) * 256 +
                ((4 * (db ^ y) + x) << 4) + 8 * (lane & 1);
  }

  // ---- DMA of one tile: wave w moves rows 4*i .. 4*i+3 for
  // i in [w*kOpsPerMat, (w+1)*kOpsPerMat) of K and of V.  The byte offset
  // of a lane's 16 bytes is page * page_bytes + slot * tok_bytes +
  // (head and swizzled chunk), the last part fixed per lane and row.
  const int pmask = (1 << p.log2_page) - 1;
  const unsigned tok_bytes = (unsigned)p.Hkv * kHeadDim * 2;
  const unsigned page_bytes = tok_bytes << p.log2_page;
  const int lrow = lane >> 4, lchunk = lane & 15;
  unsigned k_lane[kOpsPerMat], v_lane[kOpsPerMat];
#pragma unroll
  for (int k = 0; k < kOpsPerMat; ++k) {
    const int row = 4 * (wave * kOpsPerMat + k) + lrow;
    k_lane[k] = g * kHeadDim * 2 + ((lchunk ^ (row & 15)) << 4);
    v_lane[k] = g * kHeadDim * 2 + ((lchunk ^ (4 * (row & 3))) << 4);
  }
  const char* kbase = reinterpret_cast<const char*>(p.k);
  const char* vbase = reinterpret_cast<const char*>(p.v);
  // Fast path: with pages of >= 16 tokens the 16 rows a wave moves
  // (4*kOpsPerMat rows starting at a multiple of 16) lie in one page, so
  // the page lookup is wave-uniform and the loads use an SGPR base plus a
  // per-lane offset fixed for the whole loop.
  static_assert(4 * kOpsPerMat == 16, "a wave moves 16 rows per matrix");
  const bool fast_pages = p.log2_page >= 4;
  unsigned k_row_off[kOpsPerMat], v_row_off[kOpsPerMat];
#pragma unroll
  for (int k = 0; k < kOpsPerMat; ++k) {
    const int r16 = 4 * k + lrow;  // row within the wave's 16
    k_row_off[k] = r16 * tok_bytes + ((lchunk ^ (r16 & 15)) << 4);
    v_row_off[k] = r16 * tok_bytes + ((lchunk ^ (4 * (r16 & 3))) << 4);
  }
  // fast-path DMA of tile t, issued in pieces: plan (page lookup) first,
  // then parts k = 0 .. kOpsPerMat-1 (one K and one V instruction each)
  struct DmaPlan {
    const char* kb0;
    const char* vb0;
    unsigned st;
  };
  auto fast_ok = [&](int t) {
    return fast_pages && kbeg + t * kKeyTile + 16 * wave + 15 < kend;
  };
  auto dma_plan = [&](int t) -> DmaPlan {
    const int w0 = kbeg + t * kKeyTile + 16 * wave;
    const int pi = clampi((w0 >> p.log2_page) - lp0, 0, kPageCache - 1);
    const unsigned pgu = (unsigned)__builtin_amdgcn_readfirstlane(pg_lds[pi]);
    const size_t off = (size_t)pgu * page_bytes +
                       (unsigned)(w0 & pmask) * tok_bytes + g * kHeadDim * 2;
    return DmaPlan{kbase + off, vbase + off,
                   ring_base + (unsigned)(t % kStages) * kTileBytes};
  };
  auto dma_part = [&](const DmaPlan& dp, int k) {
    const unsigned dst = dp.st + (wave * kOpsPerMat + k) * 1024;
    dma16_sbase(dp.kb0, k_row_off[k], dst);
    dma16_sbase(dp.vb0, v_row_off[k], dst + kVOff);
  };
  auto issue = [&](int t) {
    const int t0 = kbeg + t * kKeyTile;
    const unsigned st = ring_base + (unsigned)(t % kStages) * kTileBytes;
    const int w0 = t0 + 16 * wave;  // first position this wave moves
    if (fast_pages && w0 + 15 < kend) {
      const int pi = clampi((w0 >> p.log2_page) - lp0, 0, kPageCache - 1);
      const unsigned pgu = (unsigned)__builtin_amdgcn_readfirstlane(pg_lds[pi]);
      const size_t off = (size_t)pgu * page_bytes +
                         (unsigned)(w0 & pmask) * tok_bytes + g * kHeadDim * 2;
      const char* kb0 = kbase + off;
      const char* vb0 = vbase + off;
#pragma unroll
      for (int k = 0; k < kOpsPerMat; ++k) {
        const unsigned dst = st + (wave * kOpsPerMat + k) * 1024;
        dma16_sbase(kb0, k_row_off[k], dst);
        dma16_sbase(vb0, v_row_off[k], dst + kVOff);
      }
      return;
    }
    int pg[kOpsPerMat], slot[kOpsPerMat];
#pragma unroll
    for (int k = 0; k < kOpsPerMat; ++k) {  // page ids first, one LDS wait
      const int pos = min(t0 + 4 * (wave * kOpsPerMat + k) + lrow, kend - 1);
      slot[k] = pos & pmask;
      pg[k] = pg_lds[clampi((pos >> p.log2_page) - lp0, 0, kPageCache - 1)];
    }
#pragma unroll
    for (int k = 0; k < kOpsPerMat; ++k) {
      const int i = wave * kOpsPerMat + k;
      const size_t off = (size_t)(unsigned)pg[k] * page_bytes +
                         (unsigned)slot[k] * tok_bytes;
      const unsigned dst = __builtin_amdgcn_readfirstlane(st + i * 1024);
      dma16(kbase + off + k_lane[k], dst);
      dma16(vbase + off + v_lane[k], dst + kVOff);
    }
  };

  // ---- S^T = K Q^T of tile t, in two halves of the head dimension
  // (kc = 4h .. 4h+3) so that only half of the K fragments are live at a
  // time; 2*QB accumulation chains.
  auto read_k_half = [&](int t, int h, bf16x8 (&kf)[2][4]) {
    const unsigned st = ring_base + (unsigned)(t % kStages) * kTileBytes;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        kf[kb][c] = lds_read16(st + kb * 32 * 256 + k_off[4 * h + c]);
      }
    }
  };
  auto qk_half = [&](bf16x8 (&kf)[2][4], f32x16 (&S)[QB][2], int h) {
    if (h == 0) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        S[qb][0] = f32x16{};
        S[qb][1] = f32x16{};
      }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          S[qb][kb] = mfma32x32x16(kf[kb][c], qf[qb][4 * h + c], S[qb][kb]);
        }
      }
    }
  };
  auto qk = [&](int t, f32x16 (&S)[QB][2]) {
    bf16x8 kf0[2][4], kf1[2][4];
    read_k_half(t, 0, kf0);
    read_k_half(t, 1, kf1);
    qk_half(kf0, S, 0);
    qk_half(kf1, S, 1);
  };

  // ---- 64-bit allowed-key mask of tile t for a node (tree tiles only)
  auto tile_allow = [&](int t0, int nd) -> uint64_t {
    const int nvalid = kend - t0;  // >= 1
    const int npre = P - t0;
    uint64_t allow = nvalid >= 64 ? ~0ull : ((1ull << nvalid) - 1);
    const uint64_t pre =
        npre >= 64 ? ~0ull : (npre <= 0 ? 0ull : ((1ull << npre) - 1));
    uint64_t tree = 0;
    if (npre < 64) {
      const int mrow_lds = (nd - n_lo) * nwin - wlo;
      const int j0 = t0 - P;  // tree node at tile offset 0 (may be < 0)
      if (j0 >= 0) {
        const int w0 = min(j0 >> 6, p.W - 1);
        const int sh = j0 & 63;
        tree = mk_lds[clampi(mrow_lds + w0, 0, kMaskCache - 1)] >> sh;
        if (sh != 0 && w0 + 1 < p.W) {
          tree |= mk_lds[clampi(mrow_lds + w0 + 1, 0, kMaskCache - 1)]
                  << (64 - sh);
        }
      } else {
        tree = mk_lds[clampi(mrow_lds, 0, kMaskCache - 1)] << (-j0);
      }
    }
    return allow & (pre | tree);
  };

  f32x16 o[QB][4];
  float l_run[QB];  // this lane half's share of the row sum
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
    for (int db = 0; db < 4; ++db) o[qb][db] = f32x16{};
    l_run[qb] = 0.f;
  }
  const float c2 = p.scale_log2;

  // ---- V^T fragments of tile j
  auto read_v = [&](int j, bf16x8 (&vf)[2][2][4], int kb0 = 0, int kb1 = 2) {
    const unsigned st = ring_base + (unsigned)(j % kStages) * kTileBytes;
#pragma unroll
    for (int kb = kb0; kb < kb1; ++kb) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const unsigned va = st + v_off[db] + (kb * 32 + hf * 16) * 256;
          const s16x4 lo = lds_read_tr(va);
          const s16x4 hi = lds_read_tr(va + 8 * 256);
          vf[kb][hf][db] = __builtin_bit_cast(
              bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
      }
    }
  };

  // ---- probabilities of a tile against the reference max m_ref (log2
  // units); adds their fp32 sum to l_run
  float m_ref[QB];
  auto exps = [&](f32x16 (&S)[QB][2], bf16x8 (&pf)[QB][2][2], int kb0 = 0,
                  int kb1 = 2) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float mu = (m_ref[qb] == -INFINITY) ? 0.f : m_ref[qb];
      float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
      for (int kb = kb0; kb < kb1; ++kb) {
#pragma unroll
        for (int rr = 0; rr < 16; rr += 2) {
          const float e0 = fast_exp2(fmaf(S[qb][kb][rr], c2, -mu));
          const float e1 = fast_exp2(fmaf(S[qb][kb][rr + 1], c2, -mu));
          ps0 += e0;
          ps1 += e1;
          pf[qb][kb][rr >> 3][rr & 7] = (__bf16)e0;
          pf[qb][kb][rr >> 3][(rr & 7) + 1] = (__bf16)e1;
        }
      }
      l_run[qb] += ps0 + ps1;
    }
  };

  // ---- reference max for a tile: raised (lazily) when the tile's max
  // exceeds the current one by more than kLazyRescale; alpha rescales the
  // accumulated O and l.  Returns whether any row changed its reference.
  auto next_ref = [&](f32x16 (&S)[QB][2], float (&m_new)[QB],
                      float (&alpha)[QB]) -> bool {
    bool any_need = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      // IEEE maximum (v_maximum3_f32): no NaN canonicalisation of inputs
      float tmax = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int rr = 0; rr < 16; rr += 2) {
          tmax = __builtin_elementwise_maximum(
              tmax, __builtin_elementwise_maximum(S[qb][kb][rr],
                                                  S[qb][kb][rr + 1]));
        }
      }
      tmax = __builtin_elementwise_maximum(tmax, other_half(tmax)) * c2;
      const bool need = tmax > m_ref[qb] + kLazyRescale;
      m_new[qb] = need ? tmax : m_ref[qb];
      alpha[qb] = need ? fast_exp2(m_ref[qb] - m_new[qb]) : 1.f;
      any_need |= need;
    }
    return any_need;
  };

  // ---- O^T += V^T P^T: 4*QB independent accumulation chains
  auto pv = [&](bf16x8 (&vf)[2][2][4], bf16x8 (&pf)[QB][2][2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
        for (int db = 0; db < 4; ++db) {
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            o[qb][db] = mfma32x32x16(vf[kb][hf][db], pf[qb][kb][hf], o[qb][db]);
          }
        }
      }
    }
  };

  // ---- one pipeline step over tile j.  Tile j's scores (masked, with
  // their reference max m_ref) were computed in the previous step.  In
  // branch-free blocks: S^T of tile j+1 on the matrix core while the
  // vector ALU exponentiates tile j; then PV of tile j while the ALU finds
  // tile j+1's max.  The rare rescale of O comes last.  After the last
  // tile the S^T is computed on stale LDS data and dropped.
  //
  // With dma_inbody the DMA of tile j+3 is issued from inside the step, in
  // two bursts between segments: issuing it all right after the barrier
  // makes the four waves queue 32 instructions at the CU's address unit at
  // once and stall for it.
  auto body = [&](int j, f32x16 (&Scur)[QB][2], f32x16 (&Snext)[QB][2],
                  bool mask_next, bool dma_inbody, float (&m_new)[QB],
                  float (&alpha)[QB]) -> bool {
    bf16x8 kf0[2][4], kf1[2][4];
    bf16x8 vf[2][2][4];
    bf16x8 pf[QB][2][2];
    DmaPlan dp{};
    if (dma_inbody) dp = dma_plan(j + kStages - 1);
    read_k_half(j + 1, 0, kf0);
    // segment 1: S^T MFMAs kc 0..3; the other K half, V^T of keys 0..31
    // and their probabilities are loaded and computed beside them
    qk_half(kf0, Snext, 0);
    read_k_half(j + 1, 1, kf1);
    read_v(j, vf, 0, 1);
    exps(Scur, pf, 0, 1);
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int i = 0; i < 8 * QB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 24 / (8 * QB), 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
    }
    if (dma_inbody) {
      __builtin_amdgcn_sched_barrier(0);
      dma_part(dp, 0);
      dma_part(dp, 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    // segment 2: S^T MFMAs kc 4..7, keys 32..63
    qk_half(kf1, Snext, 1);
    read_v(j, vf, 1, 2);
    exps(Scur, pf, 1, 2);
#pragma unroll
    for (int i = 0; i < 8 * QB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 16 / (8 * QB), 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
    }
    if (dma_inbody) {
      __builtin_amdgcn_sched_barrier(0);
      dma_part(dp, 2);
      dma_part(dp, 3);
      __builtin_amdgcn_sched_barrier(0);
    }
    // segment 3: PV of tile j, max of tile j+1
    pv(vf, pf);
    if (mask_next) {
      const int t1 = kbeg + (j + 1) * kKeyTile;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        apply_tile_mask(Snext[qb], tile_allow(t1, node[qb]), half);
      }
    }
    const bool r = next_ref(Snext, m_new, alpha);
#pragma unroll
    for (int i = 0; i < 16 * QB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
    }
    return r;
  };
  auto step = [&](int j, f32x16 (&Scur)[QB][2], f32x16 (&Snext)[QB][2]) {
    if (j + 1 < ntiles) {
      // tile j+1 must have landed; tile j+2 may still be in flight
      if (j + 2 < ntiles) wait_vmcnt<kOps>();
      else wait_vmcnt<0>();
    }
    __syncthreads();
    const int t1 = kbeg + (j + 1) * kKeyTile;
    float m_new[QB], alpha[QB];
    bool r;
    const bool has_next_dma = j + kStages - 1 < ntiles;
    if (j + 1 < ntiles && t1 + kKeyTile > min(P, kend)) {
      if (has_next_dma) issue(j + kStages - 1);
      r = body(j, Scur, Snext, true, false, m_new, alpha);
    } else if (has_next_dma && fast_ok(j + kStages - 1)) {
      r = body(j, Scur, Snext, false, true, m_new, alpha);
    } else {
      if (has_next_dma) issue(j + kStages - 1);
      r = body(j, Scur, Snext, false, false, m_new, alpha);
    }
    if (j + 1 >= ntiles) {  // the scores past the last tile are not data
      r = false;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) m_new[qb] = m_ref[qb];
    }
    if (__any(r)) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        l_run[qb] *= alpha[qb];
#pragma unroll
        for (int db = 0; db < 4; ++db) o[qb][db] *= alpha[qb];
      }
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) m_ref[qb] = m_new[qb];
  };

  // Make the compiler wait for the Q loads here, before the first DMA:
  // its own wait at the first use of qf would also drain the ring.
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    asm volatile("" :: "v"(qf[qb][0]), "v"(qf[qb][1]), "v"(qf[qb][2]),
                 "v"(qf[qb][3]), "v"(qf[qb][4]), "v"(qf[qb][5]),
                 "v"(qf[qb][6]), "v"(qf[qb][7]));
  }
  __syncthreads();  // page slice and mask window visible
#pragma unroll
  for (int t = 0; t < kStages - 1; ++t) {
    if (t < ntiles) issue(t);
  }
  // wait for tile 0: later tiles may stay in flight
  if (ntiles >= 3) wait_vmcnt<2 * kOps>();
  else if (ntiles == 2) wait_vmcnt<kOps>();
  else wait_vmcnt<0>();
  __syncthreads();
  f32x16 SA[QB][2], SB[QB][2];
  qk(0, SA);
  if (kbeg + kKeyTile > min(P, kend)) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      apply_tile_mask(SA[qb], tile_allow(kbeg, node[qb]), half);
    }
  }
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) m_ref[qb] = -INFINITY;
  {
    float m_new[QB], alpha[QB];
    next_ref(SA, m_new, alpha);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) m_ref[qb] = m_new[qb];
  }
  // Hot steps: tile j+1 lies wholly in the prefix and tile j+3 is a full
  // tile on the fast DMA path.  They run in a loop of their own, so that
  // its code holds no branch between step variants (a join of variants
  // makes the compiler copy the accumulators between registers).
  auto hot_step = [&](int j, f32x16 (&Scur)[QB][2], f32x16 (&Snext)[QB][2]) {
    wait_vmcnt<kOps>();
    __syncthreads();
    float m_new[QB], alpha[QB];
    const bool r = body(j, Scur, Snext, false, true, m_new, alpha);
    if (__any(r)) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        l_run[qb] *= alpha[qb];
#pragma unroll
        for (int db = 0; db < 4; ++db) o[qb][db] *= alpha[qb];
      }
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) m_ref[qb] = m_new[qb];
  };
  int n_hot = 0;
  if (fast_pages) {
    const int last = min((kend - kbeg) / kKeyTile - kStages,
                         (P - kbeg) / kKeyTile - 2);
    n_hot = max(last + 1, 0) & ~(kStages - 1);
  }
  // both loops are unrolled by the ring depth and start at a multiple of
  // it, so that every stage index is a constant
  for (int i = 0; 4 * i < n_hot; ++i) {
    const int j = 4 * i;
    hot_step(j, SA, SB);
    hot_step(j + 1, SB, SA);
    hot_step(j + 2, SA, SB);
    hot_step(j + 3, SB, SA);
  }
  for (int i = n_hot / 4; 4 * i < ntiles; ++i) {
    const int j = 4 * i;
    step(j, SA, SB);
    if (j + 1 < ntiles) step(j + 1, SB, SA);
    if (j + 2 < ntiles) step(j + 2, SA, SB);
    if (j + 3 < ntiles) step(j + 3, SB, SA);
  }
  float m_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) m_run[qb] = m_ref[qb];

  // ---- epilogue
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l_tot = l_run[qb] + other_half(l_run[qb]);
    if (!rvalid[qb]) continue;
    if (p.splits == 1) {
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      __bf16* op = p.out + qrow[qb] * kHeadDim;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          bf16x4 v4;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v4[e] = (__bf16)(o[qb][db][g4 * 4 + e] * inv);
          }
          *reinterpret_cast<bf16x4*>(op + db * 32 + g4 * 8 + half * 4) = v4;
        }
      }
      if (half == 0) {
        p.lse[qrow[qb]] =
            l_tot > 0.f ? (m_run[qb] + log2f(l_tot)) * kLn2 : -INFINITY;
      }
    } else {
      const size_t prow = (size_t)split * p.N * p.Hq + qrow[qb];
      float* pp = p.part_o + prow * kHeadDim;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          f32x4 v4 = {o[qb][db][g4 * 4 + 0], o[qb][db][g4 * 4 + 1],
                      o[qb][db][g4 * 4 + 2], o[qb][db][g4 * 4 + 3]};
          *reinterpret_cast<f32x4*>(pp + db * 32 + g4 * 8 + half * 4) = v4;
        }
      }
      if (half == 0) {
        *reinterpret_cast<f32x2*>(p.part_ml + prow * 2) =
            f32x2{m_run[qb], l_tot};
      }
    }
  }
}

}  // namespace tree_attn
