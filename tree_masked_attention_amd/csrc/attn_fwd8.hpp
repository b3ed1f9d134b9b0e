// 256-row variant of the split-KV tree-verification attention kernel, for
// (sequence, kv head) pairs with at least 256 query rows.
//
// Same operation, data layout, MFMA mapping, LDS ring format and pipeline
// as the 128-row kernel (definitions in attn_fwd.hpp); each K/V tile staged
// in LDS serves 256 rows.  Eight waves of 32 rows, two waves per SIMD: the
// vector ALU of a SIMD issues about twice as many instructions per cycle
// (and the exponential about three times as many) when two waves feed it;
// 256 registers per wave.  Each wave overlaps its own S^T MFMAs of tile
// j+1 with the softmax of tile j; scores are built one 32-key block at a
// time and the K/V operands are read from LDS a quarter tile at a time.
// The per-wave state is written over QB query blocks of 32 rows (QB = 1
// here), so that the row bookkeeping reads the same for any block count.
#pragma once

#include "attn_fwd.hpp"

namespace tree_attn {

constexpr int kRowsPerWG8 = 256;

template <bool kBalanced, bool kFp8, int D = kHeadDim>
__global__ __launch_bounds__(512, 1) void attn_fwd256_kernel(FwdParams p) {
  static_assert(D == kHeadDim || D == 64, "head dim");
  constexpr int NW = 8;
  constexpr int QB = 1;                  // 32-query blocks per wave
  constexpr int kThreads = NW * 64;
  constexpr int kEB = kFp8 ? 1 : 2;      // bytes per cached element
  constexpr int kRowB = D * kEB;         // bytes per cached (token, head)
  // 128-byte rows (fp8 with d = 128, bf16 with d = 64): 8 chunks of 16
  // bytes per row, 8 rows per DMA op; 64-byte rows (fp8 with d = 64): 4
  // chunks, 16 rows per op
  constexpr bool kNarrow = kRowB == 128;
  constexpr int kRowChunks = kRowB / 16;  // 16-byte chunks per row
  constexpr int kKSteps = D / 16;        // MFMA k-steps over the head dim
  constexpr int kDB = D / 32;            // 32-wide head-dim blocks of O
  // 1-KB DMA ops of a 64-row matrix tile; with fewer than one per wave
  // (64-byte rows), each wave moves one op, of K (waves 0-3) or of V
  constexpr int kMatOps = kRowChunks;
  constexpr bool kSplitOps = kMatOps < NW;
  // 1-KB DMA ops per wave per matrix it moves: each moves 4, 8 or 16 rows
  constexpr int kOpsPerMat = kSplitOps ? 1 : kMatOps / NW;
  constexpr int kOps = kSplitOps ? 1 : 2 * kOpsPerMat;
  constexpr int kRowsPerOp = 1024 / kRowB;
  constexpr int kDmaRows = kRowsPerOp * kOpsPerMat;  // tile rows a wave moves
  constexpr int kLog2DmaRows = kDmaRows == 8 ? 3 : 4;
  static_assert((1 << kLog2DmaRows) == kDmaRows, "shape");
  __shared__ __align__(1024) unsigned char ring[2 * kVOff];
  __shared__ int pg_lds[kPageCache];
  __shared__ uint64_t mk_lds[kMaskCache];

  // XCD-aware decode: consecutive work units (the row blocks of one
  // (sequence, kv head, split), which read the same K/V) go to one XCD.
  const int bid = blockIdx.x;
  const int L = (bid & 7) * p.per_xcd + (bid >> 3);
  if (L >= p.plan.parts) return;
  Unit un = decode_unit<kBalanced>(p.plan, L);
  if (!un.valid) return;
  const int s = un.s, g = un.g, mb = un.mb, split = un.split;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int col = lane & 31, half = lane >> 5;

  // All prologue loads are issued before any is waited for: the split's
  // page-table entries first (they need only the sequence and the split),
  // then, once the tree bounds are in, the mask words and Q.
  const int kbeg = split * un.chunk;
  const int lp0 = kbeg >> p.log2_page;
  constexpr int kPgPer = (kPageCache + kThreads - 1) / kThreads;
  int pgv[kPgPer];
  {
    const int npg_max = min(min(((un.chunk - 1) >> p.log2_page) + 2, kPageCache),
                            p.max_pps - lp0);
    const int* ptab = p.page_table + (size_t)s * p.max_pps + lp0;
#pragma unroll
    for (int k = 0; k < kPgPer; ++k) {
      const int i = tid + k * kThreads;
      pgv[k] = i < npg_max ? ptab[i] : 0;
    }
  }

  load_bounds(p.plan, un);
  const int a = un.a, B = un.B, P = un.P, T = un.T;
  const int rows = p.G * B;
  const int r0 = mb * kRowsPerWG8;
  if (r0 >= rows) return;
  if (kbeg >= T) return;
  const int kend = min(T, kbeg + un.chunk);
  const int n = (kend - kbeg + kKeyTile - 1) / kKeyTile;  // tiles, >= 1
  const int npg = min(((kend - 1) >> p.log2_page) - lp0 + 1, kPageCache);

  const int n_lo = r0 / p.G;
  const int n_hi = (min(r0 + kRowsPerWG8, rows) - 1) / p.G;
  const int nnodes = n_hi - n_lo + 1;
  const bool has_tree = kend > P;
  const int wlo = has_tree ? (max(kbeg, P) - P) >> 6 : 0;
  const int whi = has_tree ? min(p.W - 1, ((kend - 1 - P) >> 6) + 1) : 0;
  const int nwin = whi - wlo + 1;
  const int nm = has_tree ? min(nnodes * nwin, kMaskCache) : 0;
  constexpr int kMkPer = (kMaskCache + kThreads - 1) / kThreads;
  uint64_t mkv[kMkPer];
  {
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

  // ---- this lane's query rows (one per query block)
  bool rvalid[QB];
  int node[QB];
  size_t qrow[QB];
  bf16x8 qf[QB][kKSteps];  // Q^T fragments (B operand): d = kc*16 + half*8 + 0..7
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int r = r0 + (wave * QB + qb) * 32 + col;
    rvalid[qb] = r < rows;
    node[qb] = rvalid[qb] ? r / p.G : n_hi;
    qrow[qb] = (size_t)(a + node[qb]) * p.Hq + g * p.G +
               (rvalid[qb] ? r % p.G : 0);
    const __bf16* qp = p.q + qrow[qb] * D + half * 8;
#pragma unroll
    for (int kc = 0; kc < kKSteps; ++kc) {
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

  // ---- LDS operand addresses (stage 0; the stage offset is added per tile)
  const unsigned ring_base =
      (unsigned)(size_t)(__attribute__((address_space(3))) unsigned char*)ring;
  unsigned k_off[kKSteps];
#pragma unroll
  for (int kc = 0; kc < kKSteps; ++kc) {
    if constexpr (kFp8 && kRowB == 64) {
      // fp8 rows of 64 B (d = 64), chunk c stored at c ^ ((row >> 2) & 3);
      // the lane's 8 values are half of chunk kc
      k_off[kc] = ring_base + col * 64 + ((kc ^ ((col >> 2) & 3)) << 4) +
                  half * 8;
    } else if constexpr (kFp8) {
      // fp8 rows of 128 B, 16-byte chunk c stored at c ^ ((row >> 1) & 7);
      // the lane's 8 values d = kc*16 + half*8 .. +7 are half of chunk kc
      // (32-key block offsets keep the swizzle: 32 rows = 16 row pairs)
      k_off[kc] = ring_base + col * 128 + ((kc ^ ((col >> 1) & 7)) << 4) +
                  half * 8;
    } else if constexpr (kNarrow) {
      // bf16 rows of 128 B (d = 64), the same swizzle; the lane's 8
      // values are chunk 2 kc + half
      k_off[kc] = ring_base + col * 128 +
                  (((2 * kc + half) ^ ((col >> 1) & 7)) << 4);
    } else {
      k_off[kc] = ring_base + col * 256 + (((2 * kc + half) ^ (col & 15)) << 4);
    }
  }
  const int y = (lane & 15) >> 2;
  const int x = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  unsigned v_off[kDB];
#pragma unroll
  for (int db = 0; db < kDB; ++db) {
    if constexpr (kFp8) {
      // ds_read_b64_tr_b8 (attn_fwd.hpp): lanes 2r, 2r+1 of a 16-lane group
      // name row r = key 8*(r/4) + 4*half + r%4 of the 16-key block
      const int j = lane & 15, r8 = j >> 1;
      const int row = 8 * (r8 >> 2) + 4 * half + (r8 & 3);
      const int chunk = 2 * db + ((lane >> 4) & 1);
      if constexpr (kRowB == 64) {
        // rows of 64 B: chunk c stored at c ^ 2 ((row >> 2) & 1)
        v_off[db] = ring_base + kVOff + row * 64 +
                    ((chunk ^ (2 * ((row >> 2) & 1))) << 4) + 8 * (j & 1);
      } else {
        v_off[db] = ring_base + kVOff + row * 128 +
                    ((chunk ^ ((row >> 1) & 7)) << 4) + 8 * (j & 1);
      }
    } else if constexpr (kNarrow) {
      // bf16 rows of 128 B (d = 64): chunk c stored at c ^ 4 ((row >> 1) & 1)
      // (the four rows a half-wave reads then cover all banks)
      const int row = 4 * half + y;
      v_off[db] = ring_base + kVOff + row * 128 +
                  (((4 * db + x) ^ (4 * ((row >> 1) & 1))) << 4) +
                  8 * (lane & 1);
    } else {
      v_off[db] = ring_base + kVOff + (4 * half + y) * 256 +
                  ((4 * (db ^ y) + x) << 4) + 8 * (lane & 1);
    }
  }

  // ---- DMA of one tile: wave w moves rows kDmaRows*w .. of K and of V, as
  // kOpsPerMat instructions of 4 rows (lane l: row 4k + l/16, chunk l%16)
  // or 8 rows; with 64-byte rows, rows 16 (w % 4) .. of K or V.
  const int pmask = (1 << p.log2_page) - 1;
  const unsigned tok_bytes = (unsigned)p.Hkv * kRowB;
  const unsigned page_bytes = tok_bytes << p.log2_page;
  // a lane's row and 16-byte chunk within one DMA op
  const int lrow = lane / kRowChunks;
  const int lchunk = lane % kRowChunks;
  // the wave's row group within the matrix tile it moves, and (64-byte
  // rows) whether that is V
  const int dma_w = kSplitOps ? wave % kMatOps : wave;
  const bool dma_v = kSplitOps && wave >= kMatOps;
  // source chunk of the lane's 16 bytes (the LDS chunk is fixed by the
  // lane): 256-byte rows K chunk ^ (row & 15), V chunk ^ 4 (row & 3);
  // 128-byte rows K chunk ^ ((row >> 1) & 7), V the same for fp8 and
  // chunk ^ 4 ((row >> 1) & 1) for bf16; 64-byte rows K chunk ^
  // ((row >> 2) & 3), V chunk ^ 2 ((row >> 2) & 1)
  auto k_chunk = [](int c, int row) -> unsigned {
    return (unsigned)(kRowB == 64 ? c ^ ((row >> 2) & 3)
                                  : (kNarrow ? c ^ ((row >> 1) & 7)
                                             : c ^ (row & 15)));
  };
  auto v_chunk = [](int c, int row) -> unsigned {
    return (unsigned)(kRowB == 64 ? c ^ (2 * ((row >> 2) & 1))
                      : (kFp8 ? c ^ ((row >> 1) & 7)
                              : (kNarrow ? c ^ (4 * ((row >> 1) & 1))
                                         : c ^ (4 * (row & 3)))));
  };
  const char* kbase = reinterpret_cast<const char*>(p.k);
  const char* vbase = reinterpret_cast<const char*>(p.v);
  // fast path: the wave's rows lie in one page (pages of >= kDmaRows tokens)
  const bool fast_pages = p.log2_page >= kLog2DmaRows;
  unsigned k_row_off[kOpsPerMat], v_row_off[kOpsPerMat];
#pragma unroll
  for (int k = 0; k < kOpsPerMat; ++k) {
    const int rw = kRowsPerOp * k + lrow;
    const int row = kDmaRows * dma_w + rw;  // row within the tile
    k_row_off[k] = rw * tok_bytes + (k_chunk(lchunk, row) << 4);
    v_row_off[k] = rw * tok_bytes + (v_chunk(lchunk, row) << 4);
  }
  // DMA of a full tile on the fast path (pages of >= kDmaRows tokens), in
  // pieces: the page lookup first, then part k (one K and one V
  // instruction), so that a step can spread its DMA between segments
  struct DmaPlan {
    const char* kb0;
    const char* vb0;
    unsigned st;
  };
  auto dma_plan = [&](int t) -> DmaPlan {
    const int w0 = kbeg + t * kKeyTile + kDmaRows * dma_w;
    const int pi = clampi((w0 >> p.log2_page) - lp0, 0, kPageCache - 1);
    const unsigned pgu = (unsigned)__builtin_amdgcn_readfirstlane(pg_lds[pi]);
    const size_t off = (size_t)pgu * page_bytes +
                       (unsigned)(w0 & pmask) * tok_bytes + g * kRowB;
    return DmaPlan{kbase + off, vbase + off,
                   ring_base + (unsigned)(t & (kStages - 1)) * kTileBytes};
  };
  auto dma_part = [&](const DmaPlan& dp, int k) {
    const unsigned dst = dp.st + (dma_w * kOpsPerMat + k) * 1024;
    if constexpr (kSplitOps) {
      if (dma_v) {
        dma16_sbase(dp.vb0, v_row_off[k], dst + kVOff);
      } else {
        dma16_sbase(dp.kb0, k_row_off[k], dst);
      }
    } else {
      dma16_sbase(dp.kb0, k_row_off[k], dst);
      dma16_sbase(dp.vb0, v_row_off[k], dst + kVOff);
    }
  };
  auto issue = [&](int t) {
    const int t0 = kbeg + t * kKeyTile;
    const unsigned st = ring_base + (unsigned)(t & (kStages - 1)) * kTileBytes;
    const int w0 = t0 + kDmaRows * dma_w;
    if (fast_pages && w0 + kDmaRows - 1 < kend) {
      const int pi = clampi((w0 >> p.log2_page) - lp0, 0, kPageCache - 1);
      const unsigned pgu =
          (unsigned)__builtin_amdgcn_readfirstlane(pg_lds[pi]);
      const size_t off = (size_t)pgu * page_bytes +
                         (unsigned)(w0 & pmask) * tok_bytes + g * kRowB;
#pragma unroll
      for (int k = 0; k < kOpsPerMat; ++k) {
        const unsigned dst = st + (dma_w * kOpsPerMat + k) * 1024;
        if constexpr (kSplitOps) {
          if (dma_v) {
            dma16_sbase(vbase + off, v_row_off[k], dst + kVOff);
          } else {
            dma16_sbase(kbase + off, k_row_off[k], dst);
          }
        } else {
          dma16_sbase(kbase + off, k_row_off[k], dst);
          dma16_sbase(vbase + off, v_row_off[k], dst + kVOff);
        }
      }
      return;
    }
    // The lane's row and chunk are derived again here from an opaque copy
    // of the lane id: otherwise the compiler keeps the per-lane 64-bit
    // source pointers of this path live across the whole loop, runs out of
    // registers and reloads them from scratch, and its wait for those
    // reloads also waits for every DMA in flight.
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int slrow = (int)((unsigned)ln / kRowChunks);
    const int slchunk = (int)((unsigned)ln % kRowChunks);
    int pg[kOpsPerMat], slot[kOpsPerMat];
#pragma unroll
    for (int k = 0; k < kOpsPerMat; ++k) {
      const int pos = min(w0 + kRowsPerOp * k + slrow, kend - 1);
      slot[k] = pos & pmask;
      pg[k] = pg_lds[clampi((pos >> p.log2_page) - lp0, 0, kPageCache - 1)];
    }
#pragma unroll
    for (int k = 0; k < kOpsPerMat; ++k) {
      const int row = kDmaRows * dma_w + kRowsPerOp * k + slrow;
      const size_t off = (size_t)(unsigned)pg[k] * page_bytes +
                         (unsigned)slot[k] * tok_bytes + g * kRowB;
      const unsigned dst = st + (dma_w * kOpsPerMat + k) * 1024;
      if constexpr (kSplitOps) {
        if (dma_v) {
          dma16(vbase + off + (v_chunk(slchunk, row) << 4), dst + kVOff);
        } else {
          dma16(kbase + off + (k_chunk(slchunk, row) << 4), dst);
        }
      } else {
        dma16(kbase + off + (k_chunk(slchunk, row) << 4), dst);
        dma16(vbase + off + (v_chunk(slchunk, row) << 4), dst + kVOff);
      }
    }
  };

  // ---- 64-bit allowed-key mask of tile t (first key t0) for this node
  auto tile_allow = [&](int t0, int nd) -> uint64_t {
    const int nvalid = kend - t0;
    const int npre = P - t0;
    uint64_t allow = nvalid >= 64 ? ~0ull : ((1ull << nvalid) - 1);
    const uint64_t pre =
        npre >= 64 ? ~0ull : (npre <= 0 ? 0ull : ((1ull << npre) - 1));
    uint64_t tree = 0;
    if (npre < 64) {
      const int mrow_lds = (nd - n_lo) * nwin - wlo;
      const int j0 = t0 - P;
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

  f32x16 o[QB][kDB];
  float l_run[QB];  // this lane half's share of the row sum
  float m_ref[QB];  // reference max, log2 units
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
    for (int db = 0; db < kDB; ++db) o[qb][db] = f32x16{};
    l_run[qb] = 0.f;
    m_ref[qb] = -INFINITY;
  }
  // fp8: the cached values stand for code * scale[g]; the K scale folds
  // into the score scale, the V scale into the output normalisation
  float c2 = p.scale_log2;
  float v_sc = 1.f;
  if constexpr (kFp8) {
    if (p.k_scale != nullptr) c2 *= p.k_scale[g];
    if (p.v_scale != nullptr) v_sc = p.v_scale[g];
  }

  // ---- LDS operand reads.  K fragments of key block kb, head-dim chunks
  // kc = 4h .. 4h+3; V^T fragments of key block kb, 16-key half hf.
  auto read_kq = [&](int t, int kb, int h, bf16x8 (&kf)[4]) {
    const unsigned so = (unsigned)(t & (kStages - 1)) * kTileBytes;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if constexpr (kFp8) {
        kf[c] = e4m3x8_to_bf16(lds_read8(k_off[4 * h + c] + so + kb * 32 * kRowB));
      } else {
        kf[c] = lds_read16(k_off[4 * h + c] + so + kb * 32 * kRowB);
      }
    }
  };
  auto read_vq = [&](int t, int kb, int hf, bf16x8 (&vf)[kDB]) {
    const unsigned so = (unsigned)(t & (kStages - 1)) * kTileBytes;
#pragma unroll
    for (int db = 0; db < kDB; ++db) {
      if constexpr (kFp8) {
        vf[db] = e4m3x8_to_bf16(
            lds_read_tr8(v_off[db] + so + (kb * 32 + hf * 16) * kRowB));
      } else {
        const unsigned va = v_off[db] + so + (kb * 32 + hf * 16) * kRowB;
        const s16x4 lo = lds_read_tr(va);
        const s16x4 hi = lds_read_tr(va + 8 * kRowB);
        vf[db] = __builtin_bit_cast(
            bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    }
  };
  // S^T of key block kb of tile t for every query block: QB accumulation
  // chains over the head dimension, K fragments a quarter tile at a time
  auto qk_block = [&](int t, int kb, f32x16 (&S)[QB][2]) {
    bf16x8 kf0[4], kf1[4];
    read_kq(t, kb, 0, kf0);
    if constexpr (kKSteps == 8) read_kq(t, kb, 1, kf1);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) S[qb][kb] = f32x16{};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        S[qb][kb] = mfma32x32x16(kf0[c], qf[qb][c], S[qb][kb]);
      }
    }
    if constexpr (kKSteps == 8) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          S[qb][kb] = mfma32x32x16(kf1[c], qf[qb][4 + c], S[qb][kb]);
        }
      }
    }
  };
  // O^T += V^T P^T over key block kb of tile t (kDB*QB accumulation chains)
  auto pv_block = [&](int t, int kb, const bf16x8 (&pf)[QB][2][2]) {
    bf16x8 vf0[kDB], vf1[kDB];
    read_vq(t, kb, 0, vf0);
    read_vq(t, kb, 1, vf1);
#pragma unroll
    for (int db = 0; db < kDB; ++db) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        o[qb][db] = mfma32x32x16(vf0[db], pf[qb][kb][0], o[qb][db]);
      }
    }
#pragma unroll
    for (int db = 0; db < kDB; ++db) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        o[qb][db] = mfma32x32x16(vf1[db], pf[qb][kb][1], o[qb][db]);
      }
    }
  };
  // probabilities of key block kb against m_ref; adds their fp32 sums
  auto exps_block = [&](const f32x16 (&S)[QB][2], int kb,
                        bf16x8 (&pf)[QB][2][2]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float mu = (m_ref[qb] == -INFINITY) ? 0.f : m_ref[qb];
      float e[16];
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        e[rr] = fast_exp2(fmaf(S[qb][kb][rr], c2, -mu));
      }
#pragma unroll
      for (int rr = 0; rr < 16; rr += 2) {
        pf[qb][kb][rr >> 3][rr & 7] = (__bf16)e[rr];
        pf[qb][kb][rr >> 3][(rr & 7) + 1] = (__bf16)e[rr + 1];
      }
      float t8[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) t8[k] = e[2 * k] + e[2 * k + 1];
      const float t4a = (t8[0] + t8[1]) + (t8[2] + t8[3]);
      const float t4b = (t8[4] + t8[5]) + (t8[6] + t8[7]);
      l_run[qb] += t4a + t4b;
    }
  };
  // reference max for a tile, raised only past the lazy-rescale margin;
  // pm0: this lane's max over key block 0, when found earlier (else
  // -inf and both blocks are scanned here)
  auto next_ref = [&](const f32x16 (&Sx)[QB][2], float (&m_new)[QB],
                      float (&alpha)[QB], const float (&pm0)[QB],
                      bool have_pm0) -> bool {
    bool any_need = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float tmax = __builtin_elementwise_maximum(
          have_pm0 ? pm0[qb] : max16(Sx[qb][0]), max16(Sx[qb][1]));
      tmax = __builtin_elementwise_maximum(tmax, other_half(tmax)) * c2;
      const bool need = tmax > m_ref[qb] + kLazyRescale;
      m_new[qb] = need ? tmax : m_ref[qb];
      alpha[qb] = need ? fast_exp2(m_ref[qb] - m_new[qb]) : 1.f;
      any_need |= need;
    }
    return any_need;
  };

  // ---- one pipeline step over tile j.  Tile j's scores Scur (masked, with
  // reference max m_ref) come from the previous step; this step computes
  // the scores of tile j+1 on the matrix core while the vector ALU turns
  // Scur into probabilities, then PV of tile j while the ALU finds tile
  // j+1's max.  The scores are built one 32-key block at a time, so that
  // only one and a half score tiles are live.  After the last tile the
  // scores are computed on stale LDS data and dropped.
  auto body = [&](int j, f32x16 (&Scur)[QB][2], f32x16 (&Snext)[QB][2],
                  bool mask_next, bool dma_inbody, float (&m_new)[QB],
                  float (&alpha)[QB]) -> bool {
    bf16x8 pf[QB][2][2];
    DmaPlan dp{};
    if (dma_inbody) dp = dma_plan(j + kStages - 1);
    // segment 1: S^T(j+1) keys 0..31 | probabilities of keys 0..31
    qk_block(j + 1, 0, Snext);
    exps_block(Scur, 0, pf);
    // the segments are scheduled separately: without these fences the
    // scheduler mixes them and the matrix core waits more (inside a
    // segment the compiler's own interleave beat explicit interleave
    // groups by 1-2% on the long-context workload)
    __builtin_amdgcn_sched_barrier(0);
    if (dma_inbody) {  // first half of tile j+3's DMA
#pragma unroll
      for (int k = 0; k < kOpsPerMat / 2; ++k) dma_part(dp, k);
      __builtin_amdgcn_sched_barrier(0);
    }
    // segment 2: S^T(j+1) keys 32..63, PV(j) keys 0..31 | probabilities
    // of keys 32..63 and (unmasked tiles) the max over keys 0..31 of
    // tile j+1, so that the step's tail scans only keys 32..63
    qk_block(j + 1, 1, Snext);
    pv_block(j, 0, pf);
    exps_block(Scur, 1, pf);
    float pm0[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      pm0[qb] = mask_next ? -INFINITY : max16(Snext[qb][0]);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (dma_inbody) {  // second half
#pragma unroll
      for (int k = kOpsPerMat / 2; k < kOpsPerMat; ++k) dma_part(dp, k);
      __builtin_amdgcn_sched_barrier(0);
    }
    // segment 3: PV(j) keys 32..63 | max of tile j+1
    pv_block(j, 1, pf);
    if (mask_next) {
      const int t1 = kbeg + (j + 1) * kKeyTile;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        apply_tile_mask(Snext[qb], tile_allow(t1, node[qb]), half);
      }
    }
    return next_ref(Snext, m_new, alpha, pm0, !mask_next);
  };
  auto finish = [&](bool r, const float (&m_new)[QB],
                    const float (&alpha)[QB]) {
    if (__any(r)) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        l_run[qb] *= alpha[qb];
#pragma unroll
        for (int db = 0; db < kDB; ++db) o[qb][db] *= alpha[qb];
      }
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) m_ref[qb] = m_new[qb];
  };
  auto step = [&](int j, f32x16 (&Scur)[QB][2], f32x16 (&Snext)[QB][2]) {
    if (j + 1 < n) {
      // tile j+1 must have landed; tile j+2 may still be in flight
      if (j + 2 < n) wait_vmcnt<kOps>();
      else wait_vmcnt<0>();
    }
    __syncthreads();
    if (j + kStages - 1 < n) issue(j + kStages - 1);
    float m_new[QB], alpha[QB];
    bool r;
    // (one copy of the body for masked and unmasked tiles: the tail runs
    // once per workgroup, so its code size, fetched cold into the
    // instruction cache, costs more than the branch)
    const bool mk = j + 1 < n && kbeg + (j + 2) * kKeyTile > min(P, kend);
    r = body(j, Scur, Snext, mk, false, m_new, alpha);
    if (j + 1 >= n) {  // the scores past the last tile are not data
      r = false;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) m_new[qb] = m_ref[qb];
    }
    finish(r, m_new, alpha);
  };
  // hot steps: tile j+1 pure prefix, tile j+3 a full tile on the fast path
  auto hot_step = [&](int j, f32x16 (&Scur)[QB][2], f32x16 (&Snext)[QB][2]) {
    wait_vmcnt<kOps>();
    __syncthreads();
    float m_new[QB], alpha[QB];
    const bool r = body(j, Scur, Snext, false, true, m_new, alpha);
    finish(r, m_new, alpha);
  };

  // Make the compiler wait for the Q loads before the first DMA (its own
  // wait at the first use of qf would also drain the ring).
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    if constexpr (kKSteps == 8) {
      asm volatile("" :: "v"(qf[qb][0]), "v"(qf[qb][1]), "v"(qf[qb][2]),
                   "v"(qf[qb][3]), "v"(qf[qb][4]), "v"(qf[qb][5]),
                   "v"(qf[qb][6]), "v"(qf[qb][7]));
    } else {
      asm volatile("" :: "v"(qf[qb][0]), "v"(qf[qb][1]), "v"(qf[qb][2]),
                   "v"(qf[qb][3]));
    }
  }
  __syncthreads();  // page slice and mask window visible
#pragma unroll
  for (int t = 0; t < kStages - 1; ++t) {
    if (t < n) issue(t);
  }
  if (n >= 3) wait_vmcnt<2 * kOps>();
  else if (n == 2) wait_vmcnt<kOps>();
  else wait_vmcnt<0>();
  __syncthreads();
  f32x16 SA[QB][2], SB[QB][2];
  qk_block(0, 0, SA);
  qk_block(0, 1, SA);
  if (kbeg + kKeyTile > min(P, kend)) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      apply_tile_mask(SA[qb], tile_allow(kbeg, node[qb]), half);
    }
  }
  {
    float m_new[QB], alpha[QB], pm0[QB];
    next_ref(SA, m_new, alpha, pm0, false);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) m_ref[qb] = m_new[qb];
  }
  int n_hot = 0;
  if (fast_pages) {
    const int last = min((kend - kbeg) / kKeyTile - kStages,
                         (P - kbeg) / kKeyTile - 2);
    n_hot = max(last + 1, 0) & ~(kStages - 1);
  }
  // both loops are unrolled by the ring depth and start at a multiple of
  // it, so that every stage offset is a constant
  for (int i = 0; 4 * i < n_hot; ++i) {
    const int j = 4 * i;
    hot_step(j, SA, SB);
    hot_step(j + 1, SB, SA);
    hot_step(j + 2, SA, SB);
    hot_step(j + 3, SB, SA);
  }
  // the remaining steps, two per iteration (the score registers swap
  // roles every step; stage offsets are computed, not unrolled)
  for (int j = n_hot; j < n; j += 2) {
    step(j, SA, SB);
    if (j + 1 < n) step(j + 1, SB, SA);
  }

  // ---- epilogue: the normalised output in bf16 (one split) or fp16 (a
  // split's partial), each wave's rows staged through its own 8 KB of the
  // ring so that the stores write whole rows
  __syncthreads();  // every wave is done with the ring
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l_tot = l_run[qb] + other_half(l_run[qb]);
    const float inv = l_tot > 0.f ? v_sc / l_tot : 0.f;
    const unsigned stg = ring_base + (unsigned)(wave * QB + qb) * 8192;
    u32x2 pk[4 * kDB];
    // whole rows of D two-byte values from pk (d = 8c + 4 half .. +3)
    auto store_rows = [&](int row, char* base, bool coherent) {
      if constexpr (D == 128) {
        store_rows_staged(pk, stg, row, base, lane, coherent);
      } else {
        store_half_rows_staged(pk, stg, row, 0, base, lane, coherent, 128);
      }
    };
    if (un.nsplit == 1) {
#pragma unroll
      for (int c = 0; c < 4 * kDB; ++c) {
        bf16x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v4[e] = (__bf16)(o[qb][c >> 2][(c & 3) * 4 + e] * inv);
        }
        pk[c] = __builtin_bit_cast(u32x2, v4);
      }
      store_rows(rvalid[qb] ? (int)qrow[qb] : -1,
                 reinterpret_cast<char*>(p.out), false);
      if (half == 0 && rvalid[qb]) {
        p.lse[qrow[qb]] =
            l_tot > 0.f ? (m_ref[qb] + log2f(l_tot)) * kLn2 : -INFINITY;
      }
    } else {
      // scale exponent of the partial row (f16_row_exp)
      float amax = 0.f;
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          amax = __builtin_elementwise_maximum(amax,
                                               __builtin_fabsf(o[qb][db][e]));
        }
      }
      const int ex = f16_row_exp(
          __builtin_elementwise_maximum(amax, other_half(amax)) * inv);
#pragma unroll
      for (int c = 0; c < 4 * kDB; ++c) {
        f16x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v4[e] = to_f16_sat(ldexp2(o[qb][c >> 2][(c & 3) * 4 + e] * inv, -ex));
        }
        pk[c] = __builtin_bit_cast(u32x2, v4);
      }
      // the unit's partial slot: its rows in row-block order
      const int rl = (wave * QB + qb) * 32 + col;
      const size_t prow0 = (size_t)L * kRowsPerWG8;
      store_rows(rvalid[qb] ? rl : -1,
                 reinterpret_cast<char*>(p.part_o + prow0 * D),
                 p.counters != nullptr);
      if (half == 0 && rvalid[qb]) {
        float* dst = p.part_ml + (prow0 + rl) * 2;
        const uint64_t st = pack_split_stats(split_lse2(m_ref[qb], l_tot), ex);
        if (p.counters != nullptr) {
          store_coherent8(dst, st);
        } else {
          *reinterpret_cast<uint64_t*>(dst) = st;
        }
      }
    }
  }
  if (p.counters != nullptr && un.nsplit > 1) {
    // (256 rows: one round of loads, two splits at a time)
    merge_if_last<kThreads, 8, D>(p, un, rows, r0, kRowsPerWG8, tid, pg_lds);
  }
}

}  // namespace tree_attn
