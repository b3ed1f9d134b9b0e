// Split-KV tree-verification attention kernel whose waves split every
// 64-key tile in two key halves: NW = 8 waves on 128 query rows, or NW = 4
// waves on 64 rows.
//
// Same operation, data layout, MFMA mapping, LDS ring format, DMA and mask
// handling as the 256-row kernel (definitions in attn_fwd.hpp).  Wave w
// owns query rows 32 (w % (NW/2)) .. +31 of the workgroup's rows and keys
// 32 (w / (NW/2)) .. +31 of each tile.  With NW = 8, waves w and w + 4
// share a SIMD, so every SIMD holds two waves and its vector ALU issues at
// the two-wave rate (about twice the one-wave rate, three times for the
// exponential), where four waves of 32 rows would leave one wave per SIMD.
// The 64-row shape (one wave per SIMD) serves bandwidth-bound launches in
// which 64-row blocks alone give every CU a workgroup: the key range then
// needs no split, so no partials are written or merged.  Each wave keeps
// its own online-softmax state (reference max, row sum, O) over its half
// of the keys; at the end the wave of the upper half hands its state to the
// lower-half wave of the same rows through LDS, which combines the two
// (m* = max(m0, m1), weights 2^(m_c - m*)) and writes the result.  Each
// wave reads half of the K and V tile for its 32 rows.
#pragma once

#include "attn_fwd.hpp"

namespace tree_attn {

constexpr int kRowsPerWG128 = 128;
constexpr int kRowsPerWG64 = 64;
// ring offset of the epilogue's row staging (past the halves' exchange:
// 8 KB of O, 512 B of statistics and 128 B of row maxima per wave)
constexpr int kEpilogueStage = 72 * 1024;

template <int NW, bool kBalanced, bool kFp8, int D = kHeadDim>
__global__ __launch_bounds__(NW * 64, 1) void attn_fwdh_kernel(FwdParams p) {
  static_assert(NW == 8 || NW == 4, "shape");
  static_assert(D == kHeadDim || D == 64, "head dim");
  constexpr int kRows = 16 * NW;         // query rows per workgroup
  constexpr int kThreads = NW * 64;
  constexpr int kEB = kFp8 ? 1 : 2;      // bytes per cached element
  constexpr int kRowB = D * kEB;         // bytes per cached (token, head)
  // 128-byte rows (fp8 with d = 128, bf16 with d = 64): 8 chunks of 16
  // bytes per row, 8 rows per DMA op
  constexpr bool kNarrow = kRowB == 128;
  constexpr int kRowChunks = kRowB / 16;  // 16-byte chunks per row
  // 1-KB DMA ops of a 64-row matrix tile; with fewer than one per wave
  // (64-byte rows of fp8 with d = 64 on 8 waves), each wave moves one op,
  // of K (waves 0-3) or of V
  constexpr int kMatOps = kRowChunks;
  constexpr bool kSplitOps = kMatOps < NW;
  constexpr int kKSteps = D / 16;        // MFMA k-steps over the head dim
  constexpr int kDB = D / 32;            // 32-wide head-dim blocks of O
  constexpr int kHalfDB = kDB / 2;       // the blocks a wave finishes
  // Q staging DMA ops per wave (bf16 rows of D values, 1 KB per op)
  constexpr int kQOps = kRows * D * 2 / 1024 / NW;
  // 1-KB DMA ops per wave per matrix: each moves 4 bf16 or 8 fp8 rows
  constexpr int kOpsPerMat = kSplitOps ? 1 : kMatOps / NW;
  constexpr int kOps = kSplitOps ? 1 : 2 * kOpsPerMat;
  constexpr int kRowsPerOp = 1024 / kRowB;
  constexpr int kDmaRows = kRowsPerOp * kOpsPerMat;  // tile rows a wave moves
  constexpr int kLog2DmaRows = kDmaRows == 8 ? 3 : 4;
  static_assert((1 << kLog2DmaRows) == kDmaRows, "shape");
  __shared__ __align__(1024) unsigned char ring[2 * kVOff];
  __shared__ int pg_lds[kPageCache];
  __shared__ uint64_t mk_lds[kMaskCache];

  // XCD-aware numbering (consecutive units on one XCD), then the unit
  const int bid = blockIdx.x;
  const int L = (bid & 7) * p.per_xcd + (bid >> 3);
  if (L >= p.plan.parts) return;
  Unit un = decode_unit<kBalanced>(p.plan, L);
  if (!un.valid) return;
  const int s = un.s, g = un.g, mb = un.mb, split = un.split;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rg = wave % (NW / 2);  // 32-row group
  const int kh = wave / (NW / 2);  // key half of every tile (32-key block)
  const int lane = tid & 63;
  const int col = lane & 31, half = lane >> 5;

  const unsigned ring_base =
      (unsigned)(size_t)(__attribute__((address_space(3))) unsigned char*)ring;
  const unsigned pg_base =
      (unsigned)(size_t)(__attribute__((address_space(3))) int*)pg_lds;
  const unsigned mk_base =
      (unsigned)(size_t)(__attribute__((address_space(3))) uint64_t*)mk_lds;
  const int lrow = lane >> 4, lchunk = lane & 15;  // Q rows, 16-B chunks
  // a lane's row and 16-byte chunk within one K/V DMA op
  const int drow = lane / kRowChunks, dchunk = lane % kRowChunks;
  // the wave's row group within the matrix tile it moves, and (64-byte
  // rows) whether that is V
  const int dma_w = kSplitOps ? wave % kMatOps : wave;
  const bool dma_v = kSplitOps && wave >= kMatOps;

  // Prologue, two rounds of memory latency before the first tile's scores:
  // (1) the split's page-table entries go to LDS by DMA while the tree
  // bounds load, and Q (staged in ring stage 3, which tile 3 only
  // overwrites after every wave has read it) follows as soon as the bounds
  // are in; (2) once the page-table entries are in, the ancestor-mask rows
  // and tiles 0-2 are issued behind Q, and the first scores wait for Q,
  // the mask rows and tile 0.
  const int kbeg = split * un.chunk;
  const int lp0 = kbeg >> p.log2_page;
  {
    const int npg_max = min(min(((un.chunk - 1) >> p.log2_page) + 2, kPageCache),
                            p.max_pps - lp0);
    const int* ptab = p.page_table + (size_t)s * p.max_pps + lp0;
    for (int i0 = wave * 64; i0 < npg_max; i0 += kThreads) {
      if (i0 + lane < npg_max) dma4(ptab + i0 + lane, pg_base + 4 * i0);
    }
  }

  load_bounds(p.plan, un);
  const int a = un.a, B = un.B, P = un.P, T = un.T;
  const int rows = p.G * B;
  const int r0 = mb * kRows;
  if (r0 >= rows || kbeg >= T) {
    wait_vmcnt<0>();  // no DMA into LDS outlives the workgroup
    return;
  }
  const int kend = min(T, kbeg + un.chunk);
  const int n = (kend - kbeg + kKeyTile - 1) / kKeyTile;  // tiles, >= 1

  // ancestor-mask rows of the workgroup's nodes, all W words (the window
  // of words the split needs starts at word 0)
  const int n_lo = r0 / p.G;
  const int n_hi = (min(r0 + kRows, rows) - 1) / p.G;
  const int nnodes = n_hi - n_lo + 1;
  const bool has_tree = kend > P;
  const int wlo = 0;
  const int nwin = p.W;
  const int nm = has_tree ? min(nnodes * nwin, kMaskCache) : 0;

  // ---- this lane's query row
  const int r = r0 + rg * 32 + col;
  const bool rvalid = r < rows;
  const int node = rvalid ? r / p.G : n_hi;
  const size_t qrow =
      (size_t)(a + node) * p.Hq + g * p.G + (rvalid ? r % p.G : 0);
  bf16x8 qf[kKSteps];  // Q^T fragments (B operand): d = kc*16 + half*8 + 0..7,
                 // read from LDS once the prologue DMA has landed

  // Q rows r0 .. r0+kRows-1 (rows past the last one repeat it), swizzled
  // like K.  d = 128: instruction i moves rows 4i .. 4i+3; rows 0-63 go to
  // the K half of stage 3, rows 64-127 to its V half.  d = 64 (128-byte
  // rows): instruction i moves rows 8i .. 8i+7, all in the K half.
  const unsigned q_lds = ring_base + 3 * kTileBytes;
#pragma unroll
  for (int k = 0; k < kQOps; ++k) {
    const int i = kQOps * wave + k;
    if constexpr (D == 128) {
      const int rl = 4 * i + lrow;
      const int rq = min(r0 + rl, rows - 1);
      const size_t qr = (size_t)(a + rq / p.G) * p.Hq + g * p.G + rq % p.G;
      dma16(reinterpret_cast<const char*>(p.q + qr * D) +
                ((lchunk ^ (rl & 15)) << 4),
            q_lds + (i < 16 ? 0u : (unsigned)kVOff) + ((4 * i) & 63) * 256);
    } else {
      const int rl = 8 * i + (lane >> 3);
      const int rq = min(r0 + rl, rows - 1);
      const size_t qr = (size_t)(a + rq / p.G) * p.Hq + g * p.G + rq % p.G;
      dma16(reinterpret_cast<const char*>(p.q + qr * D) +
                (((lane & 7) ^ ((rl >> 1) & 7)) << 4),
            q_lds + 8 * i * 128);
    }
  }
  // the page-table slice has landed (issued before Q's ops); Q may still
  // be in flight
  wait_vmcnt<kQOps>();
  __syncthreads();  // page slice visible
  if (nm > 0) {
    const int nd = 2 * nm;  // dwords
    const char* msrc =
        reinterpret_cast<const char*>(p.masks + (size_t)(a + n_lo) * p.W);
    for (int i0 = wave * 64; i0 < nd; i0 += kThreads) {
      if (i0 + lane < nd) dma4(msrc + 4 * (i0 + lane), mk_base + 4 * i0);
    }
  }

  // ---- LDS operand addresses of this wave's key half (stage 0)
  unsigned k_off[kKSteps];
#pragma unroll
  for (int kc = 0; kc < kKSteps; ++kc) {
    if constexpr (kFp8 && kRowB == 64) {
      // fp8 rows of 64 B (d = 64), chunk c stored at c ^ ((row >> 2) & 3);
      // the lane's 8 values are half of chunk kc
      const int row = kh * 32 + col;
      k_off[kc] = ring_base + row * 64 + ((kc ^ ((row >> 2) & 3)) << 4) +
                  half * 8;
    } else if constexpr (kFp8) {
      // fp8 rows of 128 B, 16-byte chunk c stored at c ^ ((row >> 1) & 7);
      // the lane's 8 values d = kc*16 + half*8 .. +7 are half of chunk kc
      const int row = kh * 32 + col;
      k_off[kc] = ring_base + row * 128 + ((kc ^ ((row >> 1) & 7)) << 4) +
                  half * 8;
    } else if constexpr (kNarrow) {
      // bf16 rows of 128 B (d = 64), the same swizzle; the lane's 8
      // values are chunk 2 kc + half
      const int row = kh * 32 + col;
      k_off[kc] = ring_base + row * 128 +
                  (((2 * kc + half) ^ ((row >> 1) & 7)) << 4);
    } else {
      k_off[kc] = ring_base + (kh * 32 + col) * 256 +
                  (((2 * kc + half) ^ (col & 15)) << 4);
    }
  }
  const int y = (lane & 15) >> 2;
  const int x = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  unsigned v_off[kDB];
#pragma unroll
  for (int db = 0; db < kDB; ++db) {
    if constexpr (kFp8) {
      // ds_read_b64_tr_b8: in each group of 16 lanes, lanes 2r and 2r+1
      // name bytes 0-7 and 8-15 of "row" r (r = 0..7), and lane i of the
      // group receives byte i of rows 0..7.  Row r is key 8*(r/4) + 4*half
      // + r%4 of the 16-key block (the order of the probabilities' k
      // index), the 16 bytes are columns db*32 + 16*((lane >> 4) & 1) ..
      const int j = lane & 15, r8 = j >> 1;
      const int row = kh * 32 + 8 * (r8 >> 2) + 4 * half + (r8 & 3);
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
      const int row = kh * 32 + 4 * half + y;
      v_off[db] = ring_base + kVOff + row * 128 +
                  (((4 * db + x) ^ (4 * ((row >> 1) & 1))) << 4) +
                  8 * (lane & 1);
    } else {
      v_off[db] = ring_base + kVOff + (kh * 32 + 4 * half + y) * 256 +
                  ((4 * (db ^ y) + x) << 4) + 8 * (lane & 1);
    }
  }

  // ---- DMA of one tile: wave w moves rows kDmaRows*w .. of K and of V
  const int pmask = (1 << p.log2_page) - 1;
  const unsigned tok_bytes = (unsigned)p.Hkv * kRowB;
  const unsigned page_bytes = tok_bytes << p.log2_page;
  const char* kbase = reinterpret_cast<const char*>(p.k);
  const char* vbase = reinterpret_cast<const char*>(p.v);
  const bool fast_pages = p.log2_page >= kLog2DmaRows;
  // page ids are clamped to the cache when used (the table is not checked)
  const unsigned pg_last = (unsigned)max(p.num_pages - 1, 0);
  // source chunk of the lane's 16 bytes (the LDS chunk is fixed by the
  // lane): 256-byte rows K chunk ^ (row & 15), V chunk ^ 4 (row & 3) (for
  // the 16-bit transposing reads); 128-byte rows K chunk ^ ((row >> 1) & 7),
  // V the same for fp8 and chunk ^ 4 ((row >> 1) & 1) for bf16; 64-byte
  // rows K chunk ^ ((row >> 2) & 3), V chunk ^ 2 ((row >> 2) & 1)
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
  unsigned k_row_off[kOpsPerMat], v_row_off[kOpsPerMat];
#pragma unroll
  for (int k = 0; k < kOpsPerMat; ++k) {
    const int rw = kRowsPerOp * k + drow;
    const int row = kDmaRows * dma_w + rw;  // row within the tile
    k_row_off[k] = rw * tok_bytes + (k_chunk(dchunk, row) << 4);
    v_row_off[k] = rw * tok_bytes + (v_chunk(dchunk, row) << 4);
  }
  struct DmaPlan {
    const char* kb0;
    const char* vb0;
    unsigned st;
  };
  auto dma_plan = [&](int t) -> DmaPlan {
    const int w0 = kbeg + t * kKeyTile + kDmaRows * dma_w;
    const int pi = clampi((w0 >> p.log2_page) - lp0, 0, kPageCache - 1);
    const unsigned pgu =
        min((unsigned)__builtin_amdgcn_readfirstlane(pg_lds[pi]), pg_last);
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
      const DmaPlan dp = dma_plan(t);
#pragma unroll
      for (int k = 0; k < kOpsPerMat; ++k) dma_part(dp, k);
      return;
    }
    int pg[kOpsPerMat], slot[kOpsPerMat];
#pragma unroll
    for (int k = 0; k < kOpsPerMat; ++k) {
      const int pos = min(w0 + kRowsPerOp * k + drow, kend - 1);
      slot[k] = pos & pmask;
      pg[k] = clampi(pg_lds[clampi((pos >> p.log2_page) - lp0, 0,
                                   kPageCache - 1)],
                     0, p.num_pages - 1);
    }
#pragma unroll
    for (int k = 0; k < kOpsPerMat; ++k) {
      const int row = kDmaRows * dma_w + kRowsPerOp * k + drow;
      const size_t off = (size_t)(unsigned)pg[k] * page_bytes +
                         (unsigned)slot[k] * tok_bytes + g * kRowB;
      const unsigned dst = st + (dma_w * kOpsPerMat + k) * 1024;
      if constexpr (kSplitOps) {
        if (dma_v) {
          dma16(vbase + off + (v_chunk(dchunk, row) << 4), dst + kVOff);
        } else {
          dma16(kbase + off + (k_chunk(dchunk, row) << 4), dst);
        }
      } else {
        dma16(kbase + off + (k_chunk(dchunk, row) << 4), dst);
        dma16(vbase + off + (v_chunk(dchunk, row) << 4), dst + kVOff);
      }
    }
  };

  // ---- allowed keys of this wave's half of tile t (first key t0), in the
  // bit order of a 32-key block: bit kk = key t0 + 32 kh + kk
  auto half_allow = [&](int t0) -> uint32_t {
    const int nvalid = kend - t0;
    const int npre = P - t0;
    uint64_t allow = nvalid >= 64 ? ~0ull : ((1ull << nvalid) - 1);
    const uint64_t pre =
        npre >= 64 ? ~0ull : (npre <= 0 ? 0ull : ((1ull << npre) - 1));
    uint64_t tree = 0;
    if (npre < 64) {
      const int mrow_lds = (node - n_lo) * nwin - wlo;
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
    return (uint32_t)((allow & (pre | tree)) >> (32 * kh));
  };
  auto apply_half_mask = [&](f32x16& S, uint32_t allow) {
    allow >>= 4 * half;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const int kk = 8 * (rr >> 2) + (rr & 3);
      if (!((allow >> kk) & 1u)) S[rr] = -INFINITY;
    }
  };

  f32x16 o[kDB];
  float l_run = 0.f;        // this lane half's share of the row sum
  float m_ref = -INFINITY;  // reference max, log2 units
#pragma unroll
  for (int db = 0; db < kDB; ++db) o[db] = f32x16{};
  // fp8: the cached values stand for code * scale[g]; the K scale folds
  // into the score scale, the V scale into the output normalisation
  float c2 = p.scale_log2;
  float v_sc = 1.f;
  if constexpr (kFp8) {
    if (p.k_scale != nullptr) c2 *= p.k_scale[g];
    if (p.v_scale != nullptr) v_sc = p.v_scale[g];
  }

  // ---- S^T of this wave's key half of tile t (one accumulation chain over
  // the head dimension; the other wave of the SIMD fills its latency)
  auto qk_half = [&](int t, f32x16& S) {
    const unsigned so = (unsigned)(t & (kStages - 1)) * kTileBytes;
    bf16x8 kf[kKSteps];
#pragma unroll
    for (int c = 0; c < kKSteps; ++c) {
      if constexpr (kFp8) {
        kf[c] = e4m3x8_to_bf16(lds_read8(k_off[c] + so));
      } else {
        kf[c] = lds_read16(k_off[c] + so);
      }
    }
    S = f32x16{};
#pragma unroll
    for (int c = 0; c < kKSteps; ++c) S = mfma32x32x16(kf[c], qf[c], S);
  };
  // O^T += V^T P^T over this wave's key half of tile t
  auto pv_half = [&](int t, const bf16x8 (&pf)[2]) {
    const unsigned so = (unsigned)(t & (kStages - 1)) * kTileBytes;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      bf16x8 vf[kDB];
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        if constexpr (kFp8) {
          vf[db] = e4m3x8_to_bf16(lds_read_tr8(v_off[db] + so + hf * 16 * kRowB));
        } else {
          const unsigned va = v_off[db] + so + hf * 16 * kRowB;
          const s16x4 lo = lds_read_tr(va);
          const s16x4 hi = lds_read_tr(va + 8 * kRowB);
          vf[db] = __builtin_bit_cast(
              bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
      }
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        o[db] = mfma32x32x16(vf[db], pf[hf], o[db]);
      }
    }
  };
  // probabilities against m_ref; adds their fp32 sum
  auto exps_half = [&](const f32x16& S, bf16x8 (&pf)[2]) {
    const float mu = (m_ref == -INFINITY) ? 0.f : m_ref;
    float e[16];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) e[rr] = fast_exp2(fmaf(S[rr], c2, -mu));
#pragma unroll
    for (int rr = 0; rr < 16; rr += 2) {
      pf[rr >> 3][rr & 7] = (__bf16)e[rr];
      pf[rr >> 3][(rr & 7) + 1] = (__bf16)e[rr + 1];
    }
    float t8[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) t8[k] = e[2 * k] + e[2 * k + 1];
    l_run += ((t8[0] + t8[1]) + (t8[2] + t8[3])) +
             ((t8[4] + t8[5]) + (t8[6] + t8[7]));
  };
  // reference max for the next half tile (lazy raise, as in the others)
  auto next_ref = [&](const f32x16& Sx, float& m_new, float& alpha) -> bool {
    float tmax = max16(Sx);
    tmax = __builtin_elementwise_maximum(tmax, other_half(tmax)) * c2;
    const bool need = tmax > m_ref + kLazyRescale;
    m_new = need ? tmax : m_ref;
    alpha = need ? fast_exp2(m_ref - m_new) : 1.f;
    return need;
  };

  // ---- one pipeline step over tile j (this wave's half of it): S^T of
  // the next half tile on the matrix core while the vector ALU turns the
  // current scores into probabilities, then PV of tile j while the ALU
  // finds the next half tile's max.  The instruction order inside a step
  // is left to the compiler: with two waves per SIMD, explicit interleave
  // groups and scheduling fences (as the 256-row kernel uses) made this
  // kernel 2-3% slower.  After the last tile the scores are computed on
  // stale LDS data and dropped.
  auto body = [&](int j, f32x16& Scur, f32x16& Snext, bool mask_next,
                  bool dma_inbody, float& m_new, float& alpha) -> bool {
    bf16x8 pf[2];
    DmaPlan dp{};
    if (dma_inbody) dp = dma_plan(j + kStages - 1);
    // S^T(j+1) on the matrix core | probabilities of tile j
    qk_half(j + 1, Snext);
    exps_half(Scur, pf);
    if (dma_inbody) {  // first half of tile j+3's DMA
#pragma unroll
      for (int k = 0; k < kOpsPerMat / 2; ++k) dma_part(dp, k);
    }
    // PV(j) | mask and max of tile j+1
    pv_half(j, pf);
    if (mask_next) {
      apply_half_mask(Snext, half_allow(kbeg + (j + 1) * kKeyTile));
    }
    const bool need = next_ref(Snext, m_new, alpha);
    if (dma_inbody) {  // second half
#pragma unroll
      for (int k = kOpsPerMat / 2; k < kOpsPerMat; ++k) dma_part(dp, k);
    }
    return need;
  };
  auto finish = [&](bool r, float m_new, float alpha) {
    if (__any(r)) {
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < kDB; ++db) o[db] *= alpha;
    }
    m_ref = m_new;
  };
  auto step = [&](int j, f32x16& Scur, f32x16& Snext) {
    if (j + 1 < n) {
      // tile j+1 must have landed; tile j+2 may still be in flight
      if (j + 2 < n) wait_vmcnt<kOps>();
      else wait_vmcnt<0>();
    }
    __syncthreads();
    if (j + kStages - 1 < n) issue(j + kStages - 1);
    float m_new, alpha;
    bool r;
    // (one copy of the body for masked and unmasked tiles: the tail runs
    // once per workgroup, so its code size, fetched cold into the
    // instruction cache, costs more than the branch)
    const bool mk = j + 1 < n && kbeg + (j + 2) * kKeyTile > min(P, kend);
    r = body(j, Scur, Snext, mk, false, m_new, alpha);
    if (j + 1 >= n) {  // the scores past the last tile are not data
      r = false;
      m_new = m_ref;
    }
    finish(r, m_new, alpha);
  };
  // hot steps: tile j+1 pure prefix, tile j+3 a full tile on the fast path
  auto hot_step = [&](int j, f32x16& Scur, f32x16& Snext) {
    wait_vmcnt<kOps>();
    __syncthreads();
    float m_new, alpha;
    const bool r = body(j, Scur, Snext, false, true, m_new, alpha);
    finish(r, m_new, alpha);
  };

#pragma unroll
  for (int t = 0; t < kStages - 1; ++t) {
    if (t < n) issue(t);
  }
  // Q, the mask rows and tile 0 have landed; tiles 1-2 may be in flight
  if (n >= 3) wait_vmcnt<2 * kOps>();
  else if (n == 2) wait_vmcnt<kOps>();
  else wait_vmcnt<0>();
  __syncthreads();
  {
    const int rl = rg * 32 + col;
    if constexpr (D == 128) {
      const unsigned qa =
          q_lds + (rg < 2 ? 0u : (unsigned)kVOff) + (rl & 63) * 256;
#pragma unroll
      for (int kc = 0; kc < kKSteps; ++kc) {
        qf[kc] = lds_read16(qa + (((2 * kc + half) ^ (col & 15)) << 4));
      }
    } else {
      const unsigned qa = q_lds + rl * 128;
#pragma unroll
      for (int kc = 0; kc < kKSteps; ++kc) {
        qf[kc] = lds_read16(qa + (((2 * kc + half) ^ ((rl >> 1) & 7)) << 4));
      }
    }
  }
  f32x16 SA, SB;
  qk_half(0, SA);
  if (kbeg + kKeyTile > min(P, kend)) apply_half_mask(SA, half_allow(kbeg));
  {
    float m_new, alpha;
    next_ref(SA, m_new, alpha);
    m_ref = m_new;
  }
  int n_hot = 0;
  if (fast_pages) {
    const int last = min((kend - kbeg) / kKeyTile - kStages,
                         (P - kbeg) / kKeyTile - 2);
    n_hot = max(last + 1, 0) & ~(kStages - 1);
  }
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

  // ---- combine the two key halves.  Wave (rg, kh) finishes head-dim half
  // kh (O^T blocks kh kHalfDB .. +kHalfDB-1) of its 32 rows: it hands the
  // other blocks and its (max, row sum) to the partner wave (rg, 1 - kh)
  // through LDS and takes the partner's share of its own, so both waves of
  // a row group do half of the epilogue.
  float l_tot = l_run + other_half(l_run);
  // (selected by a wave-uniform branch: indexing o[] by kh would put the
  // array in scratch memory)
  f32x16 o_own[kHalfDB], o_give[kHalfDB];
  if (kh == 0) {
#pragma unroll
    for (int b = 0; b < kHalfDB; ++b) {
      o_own[b] = o[b];
      o_give[b] = o[kHalfDB + b];
    }
  } else {
#pragma unroll
    for (int b = 0; b < kHalfDB; ++b) {
      o_own[b] = o[kHalfDB + b];
      o_give[b] = o[b];
    }
  }
  __syncthreads();  // every wave is done with the ring
  {
    float* xo_out = reinterpret_cast<float*>(ring) + wave * (8 * 64 * 4);
    float* xml_out = reinterpret_cast<float*>(ring) + NW * (8 * 64 * 4) +
                     wave * 128;
#pragma unroll
    for (int b = 0; b < kHalfDB; ++b) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        *reinterpret_cast<f32x4*>(xo_out + ((b * 4 + g4) * 64 + lane) * 4) =
            f32x4{o_give[b][g4 * 4 + 0], o_give[b][g4 * 4 + 1],
                  o_give[b][g4 * 4 + 2], o_give[b][g4 * 4 + 3]};
      }
    }
    xml_out[lane] = m_ref;
    xml_out[64 + lane] = l_tot;
  }
  __syncthreads();
  const int partner = wave ^ (NW / 2);
  const float* xo_in = reinterpret_cast<const float*>(ring) +
                       partner * (8 * 64 * 4);
  const float* xml_in = reinterpret_cast<const float*>(ring) +
                        NW * (8 * 64 * 4) + partner * 128;
  // both waves form the combined statistics from the same operands in the
  // same order (key half 0 first), so they agree bit for bit
  const float m_p = xml_in[lane], l_p = xml_in[64 + lane];
  const float m0 = kh == 0 ? m_ref : m_p, m1 = kh == 0 ? m_p : m_ref;
  const float l0 = kh == 0 ? l_tot : l_p, l1 = kh == 0 ? l_p : l_tot;
  const float mx = __builtin_elementwise_maximum(m0, m1);
  const float a0 = mx == -INFINITY ? 0.f : fast_exp2(m0 - mx);
  const float a1 = mx == -INFINITY ? 0.f : fast_exp2(m1 - mx);
  const float a_own = kh == 0 ? a0 : a1, a_p = kh == 0 ? a1 : a0;
  f32x16 oc[kHalfDB];
#pragma unroll
  for (int b = 0; b < kHalfDB; ++b) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const f32x4 u =
          *reinterpret_cast<const f32x4*>(xo_in + ((b * 4 + g4) * 64 + lane) * 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        oc[b][g4 * 4 + e] = o_own[b][g4 * 4 + e] * a_own + u[e] * a_p;
      }
    }
  }
  l_tot = l0 * a0 + l1 * a1;
  m_ref = mx;

  // ---- epilogue: this wave's half of each of its rows, the normalised
  // output in bf16 (one split) or, for a split's partial, in fp16 scaled by
  // 2^-ex (the row's scale exponent, from the whole row's largest value:
  // the two waves exchange their halves' maxima), staged through LDS past
  // the exchange area so that the stores write whole half rows
  const float inv = l_tot > 0.f ? v_sc / l_tot : 0.f;
  const unsigned stg = ring_base + kEpilogueStage + wave * 4096;
  u32x2 pk[4 * kHalfDB];
  // this wave's half of each row (d = D/2 kh + 8c + 4 half .. +3 from pk)
  auto store_half = [&](int row, char* base, bool coherent) {
    if constexpr (D == 128) {
      store_half_rows_staged(pk, stg, row, kh, base, lane, coherent);
    } else {
      store_seg_rows_staged<4>(pk, stg, row, base + kh * 64, D * 2, lane,
                               coherent);
    }
  };
  if (un.nsplit == 1) {
#pragma unroll
    for (int c = 0; c < 4 * kHalfDB; ++c) {
      bf16x4 v4;
#pragma unroll
      for (int e = 0; e < 4; ++e) v4[e] = (__bf16)(oc[c >> 2][(c & 3) * 4 + e] * inv);
      pk[c] = __builtin_bit_cast(u32x2, v4);
    }
    store_half(rvalid ? (int)qrow : -1, reinterpret_cast<char*>(p.out), false);
    if (kh == 0 && half == 0 && rvalid) {
      p.lse[qrow] = l_tot > 0.f ? (m_ref + log2f(l_tot)) * kLn2 : -INFINITY;
    }
  } else {
    float amax = 0.f;
#pragma unroll
    for (int b = 0; b < kHalfDB; ++b) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        amax = __builtin_elementwise_maximum(amax, __builtin_fabsf(oc[b][e]));
      }
    }
    amax = __builtin_elementwise_maximum(amax, other_half(amax));
    float* xam = reinterpret_cast<float*>(ring) + NW * (8 * 64 * 4 + 128);
    if (half == 0) xam[wave * 32 + col] = amax;
    __syncthreads();
    amax = __builtin_elementwise_maximum(amax, xam[partner * 32 + col]);
    const int ex = f16_row_exp(amax * inv);
#pragma unroll
    for (int c = 0; c < 4 * kHalfDB; ++c) {
      f16x4 v4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v4[e] = to_f16_sat(ldexp2(oc[c >> 2][(c & 3) * 4 + e] * inv, -ex));
      }
      pk[c] = __builtin_bit_cast(u32x2, v4);
    }
    // the unit's partial slot: its rows in row-block order
    const size_t prow0 = (size_t)L * kRows;
    store_half(rvalid ? r - r0 : -1,
               reinterpret_cast<char*>(p.part_o + prow0 * D),
               p.counters != nullptr);
    if (kh == 0 && half == 0 && rvalid) {
      float* dst = p.part_ml + (prow0 + (r - r0)) * 2;
      const uint64_t st = pack_split_stats(split_lse2(m_ref, l_tot), ex);
      if (p.counters != nullptr) {
        store_coherent8(dst, st);
      } else {
        *reinterpret_cast<uint64_t*>(dst) = st;
      }
    }
  }
  if (p.counters != nullptr && un.nsplit > 1) {
    merge_if_last<kThreads, 4, D>(p, un, rows, r0, kRows, tid, pg_lds);
  }
}

}  // namespace tree_attn
