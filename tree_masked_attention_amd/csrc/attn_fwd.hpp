// Shared definitions of the split-KV tree-verification attention kernels on
// the gfx950 bf16 matrix cores (attn_fwd128h.hpp: 128 or 64 query rows per
// workgroup; attn_fwd8.hpp: 256 rows), for bf16 or fp8 (E4M3) K/V tiles.
//
// The kernels compute, for every query row (node i, q head h) of a
// sequence, softmax attention over the prefix keys plus the tree keys
// allowed by node i's ancestor bitmask (tree-causal mask of JETFLOW,
// gist.science 2606.18394, section 2 "Arquitectura Central"), over a paged
// KV cache (section 3, item 3 names a paged kernel with the tree mask
// staged on chip).
//
// Work decomposition.  The rows of one (sequence s, kv head g) pair are the
// G query heads of the group times the B_s nodes, packed node-major
// (row = i * G + h_in_group), so each K/V tile staged in LDS serves all G
// heads of the group.  A workgroup owns a block of rows and one split of
// the key range [0, P_s + B_s).  The tree keys are the last B_s positions
// of that range, so the split that reaches them applies the bitmask on its
// tail tiles (the tree-block pass).  With one split a kernel writes the
// normalised output and the LSE; otherwise it writes partials: the split's
// output normalised by its own row sum, in fp16 (a convex combination of V
// rows, so within V's range), and the running max and row sum in fp32.
// The partials are merged either by the merge kernel (a launch of its own)
// or, when the launch is given arrival counters, by the last of a row
// block's split workgroups to finish (merge_if_last below).
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
// global_load_lds_dwordx4: the load unit writes each lane's 16 bytes
// straight to LDS (lane l of an instruction lands at M0 + 16*l), so no
// registers stage the data.  The loads are issued from inline assembly and
// waited for with explicit vmcnt counts, because the compiler would
// otherwise drain every such load before each barrier and the ring would
// never hold more than one tile in flight.  Tile j+3 is issued while tile j
// is consumed.  Rows are stored unpadded with an XOR swizzle of their
// 16-byte chunks (K: chunk ^ (row & 15); V: chunk ^ 4*(row & 3)) so that
// the MFMA operand reads hit distinct LDS banks.  The split's page-table
// slice and the ancestor-mask words its tree keys need are copied to LDS
// before the ring starts, so the loop issues no other global loads.
//
// FP8 tiles (E4M3 codes, 128-byte rows): the same ring and DMA ops, each
// moving 8 rows instead of 4, with 16-byte chunk c of row r stored at
// c ^ ((r >> 1) & 7).  Each wave converts its operands to bf16 as it reads
// them (exact: every E4M3 value is a bf16 value): K by ds_read_b64 of the
// lane's 8 codes, V^T by the byte-transposing ds_read_b64_tr_b8 of the 8
// keys of its register run pair.  The K scale folds into the softmax
// scale, the V scale into the output normalisation.
//
// Softmax runs in base 2 with scale*log2(e) folded into the FMA that
// subtracts the running max; the running max is only raised when a tile's
// max exceeds it by more than 8 (log2 units), which bounds the
// probabilities by 2^8 and skips most O rescales.  The row sum accumulates
// the fp32 probabilities (before their rounding to bf16 for the PV
// product).
#pragma once

#include "attn_merge.hpp"
#include "common.hpp"
#include "split_plan.hpp"

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
  _Float16* part_o;  // [units][rows per workgroup][head dim] partials
  float* part_ml;    // [units][rows per workgroup][2] split statistics
  const float* k_scale;  // fp8 K/V: [Hkv] scale of the cached codes, or
  const float* v_scale;  // null (1); unused for bf16
  unsigned* counters;  // one arrival count per (sequence, kv head, row
                       // block), or null: the merge kernel merges
  int max_pps, num_pages, log2_page, W;
  int max_tokens;  // min(max_pps * page_size, 2^30)
  int S, N, Hq, Hkv, G;
  int per_xcd;     // units handled per XCD slot column of the grid
  SplitParams plan;  // the work units (split_plan.hpp)
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

typedef __attribute__((address_space(3))) u32x2 lds_u32x2;

__device__ __forceinline__ void lds_write8(unsigned addr, u32x2 v) {
  *(lds_u32x2*)(size_t)addr = v;
}

// Stores a wave's 32 rows of 128 two-byte values, held transposed in
// registers (lane (col, half): row col; pk[c] = columns 8c + 4 half .. +3),
// as whole 16-byte row chunks: the rows go to the wave's own 8 KB of LDS at
// stg (16-byte chunks XOR-swizzled by row), then each lane stores 16 bytes,
// four full 256-byte rows per instruction.  row: the global row index of
// this lane's row (rows of 256 bytes from base), or -1 for a row that is
// not written.  Uses only the calling wave's data: no barrier.  coherent:
// device-coherent stores, for partials that another workgroup of the same
// launch merges (merge_if_last waits for them before counting in).
__device__ __forceinline__ void store_rows_staged(const u32x2 (&pk)[16],
                                                  unsigned stg, int row,
                                                  char* base, int lane,
                                                  bool coherent = false) {
  const int col = lane & 31, half = lane >> 5;
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    lds_write8(stg + col * 256 + ((c ^ (col & 15)) << 4) + half * 8, pk[c]);
  }
  asm volatile("" ::: "memory");
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int rr = 4 * k + (lane >> 4), ch = lane & 15;
    const u32x4 v = *(const lds_u32x4*)(size_t)(stg + rr * 256 +
                                                ((ch ^ (rr & 15)) << 4));
    const int dr = __shfl(row, rr);
    if (dr >= 0) {
      char* dst = base + (size_t)dr * 256 + ch * 16;
      if (coherent) {
        // device-coherent (sc1) 16-byte store; the compiler does not track
        // it; merge_if_last_rows waits for it (vmcnt 0) before counting in
        asm volatile("global_store_dwordx4 %0, %1, off sc1"
                     :: "v"(dst), "v"(v) : "memory");
      } else {
        *reinterpret_cast<u32x4*>(dst) = v;
      }
    }
  }
}

// Same for 64 two-byte values per row: the wave's 32 rows (pk[c] =
// columns 8c + 4 half .. +3 of the 64), staged at stg (4 KB) and stored as
// 128-byte segments at byte offset 128 * hh of rows row_bytes apart (half
// rows of 256-byte rows, or whole rows of 64 values), 8 rows per
// instruction.
__device__ __forceinline__ void store_half_rows_staged(const u32x2 (&pk)[8],
                                                       unsigned stg, int row,
                                                       int hh, char* base,
                                                       int lane,
                                                       bool coherent = false,
                                                       int row_bytes = 256) {
  const int col = lane & 31, half = lane >> 5;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    lds_write8(stg + col * 128 + ((c ^ (col & 7)) << 4) + half * 8, pk[c]);
  }
  asm volatile("" ::: "memory");
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int rr = 8 * k + (lane >> 3), ch = lane & 7;
    const u32x4 v = *(const lds_u32x4*)(size_t)(stg + rr * 128 +
                                                ((ch ^ (rr & 7)) << 4));
    const int dr = __shfl(row, rr);
    if (dr >= 0) {
      char* dst = base + (size_t)dr * row_bytes + hh * 128 + ch * 16;
      if (coherent) {
        asm volatile("global_store_dwordx4 %0, %1, off sc1"
                     :: "v"(dst), "v"(v) : "memory");
      } else {
        *reinterpret_cast<u32x4*>(dst) = v;
      }
    }
  }
}

// Same for a wave's 32 rows of NC * 8 two-byte values (pk[c] = columns
// 8c + 4 half .. +3), staged at stg (NC * 512 bytes) and stored as
// NC * 16-byte segments at base + row * row_bytes, 64 / NC rows per
// instruction.
template <int NC>
__device__ __forceinline__ void store_seg_rows_staged(const u32x2 (&pk)[NC],
                                                      unsigned stg, int row,
                                                      char* base,
                                                      int row_bytes, int lane,
                                                      bool coherent) {
  static_assert(NC == 2 || NC == 4 || NC == 8 || NC == 16, "segment");
  constexpr int RPI = 64 / NC;  // rows per instruction
  const int col = lane & 31, half = lane >> 5;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    lds_write8(stg + col * (NC * 16) + ((c ^ (col & (NC - 1))) << 4) +
                   half * 8,
               pk[c]);
  }
  asm volatile("" ::: "memory");
#pragma unroll
  for (int k = 0; k < 32 / RPI; ++k) {
    const int rr = RPI * k + lane / NC, ch = lane % NC;
    const u32x4 v = *(const lds_u32x4*)(size_t)(stg + rr * (NC * 16) +
                                                ((ch ^ (rr & (NC - 1))) << 4));
    const int dr = __shfl(row, rr);
    if (dr >= 0) {
      char* dst = base + (size_t)dr * row_bytes + ch * 16;
      if (coherent) {
        asm volatile("global_store_dwordx4 %0, %1, off sc1"
                     :: "v"(dst), "v"(v) : "memory");
      } else {
        *reinterpret_cast<u32x4*>(dst) = v;
      }
    }
  }
}

// Transposing LDS read (see the file comment).
__device__ __forceinline__ s16x4 lds_read_tr(unsigned addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(size_t)addr);
}

__device__ __forceinline__ u32x2 lds_read8(unsigned addr) {
  return *(const lds_u32x2*)(size_t)addr;
}

// Transposing LDS read of bytes (ds_read_b64_tr_b8): in each group of 16
// lanes, lanes 2r and 2r+1 address bytes 0-7 and 8-15 of row r (r = 0..7)
// and lane i of the group receives byte i of rows 0..7, in row order.
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
__device__ __forceinline__ u32x2 lds_read_tr8(unsigned addr) {
  return __builtin_bit_cast(
      u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(size_t)addr));
}

// Eight E4M3 codes (byte i of w = element i) -> eight bf16, exactly.
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(u32x2 w) {
  u32x4 r;
  r[0] = e4m3x2_to_bf16x2<false>(w[0]);
  r[1] = e4m3x2_to_bf16x2<true>(w[0]);
  r[2] = e4m3x2_to_bf16x2<false>(w[1]);
  r[3] = e4m3x2_to_bf16x2<true>(w[1]);
  return __builtin_bit_cast(bf16x8, r);
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

// 4 bytes per lane from global memory to LDS at lds_base + 4 * lane.
__device__ __forceinline__ void dma4(const void* gptr, unsigned lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off"
               :: "s"(lds_base), "v"(gptr) : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// Max of a lane's 16 scores of one 32-key block, as a tree of three-way
// maxima (three dependent steps instead of eight).
__device__ __forceinline__ float max16(const f32x16& v) {
  auto mx3 = [](float a, float b, float c) {
    return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b),
                                         c);
  };
  const float a = mx3(v[0], v[1], v[2]), b = mx3(v[3], v[4], v[5]);
  const float c = mx3(v[6], v[7], v[8]), d = mx3(v[9], v[10], v[11]);
  const float e = mx3(v[12], v[13], v[14]);
  return __builtin_elementwise_maximum(mx3(a, b, c), mx3(d, e, v[15]));
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

// Epilogue of a split workgroup of a launch that merges its own partials
// (merge_if_last_rows): unit un, rows [r0, r0 + rows_per_wg) of its pair;
// RT rows per thread in the merge's rounds of loads.
template <int NT, int RT = 4, int D = kHeadDim>
__device__ __forceinline__ void merge_if_last(const FwdParams& p,
                                              const Unit& un, int rows,
                                              int r0, int rows_per_wg,
                                              int tid, int* flag_lds) {
  merge_if_last_rows<NT, D, RT>(
      p.counters + un.seg, un.nsplit, p.part_o, p.part_ml, p.out, p.lse,
      p.Hq, p.G, un.g, un.a, r0, min(r0 + rows_per_wg, rows),
      PartSlots{un.slot0, un.mblocks, rows_per_wg, r0}, tid, flag_lds);
}

}  // namespace tree_attn
