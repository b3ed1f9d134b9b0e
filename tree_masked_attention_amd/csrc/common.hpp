// Shared device-side definitions for the tree-attention kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tree_attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));

constexpr float kF16Max = 65504.f;

// fp32 -> fp16 (round to nearest even), saturated to the finite range.
__device__ __forceinline__ _Float16 to_f16_sat(float x) {
  return (_Float16)__builtin_elementwise_min(
      __builtin_elementwise_max(x, -kF16Max), kF16Max);
}

// Split partials travel in fp16 with a power-of-two scale per row: the
// exponent e >= 0 such that 2^-e * amax < 2^15 for the row's largest
// magnitude amax (e = 0 whenever amax < 2^15).  Scaling by a power of two
// is exact, so a partial keeps fp16's 11-bit precision relative to its row
// maximum over the whole bf16 range; the merge multiplies the weight of
// the partial by 2^e.
__device__ __forceinline__ int f16_row_exp(float amax) {
  const int e = __builtin_amdgcn_frexp_expf(amax) - 15;
  return e > 0 ? e : 0;
}

__device__ __forceinline__ float ldexp2(float x, int e) {
  return __builtin_amdgcn_ldexpf(x, e);
}

constexpr int kHeadDim = 128;
constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.442695040888963407f;

__device__ __forceinline__ int clampi(int x, int lo, int hi) {
  return x < lo ? lo : (x > hi ? hi : x);
}

// Device-coherent 8-byte store and load (relaxed atomics at agent scope:
// the sc1 bit, so the data bypass this XCD's L2, whose lines other XCDs do
// not see).  Used for data that another workgroup of the same launch reads
// after an arrival counter says it is complete; no cache-wide writeback or
// invalidate is needed for it.
__device__ __forceinline__ void store_coherent8(void* p, uint64_t v) {
  __hip_atomic_store(static_cast<uint64_t*>(p), v, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t load_coherent8(const void* p) {
  return __hip_atomic_load(static_cast<uint64_t*>(const_cast<void*>(p)),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// 2^x on the hardware exponential unit (exact 0 for -inf).
__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);
}

// Value of the other lane half (lane ^ 32).
__device__ __forceinline__ float other_half(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  // r[0]: lanes 32..63 now hold lanes 0..31; r[1]: lanes 0..31 hold 32..63
  return __builtin_bit_cast(float, __lane_id() < 32 ? r[1] : r[0]);
}

// Two E4M3 codes (bytes 2 kHi, 2 kHi + 1 of w) -> two bf16 in one word,
// by the direct conversion v_cvt_scalef32_pk_bf16_fp8 with scale 1.  Every
// E4M3 value is a bf16 value, so the conversion is exact; on gfx950 it
// gives the bits of v_cvt_pk_f32_fp8 followed by a truncation to bf16 for
// all 256 codes in every byte position (NaN codes included), and that
// instruction decodes OCP E4M3 (both checked on the device against the
// format's definition).
template <bool kHi>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(
      uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, kHi));
}

// D = A(32x16) * B(16x32) + C on the bf16 matrix cores, fp32 accumulate.
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

}  // namespace tree_attn
