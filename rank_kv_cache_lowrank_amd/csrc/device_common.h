// Device helpers shared by the decode and append kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lr {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(unsigned)))) unsigned u32x2;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kGroup = 32;        // int4 quantisation group along the rank
constexpr int kGroupBytes = 16;   // packed bytes per group

#define LR_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// ---- s_waitcnt helpers (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4]<<14)
#define LR_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14))
#define LR_WAIT_LGKM0() __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14))

// Wait until at most n vector-memory instructions of this wave are outstanding (n in 0..63).
__device__ __forceinline__ void wait_vmcnt(int n) {
#define LR_C4(b) case b: LR_WAIT_VM(b); break; case b + 1: LR_WAIT_VM(b + 1); break; \
                 case b + 2: LR_WAIT_VM(b + 2); break; case b + 3: LR_WAIT_VM(b + 3); break;
  switch (n) {
    LR_C4(0) LR_C4(4) LR_C4(8) LR_C4(12) LR_C4(16) LR_C4(20) LR_C4(24) LR_C4(28)
    LR_C4(32) LR_C4(36) LR_C4(40) LR_C4(44) LR_C4(48) LR_C4(52) LR_C4(56) LR_C4(60)
    default: LR_WAIT_VM(0); break;
  }
#undef LR_C4
}

// Workgroup barrier that orders LDS traffic only: this wave's LDS writes complete, then all
// waves meet. (No global-memory fence: outstanding direct-to-LDS loads are waited for with
// wait_vmcnt by the code that owns them.)
__device__ __forceinline__ void barrier_lds() {
  asm volatile("" ::: "memory");
  LR_WAIT_LGKM0();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// 16 bytes per lane from global memory straight into LDS: lane l writes lds_base + 16*l.
// The latents are read once per decode step, so the loads carry the nontemporal hint (cache
// policy bit NT); measured on MI355X this raises a streaming ring from ~5.7 to ~7 TB/s.
constexpr int kCachePolicyNT = 2;
__device__ __forceinline__ void dma16(const void* g, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, LR_LDS(lds_wave_base), 16, 0, kCachePolicyNT);
}

// Value operand through the gfx950 transpose read: within each 16-lane group g, lane j's element
// e comes from the address given by lane 16g + 4e + j/4, at element offset j%4. Lane
// 16g + 4e + q therefore points at row 4g+e, column 4q of the 16-column block, and every lane j
// receives column j of rows 4g .. 4g+3: the A operand of the 16x16x16 product with K = token.
__device__ __forceinline__ bf16x4 v_operand_tr(const unsigned char* p) {
  return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                        (__attribute__((address_space(3))) s16x4*)(p)));
}

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }  // RNE

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Reductions across the 4 lane groups (lanes l, l^16, l^32, l^48). gfx950's permlane swaps
// return, for every lane, the pair {own value, value of lane l^16} (resp. l^32) without an LDS
// round trip; the order inside the pair differs between lanes, the max / sum does not.
// The second operand passes through an empty asm so that the compiler cannot treat the two
// results of a swap of a value with itself as equal (it would fold the pair to one element).
__device__ __forceinline__ void swap_pair16(float v, float& a, float& b) {
  unsigned x = __builtin_bit_cast(unsigned, v), y = x;
  asm volatile("" : "+v"(y));
  auto p = __builtin_amdgcn_permlane16_swap(x, y, false, false);
  a = __builtin_bit_cast(float, (unsigned)p[0]);
  b = __builtin_bit_cast(float, (unsigned)p[1]);
}
__device__ __forceinline__ void swap_pair32(float v, float& a, float& b) {
  unsigned x = __builtin_bit_cast(unsigned, v), y = x;
  asm volatile("" : "+v"(y));
  auto p = __builtin_amdgcn_permlane32_swap(x, y, false, false);
  a = __builtin_bit_cast(float, (unsigned)p[0]);
  b = __builtin_bit_cast(float, (unsigned)p[1]);
}
__device__ __forceinline__ float wave_max_lg(float v) {
  float a, b;
  swap_pair16(v, a, b);
  swap_pair32(fmaxf(a, b), a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float wave_sum_lg(float v) {
  float a, b;
  swap_pair16(v, a, b);
  swap_pair32(a + b, a, b);
  return a + b;
}

// ---- int4 groups of 32: element value = fma(code, scale, zero) in float32 (one rounding).
__device__ __forceinline__ float dequant_one(unsigned code, float scale, float zero) {
  return __builtin_fmaf((float)code, scale, zero);
}

__device__ __forceinline__ float half_lo(unsigned w) {
  _Float16 h = __builtin_bit_cast(_Float16, (unsigned short)(w & 0xFFFFu));
  return (float)h;
}
__device__ __forceinline__ float half_hi(unsigned w) {
  _Float16 h = __builtin_bit_cast(_Float16, (unsigned short)(w >> 16));
  return (float)h;
}

}  // namespace lr
