// dsa_device.hpp -- gfx950 device helpers shared by the DSA kernels.
//
// Number formats are decoded with gfx950's conversion instructions:
//  * v_cvt_scalef32_pk_bf16_fp8 turns two OCP e4m3 codes into two bf16
//    values; every e4m3 value is a bf16 value, so this is exact.
//  * v_cvt_scalef32_pk_bf16_fp4 turns two e2m1 codes into two bf16 values
//    times a scale; the instruction takes only the exponent field of its fp32
//    scale, i.e. it applies a power of two -- exactly an E8M0 block scale
//    (measured on the device for all nibbles and several scales).
//  * NVFP4 block scales are e4m3 (not powers of two), so NVFP4 elements go
//    through fp32: e2m1 -> f32, times the decoded block scale (exact: at most
//    6 significant bits), -> bf16 (exact).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(8))) int i32x8_t;

constexpr int kPage = 64;       // tokens per cache page
constexpr int kIdxHeads = 32;   // indexer heads
constexpr int kIdxDim = 128;    // indexer head dim
constexpr int kLatDim = 576;    // MLA latent dims (512 no-rope + 64 rope)
constexpr int kVDim = 512;      // value dims = the no-rope part
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ bf16x4_t cat2(bf16x2_t a, bf16x2_t b) { return __builtin_shufflevector(a, b, 0, 1, 2, 3); }
__device__ __forceinline__ bf16x8_t cat4(bf16x4_t a, bf16x4_t b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Four e4m3 codes (byte i = element i) -> bf16, exact.
__device__ __forceinline__ bf16x4_t e4m3x4_bf16(uint32_t w) {
  return cat2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false),
              __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
}
__device__ __forceinline__ bf16x8_t e4m3x8_bf16(uint32_t lo, uint32_t hi) {
  return cat4(e4m3x4_bf16(lo), e4m3x4_bf16(hi));
}

// Eight e2m1 codes (element 2i in the low nibble of byte i) times 2^(e8m0-127) -> bf16, exact
// for the exponent range of these data.  `pow2` is the scale as an fp32 power of two.
__device__ __forceinline__ bf16x8_t e2m1x8_bf16(uint32_t w, float pow2) {
  return cat4(cat2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, pow2, 0),
                   __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, pow2, 1)),
              cat2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, pow2, 2),
                   __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, pow2, 3)));
}

// E8M0 byte -> the fp32 whose exponent field holds it (the scale operand of the fp4 conversion).
__device__ __forceinline__ float e8m0_pow2(uint32_t e) { return __uint_as_float((e & 0xFFu) << 23); }

// One e4m3 code -> fp32 (exact).
__device__ __forceinline__ float e4m3_f32(uint32_t code) {
  f32x2_t v = __builtin_amdgcn_cvt_pk_f32_fp8(code, false);
  return v[0];
}

// bf16 <- fp32, round to nearest even (exact when the value has <= 8 significant bits).
__device__ __forceinline__ bf16x2_t f32x2_bf16(float a, float b) {
  bf16x2_t r;
  r[0] = (__bf16)a;
  r[1] = (__bf16)b;
  return r;
}

// Eight NVFP4 elements (one dword of e2m1 pairs) times their e4m3 block scale -> bf16, exact.
__device__ __forceinline__ bf16x8_t nvfp4x8_bf16(uint32_t w, float bscale) {
  f32x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  f32x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
  f32x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
  f32x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  return cat4(cat2(f32x2_bf16(p0[0] * bscale, p0[1] * bscale), f32x2_bf16(p1[0] * bscale, p1[1] * bscale)),
              cat2(f32x2_bf16(p2[0] * bscale, p2[1] * bscale), f32x2_bf16(p3[0] * bscale, p3[1] * bscale)));
}

__device__ __forceinline__ f32x16_t mfma_32x32x16_bf16(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma_16x16x32_bf16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Sum of lane l and lane l^32 (the two halves of a wave), in every lane.
__device__ __forceinline__ float sum_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Order-preserving map of an fp32 score to uint32: larger key <=> larger value; -0 maps to +0.
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Its inverse (the float whose key is k).
__device__ __forceinline__ float key_score(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

__device__ __forceinline__ void flag_error(int32_t *err, uint32_t bits) {
  if (err) atomicOr(err, (int32_t)bits);
}

// Wave-wide inclusive prefix sum (wave64): Hillis-Steele steps inside each 16-lane row with
// DPP row shifts, then the row totals carried across rows with DPP row broadcasts.  Lanes
// whose DPP source is out of range (or whose row is masked off) receive 0 through `old`.
__device__ __forceinline__ int wave_scan_incl(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2, 3
  return x;
}

// Wave-wide max / min of uint32 (the result in every lane), same DPP pattern.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  int v = (int)x;
  v = (int)max((uint32_t)v, (uint32_t)__builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false));
  v = (int)max((uint32_t)v, (uint32_t)__builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false));
  v = (int)max((uint32_t)v, (uint32_t)__builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false));
  v = (int)max((uint32_t)v, (uint32_t)__builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false));
  v = (int)max((uint32_t)v, (uint32_t)__builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false));
  v = (int)max((uint32_t)v, (uint32_t)__builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false));
  return (uint32_t)__builtin_amdgcn_readlane(v, 63);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) { return ~wave_max_u32(~x); }

// Block-wide inclusive scan of one int per thread (blockDim.x == NT).  `tmp` holds NT / 64 ints.
template <int NT>
__device__ __forceinline__ int block_scan_incl(int v, int *tmp, int &total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  v = wave_scan_incl(v);
  if (lane == 63) tmp[wid] = v;
  __syncthreads();
  int base = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int t = tmp[w];
    base += w < wid ? t : 0;
    total += t;
  }
  __syncthreads();
  return v + base;
}

__device__ __forceinline__ int block_scan_incl_256(int v, int *tmp, int &total) {
  return block_scan_incl<256>(v, tmp, total);
}

}  // namespace dsa
