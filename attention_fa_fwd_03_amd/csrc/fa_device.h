// Device-side building blocks for the gfx950 (CDNA4) attention kernels.
//
// Everything here is written for 64-lane wavefronts and the gfx950 matrix
// cores.  Lane layouts of the builtins used below (verified on the hardware
// with an in-bounds layout probe):
//
//  v_mfma_f32_32x32x16_bf16  A[32 x 16], B[16 x 32], C[32 x 32]
//    lane l holds A[l%32][(l/32)*8 + e] and B[(l/32)*8 + e][l%32], e = 0..7;
//    C register i of lane l is C[(i/4)*8 + (l/32)*4 + i%4][l%32], i = 0..15.
//  ds_read_b64_tr_b16 (8 bytes per lane, transposed inside each group of 16
//    lanes): if lane j of a group points at four 16-bit values src[j][0..3],
//    lane i of the group receives out[t] = src[4t + i/4][i%4], t = 0..3.
//  v_permlane32_swap x, x: returns (x from lane l&31, x from lane (l&31)+32).
//  v_cvt_scalef32_pk_bf16_fp8: two OCP E4M3 bytes -> two bf16 (exact).
//  global_load_lds_dwordx4: lane l's 16 bytes land at LDS base + 16*l.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

#define FA_LDS __attribute__((address_space(3)))
#define FA_GLOBAL __attribute__((address_space(1)))
#define FA_CONST __attribute__((address_space(4)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Running-max floor: a large finite value so that rows with no visible key
// never evaluate (-inf) - (-inf).
constexpr float kMaxFloor = -3.0e38f;

// s_waitcnt immediate for "vector memory count <= n" (gfx9 encoding), leaving
// the LDS/scalar and export counters unconstrained.
__device__ __forceinline__ constexpr int vmcnt_imm(int n) {
  return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8);
}
#define FA_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(::fa::vmcnt_imm(n))

// Wave-uniform load of read-only metadata through the scalar cache (s_load):
// it is tracked by the LDS/scalar counter, so it never waits behind the
// vector-memory data loads that are in flight.
__device__ __forceinline__ int load_uniform_i32(const int32_t* base, int64_t idx) {
  const FA_CONST int32_t* p = (const FA_CONST int32_t*)(base);
  return p[idx];
}

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float rcp_hw(float x) { return __builtin_amdgcn_rcpf(x); }

// Value of x held by the lane 32 positions away (l ^ 32).
__device__ __forceinline__ float partner32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  int lane = __lane_id();
  return __uint_as_float(lane < 32 ? r[1] : r[0]);
}

// max over the two lanes {l, l^32}
__device__ __forceinline__ float max_pair32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float sum_pair32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ bf16x8 lds_read_b128(const char FA_LDS* p) {
  return *reinterpret_cast<const bf16x8 FA_LDS*>(p);
}

__device__ __forceinline__ bf16x4 lds_read_tr16(const char FA_LDS* __restrict__ p) {
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<s16x4 FA_LDS*>(const_cast<char FA_LDS*>(p)));
  return __builtin_bit_cast(bf16x4, v);
}

// 16 bytes from global memory straight into LDS (base + 16*lane).
__device__ __forceinline__ void global_to_lds16(const void* gsrc, char FA_LDS* lds_base) {
  __builtin_amdgcn_global_load_lds((const FA_GLOBAL void*)(gsrc), (FA_LDS void*)(lds_base), 16, 0, 0);
}

// Buffer descriptor over [base, base + 2^31): raw (unstrided) 32-bit
// offsets; loads past the end return zeros.  The third word is the gfx9
// default (32-bit data format).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff, 0x00020000);
}

// 16 bytes at byte offset voff of the descriptor's range straight into LDS
// (base + 16*lane).
__device__ __forceinline__ void buffer_to_lds16(__amdgpu_buffer_rsrc_t rs, unsigned voff, char FA_LDS* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (FA_LDS void*)(lds_base), 16, voff, 0, 0, 0);
}

// 8 OCP E4M3 bytes -> 8 bf16 (exact).
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(i32x2 w) {
  bf16x8 r;
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, false);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, true);
  bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, false);
  bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, true);
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// Power-of-two scale for the E4M3 split of one query row whose largest
// magnitude is amax: returns 2^e with amax * 2^e in [128, 256), so every
// scaled value stays below the E4M3 maximum (448) and the row's large values
// keep both parts in the normal range; *inv = 2^-e.  e is clamped to
// [-126, 126]; an all-zero row takes e = 0.
__device__ __forceinline__ float split_scale(float amax, float* inv) {
  int E;
  (void)frexpf(amax, &E);            // amax = m 2^E, m in [0.5, 1)
  int e = amax > 0.0f ? 8 - E : 0;
  e = min(max(e, -126), 126);
  *inv = ldexpf(1.0f, -e);
  return ldexpf(1.0f, e);
}

// Eight bf16 values x -> E4M3 parts (hi, lo) of scale * x, with
// scale * x ~= hi + lo: the two 3-bit mantissas carry each value to about
// 2^-8 relative (values far below the row's maximum to about 2^-17 of that
// maximum, absolute), and each part times an E4M3 operand is exact in an
// FP8 product.  scale comes from split_scale of the row's maximum.
__device__ __forceinline__ void split_e4m3(bf16x8 x, float scale, i32x2& hi, i32x2& lo) {
  float f[8], r[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = scale * (float)x[e];
  int h0 = 0, h1 = 0, l0 = 0, l1 = 0;
  h0 = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], h0, false);
  h0 = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], h0, true);
  h1 = __builtin_amdgcn_cvt_pk_fp8_f32(f[4], f[5], h1, false);
  h1 = __builtin_amdgcn_cvt_pk_fp8_f32(f[6], f[7], h1, true);
  r[0] = f[0] - __builtin_amdgcn_cvt_f32_fp8(h0, 0);
  r[1] = f[1] - __builtin_amdgcn_cvt_f32_fp8(h0, 1);
  r[2] = f[2] - __builtin_amdgcn_cvt_f32_fp8(h0, 2);
  r[3] = f[3] - __builtin_amdgcn_cvt_f32_fp8(h0, 3);
  r[4] = f[4] - __builtin_amdgcn_cvt_f32_fp8(h1, 0);
  r[5] = f[5] - __builtin_amdgcn_cvt_f32_fp8(h1, 1);
  r[6] = f[6] - __builtin_amdgcn_cvt_f32_fp8(h1, 2);
  r[7] = f[7] - __builtin_amdgcn_cvt_f32_fp8(h1, 3);
  l0 = __builtin_amdgcn_cvt_pk_fp8_f32(r[0], r[1], l0, false);
  l0 = __builtin_amdgcn_cvt_pk_fp8_f32(r[2], r[3], l0, true);
  l1 = __builtin_amdgcn_cvt_pk_fp8_f32(r[4], r[5], l1, false);
  l1 = __builtin_amdgcn_cvt_pk_fp8_f32(r[6], r[7], l1, true);
  hi = i32x2{h0, h1};
  lo = i32x2{l0, l1};
}

__device__ __forceinline__ float amax8(bf16x8 x, float m) {
#pragma unroll
  for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf((float)x[e]));
  return m;
}

// 16 OCP E4M3 bytes -> 16 bf16 (exact).
__device__ __forceinline__ void fp8x16_to_bf16(i32x4 w, bf16x8& lo, bf16x8& hi) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[d], 1.0f, false);
    bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[d], 1.0f, true);
    if (d < 2) {
      lo[4 * d + 0] = a[0]; lo[4 * d + 1] = a[1]; lo[4 * d + 2] = b[0]; lo[4 * d + 3] = b[1];
    } else {
      hi[4 * (d - 2) + 0] = a[0]; hi[4 * (d - 2) + 1] = a[1];
      hi[4 * (d - 2) + 2] = b[0]; hi[4 * (d - 2) + 3] = b[1];
    }
  }
}

// w with its bytes k..15 cleared (k <= 0: all cleared; k >= 16: unchanged).
// Cache bytes past a sequence's end that share a load with live bytes may
// hold anything, NaN codes included; their scores are removed by select, but
// a NaN value would survive the zero weight of its product, so such value
// bytes are cleared before they reach a product.
__device__ __forceinline__ i32x4 keep_bytes(i32x4 w, int k) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = k - 4 * j;
    const unsigned m = n >= 4 ? 0xffffffffu : (n <= 0 ? 0u : (1u << (8 * n)) - 1u);
    w[j] &= (int)m;
  }
  return w;
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

}  // namespace fa
