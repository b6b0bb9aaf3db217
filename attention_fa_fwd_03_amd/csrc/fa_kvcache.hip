// FP8 E4M3 KV-cache write for gfx950: quantise token-major bf16 K/V rows and
// place them in head-major or vectorised paged caches.
//
// Method: the fp8 KV-cache page ("flash_attention: prologue fusion, ...",
// part 3) quantises K/V on the GPU with a scale from the largest magnitude
// over 448, and the paged FP8 PR reads per-tensor descales amax/448.  Here:
//   descale = max(amax / 448, 2^-126)   (or a descale the caller gives),
//   code    = E4M3(x * (1 / descale)),  nearest, ties to even, saturating
// with every step in fp32 (the division correctly rounded).
//
// The work is bound by HBM bandwidth (2 bytes read, 1 written per element):
// one thread converts one 16-element chunk of one (token, kv-head) row — two
// 16-byte loads, one 16-byte store into a head-major page row or a
// vectorised K column; a vectorised V chunk is 16 head dims of one key,
// which that layout keeps 16 bytes apart, so it takes byte stores.  The
// per-tensor maximum is a two-step reduction (per-block partial maxima, then
// one workgroup) so that no atomics or pre-cleared memory are involved.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

constexpr int kKvThreads = 256;
constexpr float kE4M3Max = 448.0f;
constexpr float kFltMin = 1.17549435e-38f;   // 2^-126

// fp32 -> E4M3 code: nearest, ties to even; |y| >= 448 (and infinity)
// saturates to +-448; NaN gives 0x7F with y's sign.  Integer arithmetic on
// the fp32 fields, so the rounding is exact by construction.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return sign | 0x7fu;
  if (a >= 0x43e00000u) return sign | 0x7eu;             // 448.0f
  if (a < 0x3c800000u) {                                 // below 2^-6: steps of 2^-9
    const float q = __builtin_rintf(__uint_as_float(a) * 512.0f);
    return sign | (uint32_t)q;
  }
  // normal: exponent field (biased 7) and the top 3 mantissa bits; the 20
  // dropped bits round to nearest, ties to even (a carry out of the
  // mantissa moves into the exponent, and cannot pass 448 here)
  uint32_t code = ((((a >> 23) - 127u + 7u) << 3) | ((a >> 20) & 7u));
  const uint32_t rem = a & 0xfffffu;
  if (rem > 0x80000u || (rem == 0x80000u && (code & 1u))) code += 1u;
  return sign | code;
}

__device__ __forceinline__ uint32_t pack4(float a, float b, float c, float d, float inv) {
  return e4m3_code(a * inv) | (e4m3_code(b * inv) << 8) | (e4m3_code(c * inv) << 16) | (e4m3_code(d * inv) << 24);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

// Per-block maxima of |k| (blocks [0, nb_k)) and |v| (blocks [nb_k, nb_k + nb_v)).
__global__ __launch_bounds__(kKvThreads) void fa_kv_amax_kernel(const KvAmaxArgs a) {
  __shared__ float red[kKvThreads / 64];
  const bool is_k = (int)blockIdx.x < a.nb_k;
  const bf16* x = is_k ? a.k : a.v;
  const int64_t n = is_k ? a.n_k : a.n_v;               // elements, a multiple of 8
  const int nb = is_k ? a.nb_k : a.nb_v;
  const int blk = is_k ? (int)blockIdx.x : (int)blockIdx.x - a.nb_k;
  float m = 0.0f;
  for (int64_t i = ((int64_t)blk * kKvThreads + threadIdx.x) * 8; i < n; i += (int64_t)nb * kKvThreads * 8) {
    const bf16x8 w = *reinterpret_cast<const bf16x8*>(x + i);
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf((float)w[e]));
  }
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float r = red[0];
    for (int w = 1; w < kKvThreads / 64; ++w) r = fmaxf(r, red[w]);
    a.partial[blockIdx.x] = r;
  }
}

// One workgroup: descale = max(amax / 448, 2^-126) for K and V.
__global__ __launch_bounds__(kKvThreads) void fa_kv_descale_kernel(const KvAmaxArgs a) {
  __shared__ float red[2][kKvThreads / 64];
  float mk = 0.0f, mv = 0.0f;
  for (int i = threadIdx.x; i < a.nb_k; i += kKvThreads) mk = fmaxf(mk, a.partial[i]);
  for (int i = threadIdx.x; i < a.nb_v; i += kKvThreads) mv = fmaxf(mv, a.partial[a.nb_k + i]);
  mk = wave_max(mk);
  mv = wave_max(mv);
  if ((threadIdx.x & 63) == 0) {
    red[0][threadIdx.x >> 6] = mk;
    red[1][threadIdx.x >> 6] = mv;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kKvThreads / 64; ++w) {
      mk = fmaxf(mk, red[0][w]);
      mv = fmaxf(mv, red[1][w]);
    }
    *a.k_descale = fmaxf(__fdiv_rn(mk, kE4M3Max), kFltMin);
    *a.v_descale = fmaxf(__fdiv_rn(mv, kE4M3Max), kFltMin);
  }
}

// Item i < T*Hkv*ck: K chunk (t, g, c); then T*Hkv*cv V chunks.
template <bool VEC>
__global__ __launch_bounds__(kKvThreads) void fa_kv_write_kernel(const KvWriteArgs a) {
  const int ck = a.d_qk >> 4, cv = a.d_v >> 4;
  const int64_t nk = a.T * a.Hkv * ck, ntot = nk + a.T * a.Hkv * cv;
  const float inv_k = __fdiv_rn(1.0f, *a.k_descale), inv_v = __fdiv_rn(1.0f, *a.v_descale);
  const int64_t cap = (int64_t)a.num_pages << a.page_shift;
  const int pmask = (1 << a.page_shift) - 1;
  for (int64_t i = (int64_t)blockIdx.x * kKvThreads + threadIdx.x; i < ntot; i += (int64_t)gridDim.x * kKvThreads) {
    const bool is_k = i < nk;
    const int64_t j = is_k ? i : i - nk;
    const int nc = is_k ? ck : cv, D = is_k ? a.d_qk : a.d_v;
    const int c = (int)(j % nc);
    const int64_t tg = j / nc;                          // t * Hkv + g
    const int64_t t = tg / a.Hkv;
    const int g = (int)(tg - t * a.Hkv);
    const int64_t slot = a.slot_mapping[t];
    if (slot < 0 || slot >= cap) continue;
    const int64_t p = slot >> a.page_shift;
    const int s = (int)(slot & pmask);
    const bf16* src = (is_k ? a.k : a.v) + tg * D + c * 16;
    const bf16x8 lo = *reinterpret_cast<const bf16x8*>(src);
    const bf16x8 hi = *reinterpret_cast<const bf16x8*>(src + 8);
    const float inv = is_k ? inv_k : inv_v;
    i32x4 w;
    w[0] = (int)pack4((float)lo[0], (float)lo[1], (float)lo[2], (float)lo[3], inv);
    w[1] = (int)pack4((float)lo[4], (float)lo[5], (float)lo[6], (float)lo[7], inv);
    w[2] = (int)pack4((float)hi[0], (float)hi[1], (float)hi[2], (float)hi[3], inv);
    w[3] = (int)pack4((float)hi[4], (float)hi[5], (float)hi[6], (float)hi[7], inv);
    const int64_t ps = (int64_t)1 << a.page_shift;
    uint8_t* blk = reinterpret_cast<uint8_t*>(is_k ? a.k_cache : a.v_cache) + p * a.Hkv * ps * D + (int64_t)g * ps * D;
    if (!VEC) {
      *reinterpret_cast<i32x4*>(blk + (int64_t)s * D + c * 16) = w;
    } else if (is_k) {
      *reinterpret_cast<i32x4*>(blk + (int64_t)c * ps * 16 + s * 16) = w;
    } else {
      // V [page/16, Dv, 16]: dim d of key s at (s/16) Dv 16 + d 16 + s%16
      uint8_t* col = blk + (int64_t)(s >> 4) * D * 16 + (int64_t)c * 16 * 16 + (s & 15);
#pragma unroll
      for (int e = 0; e < 16; ++e) col[e * 16] = (uint8_t)((uint32_t)w[e >> 2] >> (8 * (e & 3)));
    }
  }
}

hipError_t kv_amax_dispatch(const KvAmaxArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(fa_kv_amax_kernel, dim3(a.nb_k + a.nb_v), dim3(kKvThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fa_kv_descale_kernel, dim3(1), dim3(kKvThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t kv_write_dispatch(const KvWriteArgs& a, bool vec, int blocks, hipStream_t stream) {
  if (vec) hipLaunchKernelGGL(fa_kv_write_kernel<true>, dim3(blocks), dim3(kKvThreads), 0, stream, a);
  else hipLaunchKernelGGL(fa_kv_write_kernel<false>, dim3(blocks), dim3(kKvThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace fa
