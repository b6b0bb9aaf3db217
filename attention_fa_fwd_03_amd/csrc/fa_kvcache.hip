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
// a workgroup quantises 16 consecutive tokens into LDS with contiguous
// reads, then writes each destination run contiguously when the tokens fill
// one 16-slot block of a page (16 page rows, 256-byte vectorised K columns,
// 16-byte vectorised V vectors of 16 keys each), else token by token.  The
// per-tensor maximum is a two-step reduction (per-block partial maxima, then
// one workgroup) so that no atomics or pre-cleared memory are involved.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

constexpr int kKvThreads = 256;
constexpr int kBatch = 4;                    // row chunks whose loads are in flight together per thread
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

// A workgroup takes a group of 16 consecutive tokens and a range of
// kv-heads [h0, h0 + nh).  Phase 1 reads the group's rows (contiguous:
// heads h0.. of a token are adjacent) and quantises them into LDS, token by
// token.  Phase 2 writes the caches in their own order: when the 16 tokens
// fill one 16-slot block of one page in order (a prefill fill), every
// destination run is contiguous — 16 page rows (head-major), 256-byte K
// columns, whole 16-byte V vectors (vectorised); otherwise each token goes
// to its own slot.
template <bool VEC>
__global__ __launch_bounds__(kKvThreads) void fa_kv_write_kernel(const KvWriteArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t kv_lds[];
  __shared__ int64_t sl[16];
  const int ck = a.d_qk >> 4, cv = a.d_v >> 4;
  const int h0 = (int)blockIdx.y * a.heads_per_pass;
  const int nh = (int)min((int64_t)a.heads_per_pass, a.Hkv - h0);
  const int rk = nh * a.d_qk, rv = nh * a.d_v;            // LDS bytes per token
  uint8_t* lk = kv_lds;
  uint8_t* lv = kv_lds + 16 * rk;
  const float inv_k = __fdiv_rn(1.0f, *a.k_descale), inv_v = __fdiv_rn(1.0f, *a.v_descale);
  const int64_t cap = a.num_pages << a.page_shift;
  const int64_t ps = (int64_t)1 << a.page_shift;
  const int pmask = (int)ps - 1;
  const int per = nh * (ck + cv);
  for (int64_t t0 = (int64_t)blockIdx.x * 16; t0 < a.T; t0 += (int64_t)gridDim.x * 16) {
    const int n = (int)min((int64_t)16, a.T - t0);
    __syncthreads();                                     // the previous group is written out
    if (threadIdx.x < 16) sl[threadIdx.x] = threadIdx.x < n ? a.slot_mapping[t0 + threadIdx.x] : -1;
    // phase 1: rows -> codes in LDS (tokens past the end contribute zeros,
    // never stored); kBatch items' loads are issued before any is converted
    for (int base = threadIdx.x; base < 16 * per; base += kBatch * kKvThreads) {
      bf16x8 lo[kBatch], hi[kBatch];
      int dst[kBatch];
      float inv[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int item = base + u * kKvThreads;
        const int tok = item / per, q = item - tok * per;
        const bool is_k = q < nh * ck;
        const int qq = is_k ? q : q - nh * ck;
        dst[u] = item < 16 * per ? (is_k ? tok * rk : 16 * rk + tok * rv) + qq * 16 : -1;
        inv[u] = is_k ? inv_k : inv_v;
        lo[u] = hi[u] = bf16x8{};
        if (item < 16 * per && tok < n) {
          const int64_t t = t0 + tok;
          const bf16* src = is_k ? a.k + (t * a.Hkv + h0) * a.d_qk + qq * 16 : a.v + (t * a.Hkv + h0) * a.d_v + qq * 16;
          lo[u] = *reinterpret_cast<const bf16x8*>(src);
          hi[u] = *reinterpret_cast<const bf16x8*>(src + 8);
        }
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        if (dst[u] < 0) continue;
        i32x4 w;
        w[0] = (int)pack4((float)lo[u][0], (float)lo[u][1], (float)lo[u][2], (float)lo[u][3], inv[u]);
        w[1] = (int)pack4((float)lo[u][4], (float)lo[u][5], (float)lo[u][6], (float)lo[u][7], inv[u]);
        w[2] = (int)pack4((float)hi[u][0], (float)hi[u][1], (float)hi[u][2], (float)hi[u][3], inv[u]);
        w[3] = (int)pack4((float)hi[u][4], (float)hi[u][5], (float)hi[u][6], (float)hi[u][7], inv[u]);
        *reinterpret_cast<i32x4*>(kv_lds + dst[u]) = w;
      }
    }
    __syncthreads();
    const int64_t s0 = sl[0];
    bool whole = ps >= 16 && n == 16 && s0 >= 0 && s0 + 15 < cap && (s0 & 15) == 0;
#pragma unroll
    for (int i = 1; i < 16; ++i) whole = whole && sl[i] == s0 + i;
    if (whole) {
      const int64_t p = s0 >> a.page_shift;
      const int s = (int)(s0 & pmask);
      // K, in destination order: vectorised (head g, column c, token i),
      // head-major (head g, token i, chunk c); the last index fastest
      for (int item = threadIdx.x; item < 16 * nh * ck; item += kKvThreads) {
        int g, i, c;
        if (VEC) {
          i = item & 15;
          const int gc = item >> 4;
          g = gc / ck;
          c = gc - g * ck;
        } else {
          const int gi = item / ck;
          c = item - gi * ck;
          g = gi >> 4;
          i = gi & 15;
        }
        const i32x4 w = *reinterpret_cast<const i32x4*>(lk + i * rk + (g * ck + c) * 16);
        uint8_t* blk = reinterpret_cast<uint8_t*>(a.k_cache) + (p * a.Hkv + h0 + g) * ps * a.d_qk;
        if (VEC) *reinterpret_cast<i32x4*>(blk + (int64_t)c * ps * 16 + (s + i) * 16) = w;
        else *reinterpret_cast<i32x4*>(blk + (int64_t)(s + i) * a.d_qk + c * 16) = w;
      }
      if (VEC) {
        // V vectors: (head g, dim d) gathers byte d of the 16 tokens
        for (int col = threadIdx.x; col < nh * a.d_v; col += kKvThreads) {
          const int g = col / a.d_v, d = col - g * a.d_v;
          uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
          for (int i = 0; i < 16; ++i) w[i >> 2] |= (uint32_t)lv[i * rv + col] << (8 * (i & 3));
          uint8_t* dst = reinterpret_cast<uint8_t*>(a.v_cache) + (p * a.Hkv + h0 + g) * ps * a.d_v +
                         (int64_t)(s >> 4) * a.d_v * 16 + (int64_t)d * 16;
          *reinterpret_cast<i32x4*>(dst) = i32x4{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
        }
      } else {
        for (int item = threadIdx.x; item < 16 * nh * cv; item += kKvThreads) {
          const int gi = item / cv, c = item - gi * cv, g = gi >> 4, i = gi & 15;
          const i32x4 w = *reinterpret_cast<const i32x4*>(lv + i * rv + (g * cv + c) * 16);
          uint8_t* blk = reinterpret_cast<uint8_t*>(a.v_cache) + (p * a.Hkv + h0 + g) * ps * a.d_v;
          *reinterpret_cast<i32x4*>(blk + (int64_t)(s + i) * a.d_v + c * 16) = w;
        }
      }
    } else {
      // token by token: (token i, head g, chunk c), c fastest
      for (int item = threadIdx.x; item < n * per; item += kKvThreads) {
        const int i = item / per, q = item - i * per;
        const int64_t slot = sl[i];
        if (slot < 0 || slot >= cap) continue;
        const int64_t p = slot >> a.page_shift;
        const int s = (int)(slot & pmask);
        const bool is_k = q < nh * ck;
        const int qq = is_k ? q : q - nh * ck, nc = is_k ? ck : cv, D = is_k ? a.d_qk : a.d_v;
        const int g = qq / nc, c = qq - g * nc;
        const i32x4 w = *reinterpret_cast<const i32x4*>((is_k ? lk + i * rk : lv + i * rv) + qq * 16);
        uint8_t* blk = reinterpret_cast<uint8_t*>(is_k ? a.k_cache : a.v_cache) + (p * a.Hkv + h0 + g) * ps * D;
        if (!VEC) {
          *reinterpret_cast<i32x4*>(blk + (int64_t)s * D + c * 16) = w;
        } else if (is_k) {
          *reinterpret_cast<i32x4*>(blk + (int64_t)c * ps * 16 + s * 16) = w;
        } else {
          uint8_t* col = blk + (int64_t)(s >> 4) * D * 16 + (int64_t)c * 256 + (s & 15);
#pragma unroll
          for (int e = 0; e < 16; ++e) col[e * 16] = (uint8_t)((uint32_t)w[e >> 2] >> (8 * (e & 3)));
        }
      }
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

hipError_t kv_write_dispatch(const KvWriteArgs& a, bool vec, hipStream_t stream) {
  const int64_t groups = (a.T + 15) / 16;
  const dim3 grid((unsigned)(groups < 8192 ? groups : 8192), (unsigned)((a.Hkv + a.heads_per_pass - 1) / a.heads_per_pass));
  const size_t lds = (size_t)16 * a.heads_per_pass * (a.d_qk + a.d_v);
  if (vec) hipLaunchKernelGGL(fa_kv_write_kernel<true>, grid, dim3(kKvThreads), lds, stream, a);
  else hipLaunchKernelGGL(fa_kv_write_kernel<false>, grid, dim3(kKvThreads), lds, stream, a);
  return hipGetLastError();
}

}  // namespace fa
