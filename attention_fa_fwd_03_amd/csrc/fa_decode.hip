// Split-KV decode over a paged FP8 E4M3 cache, and the split combine, for gfx950.
//
// Decode is bound by HBM bandwidth: every cache byte is read once, and the
// q-heads that share a kv-head (GQA) are packed into the rows of one matrix
// product so that they share that read.  Each wavefront is an independent
// worker for one (split, sequence, kv-head): it walks keys [split*L,
// (split+1)*L) in tiles of 32 keys and writes a partial result
// (O normalised by its own denominator, and its natural-log LSE) to the
// workspace; the combine kernel merges the partials of a row by their LSE
// weights (LSE PR: split-K partials are finalised from per-split (m, l)).
//
// Per tile:  S^T[32 keys x 32 rows] = K . Q^T with bf16 MFMA, then
// O^T += V^T P^T.  Decode is a streaming read, so the kernel is built to keep
// many cache bytes in flight: K and V of a tile are loaded straight into
// registers with 16-byte loads, one tile ahead in two register
// sets, so every wait is an exact count of ordinary loads.  K rows feed the
// Q.K^T product from registers (two lanes per key row, converted exactly from
// E4M3 to bf16); the contraction runs over head-dim positions in the order
// d = 32p + 16h + 8u + e (h = lane/32).  The V tile is written by the wave
// into its own LDS tile and read back transposed with ds_read_b64_tr_b8 as
// the A operand of O^T += V^T P^T.  The Q fragments (same d order) are kept
// in LDS, each lane reading back its own bytes, which leaves the registers
// to the loads in flight.
//
// Page lookups are bounded to the sequence's own pages and every byte offset
// is 64-bit, so caches beyond 4 GiB are addressed correctly; keys past
// seqlen_k are clamped for the load and removed by select before the softmax.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

constexpr int kDecWaves = 4;
constexpr int kDecKT = 32;       // keys per tile

// V tile rows are 128 bytes (alternating halves of the 64-bank LDS); the
// transposed reads take rows {0-3, 8-11} (+4 for lanes 32-63) at 2 chunks per
// 32 lanes.  Spreading rows {0, 2, 8, 10} over even chunk offsets makes the
// 32 accesses hit distinct banks.
__device__ __forceinline__ int dec_vswz(int r) { return 2 * (((r >> 1) & 1) | (((r >> 3) & 1) << 1)); }

__device__ __forceinline__ i32x2 lds_read_tr8(const char FA_LDS* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((i32x2 FA_LDS*)(p));
}

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

template <int DQK, int DV>
__global__ __launch_bounds__(kDecWaves * 64) __attribute__((amdgpu_waves_per_eu(2)))
void fa_decode_kernel(const DecodeArgs a) {
  static_assert(DQK % 32 == 0 && DV % 128 == 0, "decode tile shapes");
  constexpr int kVTile = kDecKT * DV;            // fp8 bytes per V tile
  constexpr int kVLoads = kVTile / 1024;         // 16-byte V loads per lane per tile
  constexpr int kKLoads = DQK / 32;              // 16-byte K loads per lane per tile
  constexpr int kQBytes = DQK / 16 * 1024;       // Q fragments of one wave, lane-major
  constexpr int kWaveLds = kQBytes + kVTile;
  __shared__ __attribute__((aligned(1024))) char lds_raw[kDecWaves * kWaveLds];

  // the wavefront index is uniform within a wavefront; readfirstlane lets the
  // compiler keep everything derived from it in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int wi = blockIdx.x * kDecWaves + wave;
  const int units = a.n_split * a.B * a.Hkv;
  if (wi >= units) return;
  const int g = wi % a.Hkv;
  const int b = (wi / a.Hkv) % a.B;
  const int split = wi / (a.Hkv * a.B);
  char FA_LDS* qlds = (char FA_LDS*)(lds_raw) + wave * kWaveLds;
  char FA_LDS* vlds = qlds + kQBytes;

  const int skv = (int)min((int64_t)a.seqlen_k[b], (int64_t)a.max_pages << a.page_shift);   // bounded page-table lookups
  const int qs = a.cu_q[b];
  const int sq = a.cu_q[b + 1] - qs;
  const int R = sq * a.group;
  if (R <= 0) return;
  const int r = lane & 31;
  const bool rvalid = r < R;
  const int qi = rvalid ? r / a.group : 0;
  const int h = g * a.group + (rvalid ? r % a.group : 0);
  const int64_t tok = qs + qi;
  const int k_lo = split * a.split_len;
  const int k_hi = min(skv, k_lo + a.split_len);
  if (k_lo >= k_hi) {
    if (lane < 32 && rvalid) a.part_lse[((int64_t)split * a.total_q + tok) * a.Hq + h] = -INFINITY;
    return;
  }

  const int delta = skv - sq;
  const int ip = qi + delta;
  int my_hi = k_hi - 1, my_lo = k_lo;
  if (a.causal) my_hi = min(my_hi, ip);
  if (a.win_right >= 0) my_hi = min(my_hi, ip + a.win_right);
  if (a.win_left >= 0) my_lo = max(my_lo, ip - a.win_left);

  const float kdesc = *a.k_descale, vdesc = *a.v_descale;
  const float C = a.qk_scale * kLog2e * kdesc;
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.k);
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(a.v);
  const int32_t* bt = a.block_table + (int64_t)b * a.max_pages;
  const int pmask = (1 << a.page_shift) - 1;

  // This lane's V pieces: piece n is tile row v_row[n], source chunk
  // v_chunk[n] (16 bytes), stored at LDS byte n*1024 + 16*lane of the V tile.
  int v_row[kVLoads], v_chunk[kVLoads];
#pragma unroll
  for (int n = 0; n < kVLoads; ++n) {
    const int byte = n * 1024 + lane * 16;
    v_row[n] = byte / DV;
    v_chunk[n] = ((byte % DV) >> 4) ^ dec_vswz(v_row[n]);
  }

  // Load tile t's K rows and V pieces into registers.  Pages hold whole
  // 32-key tiles (page_size >= 32, checked by the host): one wave-uniform
  // scalar page lookup per tile, clamped to the cache; rows past k_hi re-read
  // the last key (masked before the softmax).
  auto load_tile = [&](int t, i32x4 (&kr)[kKLoads], i32x4 (&vr)[kVLoads]) {
    const int k0 = k_lo + t * kDecKT;
    const int64_t page = min(max(load_uniform_i32(bt, k0 >> a.page_shift), 0), a.num_pages - 1);
    const uint8_t* kpage = kbase + page * a.k_pg + (int64_t)g * a.k_sh;
    const uint8_t* vpage = vbase + page * a.v_pg + (int64_t)g * a.v_sh;
    const int jk = min(k0 + (lane & 31), k_hi - 1);
    const uint8_t* krow = kpage + (int64_t)(jk & pmask) * a.k_st + (lane >> 5) * 16;
#pragma unroll
    for (int p = 0; p < kKLoads; ++p)
      kr[p] = *reinterpret_cast<const i32x4*>(krow + 32 * p);
#pragma unroll
    for (int n = 0; n < kVLoads; ++n) {
      const int jv = min(k0 + v_row[n], k_hi - 1);
      vr[n] = *(
          reinterpret_cast<const i32x4*>(vpage + (int64_t)(jv & pmask) * a.v_st + v_chunk[n] * 16));
    }
  };

  const int ntiles = (k_hi - k_lo + kDecKT - 1) / kDecKT;
  const int last = ntiles - 1;
  f32x16 oacc[DV / 32];
#pragma unroll
  for (int d = 0; d < DV / 32; ++d) oacc[d] = f32x16{};
  float m_run = kMaxFloor, l_run = 0.0f;

  // body(t): tile t is in (kc, vc); tile t+1 is in flight in the other set.
  // After the products have consumed kc and the V pieces are in LDS, tile t+2
  // is loaded into (kc, vc).  Loads past the last tile re-read the last one.
  auto body = [&](int t, i32x4 (&kc)[kKLoads], i32x4 (&vc)[kVLoads]) {
    // ---- S^T = K Q^T ----  (two accumulation chains, summed at the end)
    f32x16 sacc2[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int p = 0; p < kKLoads; ++p) {
      bf16x8 lo, hi;
      fp8x16_to_bf16(kc[p], lo, hi);
      const bf16x8 q0 = *reinterpret_cast<const bf16x8 FA_LDS*>(qlds + ((2 * p) * 64 + lane) * 16);
      const bf16x8 q1 = *reinterpret_cast<const bf16x8 FA_LDS*>(qlds + ((2 * p + 1) * 64 + lane) * 16);
      sacc2[0] = mfma32(lo, q0, sacc2[0]);
      sacc2[1] = mfma32(hi, q1, sacc2[1]);
    }
    f32x16 sacc = sacc2[0] + sacc2[1];
    // V pieces of tile t into this wave's LDS tile (the transposed reads of
    // tile t-1 were consumed, hence complete, before this point)
#pragma unroll
    for (int n = 0; n < kVLoads; ++n) *reinterpret_cast<i32x4 FA_LDS*>(vlds + n * 1024 + lane * 16) = vc[n];
    load_tile(min(t + 2, last), kc, vc);

    const int k0 = k_lo + t * kDecKT;
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int j = k0 + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
      const float val = (j >= my_lo && j <= my_hi) ? sacc[i] : -INFINITY;
      sacc[i] = val;
      mx = fmaxf(mx, val);
    }
    mx = max_pair32(mx);
    const float m_new = fmaxf(m_run, mx * C);
    if (__builtin_amdgcn_ballot_w64(m_new > m_run + 8.0f) != 0) {
      const float alpha = exp2_hw(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < DV / 32; ++d)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[d][i] *= alpha;
    }
    bf16x8 pf[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = exp2_hw(fmaf(sacc[i], C, -m_run));
      l_run += p;
      pf[i >> 3][i & 7] = (bf16)p;
    }
    // ---- O^T += V^T P^T ----
    const int grp = lane >> 4, i16 = lane & 15;
    const int hsel = grp >> 1;
    const int tt = i16 >> 1, qq = i16 & 1;
    const int key_in = tt < 4 ? hsel * 4 + tt : 8 + hsel * 4 + (tt - 4);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int rr = u * 16 + key_in;
#pragma unroll
      for (int d = 0; d < DV / 32; ++d) {
        const int c = d * 2 + (grp & 1);
        const i32x2 raw = lds_read_tr8(vlds + rr * DV + ((c ^ dec_vswz(rr)) << 4) + qq * 8);
        oacc[d] = mfma32(fp8x8_to_bf16(raw), pf[u], oacc[d]);
      }
    }
  };

  i32x4 kA[kKLoads], vA[kVLoads], kB[kKLoads], vB[kVLoads];
  load_tile(0, kA, vA);
  load_tile(min(1, last), kB, vB);
  // Q is staged while the first two tiles are in flight
  // Q fragments: step s = 2p + u holds d = 32p + 16*(lane/32) + 8u + e; lane
  // l's fragment of step s lives at LDS byte (s*64 + l)*16 of this wave.
  {
    const bf16* qp = a.q + tok * a.q_st + (int64_t)h * a.q_sh + (lane >> 5) * 16;
#pragma unroll
    for (int p = 0; p < DQK / 32; ++p) {
      bf16x8 x0 = *reinterpret_cast<const bf16x8*>(qp + 32 * p);
      bf16x8 x1 = *reinterpret_cast<const bf16x8*>(qp + 32 * p + 8);
      if (!rvalid) { x0 = bf16x8{}; x1 = bf16x8{}; }
      *reinterpret_cast<bf16x8 FA_LDS*>(qlds + ((2 * p) * 64 + lane) * 16) = x0;
      *reinterpret_cast<bf16x8 FA_LDS*>(qlds + ((2 * p + 1) * 64 + lane) * 16) = x1;
    }
  }
  int t = 0;
  for (; t + 1 < ntiles; t += 2) {
    body(t, kA, vA);
    body(t + 1, kB, vB);
  }
  if (t < ntiles) body(t, kA, vA);

  // ---- partial epilogue ----
  const float l_tot = sum_pair32(l_run);
  if (rvalid) {
    const float inv = l_tot > 0.0f ? vdesc / l_tot : 0.0f;
    float* po = a.part_o + (((int64_t)split * a.total_q + tok) * a.Hq + h) * DV + (lane >> 5) * 4;
#pragma unroll
    for (int d = 0; d < DV / 32; ++d)
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        f32x4 w;
        w[0] = oacc[d][gi * 4 + 0] * inv;
        w[1] = oacc[d][gi * 4 + 1] * inv;
        w[2] = oacc[d][gi * 4 + 2] * inv;
        w[3] = oacc[d][gi * 4 + 3] * inv;
        *reinterpret_cast<f32x4*>(po + d * 32 + gi * 8) = w;
      }
    if (lane < 32)
      a.part_lse[((int64_t)split * a.total_q + tok) * a.Hq + h] =
          l_tot > 0.0f ? (m_run + log2_hw(l_tot)) * kLn2 : -INFINITY;
  }
}

// Merge split partials: one wavefront per (token, q-head).
template <int DV>
__global__ __launch_bounds__(256) void fa_combine_kernel(const CombineArgs a) {
  constexpr int kPer = DV / 64;
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.total_q * a.Hq) return;
  const int64_t tok = row / a.Hq;
  const int h = (int)(row % a.Hq);
  float m = -INFINITY;
  for (int s = 0; s < a.n_split; ++s) m = fmaxf(m, a.part_lse[((int64_t)s * a.total_q + tok) * a.Hq + h]);
  float acc[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) acc[e] = 0.0f;
  float lse = -INFINITY, inv = 0.0f;
  if (m > -INFINITY) {
    float sum = 0.0f;
    for (int s = 0; s < a.n_split; ++s) {
      const float ls = a.part_lse[((int64_t)s * a.total_q + tok) * a.Hq + h];
      if (ls > -INFINITY) {
        const float w = exp2_hw((ls - m) * kLog2e);
        sum += w;
        const float* po = a.part_o + (((int64_t)s * a.total_q + tok) * a.Hq + h) * DV + lane * kPer;
#pragma unroll
        for (int e = 0; e < kPer; ++e) acc[e] += w * po[e];
      }
    }
    inv = 1.0f / sum;
    lse = m + log2_hw(sum) * kLn2;
  }
  bf16* op = a.o + tok * a.o_st + (int64_t)h * a.o_sh + lane * kPer;
#pragma unroll
  for (int e = 0; e < kPer; ++e) op[e] = (bf16)(acc[e] * inv);
  if (lane == 0) a.lse[(int64_t)h * a.total_q + tok] = lse;
}

hipError_t decode_dispatch(const DecodeArgs& a, int dqk, int dv, bool fp8, hipStream_t stream, bool* supported) {
  *supported = true;
  const int units = a.n_split * a.B * a.Hkv;
  const dim3 grid((units + kDecWaves - 1) / kDecWaves);
  if (fp8 && dqk == 192 && dv == 128) {
    hipLaunchKernelGGL((fa_decode_kernel<192, 128>), grid, dim3(kDecWaves * 64), 0, stream, a);
    return hipGetLastError();
  }
  if (fp8 && dqk == 128 && dv == 128) {
    hipLaunchKernelGGL((fa_decode_kernel<128, 128>), grid, dim3(kDecWaves * 64), 0, stream, a);
    return hipGetLastError();
  }
  *supported = false;
  return hipSuccess;
}

hipError_t combine_dispatch(const CombineArgs& a, int dv, hipStream_t stream, bool* supported) {
  *supported = true;
  const int64_t rows = a.total_q * a.Hq;
  const dim3 grid((unsigned)((rows + 3) / 4));
  if (dv == 128) {
    hipLaunchKernelGGL((fa_combine_kernel<128>), grid, dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  *supported = false;
  return hipSuccess;
}

}  // namespace fa
