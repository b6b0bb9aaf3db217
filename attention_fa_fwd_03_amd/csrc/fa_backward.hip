// Attention backward pass (dQ, dK, dV) for gfx950, recomputing the
// probabilities from the forward's saved LSE.
//
// Method (SM90 FlashAttention page, backward commit; LSE page, Summary):
// Delta_i = dO_i . O_i per row and head (the page's preprocess; here the dQ
// kernel computes it for its own rows and runs first); with
// P = exp(scale q.k - LSE) the gradients are
//   dV = P^T dO,  dS = P * (dO V^T - Delta),  dK = scale dS^T Q,  dQ = scale dS K.
// The page's kernel walks key tiles, loops over query tiles and adds dQ
// with atomics; here dK/dV and dQ are two kernels that each recompute S and
// dP, so every output is written once by one wavefront and summed in fp32
// in a fixed order (deterministic, no atomics, no pre-cleared memory).
//
// Products are v_mfma_f32_32x32x16_bf16, oriented as in the forward kernel
// so that each accumulator feeds the next product without moving data
// between lanes:
//   dK/dV kernel (a wavefront owns 32 keys, K and V^T fragments in
//   registers; 64-row Q / dO tiles staged in LDS):
//     S  [rows x keys] = Q K^T        A = Q rows from LDS, B = K in registers
//     dP [rows x keys] = dO V^T       A = dO rows from LDS, B = V in registers
//     dV^T [d x keys] += dO^T P       A = dO read transposed, B = P in registers
//     dK^T [d x keys] += Q^T dS       A = Q read transposed,  B = dS in registers
//   dQ kernel (a wavefront owns 32 query rows, Q and dO fragments in
//   registers; 64-key K / V tiles staged in LDS):
//     S^T [keys x rows] = K Q^T,  dP^T = V dO^T,  dQ^T [d x rows] += K^T dS^T
// The B operand taken from a 32x32 accumulator enumerates its 16 rows (or
// keys) per step with bits 2 and 3 swapped, and the transposed reads fetch
// rows in that same order (as in the forward's P.V).
//
// Rows with no visible key have LSE = -inf: their P is 0 (the log2-domain
// LSE is replaced by +inf), so they contribute nothing.  Masking is by
// select, never by multiply.
#include "fa_device.h"
#include "fa_kernels.h"
#include "fa_prefill_common.h"

namespace fa {

constexpr int kBwWaves = 4;
constexpr int kBwThreads = 64 * kBwWaves;
constexpr int kBwTile = 64;        // rows of a staged Q/dO tile, keys of a staged K/V tile
constexpr int kBwKeys = 32 * kBwWaves;   // keys per dK/dV workgroup
constexpr int kBwRowsQ = 32 * kBwWaves;  // query rows per dQ workgroup

struct BwSeq {
  int64_t qstart, kstart;
  int sq, skv;
};

__device__ __forceinline__ BwSeq bw_seq(const BwdArgs& a, int b) {
  BwSeq s;
  if (a.cu_q) {
    s.qstart = a.cu_q[b];
    s.sq = a.cu_q[b + 1] - a.cu_q[b];
    s.kstart = a.cu_k[b];
    s.skv = a.cu_k[b + 1] - a.cu_k[b];
  } else {
    s.qstart = (int64_t)b * a.Sq;
    s.sq = a.Sq;
    s.kstart = (int64_t)b * a.Skv;
    s.skv = a.Skv;
  }
  return s;
}

// index of (sequence b, head h, row i) in the LSE / Delta layout
__device__ __forceinline__ int64_t bw_lse_index(const BwdArgs& a, int b, int h, int64_t qstart, int i) {
  if (a.cu_q) return (int64_t)h * a.lse_tq + qstart + i;
  return ((int64_t)b * a.Hq + h) * a.Sq + i;
}

// Row swizzle of the Q / dO tiles of the 16-key dK/dV kernel (256-byte
// rows): its transposed reads take 8 rows (two groups of four) x 2 adjacent
// chunks per pass, its A fragments 16 rows x 1 chunk per 16 lanes.  With
// r = 4 g + i (i < 4) inside 16 rows, the chunk pair index is 2 i + the
// parity of g and g / 2 and bit 0 is bit 1 of g: any two of the four
// groups then fill 8 different chunk pairs, and the 16 rows 16 different
// chunks (the forward's map sends rows r and r + 4 to the same pair).
__device__ __forceinline__ int swz_bw16(int r) {
  const int g = (r >> 2) & 3, i = r & 3;
  return ((2 * i + ((g ^ (g >> 1)) & 1)) << 1) | ((g >> 1) & 1);
}

// 64 rows x D bf16 of a packed tensor -> swizzled LDS tile, one 1 KB
// buffer load to LDS per wavefront instruction (lane l fills 16 bytes at
// 16 l of its KB: tile row r, stored chunk pos = source chunk pos ^ swz(r),
// swz_bw16 when ALT).  Rows at or past nrows re-read the last row (their
// results are masked).
template <int D, bool ALT = false>
struct RowStager {
  static constexpr int kRow = D * 2;
  static constexpr int kPerWave = kBwTile * kRow / 1024 / kBwWaves;
  static_assert(kPerWave >= 1, "tile too small");
  int row[kPerWave], col[kPerWave];   // tile row and source element column of each piece
  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int byte = (wave * kPerWave + i) * 1024 + lane * 16;
      row[i] = byte / kRow;
      col[i] = ((((byte % kRow) >> 4) ^ (ALT ? swz_bw16(row[i]) : swz<kRow>(row[i]))) << 3);
    }
  }
  // Whole tiles (rows r0..r0+63 all inside the sequence, row stride below
  // 2^24 elements): one buffer descriptor at row r0 and 32-bit per-lane
  // offsets computed once per stride, no per-piece address arithmetic.
  __device__ __forceinline__ void offsets(int64_t st, unsigned (&off)[kPerWave]) const {
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) off[i] = ((unsigned)row[i] * (unsigned)st + (unsigned)col[i]) * 2u;
  }
  __device__ __forceinline__ void issue_whole(const bf16* base, int64_t st, int r0, const unsigned (&off)[kPerWave],
                                              char FA_LDS* tile, int wave) const {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(base + (int64_t)r0 * st);
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) buffer_to_lds16(rs, off[i], tile + (wave * kPerWave + i) * 1024);
  }
  // Tiles that may run past the sequence's end: the same buffer copies, rows
  // at or past nrows re-reading row nrows - 1.  Offsets count from row r0
  // (at most 63 rows of a stride below 2^24 elements: below 2^31 bytes).
  // Only buffer copies are used: a global_load_lds anywhere in a loop makes
  // the compiler wait for every LDS read in it with lgkmcnt(0).
  __device__ __forceinline__ void issue_clamped(const bf16* base, int64_t st, int r0, int nrows, char FA_LDS* tile,
                                                int wave) const {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(base + (int64_t)r0 * st);
    const int last = nrows - 1 - r0;
#pragma unroll
    for (int i = 0; i < kPerWave; ++i)
      buffer_to_lds16(rs, ((unsigned)min(row[i], last) * (unsigned)st + (unsigned)col[i]) * 2u,
                      tile + (wave * kPerWave + i) * 1024);
  }
};

// A fragment of O^T-style products read transposed from a swizzled tile of
// 64 rows: rows {16u + swap23 order} x 32 columns [32 dblk, +32).
template <int kRow>
__device__ __forceinline__ bf16x8 tr_fragment(const char FA_LDS* tile, int u, int dblk, int lane) {
  const int grp = lane >> 4, i16 = lane & 15;
  const int r1 = u * 16 + (grp >> 1) * 4 + (i16 >> 2);
  const int r2 = r1 + 8;
  const int dcol = dblk * 32 + (grp & 1) * 16 + 4 * (i16 & 3);
  const int chunk = dcol >> 3, half = (dcol >> 2) & 1;
  const bf16x4 lo4 = lds_read_tr16(tile + r1 * kRow + ((chunk ^ swz<kRow>(r1)) << 4) + half * 8);
  const bf16x4 hi4 = lds_read_tr16(tile + r2 * kRow + ((chunk ^ swz<kRow>(r2)) << 4) + half * 8);
  bf16x8 f;
  f[0] = lo4[0]; f[1] = lo4[1]; f[2] = lo4[2]; f[3] = lo4[3];
  f[4] = hi4[0]; f[5] = hi4[1]; f[6] = hi4[2]; f[7] = hi4[3];
  return f;
}

// natural-log LSE -> log2 domain, with rows that see no key sent to +inf
__device__ __forceinline__ float lse_log2(float lse) { return lse == -INFINITY ? INFINITY : lse * kLog2e; }

// ---------------------------------------------------------------- dK, dV
// Workgroup = (sequence, kv-head, 128 keys); wavefront w owns keys
// [k0 + 32 w, +32).  Steps walk the q-heads of the group and, per head, the
// 64-row query tiles that can see any of the workgroup's keys; the Q / dO
// tiles (and their LSE / Delta rows) of the next step load while the
// current one is computed.
// MODE 0 computes both; at D = 128 the K / V fragments and both
// accumulators alone take 192 registers (one wavefront per SIMD), so there
// MODE 1 (dV: S and dV^T += dO^T P) and MODE 2 (dK: S, dP and dK^T += Q^T dS)
// run as two kernels of half the registers, two wavefronts per SIMD each.
template <int D, int MODE>
__global__ __launch_bounds__(kBwThreads) __attribute__((amdgpu_waves_per_eu((D > 64 && MODE == 0) ? 1 : 2)))
void fa_bwd_dkdv_kernel(const BwdArgs a) {
  constexpr bool DOV = MODE != 2, DOK = MODE != 1;
  constexpr int kRow = D * 2;
  constexpr int kTileB = kBwTile * kRow;
  constexpr int kStage = 2 * kTileB + 2 * kBwTile * 4;
  __shared__ __attribute__((aligned(1024))) char lds_raw[2 * kStage];
  char FA_LDS* lds = (char FA_LDS*)(lds_raw);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  // the forward's workgroup order (wg_tile) with key blocks for query
  // tiles: causal calls take key blocks near the start first (they see the
  // most rows), an XCD's (sequence, kv-head) slots in groups of 4 (the
  // backward's units are small enough to balance in smaller groups, which
  // keep fewer slots' Q / dO tiles streaming through an L2) with the slot
  // rotated per level; otherwise all key blocks of one slot in a row
  int bg, lvl;
  wg_tile<4>(a.causal != 0, bg, lvl);
  if (bg >= a.B * a.Hkv) return;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const BwSeq sv = bw_seq(a, b);
  const int k0 = ((int)gridDim.y - 1 - lvl) * kBwKeys;
  if (k0 >= sv.skv) return;
  const int key = k0 + wave * 32 + (lane & 31);
  const bool kvalid = key < sv.skv;
  const int delta_al = sv.skv - sv.sq;

  // K and V fragments of this lane's key (B operands): d = 16 s + 8 (lane/32) + e
  bf16x8 kf[D / 16], vf[D / 16];
  {
    const int64_t kr = sv.kstart + min(key, sv.skv - 1);
    const bf16* kp = a.k + kr * a.k_st + (int64_t)g * a.k_sh + (lane >> 5) * 8;
    const bf16* vp = a.v + kr * a.v_st + (int64_t)g * a.v_sh + (lane >> 5) * 8;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      kf[s] = kvalid ? *reinterpret_cast<const bf16x8*>(kp + 16 * s) : bf16x8{};
      vf[s] = (DOK && kvalid) ? *reinterpret_cast<const bf16x8*>(vp + 16 * s) : bf16x8{};
    }
  }
  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int d = 0; d < D / 32; ++d) dk[d] = dv[d] = f32x16{};

  // query rows that see any key of [k0, j1]
  const int j1 = min(k0 + kBwKeys, sv.skv) - 1;
  int r_lo = 0, r_hi = sv.sq - 1;
  if (a.causal) r_lo = max(r_lo, k0 - delta_al);
  if (a.win_right >= 0) r_lo = max(r_lo, k0 - delta_al - a.win_right);
  if (a.win_left >= 0) r_hi = min(r_hi, j1 + a.win_left - delta_al);
  const int qb0 = r_lo >= 0 ? r_lo / kBwTile : 0;
  const int nqb = r_lo <= r_hi ? r_hi / kBwTile - qb0 + 1 : 0;
  const int nsteps = nqb * a.group;
  const float C = a.qk_scale * kLog2e;

  RowStager<D> st;
  st.init(wave, lane);
  auto stage_ptr = [&](int i) { return lds + i * kStage; };
  float ld_lse = 0.0f, ld_delta = 0.0f;
  // loads of step n into stage buffer sb: Q and dO by DMA, LSE / Delta to registers
  auto issue = [&](int n, int sb) {
    const int h = g * a.group + n / nqb;
    const int r0 = (qb0 + n % nqb) * kBwTile;
    char FA_LDS* sp = stage_ptr(sb);
    st.issue_clamped(a.q + sv.qstart * a.q_st + (int64_t)h * a.q_sh, a.q_st, r0, sv.sq, sp, wave);
    st.issue_clamped(a.dout + sv.qstart * a.o_st + (int64_t)h * a.o_sh, a.o_st, r0, sv.sq, sp + kTileB, wave);
    if (tid < kBwTile) {
      const int r = min(r0 + tid, sv.sq - 1);
      const int64_t li = bw_lse_index(a, b, h, sv.qstart, r);
      ld_lse = a.lse[li];
      ld_delta = a.delta[li];
    }
  };
  auto publish = [&](int sb) {
    if (tid < kBwTile) {
      float FA_LDS* lp = reinterpret_cast<float FA_LDS*>(stage_ptr(sb) + 2 * kTileB);
      lp[tid] = lse_log2(ld_lse);
      lp[kBwTile + tid] = ld_delta;
    }
  };

  if (nsteps > 0) {
    issue(0, 0);
    FA_WAIT_VMCNT(0);
    publish(0);
  }
  for (int n = 0; n < nsteps; ++n) {
    const int sb = n & 1;
    __syncthreads();   // step n visible; everyone is done with the other buffer
    if (n + 1 < nsteps) issue(n + 1, sb ^ 1);
    const char FA_LDS* qt = stage_ptr(sb);
    const char FA_LDS* dt = qt + kTileB;
    const float FA_LDS* lse2 = reinterpret_cast<const float FA_LDS*>(qt + 2 * kTileB);
    const float FA_LDS* dl = lse2 + kBwTile;
    const int r0 = (qb0 + n % nqb) * kBwTile;

    // every row of the tile sees every key of this wavefront: no per-score mask
    const int kw0 = k0 + wave * 32, kw1 = kw0 + 31;
    bool full = kw1 < sv.skv && r0 + kBwTile <= sv.sq;
    if (a.causal) full = full && kw1 <= r0 + delta_al;
    if (a.win_right >= 0) full = full && kw1 <= r0 + delta_al + a.win_right;
    if (a.win_left >= 0) full = full && kw0 >= r0 + kBwTile - 1 + delta_al - a.win_left;
    // the tile's two 32-row halves one after the other (keeps the S / dP
    // accumulators of one half live at a time)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      // S and dP for rows [32 rb, +32)
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int stp = 0; stp < D / 16; ++stp) {
        const int r = rb * 32 + (lane & 31);
        const int off = r * kRow + (((2 * stp + (lane >> 5)) ^ swz<kRow>(r)) << 4);
        s = mfma32(lds_read_b128(qt + off), kf[stp], s);
        if (DOK) dp = mfma32(lds_read_b128(dt + off), vf[stp], dp);
      }
      // P and dS (register i: row 32 rb + 8 (i/4) + 4 (lane/32) + i%4)
      bf16x8 pf[2], dsf[2];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int rr = rb * 32 + q4 * 8 + (lane >> 5) * 4;
        const f32x4 l4 = *reinterpret_cast<const f32x4 FA_LDS*>(lse2 + rr);
        const f32x4 d4 = *reinterpret_cast<const f32x4 FA_LDS*>(dl + rr);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = q4 * 4 + e;
          float p = exp2_hw(fmaf(s[i], C, -l4[e]));
          if (!full) {
            const int qi = r0 + rr + e;
            const int ip = qi + delta_al;
            bool vis = kvalid && qi < sv.sq;
            if (a.causal) vis = vis && key <= ip;
            if (a.win_right >= 0) vis = vis && key <= ip + a.win_right;
            if (a.win_left >= 0) vis = vis && key >= ip - a.win_left;
            p = vis ? p : 0.0f;
          }
          if (DOV) pf[i >> 3][i & 7] = (bf16)p;
          if (DOK) dsf[i >> 3][i & 7] = (bf16)(p * (dp[i] - d4[e]));
        }
      }
      // dV^T += dO^T P and dK^T += Q^T dS over these 32 rows
#pragma unroll
      for (int uu = 0; uu < 2; ++uu) {
#pragma unroll
        for (int d = 0; d < D / 32; ++d) {
          if (DOV) dv[d] = mfma32(tr_fragment<kRow>(dt, rb * 2 + uu, d, lane), pf[uu], dv[d]);
          if (DOK) dk[d] = mfma32(tr_fragment<kRow>(qt, rb * 2 + uu, d, lane), dsf[uu], dk[d]);
        }
      }
    }
    if (n + 1 < nsteps) {
      FA_WAIT_VMCNT(0);
      publish(sb ^ 1);
    }
  }

  // dK^T / dV^T register i of block d: dim 32 d + 8 (i/4) + 4 (lane/32) + i%4
  if (kvalid) {
    const int64_t kr = sv.kstart + key;
    bf16* kp = a.dk + kr * a.k_st + (int64_t)g * a.k_sh + (lane >> 5) * 4;
    bf16* vp = a.dv + kr * a.v_st + (int64_t)g * a.v_sh + (lane >> 5) * 4;
#pragma unroll
    for (int d = 0; d < D / 32; ++d) {
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        bf16x4 wk, wv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          wk[e] = (bf16)(dk[d][gi * 4 + e] * a.qk_scale);
          wv[e] = (bf16)dv[d][gi * 4 + e];
        }
        if (DOK) *reinterpret_cast<bf16x4*>(kp + d * 32 + gi * 8) = wk;
        if (DOV) *reinterpret_cast<bf16x4*>(vp + d * 32 + gi * 8) = wv;
      }
    }
  }
}

// ---------------------------------------------------------------- dK + dV, 16 keys per wavefront
// One kernel for both gradients at D = 128: a wavefront owns 16 keys, so its
// K and V fragments (2 x 16 registers) and its dK^T, dV^T accumulators
// (2 x 32) leave room for two wavefronts per SIMD, and S and dP are
// computed once per (row, key) for both gradients.  Products are
// v_mfma_f32_16x16x32_bf16 (lane l: A row / B column l%16, the 8 contraction
// slots 8 (l/16) + j; accumulator: column l%16, rows 4 (l/16) + i):
//   S  [16 rows x 16 keys] = Q K^T     A = Q rows from LDS, B = K in registers
//   dP [16 rows x 16 keys] = dO V^T    A = dO rows from LDS, B = V in registers
//   dV^T [16 d x keys] += dO^T P       over 32 rows: A = dO read transposed,
//   dK^T [16 d x keys] += Q^T dS         B = P / dS from two row blocks' accumulators
// Contraction slot j of lane group g = l/16 holds row 4 g + j (j < 4) or
// 16 + 4 g + j - 4 (the rows the two accumulators give that lane); the
// transposed reads fetch the same rows (any bijection of the summed rows
// serves, as long as both operands use it).
constexpr int kBw16Keys = 16 * kBwWaves;   // keys per workgroup

__device__ __forceinline__ f32x4 bw_mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// A fragment of a 16x16x32 transposed product from a 64-row tile (swz_bw16):
// columns [16 dblk, +16) (lane l: column 16 dblk + l%16) and the 32 rows
// 32 half + {4 g + [0, 4), 16 + 4 g + [0, 4)} of lane group g.
template <int kRow>
__device__ __forceinline__ bf16x8 tr_fragment16(const char FA_LDS* tile, int half, int dblk, int lane) {
  const int grp = lane >> 4, i16 = lane & 15;
  const int r1 = half * 32 + 4 * grp + (i16 >> 2);
  const int r2 = r1 + 16;
  const int dcol = dblk * 16 + 4 * (i16 & 3);
  const int chunk = dcol >> 3, hv = (dcol >> 2) & 1;
  const bf16x4 lo4 = lds_read_tr16(tile + r1 * kRow + ((chunk ^ swz_bw16(r1)) << 4) + hv * 8);
  const bf16x4 hi4 = lds_read_tr16(tile + r2 * kRow + ((chunk ^ swz_bw16(r2)) << 4) + hv * 8);
  bf16x8 f;
  f[0] = lo4[0]; f[1] = lo4[1]; f[2] = lo4[2]; f[3] = lo4[3];
  f[4] = hi4[0]; f[5] = hi4[1]; f[6] = hi4[2]; f[7] = hi4[3];
  return f;
}

template <int D>
__global__ __launch_bounds__(kBwThreads) __attribute__((amdgpu_waves_per_eu(2)))
void fa_bwd_dkdv16_kernel(const BwdArgs a) {
  static_assert(D == 128, "swz_bw16 is a map on the 16 chunks of 256-byte rows");
  constexpr int kRow = D * 2;
  constexpr int kTileB = kBwTile * kRow;
  constexpr int kStage = 2 * kTileB + 2 * kBwTile * 4;
  constexpr int NS = D / 32;                 // contraction steps of S and dP
  constexpr int ND = D / 16;                 // 16-wide output blocks of dK^T, dV^T
  __shared__ __attribute__((aligned(1024))) char lds_raw[2 * kStage];
  char FA_LDS* lds = (char FA_LDS*)(lds_raw);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int grp = lane >> 4;
  // workgroup order as in the 32-key kernel (wg_tile, key blocks near the
  // start first for causal calls)
  int bg, lvl;
  wg_tile<4>(a.causal != 0, bg, lvl);
  if (bg >= a.B * a.Hkv) return;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const BwSeq sv = bw_seq(a, b);
  const int k0 = ((int)gridDim.y - 1 - lvl) * kBw16Keys;
  if (k0 >= sv.skv) return;
  const int key = k0 + wave * 16 + (lane & 15);
  const bool kvalid = key < sv.skv;
  const int delta_al = sv.skv - sv.sq;

  // K and V fragments of this lane's key (B operands): d = 32 s + 8 grp + e
  bf16x8 kf[NS], vf[NS];
  {
    const int64_t kr = sv.kstart + min(key, sv.skv - 1);
    const bf16* kp = a.k + kr * a.k_st + (int64_t)g * a.k_sh + grp * 8;
    const bf16* vp = a.v + kr * a.v_st + (int64_t)g * a.v_sh + grp * 8;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      kf[s] = kvalid ? *reinterpret_cast<const bf16x8*>(kp + 32 * s) : bf16x8{};
      vf[s] = kvalid ? *reinterpret_cast<const bf16x8*>(vp + 32 * s) : bf16x8{};
    }
  }
  f32x4 dk[ND], dv[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) dk[d] = dv[d] = f32x4{};

  // rows that see this lane's key: [my_qlo, my_qlo + my_cnt) (causal:
  // i + delta >= key; windows: key - delta - right <= i <= key - delta + left)
  int my_qlo = 0, my_qhi = sv.sq - 1;
  if (a.causal) my_qlo = max(my_qlo, key - delta_al);
  if (a.win_right >= 0) my_qlo = max(my_qlo, key - delta_al - a.win_right);
  if (a.win_left >= 0) my_qhi = min(my_qhi, key - delta_al + a.win_left);
  const unsigned my_cnt = kvalid ? (unsigned)max(my_qhi - my_qlo + 1, 0) : 0u;

  // query rows that see any key of [k0, j1]
  const int j1 = min(k0 + kBw16Keys, sv.skv) - 1;
  int r_lo = 0, r_hi = sv.sq - 1;
  if (a.causal) r_lo = max(r_lo, k0 - delta_al);
  if (a.win_right >= 0) r_lo = max(r_lo, k0 - delta_al - a.win_right);
  if (a.win_left >= 0) r_hi = min(r_hi, j1 + a.win_left - delta_al);
  const int qb0 = r_lo >= 0 ? r_lo / kBwTile : 0;
  const int nqb = r_lo <= r_hi ? r_hi / kBwTile - qb0 + 1 : 0;
  const int nsteps = nqb * a.group;
  const float C = a.qk_scale * kLog2e;

  RowStager<D, true> st;
  st.init(wave, lane);
  unsigned offq[RowStager<D, true>::kPerWave], offo[RowStager<D, true>::kPerWave];
  st.offsets(a.q_st, offq);
  st.offsets(a.o_st, offo);
  auto stage_ptr = [&](int i) { return lds + i * kStage; };
  float ld_lse = 0.0f, ld_delta = 0.0f;
  auto issue = [&](int n, int sb) {
    const int h = g * a.group + n / nqb;
    const int r0 = (qb0 + n % nqb) * kBwTile;
    char FA_LDS* sp = stage_ptr(sb);
    const bf16* qb = a.q + sv.qstart * a.q_st + (int64_t)h * a.q_sh;
    const bf16* ob = a.dout + sv.qstart * a.o_st + (int64_t)h * a.o_sh;
    if (r0 + kBwTile <= sv.sq) {
      st.issue_whole(qb, a.q_st, r0, offq, sp, wave);
      st.issue_whole(ob, a.o_st, r0, offo, sp + kTileB, wave);
    } else {
      st.issue_clamped(qb, a.q_st, r0, sv.sq, sp, wave);
      st.issue_clamped(ob, a.o_st, r0, sv.sq, sp + kTileB, wave);
    }
    if (tid < kBwTile) {
      const int64_t l0 = bw_lse_index(a, b, h, sv.qstart, 0);   // rows of one (sequence, head) are contiguous
      const int r = min(r0 + tid, sv.sq - 1);
      ld_lse = a.lse[l0 + r];
      ld_delta = a.delta[l0 + r];
    }
  };
  auto publish = [&](int sb) {
    if (tid < kBwTile) {
      float FA_LDS* lp = reinterpret_cast<float FA_LDS*>(stage_ptr(sb) + 2 * kTileB);
      lp[tid] = lse_log2(ld_lse);
      lp[kBwTile + tid] = ld_delta;
    }
  };

  if (nsteps > 0) {
    issue(0, 0);
    FA_WAIT_VMCNT(0);
    publish(0);
  }
  for (int n = 0; n < nsteps; ++n) {
    const int sb = n & 1;
    __syncthreads();   // step n visible; everyone is done with the other buffer
    if (n + 1 < nsteps) issue(n + 1, sb ^ 1);
    const char FA_LDS* qt = stage_ptr(sb);
    const char FA_LDS* dt = qt + kTileB;
    const float FA_LDS* lse2 = reinterpret_cast<const float FA_LDS*>(qt + 2 * kTileB);
    const float FA_LDS* dl = lse2 + kBwTile;
    const int r0 = (qb0 + n % nqb) * kBwTile;

    // every row of the tile sees every key of this wavefront: no per-score mask
    const int kw0 = k0 + wave * 16, kw1 = kw0 + 15;
    bool full = kw1 < sv.skv && r0 + kBwTile <= sv.sq;
    if (a.causal) full = full && kw1 <= r0 + delta_al;
    if (a.win_right >= 0) full = full && kw1 <= r0 + delta_al + a.win_right;
    if (a.win_left >= 0) full = full && kw0 >= r0 + kBwTile - 1 + delta_al - a.win_left;
    // S and dP of all 64 rows (four 16-row blocks) first, then P and dS,
    // then the dV / dK products.  Each product's A fragment is read kAhead
    // products before it, in a fixed order (one scheduling barrier per
    // product), so a wavefront waits only for reads kAhead products old.
    constexpr int NSP = 2 * 4 * NS;            // S and dP products: (block rb, step, S | dP)
    constexpr int NKV = 2 * 2 * ND;            // dV and dK products: (half, block d, dV | dK)
    constexpr int kAhead = 4;
    auto sp_read = [&](int i) {
      const int rb = i / (2 * NS), stp = (i >> 1) % NS;
      const int r = rb * 16 + (lane & 15);
      return lds_read_b128(((i & 1) ? dt : qt) + r * kRow + (((4 * stp + grp) ^ swz_bw16(r)) << 4));
    };
    auto kv_read = [&](int i) {
      return tr_fragment16<kRow>((i & 1) ? qt : dt, i / (2 * ND), (i >> 1) % ND, lane);
    };
    f32x4 s[4], dp[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) s[rb] = dp[rb] = f32x4{};
    bf16x8 af[NSP];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) af[i] = sp_read(i);
#pragma unroll
    for (int i = 0; i < NSP; ++i) {
      if (i + kAhead < NSP) af[i + kAhead] = sp_read(i + kAhead);
      const int rb = i / (2 * NS), stp = (i >> 1) % NS;
      if (i & 1) dp[rb] = bw_mfma16(af[i], vf[stp], dp[rb]);
      else s[rb] = bw_mfma16(af[i], kf[stp], s[rb]);
      __builtin_amdgcn_sched_barrier(0);
    }
    // P (in place of S): accumulator register i of block rb is row
    // 16 rb + 4 grp + i
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const f32x4 l4 = *reinterpret_cast<const f32x4 FA_LDS*>(lse2 + rb * 16 + grp * 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) s[rb][i] = exp2_hw(fmaf(s[rb][i], C, -l4[i]));
    }
    if (!full) {
      // the bounds pass through an opaque copy made here, so the selects stay
      // inside this branch instead of being speculated onto every tile
      int base = r0 + grp * 4 - my_qlo;
      unsigned cnt = my_cnt;
      asm volatile("" : "+v"(base), "+v"(cnt));
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          s[rb][i] = (unsigned)(base + rb * 16 + i) < cnt ? s[rb][i] : 0.0f;
    }
    // dS = P (dP - Delta); half hf takes blocks 2 hf and 2 hf + 1
    bf16x8 pf[2], dsf[2];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const f32x4 d4 = *reinterpret_cast<const f32x4 FA_LDS*>(dl + rb * 16 + grp * 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pf[rb >> 1][(rb & 1) * 4 + i] = (bf16)s[rb][i];
        dsf[rb >> 1][(rb & 1) * 4 + i] = (bf16)(s[rb][i] * (dp[rb][i] - d4[i]));
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    bf16x8 tf[NKV];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) tf[i] = kv_read(i);
    // dV^T += dO^T P and dK^T += Q^T dS over the two 32-row halves
#pragma unroll
    for (int i = 0; i < NKV; ++i) {
      if (i + kAhead < NKV) tf[i + kAhead] = kv_read(i + kAhead);
      const int hf = i / (2 * ND), d = (i >> 1) % ND;
      if (i & 1) dk[d] = bw_mfma16(tf[i], dsf[hf], dk[d]);
      else dv[d] = bw_mfma16(tf[i], pf[hf], dv[d]);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (n + 1 < nsteps) {
      FA_WAIT_VMCNT(0);
      publish(sb ^ 1);
    }
  }

  // dK^T / dV^T register i of block d: dim 16 d + 4 grp + i of this lane's key
  if (kvalid) {
    const int64_t kr = sv.kstart + key;
    bf16* kp = a.dk + kr * a.k_st + (int64_t)g * a.k_sh + grp * 4;
    bf16* vp = a.dv + kr * a.v_st + (int64_t)g * a.v_sh + grp * 4;
#pragma unroll
    for (int d = 0; d < ND; ++d) {
      bf16x4 wk, wv;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        wk[i] = (bf16)(dk[d][i] * a.qk_scale);
        wv[i] = (bf16)dv[d][i];
      }
      *reinterpret_cast<bf16x4*>(kp + d * 16) = wk;
      *reinterpret_cast<bf16x4*>(vp + d * 16) = wv;
    }
  }
}

// ---------------------------------------------------------------- dQ
// Workgroup = (sequence, q-head, 128 query rows), as the forward kernel;
// 64-key K / V tiles stream through two LDS stages.  It also computes and
// stores Delta of its rows, so it runs before the dK / dV kernel.
template <int D>
__global__ __launch_bounds__(kBwThreads) __attribute__((amdgpu_waves_per_eu(2)))
void fa_bwd_dq_kernel(const BwdArgs a) {
  constexpr int kRow = D * 2;
  constexpr int kTileB = kBwTile * kRow;
  constexpr int kStage = 2 * kTileB;
  __shared__ __attribute__((aligned(1024))) char lds_raw[2 * kStage];
  char FA_LDS* lds = (char FA_LDS*)(lds_raw);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  // the forward's workgroup order (wg_tile): causal calls start with the
  // longest query tiles (the last ones), so the grid ends on short tiles,
  // an XCD's (sequence, head) slots in groups of 4 with the slot rotated per
  // level; otherwise all query tiles of one slot in a row
  int bh, qt;
  wg_tile<4>(a.causal != 0, bh, qt);
  if (bh >= a.B * a.Hq) return;
  const int b = bh / a.Hq, h = bh % a.Hq, g = h / a.group;
  const BwSeq sv = bw_seq(a, b);
  const int q0 = qt * kBwRowsQ;
  if (q0 >= sv.sq) return;
  const int q1 = min(q0 + kBwRowsQ, sv.sq);
  const int delta_al = sv.skv - sv.sq;
  const int qrow = q0 + wave * 32 + (lane & 31);
  const bool qvalid = qrow < sv.sq;
  const int ip = qrow + delta_al;

  // Q and dO fragments of this lane's row (B operands)
  bf16x8 qf[D / 16], of[D / 16];
  {
    const int64_t t = sv.qstart + (qvalid ? qrow : 0);
    const bf16* qp = a.q + t * a.q_st + (int64_t)h * a.q_sh + (lane >> 5) * 8;
    const bf16* op = a.dout + t * a.o_st + (int64_t)h * a.o_sh + (lane >> 5) * 8;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      qf[s] = qvalid ? *reinterpret_cast<const bf16x8*>(qp + 16 * s) : bf16x8{};
      of[s] = qvalid ? *reinterpret_cast<const bf16x8*>(op + 16 * s) : bf16x8{};
    }
  }
  // Delta of this lane's row: its half of dO . O (the d values of of[]),
  // plus the other half from lane ^ 32; written for the dK / dV kernel,
  // which runs after this one
  float dlt = 0.0f;
  {
    const int64_t t = sv.qstart + (qvalid ? qrow : 0);
    const bf16* opo = a.o + t * a.o_st + (int64_t)h * a.o_sh + (lane >> 5) * 8;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const bf16x8 ov = qvalid ? *reinterpret_cast<const bf16x8*>(opo + 16 * s) : bf16x8{};
#pragma unroll
      for (int e = 0; e < 8; ++e) dlt = fmaf((float)ov[e], (float)of[s][e], dlt);
    }
    dlt += __shfl_xor(dlt, 32);
  }
  float lse2 = INFINITY;
  if (qvalid) {
    const int64_t li = bw_lse_index(a, b, h, sv.qstart, qrow);
    lse2 = lse_log2(a.lse[li]);
    if (lane < 32) a.delta[li] = dlt;
  }
  f32x16 dq[D / 32];
#pragma unroll
  for (int d = 0; d < D / 32; ++d) dq[d] = f32x16{};

  // key tiles that any row of the workgroup sees
  auto row_hi = [&](int i) {
    int hi = sv.skv - 1;
    if (a.causal) hi = min(hi, i + delta_al);
    if (a.win_right >= 0) hi = min(hi, i + delta_al + a.win_right);
    return hi;
  };
  auto row_lo = [&](int i) {
    int lo = 0;
    if (a.win_left >= 0) lo = max(lo, i + delta_al - a.win_left);
    return lo;
  };
  const int lo_min = row_lo(q0), hi_max = row_hi(q1 - 1);
  const int t_begin = lo_min / kBwTile;
  const int t_end = hi_max >= lo_min ? hi_max / kBwTile : t_begin - 1;
  const int my_lo = row_lo(qrow), my_hi = row_hi(qrow);
  const unsigned my_cnt = qvalid ? (unsigned)max(my_hi - my_lo + 1, 0) : 0u;   // keys [my_lo, my_lo + my_cnt)
  // this wavefront's rows [wq0, wq1]: the intersection of their key ranges
  const int wq0 = q0 + wave * 32, wq1 = wq0 + 31;
  const bool wave_rows_full = wq1 < sv.sq;
  const int wave_lo_max = row_lo(wq1), wave_hi_min = row_hi(wq0);
  const float C = a.qk_scale * kLog2e;

  RowStager<D> st;
  st.init(wave, lane);
  // whole tiles share one set of 32-bit offsets (K and V rows have the same
  // stride here: D_qk = D_v)
  unsigned offk[RowStager<D>::kPerWave];
  st.offsets(a.k_st, offk);
  const bool whole_ok = a.k_st == a.v_st;
  auto stage_ptr = [&](int i) { return lds + i * kStage; };
  const bf16* kbase = a.k + sv.kstart * a.k_st + (int64_t)g * a.k_sh;
  const bf16* vbase = a.v + sv.kstart * a.v_st + (int64_t)g * a.v_sh;
  auto issue = [&](int t, int sb) {
    if (whole_ok && (t + 1) * kBwTile <= sv.skv) {
      st.issue_whole(kbase, a.k_st, t * kBwTile, offk, stage_ptr(sb), wave);
      st.issue_whole(vbase, a.v_st, t * kBwTile, offk, stage_ptr(sb) + kTileB, wave);
    } else {
      st.issue_clamped(kbase, a.k_st, t * kBwTile, sv.skv, stage_ptr(sb), wave);
      st.issue_clamped(vbase, a.v_st, t * kBwTile, sv.skv, stage_ptr(sb) + kTileB, wave);
    }
  };
  if (t_begin <= t_end) {
    issue(t_begin, 0);
    FA_WAIT_VMCNT(0);
  }
  for (int t = t_begin; t <= t_end; ++t) {
    const int sb = (t - t_begin) & 1;
    __syncthreads();
    if (t + 1 <= t_end) issue(t + 1, sb ^ 1);
    const char FA_LDS* kt = stage_ptr(sb);
    const char FA_LDS* vt = kt + kTileB;
    const int k0 = t * kBwTile;

    // S^T and dP^T for keys [32 kb, +32) of the tile; each product's K / V
    // fragment is read kAheadQ products before it, in a fixed order
    constexpr int NP = 4 * (D / 16);           // (step, key block, S | dP)
    constexpr int kAheadQ = 2;                 // 4 measured the same, 6 spills
    auto kv_frag = [&](int i) {
      const int stp = i >> 2, kb = (i >> 1) & 1;
      const int r = kb * 32 + (lane & 31);
      return lds_read_b128(((i & 1) ? vt : kt) + r * kRow + (((2 * stp + (lane >> 5)) ^ swz<kRow>(r)) << 4));
    };
    f32x16 s[2] = {f32x16{}, f32x16{}}, dp[2] = {f32x16{}, f32x16{}};
    bf16x8 fr[NP];
#pragma unroll
    for (int i = 0; i < kAheadQ; ++i) fr[i] = kv_frag(i);
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      if (i + kAheadQ < NP) fr[i + kAheadQ] = kv_frag(i + kAheadQ);
      const int stp = i >> 2, kb = (i >> 1) & 1;
      if (i & 1) dp[kb] = mfma32(fr[i], of[stp], dp[kb]);
      else s[kb] = mfma32(fr[i], qf[stp], s[kb]);
      __builtin_amdgcn_sched_barrier(0);
    }
    // P^T in place of S^T (register i of key block kb: key 32 kb + 8 (i/4) +
    // 4 (lane/32) + i%4), then the mask, then dS^T; tiles inside every row's
    // key range of this wavefront skip the mask
    const bool full = wave_rows_full && k0 >= wave_lo_max && k0 + kBwTile - 1 <= wave_hi_min;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = exp2_hw(fmaf(s[kb][i], C, -lse2));
    if (!full) {
      // the bounds pass through an opaque copy made here, so the selects stay
      // inside this branch instead of being speculated onto every tile
      int base = k0 + (lane >> 5) * 4 - my_lo;
      unsigned cnt = my_cnt;
      asm volatile("" : "+v"(base), "+v"(cnt));
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          s[kb][i] = (unsigned)(base + kb * 32 + (i >> 2) * 8 + (i & 3)) < cnt ? s[kb][i] : 0.0f;
    }
    bf16x8 dsf[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) dsf[kb * 2 + (i >> 3)][i & 7] = (bf16)(s[kb][i] * (dp[kb][i] - dlt));
    // dQ^T += K^T dS^T over the tile's 64 keys
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int d = 0; d < D / 32; ++d) dq[d] = mfma32(tr_fragment<kRow>(kt, u, d, lane), dsf[u], dq[d]);
    }
    if (t + 1 <= t_end) FA_WAIT_VMCNT(0);
  }

  if (qvalid) {
    bf16* qp = a.dq + (sv.qstart + qrow) * a.q_st + (int64_t)h * a.q_sh + (lane >> 5) * 4;
#pragma unroll
    for (int d = 0; d < D / 32; ++d) {
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (bf16)(dq[d][gi * 4 + e] * a.qk_scale);
        *reinterpret_cast<bf16x4*>(qp + d * 32 + gi * 8) = w;
      }
    }
  }
}

template <int D>
static hipError_t launch_bwd(const BwdArgs& a, int max_sq, int max_skv, hipStream_t stream) {
  // dQ first: it also writes Delta, which the dK / dV kernel reads
  if (max_sq > 0) {
    // grid x: slots rounded up to a multiple of the 8 XCDs (wg_tile's map)
    hipLaunchKernelGGL(fa_bwd_dq_kernel<D>, dim3((a.B * a.Hq + 7) / 8 * 8, (max_sq + kBwRowsQ - 1) / kBwRowsQ),
                       dim3(kBwThreads), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (max_skv > 0) {
    if constexpr (D > 64) {
      const dim3 grid((a.B * a.Hkv + 7) / 8 * 8, (max_skv + kBw16Keys - 1) / kBw16Keys);
      hipLaunchKernelGGL((fa_bwd_dkdv16_kernel<D>), grid, dim3(kBwThreads), 0, stream, a);
    } else {
      const dim3 grid((a.B * a.Hkv + 7) / 8 * 8, (max_skv + kBwKeys - 1) / kBwKeys);
      hipLaunchKernelGGL((fa_bwd_dkdv_kernel<D, 0>), grid, dim3(kBwThreads), 0, stream, a);
    }
  }
  return hipGetLastError();
}

hipError_t bwd_dispatch(const BwdArgs& a, int d, int max_sq, int max_skv, hipStream_t stream, bool* supported) {
  *supported = true;
  if (d == 64) return launch_bwd<64>(a, max_sq, max_skv, stream);
  if (d == 128) return launch_bwd<128>(a, max_sq, max_skv, stream);
  *supported = false;
  return hipSuccess;
}

}  // namespace fa
