// Fused attention forward (prefill / dense / varlen / paged) for gfx950.
//
// One workgroup = 4 wavefronts = 128 query rows of one (sequence, q-head);
// each wavefront owns 32 query rows.  The key axis is walked in tiles of 64
// keys staged in LDS (double buffered).  Per tile and wavefront:
//
//   S^T[64 x 32]  = K_tile . Q^T          v_mfma_f32_32x32x16_bf16, A = K from LDS,
//                                          B = Q fragments kept in registers
//   online softmax on S^T                 lane l owns query row l%32; the row
//                                          max needs one permlane32 swap
//   O^T[Dv x 32] += V_tile^T . P^T        A = V read transposed from LDS
//                                          (ds_read_b64_tr_b16), B = P in registers
//
// Computing the transposed products keeps every per-row quantity (running
// max, denominator, rescale factor, output scaling) lane-local.  The P^T
// operand taken straight from the S^T accumulator enumerates the 16 keys of
// an MFMA step in the order that swaps bits 2 and 3 of the key index; the V
// transposed reads fetch rows in that same order, so K and V stay paired.
//
// Softmax works in the log2 domain: the running max m is kept in units of
// scale*log2(e)*logit so that p = exp2(fma(x, C, -m)) is one FMA and one
// v_exp_f32 per score (method: LSE PR, "log2 domain with the logit scale
// folded"; the paged FP8 PR folds the K descale into that same constant).
// The output is rescaled only when some row's max grows by more than 2^8
// (lazy rescaling, paged FP8 PR review), which leaves the result unchanged.
//
// Masking is by select to -inf (never by multiply, so NaN bytes in unused
// cache slots cannot leak), with rows that see no key producing O = 0 and
// LSE = -inf.  Tiles wholly outside the causal / window range or inactive in
// the block mask are skipped; tiles wholly inside skip the per-score mask.
//
// K/V staging: bf16 K/V go global -> LDS with global_load_lds_dwordx4 (no
// registers); FP8 E4M3 K/V are loaded to registers one tile ahead, converted
// exactly to bf16 and written to LDS.  LDS rows are 16-byte-chunk XOR
// swizzled (chunk c of row r stored at c ^ (r & 7)) so that both the K reads
// and the transposed V reads are bank-conflict free.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

constexpr int BM = 128;
constexpr int BN = 64;
constexpr int NTHREADS = 256;
constexpr float kLazyTau = 8.0f;

template <int DQK, int DV, bool FP8>
struct PrefillTraits {
  static constexpr int kRowK = DQK * 2;            // bytes per bf16 K row in LDS
  static constexpr int kRowV = DV * 2;
  static constexpr int kTileK = BN * kRowK;
  static constexpr int kTileV = BN * kRowV;
  static constexpr int kStage = kTileK + kTileV;
  static constexpr int kLds = 2 * kStage;
  static constexpr int kKItems = BN * DQK / 16;    // 16-byte source items per K tile (fp8)
  static constexpr int kVItems = BN * DV / 16;
  static constexpr int kKPer = (kKItems + NTHREADS - 1) / NTHREADS;
  static constexpr int kVPer = (kVItems + NTHREADS - 1) / NTHREADS;
};

struct SeqView {
  int b, h, g;
  int sq, skv;            // lengths of this sequence
  int64_t qstart, kstart; // first token row (packed Q/O; contiguous K/V)
};

// Element offset of key row j.  `tile_page` is the wave-uniform page of the
// tile when pages hold at least one whole tile (page_size >= 64), else -1
// and each row looks its page up.
__device__ __forceinline__ int64_t key_row_offset(const PrefillArgs& a, const SeqView& sv, int j,
                                                  int64_t tok_stride, int64_t head_stride,
                                                  int64_t page_stride, bool paged, int tile_page) {
  if (paged) {
    int page = tile_page >= 0 ? tile_page : a.block_table[(int64_t)sv.b * a.max_pages + (j >> a.page_shift)];
    page = min(max(page, 0), a.num_pages - 1);      // never read outside the cache
    const int slot = j & ((1 << a.page_shift) - 1);
    return (int64_t)page * page_stride + (int64_t)sv.g * head_stride + (int64_t)slot * tok_stride;
  }
  return (sv.kstart + j) * tok_stride + (int64_t)sv.g * head_stride;
}

// Page of tile k0 when a page spans whole tiles (scalar load), else -1.
__device__ __forceinline__ int tile_page_of(const PrefillArgs& a, const SeqView& sv, int k0, bool paged) {
  if (!paged || a.page_shift < 6) return -1;
  return load_uniform_i32(a.block_table, (int64_t)sv.b * a.max_pages + (k0 >> a.page_shift));
}

// Issue the bf16 copy of one K or V tile into LDS (global_load_lds).
template <int D, bool PAGED>
__device__ __forceinline__ void stage_bf16(const PrefillArgs& a, const SeqView& sv, const bf16* base,
                                           int64_t tok_stride, int64_t head_stride, int64_t page_stride,
                                           char FA_LDS* tile, int k0, int tile_page) {
  constexpr int kRow = D * 2;
  constexpr int kInstr = BN * kRow / 1024;          // 1 KB per wave instruction
  constexpr int kPerWave = kInstr / 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < kPerWave; ++i) {
    const int n = wave * kPerWave + i;
    const int byte = n * 1024 + lane * 16;
    const int r = byte / kRow;
    const int pos = (byte % kRow) >> 4;
    const int c = pos ^ (r & 7);
    int j = k0 + r;
    j = j < sv.skv ? j : sv.skv - 1;                 // clamp: tail rows are masked anyway
    const int64_t off = key_row_offset(a, sv, j, tok_stride, head_stride, page_stride, PAGED, tile_page);
    global_to_lds16(base + off + c * 8, tile + n * 1024);
  }
}

template <int D>
struct Fp8Regs {
  static constexpr int kItems = BN * D / 16;
  static constexpr int kPer = (kItems + NTHREADS - 1) / NTHREADS;
  i32x4 w[kPer];
};

template <int D, bool PAGED>
__device__ __forceinline__ void load_fp8(const PrefillArgs& a, const SeqView& sv, const uint8_t* base,
                                         int64_t tok_stride, int64_t head_stride, int64_t page_stride,
                                         Fp8Regs<D>& regs, int k0, int tile_page) {
  constexpr int kPerRow = D / 16;
#pragma unroll
  for (int it = 0; it < Fp8Regs<D>::kPer; ++it) {
    const int idx = it * NTHREADS + threadIdx.x;
    if (Fp8Regs<D>::kItems % NTHREADS == 0 || idx < Fp8Regs<D>::kItems) {
      const int r = idx / kPerRow, f = idx % kPerRow;
      int j = k0 + r;
      j = j < sv.skv ? j : sv.skv - 1;
      const int64_t off = key_row_offset(a, sv, j, tok_stride, head_stride, page_stride, PAGED, tile_page);
      regs.w[it] = *reinterpret_cast<const i32x4*>(base + off + f * 16);
    }
  }
}

template <int D>
__device__ __forceinline__ void store_fp8(const Fp8Regs<D>& regs, char FA_LDS* tile) {
  constexpr int kPerRow = D / 16;
  constexpr int kRow = D * 2;
#pragma unroll
  for (int it = 0; it < Fp8Regs<D>::kPer; ++it) {
    const int idx = it * NTHREADS + threadIdx.x;
    if (Fp8Regs<D>::kItems % NTHREADS == 0 || idx < Fp8Regs<D>::kItems) {
      const int r = idx / kPerRow, f = idx % kPerRow;
      bf16x8 lo, hi;
      fp8x16_to_bf16(regs.w[it], lo, hi);
      char FA_LDS* row = tile + r * kRow;
      *reinterpret_cast<bf16x8 FA_LDS*>(row + (((2 * f) ^ (r & 7)) << 4)) = lo;
      *reinterpret_cast<bf16x8 FA_LDS*>(row + (((2 * f + 1) ^ (r & 7)) << 4)) = hi;
    }
  }
}

__device__ __forceinline__ bool tile_active(const PrefillArgs& a, const SeqView& sv, int q0, int t) {
  if (!a.bmask) return true;
  const int64_t row = ((int64_t)sv.b * a.Hq + sv.h) * a.bm_nqb + q0 / a.bm_bq;
  return a.bmask[row * a.bm_nkb + (t * BN) / a.bm_bk] != 0;
}

template <int DQK, int DV, bool FP8, bool PAGED, int MODS>
__global__ __launch_bounds__(NTHREADS) __attribute__((amdgpu_waves_per_eu(2)))
void fa_prefill_kernel(const PrefillArgs a) {
  using T = PrefillTraits<DQK, DV, FP8>;
  __shared__ __attribute__((aligned(1024))) char lds_raw[T::kLds];
  char FA_LDS* lds = (char FA_LDS*)(lds_raw);

  constexpr bool ALIBI = (MODS & kModAlibi) != 0;
  constexpr bool SOFTCAP = (MODS & kModSoftcap) != 0;
  constexpr bool ANYMOD = ALIBI || SOFTCAP;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int bh = blockIdx.x;
  const int qt = (int)gridDim.y - 1 - (int)blockIdx.y;   // longest causal tiles first
  SeqView sv;
  sv.b = bh / a.Hq;
  sv.h = bh % a.Hq;
  sv.g = sv.h / a.group;
  if (a.cu_q) {
    const int s0 = a.cu_q[sv.b], s1 = a.cu_q[sv.b + 1];
    sv.qstart = s0;
    sv.sq = s1 - s0;
  } else {
    sv.qstart = (int64_t)sv.b * a.Sq;
    sv.sq = a.Sq;
  }
  if (PAGED) {
    sv.kstart = 0;
    sv.skv = (int)min((int64_t)a.seqlen_k[sv.b], (int64_t)a.max_pages << a.page_shift);   // bounded page-table lookups
  } else if (a.cu_k) {
    const int s0 = a.cu_k[sv.b], s1 = a.cu_k[sv.b + 1];
    sv.kstart = s0;
    sv.skv = s1 - s0;
  } else {
    sv.kstart = (int64_t)sv.b * a.Skv;
    sv.skv = a.Skv;
  }
  const int q0 = qt * BM;
  if (q0 >= sv.sq) return;
  const int q1 = min(q0 + BM, sv.sq);
  const int delta = sv.skv - sv.sq;

  // Visible key interval of a row i (aligned position i' = i + delta).
  auto row_hi = [&](int i) {
    int hi = sv.skv - 1;
    if (a.causal) hi = min(hi, i + delta);
    if (a.win_right >= 0) hi = min(hi, i + delta + a.win_right);
    return hi;
  };
  auto row_lo = [&](int i) {
    int lo = 0;
    if (a.win_left >= 0) lo = max(lo, i + delta - a.win_left);
    return lo;
  };

  const int lo_min = row_lo(q0), hi_max = row_hi(q1 - 1);
  int t_begin = lo_min / BN, t_end = hi_max >= 0 ? hi_max / BN : -1;
  if (hi_max < lo_min) t_end = t_begin - 1;

  // ---- per-lane query row and its Q fragments (B operand of S^T = K Q^T) ----
  const int qrow = q0 + wave * 32 + (lane & 31);
  const bool qvalid = qrow < sv.sq;
  bf16x8 qf[DQK / 16];
  {
    const bf16* qp = a.q + (sv.qstart + (qvalid ? qrow : 0)) * a.q_st + (int64_t)sv.h * a.q_sh + (lane >> 5) * 8;
#pragma unroll
    for (int s = 0; s < DQK / 16; ++s) {
      bf16x8 v = *reinterpret_cast<const bf16x8*>(qp + s * 16);
      if (!qvalid) v = bf16x8{};
      qf[s] = v;
    }
  }
  const int my_lo = row_lo(qrow), my_hi = row_hi(qrow);
  const int wq0 = q0 + wave * 32;
  const int wave_lo_max = row_lo(wq0 + 31), wave_hi_min = row_hi(wq0);

  float kdesc = 1.0f, vdesc = 1.0f;
  if (FP8) {
    kdesc = *a.k_descale;
    vdesc = *a.v_descale;
  }
  // C: multiplier from the raw MFMA dot product to log2-domain scaled logits
  const float C = ANYMOD ? 1.0f : a.qk_scale * kLog2e * kdesc;
  const float raw_scale = a.qk_scale * kdesc;      // raw dot -> natural scaled logit
  const float cap = a.softcap, inv_cap = SOFTCAP ? 1.0f / a.softcap : 0.0f;
  const int ip = qrow + delta;

  f32x16 oacc[DV / 32];
#pragma unroll
  for (int d = 0; d < DV / 32; ++d) oacc[d] = f32x16{};
  float m_run = kMaxFloor, l_run = 0.0f;

  // find first active tile
  while (t_begin <= t_end && !tile_active(a, sv, q0, t_begin)) ++t_begin;

  char FA_LDS* stage0 = lds;
  char FA_LDS* stage1 = lds + T::kStage;
  const int64_t kpg = a.k_pg, vpg = a.v_pg;

  Fp8Regs<DQK> kreg;
  Fp8Regs<DV> vreg;

  if (t_begin <= t_end) {
    const int tp = tile_page_of(a, sv, t_begin * BN, PAGED);
    if (FP8) {
      load_fp8<DQK, PAGED>(a, sv, reinterpret_cast<const uint8_t*>(a.k), a.k_st, a.k_sh, kpg, kreg, t_begin * BN, tp);
      load_fp8<DV, PAGED>(a, sv, reinterpret_cast<const uint8_t*>(a.v), a.v_st, a.v_sh, vpg, vreg, t_begin * BN, tp);
      store_fp8<DQK>(kreg, stage0);
      store_fp8<DV>(vreg, stage0 + T::kTileK);
    } else {
      stage_bf16<DQK, PAGED>(a, sv, reinterpret_cast<const bf16*>(a.k), a.k_st, a.k_sh, kpg, stage0, t_begin * BN, tp);
      stage_bf16<DV, PAGED>(a, sv, reinterpret_cast<const bf16*>(a.v), a.v_st, a.v_sh, vpg, stage0 + T::kTileK, t_begin * BN, tp);
      FA_WAIT_VMCNT(0);
    }
    __syncthreads();
  }

  int cur = 0;
  for (int t = t_begin; t <= t_end;) {
    int tn = t + 1;
    while (tn <= t_end && !tile_active(a, sv, q0, tn)) ++tn;
    const bool has_next = tn <= t_end;
    char FA_LDS* sc = cur ? stage1 : stage0;
    char FA_LDS* sn = cur ? stage0 : stage1;
    if (has_next) {
      const int tp = tile_page_of(a, sv, tn * BN, PAGED);
      if (FP8) {
        load_fp8<DQK, PAGED>(a, sv, reinterpret_cast<const uint8_t*>(a.k), a.k_st, a.k_sh, kpg, kreg, tn * BN, tp);
        load_fp8<DV, PAGED>(a, sv, reinterpret_cast<const uint8_t*>(a.v), a.v_st, a.v_sh, vpg, vreg, tn * BN, tp);
      } else {
        stage_bf16<DQK, PAGED>(a, sv, reinterpret_cast<const bf16*>(a.k), a.k_st, a.k_sh, kpg, sn, tn * BN, tp);
        stage_bf16<DV, PAGED>(a, sv, reinterpret_cast<const bf16*>(a.v), a.v_st, a.v_sh, vpg, sn + T::kTileK, tn * BN, tp);
      }
    }

    const int k0 = t * BN;
    // ---------------- S^T = K Q^T ----------------
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sacc[kb] = f32x16{};
      const int r = kb * 32 + (lane & 31);
      const char FA_LDS* rowp = sc + r * T::kRowK;
#pragma unroll
      for (int s = 0; s < DQK / 16; ++s) {
        const int c = s * 2 + (lane >> 5);
        const bf16x8 kf = lds_read_b128(rowp + ((c ^ (r & 7)) << 4));
        sacc[kb] = mfma32(kf, qf[s], sacc[kb]);
      }
    }

    // ---------------- scores, masking ----------------
    const bool need_mask = !(k0 >= wave_lo_max && k0 + BN - 1 <= wave_hi_min);
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int j = k0 + kb * 32 + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
        float val = sacc[kb][i];
        if (ANYMOD) {
          float s = val * raw_scale;
          if (SOFTCAP) s = cap * tanh_fast(s * inv_cap);
          if (ALIBI) s -= a.alibi_slope * fabsf((float)(ip - j));
          val = s * kLog2e;
        }
        if (need_mask) val = (j >= my_lo && j <= my_hi) ? val : -INFINITY;
        sacc[kb][i] = val;
        mx = fmaxf(mx, val);
      }
    }
    mx = max_pair32(mx);
    const float m_new = fmaxf(m_run, mx * C);
    const bool grow = m_new > m_run + kLazyTau;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float alpha = exp2_hw(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < DV / 32; ++d)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[d][i] *= alpha;
    }
    bf16x8 pf[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = exp2_hw(fmaf(sacc[kb][i], C, -m_run));
        l_run += p;
        pf[kb * 2 + (i >> 3)][i & 7] = (bf16)p;
      }
    }

    // ---------------- O^T += V^T P^T ----------------
    {
      const char FA_LDS* vt = sc + T::kTileK;
      const int grp = lane >> 4, i16 = lane & 15;
      const int hsel = grp >> 1;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r1 = u * 16 + hsel * 4 + (i16 >> 2);
        const int r2 = r1 + 8;
#pragma unroll
        for (int d = 0; d < DV / 32; ++d) {
          const int dcol = d * 32 + (grp & 1) * 16 + 4 * (i16 & 3);
          const int chunk = dcol >> 3, half = (dcol >> 2) & 1;
          const bf16x4 lo4 = lds_read_tr16(vt + r1 * T::kRowV + ((chunk ^ (r1 & 7)) << 4) + half * 8);
          const bf16x4 hi4 = lds_read_tr16(vt + r2 * T::kRowV + ((chunk ^ (r2 & 7)) << 4) + half * 8);
          bf16x8 vf;
          vf[0] = lo4[0]; vf[1] = lo4[1]; vf[2] = lo4[2]; vf[3] = lo4[3];
          vf[4] = hi4[0]; vf[5] = hi4[1]; vf[6] = hi4[2]; vf[7] = hi4[3];
          oacc[d] = mfma32(vf, pf[u], oacc[d]);
        }
      }
    }

    if (has_next) {
      if (FP8) {
        store_fp8<DQK>(kreg, sn);
        store_fp8<DV>(vreg, sn + T::kTileK);
      } else {
        FA_WAIT_VMCNT(0);
      }
    }
    __syncthreads();
    cur ^= 1;
    t = tn;
  }

  // ---------------- epilogue ----------------
  const float l_tot = sum_pair32(l_run);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  const float osc = inv * vdesc;
  if (qvalid) {
    bf16* op = a.o + (sv.qstart + qrow) * a.o_st + (int64_t)sv.h * a.o_sh + (lane >> 5) * 4;
#pragma unroll
    for (int d = 0; d < DV / 32; ++d) {
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        bf16x4 w;
        w[0] = (bf16)(oacc[d][gi * 4 + 0] * osc);
        w[1] = (bf16)(oacc[d][gi * 4 + 1] * osc);
        w[2] = (bf16)(oacc[d][gi * 4 + 2] * osc);
        w[3] = (bf16)(oacc[d][gi * 4 + 3] * osc);
        *reinterpret_cast<bf16x4*>(op + d * 32 + gi * 8) = w;
      }
    }
    if (lane < 32) {
      const float lse = l_tot > 0.0f ? (m_run + log2_hw(l_tot)) * kLn2 : -INFINITY;
      int64_t li;
      if (a.cu_q) li = (int64_t)sv.h * a.lse_tq + sv.qstart + qrow;
      else li = ((int64_t)sv.b * a.Hq + sv.h) * a.Sq + qrow;
      a.lse[li] = lse;
    }
  }
}

template <int DQK, int DV, bool FP8, bool PAGED, int MODS>
static hipError_t launch_prefill(const PrefillArgs& a, int n_bh, int n_qtiles, hipStream_t stream) {
  dim3 grid(n_bh, n_qtiles);
  hipLaunchKernelGGL((fa_prefill_kernel<DQK, DV, FP8, PAGED, MODS>), grid, dim3(NTHREADS), 0, stream, a);
  return hipGetLastError();
}

// Instantiated shapes: (D_qk, D_v) in {(64,64), (128,128)} for bf16 K/V
// (dense, varlen, paged) with every score-mod combination; (192,128) and
// (128,128) for FP8 E4M3 paged caches without score mods.
hipError_t prefill_dispatch(const PrefillArgs& a, int dqk, int dv, bool fp8, bool paged, int mods,
                            int n_bh, int n_qtiles, hipStream_t stream, bool* supported) {
  *supported = true;
#define FA_CASE(DQ, DVV, F8, PG, MD)                                                     \
  if (dqk == DQ && dv == DVV && fp8 == F8 && paged == PG && mods == MD)                  \
    return launch_prefill<DQ, DVV, F8, PG, MD>(a, n_bh, n_qtiles, stream);
#define FA_MODS4(DQ, DVV, F8, PG) \
  FA_CASE(DQ, DVV, F8, PG, 0) FA_CASE(DQ, DVV, F8, PG, 1) FA_CASE(DQ, DVV, F8, PG, 2) FA_CASE(DQ, DVV, F8, PG, 3)
  FA_MODS4(64, 64, false, false)
  FA_MODS4(128, 128, false, false)
  FA_CASE(128, 128, false, true, 0)
  FA_CASE(64, 64, false, true, 0)
  FA_CASE(192, 128, true, true, 0)
  FA_CASE(128, 128, true, true, 0)
#undef FA_MODS4
#undef FA_CASE
  *supported = false;
  return hipSuccess;
}

}  // namespace fa
