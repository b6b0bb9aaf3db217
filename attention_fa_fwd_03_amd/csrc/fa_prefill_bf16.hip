// Fused attention forward for bf16 K/V (dense, varlen and bf16 pages) on
// gfx950, with a software-pipelined tile loop.
//
// Work split as in the other prefill kernels: a workgroup of 4 wavefronts
// takes 128 query rows of one (sequence, q-head), 32 rows per wavefront, and
// walks the key axis in tiles of 64; two workgroups share each CU.  The
// products are the transposed ones (S^T = K Q^T, O^T += V^T P^T on
// v_mfma_f32_32x32x16_bf16) so that every per-row quantity stays in its lane.
//
// What this kernel changes is the order of work inside a wavefront.  A
// matrix product keeps the matrix core busy for 32 cycles, and the vector
// instructions that the same wavefront issues in that shadow cost next to
// nothing; vector work of the other wavefront on the SIMD overlaps it far
// less (measured on the hardware).  So each tile step pairs matrix work of
// one tile with the vector work of another:
//
//   A(n):  S_{n+1} = K_{n+1} Q^T          ||  P_n = exp2(X_n) -> bf16, row sums of P_n
//   B(n):  O^T += V_n^T P_n^T             ||  row max of S_{n+1},
//                                              X_{n+1} = S_{n+1} * C - m
//
// where X is the score already centred on the running max m (log2 domain,
// logit scale folded into the constant C: the LSE PR's folded scale).  The
// output is rescaled only when some row's max grows by more than 2^8 (lazy
// rescaling, paged FP8 PR review); exp2 arguments never exceed 8.
//
// K and V sit in separate two-slot LDS rings (64 KiB at D = 128): at the top
// of step n one barrier publishes K_{n+1} and V_n and frees the slots of K_n
// and V_{n-1}, into which K_{n+2} and V_{n+1} are copied (LDS DMA) during
// the step.  Scores of tiles that straddle a row's key interval (causal
// diagonal, window edges, sequence tail) are masked by select to -inf before
// the max; score mods (soft-cap, ALiBi) are applied to S_{n+1} before it.
#include "fa_prefill_common.h"

#include <type_traits>

namespace fa {

template <int D, bool PAGED, int MODS, bool BMASK>
__global__ __launch_bounds__(NTHREADS) __attribute__((amdgpu_waves_per_eu(2)))
void fa_prefill_bf16_kernel(const PrefillArgs a) {
  constexpr int kRow = D * 2;                 // bytes per K / V row in LDS
  constexpr int kTile = BN * kRow;
  constexpr int ND = D / 32;                  // 32-wide output blocks
  constexpr int NQK = D / 8;                  // Q.K products per tile: (D/16 steps) x (2 key blocks)
  constexpr int NPV = 4 * ND;                 // P.V products per tile: (4 key steps) x ND
  constexpr int kAheadK = 4;                  // K fragments read this many products ahead
  constexpr int kAheadV = 4;
  __shared__ __attribute__((aligned(1024))) char lds_raw[4 * kTile];
  char FA_LDS* lds = (char FA_LDS*)(lds_raw);
  auto kslot = [&](int s) { return lds + s * kTile; };
  auto vslot = [&](int s) { return lds + (2 + s) * kTile; };

  constexpr bool ALIBI = (MODS & kModAlibi) != 0;
  constexpr bool SOFTCAP = (MODS & kModSoftcap) != 0;
  constexpr bool ANYMOD = ALIBI || SOFTCAP;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  int bh, qt;
  wg_tile(a.causal != 0, bh, qt);
  if (bh >= a.n_bh) return;
  SeqView sv;
  seq_view(a, bh, PAGED, sv);
  const int q0 = qt * BM;
  if (q0 >= sv.sq) return;
  const int q1 = min(q0 + BM, sv.sq);
  const int delta = sv.skv - sv.sq;

  // visible key interval [row_lo(i), row_hi(i)] of query row i (aligned
  // position i + delta); empty when row_hi < row_lo
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
  const int t_begin = lo_min / BN;
  const int t_end = (hi_max >= 0 && hi_max >= lo_min) ? hi_max / BN : t_begin - 1;

  // per-lane query row and its Q fragments (B operand of S^T = K Q^T)
  const int qrow = q0 + wave * 32 + (lane & 31);
  const bool qvalid = qrow < sv.sq;
  bf16x8 qf[D / 16];
  {
    const bf16* qp = reinterpret_cast<const bf16*>(a.q) + (sv.qstart + (qvalid ? qrow : 0)) * a.q_st +
                     (int64_t)sv.h * a.q_sh + (lane >> 5) * 8;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      bf16x8 v = *reinterpret_cast<const bf16x8*>(qp + s * 16);
      if (!qvalid) v = bf16x8{};
      qf[s] = v;
    }
  }
  const int my_lo = row_lo(qrow), my_hi = row_hi(qrow);
  const unsigned my_cnt = (unsigned)max(my_hi - my_lo + 1, 0);
  const int wq0 = q0 + wave * 32;
  const int wq1 = min(wq0 + 31, q1 - 1);
  const int wave_lo_max = row_lo(wq1), wave_hi_min = row_hi(wq0);
  // the last key this wavefront's rows can see (-1 if every row is past the
  // sequence's end): tiles after it would only add zero products
  const int wave_hi_max = wq0 < q1 ? row_hi(wq1) : -1;
  auto wave_reaches = [&](int t) { return t * BN <= wave_hi_max; };

  // C: raw dot product -> log2-domain scaled logit (mods: applied explicitly)
  const float C = ANYMOD ? 1.0f : a.qk_scale * kLog2e;
  // Mods in the log2 domain with every constant folded.  Soft-cap:
  // c tanh(x / c) log2(e) = c' - 2 c' / (1 + 2^(k s)) for the raw score s,
  // k = 2 scale log2(e) / c and c' = c log2(e) (tanh(u) = 1 - 2 / (1 + e^{2u});
  // +-inf from the exponential give +-c', the correct limits): one multiply,
  // exp2, add, reciprocal and FMA per score.  ALiBi: - slope log2(e) |i' - j|
  // by one FMA with an absolute-value operand.
  const float lin2 = a.qk_scale * kLog2e;
  const float cap_k = SOFTCAP ? 2.0f * a.qk_scale * kLog2e / a.softcap : 0.0f;
  const float cap_c = SOFTCAP ? a.softcap * kLog2e : 0.0f;
  const float slope2 = ALIBI ? a.alibi_slope * kLog2e : 0.0f;
  const int ip = qrow + delta;
  const int lane_key = (lane >> 5) * 4;      // key offset of this lane's S^T registers

  f32x16 oacc[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) oacc[d] = f32x16{};
  float m_run = kMaxFloor, l_run = 0.0f;

  // next active tile at or after t (t_end + 1 when none): every tile, or
  // with a block mask the tiles active for this workgroup's query tile
  MaskBits mb;
  if (BMASK) mb.init(a, sv, q0);
  auto next_tile = [&](int t) {
    if (!BMASK) return t;
    for (; t <= t_end; ++t)
      if (mb.tile_bits(t)) return t;
    return t;
  };

  // K and V rows have the same width and layout here (D_qk = D_v, equal
  // strides), so one set of per-lane DMA offsets serves both
  Bf16Stager<D, PAGED> dma;
  dma.init(a.k_st, wave, lane);
  constexpr int kPieces = Bf16Stager<D, PAGED>::kPerWave;   // DMA instructions per tile and operand
  const bool small_pages = PAGED && a.page_shift < 6;
  auto issue_k = [&](int t, char FA_LDS* dst) {
    const int k0 = t * BN;
    dma.issue(a, sv, reinterpret_cast<const bf16*>(a.k), a.k_st, a.k_sh, a.k_pg, dst, k0,
               k0 + BN <= sv.skv && !small_pages, wave, lane);
  };
  auto issue_v = [&](int t, char FA_LDS* dst) {
    const int k0 = t * BN;
    dma.issue(a, sv, reinterpret_cast<const bf16*>(a.v), a.k_st, a.k_sh, a.v_pg, dst, k0,
               k0 + BN <= sv.skv && !small_pages, wave, lane);
  };

  // LDS offsets of this lane's fragments.  K: row lane%32 (+32 for key
  // block 1) at stored chunk (2s + lane/32) ^ swz(row); with the row's
  // swizzle split into its low bit (fixed per lane) and the rest, that is
  // kx ^ 32 s, kx holding the row, the low bit and the swizzle's high bits.
  // V^T fragment of output block d: rows rr and rr + 8 of each 16-key step
  // (the swizzle depends on the row modulo 16 only, so the steps are
  // immediate offsets).
  int kx;
  {
    const int r = lane & 31, sw = swz<kRow>(r);
    kx = r * kRow + ((((lane >> 5) ^ sw) & 1) << 4) + ((sw & ~1) << 4);
  }
  int voff[ND][2];
  {
    const int grp = lane >> 4, i16 = lane & 15;
#pragma unroll
    for (int d = 0; d < ND; ++d)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int rr = (grp >> 1) * 4 + (i16 >> 2) + h * 8;
        const int dcol = d * 32 + (grp & 1) * 16 + 4 * (i16 & 3);
        voff[d][h] = rr * kRow + (((dcol >> 3) ^ swz<kRow>(rr)) << 4) + ((dcol >> 2) & 1) * 8;
      }
  }
  auto kread = [&](const char FA_LDS* kt, int n) {
    return lds_read_b128(kt + (kx ^ (32 * (n >> 1))) + (n & 1) * 32 * kRow);
  };
  auto vread = [&](const char FA_LDS* vt, int n) {
    const int u = n / ND, d = n % ND;
    const bf16x4 lo4 = lds_read_tr16(vt + voff[d][0] + u * 16 * kRow);
    const bf16x4 hi4 = lds_read_tr16(vt + voff[d][1] + u * 16 * kRow);
    bf16x8 v;
    v[0] = lo4[0]; v[1] = lo4[1]; v[2] = lo4[2]; v[3] = lo4[3];
    v[4] = hi4[0]; v[5] = hi4[1]; v[6] = hi4[2]; v[7] = hi4[3];
    return v;
  };

  // score mods and masks of tile t, in place (log2-domain result when ANYMOD)
  auto prep = [&](f32x16 (&s)[2], int t) {
    const int k0 = t * BN;
    if (ANYMOD) {
      // i' - j of register (kb, i) is d0 - (32 kb + 8 (i/4) + i%4), exact in
      // fp32 below 2^24 keys apart
      const float d0 = (float)(ip - k0 - lane_key);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float x;
          if (SOFTCAP) x = fmaf(rcp_hw(1.0f + exp2_hw(s[kb][i] * cap_k)), -2.0f * cap_c, cap_c);
          else x = s[kb][i] * lin2;
          if (ALIBI) x = fmaf(-slope2, fabsf(d0 - (float)(kb * 32 + (i >> 2) * 8 + (i & 3))), x);
          s[kb][i] = x;
        }
    }
    if (!(k0 >= wave_lo_max && k0 + BN - 1 <= wave_hi_min)) {
      // keeps this a real branch: selects would otherwise run on every tile
      asm volatile("" ::);
      const int base = k0 + lane_key - my_lo;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const unsigned rel = (unsigned)(base + kb * 32 + (i >> 2) * 8 + (i & 3));
          s[kb][i] = rel < my_cnt ? s[kb][i] : -INFINITY;
        }
    }
  };

  f32x16 xs[2];          // X_n: scores of the current tile centred on m_run (log2 domain)
  f32x16 sn[2];          // S_{n+1}: raw scores of the next tile, then X_{n+1}
  bf16x2 pw[16];         // P_n in bf16 pairs: pw[4u .. 4u+3] is the B operand of key step u
  const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
  auto pstep = [&](int u) {
    bf16x8 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      r[2 * j] = pw[4 * u + j][0];
      r[2 * j + 1] = pw[4 * u + j][1];
    }
    return r;
  };

  // A(n): products of S_{n+1} (HAS_NEXT) paired with P_n = exp2(X_n) and its
  // row sums (two-element dot products of the bf16 pairs, which B's products
  // use as they are)
  auto phase_a = [&](auto has_next, const char FA_LDS* kt) {
    constexpr bool HN = decltype(has_next)::value;
    float lsa0 = 0.0f, lsa1 = 0.0f;
    bf16x8 kf[NQK];
    if (HN) {
      sn[0] = f32x16{};
      sn[1] = f32x16{};
#pragma unroll
      for (int n = 0; n < kAheadK && n < NQK; ++n) kf[n] = kread(kt, n);
    }
    constexpr int NCH = HN ? NQK : 8;
#pragma unroll
    for (int n = 0; n < NCH; ++n) {
      if (HN) {
        if (n + kAheadK < NQK) kf[n + kAheadK] = kread(kt, n + kAheadK);
        sn[n & 1] = mfma32(kf[n], qf[n >> 1], sn[n & 1]);
      }
      // this chunk's share of the 32 exponentials, as bf16 pairs; the empty
      // asm keeps each pair here (P is used only in B, and would otherwise
      // be sunk past the products it is meant to hide behind)
#pragma unroll
      for (int e = n * 32 / NCH; e < (n + 1) * 32 / NCH; e += 2) {
        const int kb = e >> 4, i = e & 15;
        bf16x2 pr = {(bf16)exp2_hw(xs[kb][i]), (bf16)exp2_hw(xs[kb][i + 1])};
        asm volatile("" : "+v"(pr));
        pw[e >> 1] = pr;
        if ((e >> 1) & 1) lsa1 = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, lsa1, false);
        else lsa0 = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, lsa0, false);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    l_run += lsa0 + lsa1;
  };

  // B(n): O^T += V_n^T P_n^T paired, when a next tile exists, with its row
  // max and centring; returns nothing, updates xs (= X_{n+1}), m_run, l_run
  // and the output scale
  auto phase_b = [&](auto has_next, const char FA_LDS* vt) {
    constexpr bool HN = decltype(has_next)::value;
    bf16x8 vf[NPV];
#pragma unroll
    for (int n = 0; n < kAheadV && n < NPV; ++n) vf[n] = vread(vt, n);
    float mx0 = -INFINITY, mx1 = -INFINITY;
    float m_use = m_run;
    bool resc = false;
    constexpr int HALF = NPV / 2;
#pragma unroll
    for (int n = 0; n < NPV; ++n) {
      if (n + kAheadV < NPV) vf[n + kAheadV] = vread(vt, n + kAheadV);
      oacc[n % ND] = mfma32(vf[n], pstep(n / ND), oacc[n % ND]);
      if (HN) {
        if (n < HALF) {
          // row max of S_{n+1}: 32 values over the first half
#pragma unroll
          for (int e = n * 16 / HALF; e < (n + 1) * 16 / HALF; ++e) {
            // maximum (NaN-propagating) needs no operand canonicalisation
            const float v = __builtin_elementwise_maximum(sn[0][e], sn[1][e]);
            if (e & 1) mx1 = __builtin_elementwise_maximum(mx1, v);
            else mx0 = __builtin_elementwise_maximum(mx0, v);
          }
        } else {
          if (n == HALF) {
            const float m_new = fmaxf(m_run, max_pair32(__builtin_elementwise_maximum(mx0, mx1)) * C);
            resc = __builtin_amdgcn_ballot_w64(m_new > m_run + kLazyTau) != 0;
            m_use = resc ? m_new : m_run;
          }
          // X_{n+1} = S_{n+1} * C - m over the second half
#pragma unroll
          for (int e = (n - HALF) * 32 / HALF; e < (n - HALF + 1) * 32 / HALF; ++e) {
            const int kb = e >> 4, i = e & 15;
            float x = fmaf(sn[kb][i], C, -m_use);
            asm volatile("" : "+v"(x));
            sn[kb][i] = x;
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (HN) {
      if (resc) {
        const float alpha = exp2_hw(m_run - m_use);
        m_run = m_use;
        l_run *= alpha;
#pragma unroll
        for (int d = 0; d < ND; ++d)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[d][i] *= alpha;
      }
      xs[0] = sn[0];
      xs[1] = sn[1];
    }
  };

  int tc = next_tile(t_begin);
  if (tc <= t_end) {
    int tn = next_tile(tc + 1);
    // prologue: K_0, V_0 (and K_1) in flight; S_0 -> X_0
    issue_k(tc, kslot(0));
    issue_v(tc, vslot(0));
    if (tn <= t_end) {
      issue_k(tn, kslot(1));
      FA_WAIT_VMCNT(kPieces);
    } else {
      FA_WAIT_VMCNT(0);
    }
    __syncthreads();
    {
      const char FA_LDS* kt = kslot(0);
      xs[0] = f32x16{};
      xs[1] = f32x16{};
      bf16x8 kf[NQK];
#pragma unroll
      for (int n = 0; n < kAheadK && n < NQK; ++n) kf[n] = kread(kt, n);
#pragma unroll
      for (int n = 0; n < NQK; ++n) {
        if (n + kAheadK < NQK) kf[n + kAheadK] = kread(kt, n + kAheadK);
        xs[n & 1] = mfma32(kf[n], qf[n >> 1], xs[n & 1]);
        __builtin_amdgcn_sched_barrier(0);
      }
      prep(xs, tc);
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, xs[kb][i]);
      m_run = fmaxf(m_run, max_pair32(mx) * C);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) xs[kb][i] = fmaf(xs[kb][i], C, -m_run);
    }
    // step n: K_{n+1} and V_n published at its barrier.  Every wavefront
    // takes part in every barrier and issues its share of every copy; it
    // computes the tiles up to its last visible key (a tile before its
    // first visible key is computed and masked, contributing nothing).
    int n = 0;
    auto publish = [&]() {
      // publish K_{n+1} and V_n; every wavefront is done with K_n and V_{n-1}
      FA_WAIT_VMCNT(0);
      __syncthreads();
      const int tnn = tn <= t_end ? next_tile(tn + 1) : t_end + 1;
      if (tnn <= t_end) issue_k(tnn, kslot(n & 1));
      if (tn <= t_end) issue_v(tn, vslot((n + 1) & 1));
      return tnn;
    };
    while (tn <= t_end && wave_reaches(tn)) {
      const int tnn = publish();
      phase_a(std::true_type{}, kslot((n + 1) & 1));
      prep(sn, tn);
      phase_b(std::true_type{}, vslot(n & 1));
      ++n;
      tc = tn;
      tn = tnn;
    }
    // the last tile this wavefront computes: P.V only
    {
      const int tnn = publish();
      if (wave_reaches(tc)) {
        phase_a(std::false_type{}, kslot(0));
        phase_b(std::false_type{}, vslot(n & 1));
      }
      ++n;
      tc = tn;
      tn = tnn;
    }
    // tiles past this wavefront's keys: barriers and copies only
    while (tc <= t_end) {
      const int tnn = publish();
      ++n;
      tc = tn;
      tn = tnn;
    }
  }

  // ---------------- epilogue ----------------
  const float l_tot = sum_pair32(l_run);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  // the K ring is free here: every wavefront is past its last barrier, no
  // copy is in flight and K is not read again
  store_o_rows<D>(oacc, inv, lds + wave * 32 * kRow,
                  a.o + (sv.qstart + wq0) * a.o_st + (int64_t)sv.h * a.o_sh, a.o_st, sv.sq - wq0, lane);
  if (qvalid && lane < 32) {
    const float lse = l_tot > 0.0f ? (m_run + log2_hw(l_tot)) * kLn2 : -INFINITY;
    int64_t li;
    if (a.cu_q) li = (int64_t)sv.h * a.lse_tq + sv.qstart + qrow;
    else li = ((int64_t)sv.b * a.Hq + sv.h) * a.Sq + qrow;
    a.lse[li] = lse;
  }
}

template <int D, bool PAGED, int MODS>
static hipError_t launch_bf16(const PrefillArgs& a, int n_bh, int n_qtiles, hipStream_t stream) {
  dim3 grid((n_bh + 7) / 8 * 8, n_qtiles);
  if (a.bmask)
    hipLaunchKernelGGL((fa_prefill_bf16_kernel<D, PAGED, MODS, true>), grid, dim3(NTHREADS), 0, stream, a);
  else
    hipLaunchKernelGGL((fa_prefill_bf16_kernel<D, PAGED, MODS, false>), grid, dim3(NTHREADS), 0, stream, a);
  return hipGetLastError();
}

// bf16 K/V: head dims 64 and 128 (D_qk = D_v), contiguous (dense, varlen)
// or in bf16 pages, with every score-mod combination.
hipError_t prefill_bf16_dispatch(const PrefillArgs& a, int d, bool paged, int mods, int n_bh, int n_qtiles,
                                 hipStream_t stream, bool* supported) {
  *supported = true;
#define FA_CASE(DD, PG, MD) \
  if (d == DD && paged == PG && mods == MD) return launch_bf16<DD, PG, MD>(a, n_bh, n_qtiles, stream);
  FA_CASE(64, false, 0) FA_CASE(64, false, 1) FA_CASE(64, false, 2) FA_CASE(64, false, 3)
  FA_CASE(128, false, 0) FA_CASE(128, false, 1) FA_CASE(128, false, 2) FA_CASE(128, false, 3)
  FA_CASE(64, true, 0) FA_CASE(64, true, 1) FA_CASE(64, true, 2) FA_CASE(64, true, 3)
  FA_CASE(128, true, 0) FA_CASE(128, true, 1) FA_CASE(128, true, 2) FA_CASE(128, true, 3)
#undef FA_CASE
  *supported = false;
  return hipSuccess;
}

}  // namespace fa
