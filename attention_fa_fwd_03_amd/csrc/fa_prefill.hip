// Fused attention forward over FP8 E4M3 paged caches (head-major or
// vectorised pages) for gfx950.  bf16 K/V are served by the
// software-pipelined kernel in fa_prefill_bf16.hip.  Score mods (ALiBi,
// soft-cap) run in one variant of this kernel; block masks and windows are
// runtime arguments of every variant.
//
// One workgroup = 4 wavefronts = 128 query rows of one (sequence, q-head);
// each wavefront owns 32 query rows.  A workgroup keeps its LDS ring within
// 80 KB, so two workgroups share each CU and each SIMD runs one wavefront of
// each.  The key axis is walked in tiles of 64 keys staged in LDS (a ring of
// three stages, two tiles in flight).  Per tile and wavefront:
//
//   S^T[64 x 32]  = K_tile . Q^T          v_mfma_scale_f32_32x32x64_f8f6f4 on the
//                                          E4M3 K bytes (64 dims a step, unit
//                                          scales), B = Q parts in registers
//   online softmax on S^T                 lane l owns query row l%32; the row
//                                          max needs one permlane32 swap
//   O^T[Dv x 32] += V_tile^T . P^T        v_mfma_f32_32x32x16_bf16, A = V read
//                                          transposed and converted to bf16,
//                                          B = P in registers
//
// Computing the transposed products keeps every per-row quantity (running
// max, denominator, rescale factor, output scaling) lane-local.  The P^T
// operand taken straight from the S^T accumulator enumerates the 16 keys of
// an MFMA step in the order that swaps bits 2 and 3 of the key index; the V
// transposed reads fetch rows in that same order, so K and V stay paired.
//
// Queries: E4M3 codes as given (one product per step, q_descale folded into
// the logit constant), or bf16 split per row into two E4M3 parts of 2^e q
// (hi + lo, about 2^-8 relative; each part times a K byte is exact), e from
// the row's largest magnitude so that hi stays in the E4M3 normal range;
// 2^-e and the K descale fold into that row's logit constant.
//
// Softmax works in the log2 domain: the running max m is kept in units of
// scale*log2(e)*logit so that p = exp2(fma(x, C, -m)) is one FMA and one
// v_exp_f32 per score (method: LSE PR, "log2 domain with the logit scale
// folded"; the paged FP8 PR folds the K descale into that same constant).
// The output is rescaled only when some row's max grows by more than 2^8
// (lazy rescaling, paged FP8 PR review), which leaves the result unchanged.
// The exponentials of key step u + 1 run under the P.V products of step u.
//
// Masking is by select to -inf (never by multiply, so NaN bytes in unused
// cache slots cannot leak), with rows that see no key producing O = 0 and
// LSE = -inf.  Tiles wholly outside the causal / window range are not
// loaded; a wavefront whose own 32 rows see nothing in a loaded tile skips
// its math for that tile; tiles wholly inside a wavefront's range skip the
// per-score mask.
//
// K/V staging: K and the V of head-major pages go global -> LDS with
// global_load_lds_dwordx4 (no registers) as E4M3 bytes; the P.V fragments
// of that V come from the transposing byte read (ds_read_b64_tr_b8),
// converted exactly to bf16.  For vectorised pages, and for E4M3 queries at
// D_v = 128, V is loaded to registers one tile ahead instead, converted
// exactly to bf16 and written to LDS.  LDS rows are 16-byte-chunk XOR
// swizzled so that the K reads and the transposed V reads are bank-conflict
// free.  Whole tiles take a fast addressing path (per-lane 32-bit offsets
// from one scalar tile base); the sequence tail and pages smaller than a
// tile take a clamped per-row path.
#include "fa_device.h"
#include "fa_kernels.h"
#include "fa_prefill_common.h"


namespace fa {

// VREG: FP8 V goes through registers (converted to bf16 when stored);
// otherwise FP8 V stays E4M3 in LDS and is converted when read.
template <int DQK, int DV, bool FP8, bool VREG>
struct PrefillTraits {
  static constexpr int kRowK = FP8 ? DQK : DQK * 2;           // bytes per K row in LDS (FP8 K stays E4M3)
  static constexpr int kRowV = (FP8 && !VREG) ? DV : DV * 2;  // bytes per V row (or V^T block row) in LDS
  static constexpr int kTileK = BN * kRowK;
  static constexpr int kTileV = BN * kRowV;
  static constexpr int kStage = kTileK + kTileV;
  // two workgroups per CU: at most 80 KB of LDS each; V in registers waits
  // one tile there, so two stages
  static constexpr int kStages = (!VREG && 3 * kStage <= 81920) ? 3 : 2;
  static constexpr int kLds = kStages * kStage;
};

// FP8 V tile of D columns (head-major pages): 16-byte items loaded to
// registers one tile ahead, converted exactly to bf16 and written to the
// swizzled LDS rows.
template <int D, bool PAGED>
struct Fp8Stager {
  static constexpr int kPerRow = D / 16;
  static constexpr int kItems = BN * D / 16;
  static constexpr int kPer = (kItems + NTHREADS - 1) / NTHREADS;
  static constexpr int kRow = D * 2;
  i32x4 w[kPer];
  int off[kPer];
  __device__ __forceinline__ void init(int64_t st, int tid) {
#pragma unroll
    for (int it = 0; it < kPer; ++it) {
      const int idx = min(it * NTHREADS + tid, kItems - 1);
      off[it] = (idx / kPerRow) * (int)st + (idx % kPerRow) * 16;
    }
  }
  __device__ __forceinline__ void load(const PrefillArgs& a, const SeqView& sv, const uint8_t* base, int64_t st,
                                       int64_t sh, int64_t pg, int k0, bool fast, int tid) {
    if (fast) {
      const uint8_t* tb = base + tile_base(a, sv, k0, st, sh, pg, PAGED);
#pragma unroll
      for (int it = 0; it < kPer; ++it) w[it] = *reinterpret_cast<const i32x4*>(tb + off[it]);
    } else {
#pragma unroll
      for (int it = 0; it < kPer; ++it) {
        const int idx = min(it * NTHREADS + tid, kItems - 1);
        const int r = idx / kPerRow, f = idx % kPerRow;
        w[it] = *reinterpret_cast<const i32x4*>(base + key_row_offset(a, sv, k0 + r, st, sh, pg, PAGED) + f * 16);
      }
    }
  }
  __device__ __forceinline__ void store(char FA_LDS* tile, int tid) const {
#pragma unroll
    for (int it = 0; it < kPer; ++it) {
      const int idx = it * NTHREADS + tid;
      if (kItems % NTHREADS == 0 || idx < kItems) {
        const int r = idx / kPerRow, f = idx % kPerRow;
        bf16x8 lo, hi;
        fp8x16_to_bf16(w[it], lo, hi);
        char FA_LDS* rowp = tile + r * kRow;
        *reinterpret_cast<bf16x8 FA_LDS*>(rowp + (((2 * f) ^ swz<kRow>(r)) << 4)) = lo;
        *reinterpret_cast<bf16x8 FA_LDS*>(rowp + (((2 * f + 1) ^ swz<kRow>(r)) << 4)) = hi;
      }
    }
  }
};

// Vectorised FP8 pages (paged FP8 PR review: K page [Hkv, D/16, page, 16],
// V page [Hkv, page/16, Dv, 16]).  The (page, kv-head) block starts at
// page*pg + g*sh; page_shift >= 4.

// FP8 K tile of D bytes per key, staged by LDS DMA as E4M3 bytes (no
// registers, no conversion): instruction n covers LDS bytes [1024 n, +1024),
// lane l fills 16 bytes at 16 l: tile row r, stored chunk pos = source
// chunk pos ^ swz8(r).  Head-major pages read the chunk from the key's row;
// vectorised pages from column pos ^ swz8(r) of the page.  Rows past the
// sequence re-read its last key.  BIGP (pages of at least BN keys): every
// tile lies in one page, found by one scalar lookup, and is copied by
// buffer loads with 32-bit offsets from that page.  Smaller pages take a
// per-row lookup and 64-bit addresses (global_load_lds); a kernel that
// contains one waits for all its LDS reads with lgkmcnt(0), so the two
// cases are separate kernels.
template <int D, bool VEC, bool BIGP>
struct Fp8KDma {
  static constexpr int kPerWave = BN * D / 1024 / NWAVES;
  static_assert(kPerWave >= 1 && (BN * D) % (1024 * NWAVES) == 0, "whole 1 KB pieces per wavefront");
  int off[kPerWave];   // byte offset of this lane's source chunk from the tile's first key
  __device__ __forceinline__ static void place(int i, int wave, int lane, int& row, int& col) {
    const int byte = (wave * kPerWave + i) * 1024 + lane * 16;
    row = byte / D;
    col = ((byte % D) >> 4) ^ swz8<D>(row);
  }
  __device__ __forceinline__ void init(int page_shift, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      int row, col;
      place(i, wave, lane, row, col);
      off[i] = VEC ? (col << (page_shift + 4)) + row * 16 : row * D + col * 16;
    }
  }
  __device__ __forceinline__ void issue(const PrefillArgs& a, const SeqView& sv, const uint8_t* base, int k0,
                                        bool fast, char FA_LDS* tile, int wave, int lane) const {
    const int pmask = (1 << a.page_shift) - 1;
    if (BIGP) {
      int page = load_uniform_i32(a.block_table, (int64_t)sv.b * a.max_pages + (k0 >> a.page_shift));
      page = min(max(page, 0), a.num_pages - 1);
      const uint8_t* pb = base + (int64_t)page * a.k_pg + (int64_t)sv.g * a.k_sh;
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(pb);
      if (fast) {
        const unsigned tb = (unsigned)(k0 & pmask) * (VEC ? 16 : D);
#pragma unroll
        for (int i = 0; i < kPerWave; ++i) buffer_to_lds16(rs, tb + off[i], tile + (wave * kPerWave + i) * 1024);
      } else {
#pragma unroll
        for (int i = 0; i < kPerWave; ++i) {
          int row, col;
          place(i, wave, lane, row, col);
          const unsigned j = (unsigned)(min(k0 + row, sv.skv - 1) & pmask);
          buffer_to_lds16(rs, VEC ? ((unsigned)col << (a.page_shift + 4)) + j * 16 : j * D + col * 16,
                          tile + (wave * kPerWave + i) * 1024);
        }
      }
    } else if (fast) {
      int page = load_uniform_i32(a.block_table, (int64_t)sv.b * a.max_pages + (k0 >> a.page_shift));
      page = min(max(page, 0), a.num_pages - 1);
      const uint8_t* tb = base + (int64_t)page * a.k_pg + (int64_t)sv.g * a.k_sh + (k0 & pmask) * (VEC ? 16 : D);
#pragma unroll
      for (int i = 0; i < kPerWave; ++i) global_to_lds16(tb + off[i], tile + (wave * kPerWave + i) * 1024);
    } else {
#pragma unroll
      for (int i = 0; i < kPerWave; ++i) {
        int row, col;
        place(i, wave, lane, row, col);
        const int j = min(k0 + row, sv.skv - 1);
        int page = a.block_table[(int64_t)sv.b * a.max_pages + (j >> a.page_shift)];
        page = min(max(page, 0), a.num_pages - 1);
        const uint8_t* pb = base + (int64_t)page * a.k_pg + (int64_t)sv.g * a.k_sh;
        const uint8_t* src = VEC ? pb + ((int64_t)col << (a.page_shift + 4)) + (j & pmask) * 16
                                 : pb + (int64_t)(j & pmask) * D + col * 16;
        global_to_lds16(src, tile + (wave * kPerWave + i) * 1024);
      }
    }
  }
};

// V: item idx is head dim d = idx % D of 16-key block sb = idx / D (16 bytes,
// one dim of 16 keys), so one wavefront's load covers 64 dims of one block.
// The tile is kept as V^T: row d holds the tile's 64 keys in bf16 (128
// bytes), each 16-key group in the order the P^T operand enumerates them
// (position p holds key p with bits 2 and 3 swapped), so a lane's A fragment
// is one 16-byte read.  Chunk c of row d is stored at c ^ ((d >> 1) & 7):
// the 16 rows that 16 lanes read at one chunk then fall in distinct bank
// quarters.  Value bytes past the sequence's end are cleared.
template <int D>
struct Fp8VecV {
  static constexpr int kItems = (BN / 16) * D;
  static constexpr int kPer = (kItems + NTHREADS - 1) / NTHREADS;
  static constexpr int kRow = BN * 2;
  static_assert(kItems % NTHREADS == 0, "whole V items per thread");
  i32x4 w[kPer];
  __device__ __forceinline__ void load(const PrefillArgs& a, const SeqView& sv, const uint8_t* base, int k0,
                                       bool fast, int tid) {
    const int pmask = (1 << a.page_shift) - 1;
    if (fast) {
      int page = load_uniform_i32(a.block_table, (int64_t)sv.b * a.max_pages + (k0 >> a.page_shift));
      page = min(max(page, 0), a.num_pages - 1);
      const uint8_t* tb =
          base + (int64_t)page * a.v_pg + (int64_t)sv.g * a.v_sh + ((k0 & pmask) >> 4) * (D * 16);
#pragma unroll
      for (int it = 0; it < kPer; ++it) w[it] = *reinterpret_cast<const i32x4*>(tb + (it * NTHREADS + tid) * 16);
    } else {
#pragma unroll
      for (int it = 0; it < kPer; ++it) {
        const int idx = it * NTHREADS + tid;
        const int j = k0 + (idx / D) * 16;               // first key of the block
        const int jc = min(j, sv.skv - 1);
        int page = a.block_table[(int64_t)sv.b * a.max_pages + (jc >> a.page_shift)];
        page = min(max(page, 0), a.num_pages - 1);
        const i32x4 x = *reinterpret_cast<const i32x4*>(base + (int64_t)page * a.v_pg + (int64_t)sv.g * a.v_sh +
                                                        ((jc & pmask) >> 4) * (D * 16) + (idx % D) * 16);
        w[it] = keep_bytes(x, sv.skv - j);
      }
    }
  }
  __device__ __forceinline__ void store(char FA_LDS* tile, int tid) const {
#pragma unroll
    for (int it = 0; it < kPer; ++it) {
      const int idx = it * NTHREADS + tid;
      const int d = idx % D, sb = idx / D;
      bf16x8 lo, hi;
      fp8x16_to_bf16(w[it], lo, hi);
      // keys 0-3, 8-11 | 4-7, 12-15 of the block
      const bf16x8 c0 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      const bf16x8 c1 = {lo[4], lo[5], lo[6], lo[7], hi[4], hi[5], hi[6], hi[7]};
      char FA_LDS* rowp = tile + d * kRow;
      const int sw = (d >> 1) & 7;
      *reinterpret_cast<bf16x8 FA_LDS*>(rowp + (((2 * sb) ^ sw) << 4)) = c0;
      *reinterpret_cast<bf16x8 FA_LDS*>(rowp + (((2 * sb + 1) ^ sw) << 4)) = c1;
    }
  }
};

// FP8 V tile of head-major pages, staged by LDS DMA as E4M3 bytes: tile
// rows of D bytes (key-major), chunk c of row r at c ^ swzv8<D>(r), read with
// the transposing byte read.  Rows past the sequence re-read its last key,
// whose p is 0.  Page lookups and BIGP as for K.
template <int D, bool BIGP>
struct Fp8VDma {
  static constexpr int kPerWave = BN * D / 1024 / NWAVES;
  static_assert(kPerWave >= 1 && (BN * D) % (1024 * NWAVES) == 0, "whole 1 KB pieces per wavefront");
  int off[kPerWave];   // byte offset of this lane's source chunk from the tile's first key
  __device__ __forceinline__ static void place(int i, int wave, int lane, int& row, int& col) {
    const int byte = (wave * kPerWave + i) * 1024 + lane * 16;
    row = byte / D;
    col = ((byte % D) >> 4) ^ swzv8<D>(row);
  }
  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      int row, col;
      place(i, wave, lane, row, col);
      off[i] = row * D + col * 16;
    }
  }
  __device__ __forceinline__ void issue(const PrefillArgs& a, const SeqView& sv, const uint8_t* base, int k0,
                                        bool fast, char FA_LDS* tile, int wave, int lane) const {
    const int pmask = (1 << a.page_shift) - 1;
    if (BIGP) {
      int page = load_uniform_i32(a.block_table, (int64_t)sv.b * a.max_pages + (k0 >> a.page_shift));
      page = min(max(page, 0), a.num_pages - 1);
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(base + (int64_t)page * a.v_pg + (int64_t)sv.g * a.v_sh);
      if (fast) {
        const unsigned tb = (unsigned)(k0 & pmask) * D;
#pragma unroll
        for (int i = 0; i < kPerWave; ++i) buffer_to_lds16(rs, tb + off[i], tile + (wave * kPerWave + i) * 1024);
      } else {
#pragma unroll
        for (int i = 0; i < kPerWave; ++i) {
          int row, col;
          place(i, wave, lane, row, col);
          const unsigned j = (unsigned)(min(k0 + row, sv.skv - 1) & pmask);
          buffer_to_lds16(rs, j * D + col * 16, tile + (wave * kPerWave + i) * 1024);
        }
      }
    } else if (fast) {
      int page = load_uniform_i32(a.block_table, (int64_t)sv.b * a.max_pages + (k0 >> a.page_shift));
      page = min(max(page, 0), a.num_pages - 1);
      const uint8_t* tb = base + (int64_t)page * a.v_pg + (int64_t)sv.g * a.v_sh + (k0 & pmask) * D;
#pragma unroll
      for (int i = 0; i < kPerWave; ++i) global_to_lds16(tb + off[i], tile + (wave * kPerWave + i) * 1024);
    } else {
#pragma unroll
      for (int i = 0; i < kPerWave; ++i) {
        int row, col;
        place(i, wave, lane, row, col);
        const int j = min(k0 + row, sv.skv - 1);
        int page = a.block_table[(int64_t)sv.b * a.max_pages + (j >> a.page_shift)];
        page = min(max(page, 0), a.num_pages - 1);
        global_to_lds16(base + (int64_t)page * a.v_pg + (int64_t)sv.g * a.v_sh + (int64_t)(j & pmask) * D + col * 16,
                        tile + (wave * kPerWave + i) * 1024);
      }
    }
  }
};

__device__ __forceinline__ i32x2 lds_read_tr8(const char FA_LDS* __restrict__ p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((i32x2 FA_LDS*)(p));
}

// C[32 x 32] += A B^T over 64 E4M3 products per output: lane m + 32 h holds
// bytes 32 h .. 32 h + 31 of row m of A (and of column n of B), unit scales.
// The accumulator layout is that of the bf16 32x32 product.
__device__ __forceinline__ f32x16 mfma32_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ i32x8 cat8(i32x4 x, i32x4 y) {
  return i32x8{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
}

template <int DQK, int DV, bool FP8, bool PAGED, bool VEC, bool Q8, int MODS, bool BIGP>
__global__ __launch_bounds__(NTHREADS) __attribute__((amdgpu_waves_per_eu(2)))
void fa_prefill_kernel(const PrefillArgs a) {
  // bf16 K/V go to fa_prefill_bf16_kernel.  Score mods come in one variant
  // (MODS = both bits): ALiBi is always applied there (slope 0 is the
  // identity) and the soft-cap when softcap > 0, a uniform branch per tile.
  static_assert(FP8 && (MODS == 0 || MODS == (kModAlibi | kModSoftcap)), "FP8 caches: no mods or the mods variant");
  constexpr bool ANYMOD = MODS != 0;
  static_assert(!VEC || PAGED, "vectorised pages are a page format");
  static_assert(!Q8 || FP8, "E4M3 queries go with an FP8 cache");
  // FP8 V through registers for vectorised pages and for E4M3 queries at
  // D_v = 128; E4M3 in LDS otherwise (the faster of the two, measured)
  constexpr bool VREG = FP8 && (VEC || (Q8 && DV <= 128));
  using T = PrefillTraits<DQK, DV, FP8, VREG>;
  __shared__ __attribute__((aligned(1024))) char lds_raw[T::kLds];
  char FA_LDS* lds = (char FA_LDS*)(lds_raw);


  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  int bh, qt;
  wg_tile(a.causal != 0, bh, qt);
  if (bh >= a.n_bh) return;
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
    sv.skv = (int)min((int64_t)a.seqlen_k[sv.b], (int64_t)a.max_pages << a.page_shift);   // bounded lookups
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

  // Visible key interval [row_lo(i), row_hi(i)] of query row i (aligned
  // position i' = i + delta); empty when row_hi < row_lo.
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
  // FP8 K (E4M3 products, 64 dims a step, 32 per lane): E4M3 queries as they
  // are; bf16 queries as two E4M3 parts of 2^e q (hi + lo, e per row), each
  // multiplied exactly.
  const int qrow = q0 + wave * 32 + (lane & 31);
  const bool qvalid = qrow < sv.sq;
  constexpr int kQ8 = DQK / 64;
  i32x8 qhi[kQ8], qlo[kQ8];
  float qinv = 1.0f;   // bf16 queries split into E4M3 parts: 2^-e of this row's split scale
  const int64_t qrow_off = (sv.qstart + (qvalid ? qrow : 0)) * a.q_st + (int64_t)sv.h * a.q_sh;
  {
    if (Q8) {
      const uint8_t* qp = reinterpret_cast<const uint8_t*>(a.q) + qrow_off + (lane >> 5) * 32;
#pragma unroll
      for (int s = 0; s < kQ8; ++s) {
        i32x8 v = cat8(*reinterpret_cast<const i32x4*>(qp + s * 64), *reinterpret_cast<const i32x4*>(qp + s * 64 + 16));
        if (!qvalid) v = i32x8{};
        qhi[s] = v;
        qlo[s] = i32x8{};
      }
    } else {
      // the row's power-of-two split scale from its largest magnitude (the
      // row's other half sits in lane l ^ 32)
      const bf16* qp = reinterpret_cast<const bf16*>(a.q) + qrow_off + (lane >> 5) * 32;
      bf16x8 qv[kQ8][4];
      float amax = 0.0f;
#pragma unroll
      for (int s = 0; s < kQ8; ++s)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          bf16x8 v = *reinterpret_cast<const bf16x8*>(qp + s * 64 + u * 8);
          if (!qvalid) v = bf16x8{};
          qv[s][u] = v;
          amax = amax8(v, amax);
        }
      const float qscale = split_scale(max_pair32(amax), &qinv);
#pragma unroll
      for (int s = 0; s < kQ8; ++s) {
        i32x2 h[4], l[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) split_e4m3(qv[s][u], qscale, h[u], l[u]);
        qhi[s] = i32x8{h[0][0], h[0][1], h[1][0], h[1][1], h[2][0], h[2][1], h[3][0], h[3][1]};
        qlo[s] = i32x8{l[0][0], l[0][1], l[1][0], l[1][1], l[2][0], l[2][1], l[3][0], l[3][1]};
      }
    }
  }
  const int my_lo = row_lo(qrow), my_hi = row_hi(qrow);
  const unsigned my_cnt = (unsigned)max(my_hi - my_lo + 1, 0);
  // this wavefront's rows [wq0, wq1]: union and intersection of their key ranges
  const int wq0 = q0 + wave * 32;
  const int wq1 = min(wq0 + 31, q1 - 1);
  const bool wave_rows = wq0 < q1;
  const int wave_lo_min = row_lo(wq0), wave_hi_max = row_hi(wq1);
  const int wave_lo_max = row_lo(wq1), wave_hi_min = row_hi(wq0);
  const int my_half = wave * 32 / kMaskRows;

  float kdesc = *a.k_descale;
  const float vdesc = *a.v_descale;
  if (Q8) kdesc *= *a.q_descale;         // both descales scale every logit
  else kdesc *= qinv;                    // the split carries 2^e q
  // C: multiplier from the raw MFMA dot product to log2-domain scaled logits
  // (with mods the scores are converted explicitly and C is 1)
  const float lin2 = a.qk_scale * kLog2e * kdesc;
  const float C = ANYMOD ? 1.0f : lin2;
  // Mods in the log2 domain with every constant folded (the K descale and
  // the query's split scale included).  Soft-cap: c tanh(u / c) log2(e) =
  // c' - 2 c' / (1 + 2^(k s)) for the raw dot product s, u = s scale kdesc,
  // k = 2 scale kdesc log2(e) / c and c' = c log2(e); ALiBi:
  // - slope log2(e) |i' - j| by one FMA.
  const bool capped = ANYMOD && a.softcap > 0.0f;
  const float cap_k = capped ? 2.0f * lin2 / a.softcap : 0.0f;
  const float cap_c = capped ? a.softcap * kLog2e : 0.0f;
  const float slope2 = ANYMOD ? a.alibi_slope * kLog2e : 0.0f;
  const int lane_key = (lane >> 5) * 4;            // key offset of this lane's S^T registers

  f32x16 oacc[DV / 32];
#pragma unroll
  for (int d = 0; d < DV / 32; ++d) oacc[d] = f32x16{};
  float m_run = kMaxFloor, l_run = 0.0f;

  MaskBits mb;
  mb.init(a, sv, q0);
  // next active tile at or after t (t_end + 1 when none), with its half bits
  auto next_tile = [&](int t, unsigned& hb) {
    for (; t <= t_end; ++t) {
      hb = mb.tile_bits(t);
      if (hb) return t;
    }
    hb = 0;
    return t;
  };

  const int64_t vpg = a.v_pg;
  // pages of fewer than BN keys (not BIGP): per-row page lookups
  constexpr bool small_pages = PAGED && !BIGP;
  auto fast_tile = [&](int k0) { return k0 + BN <= sv.skv && !small_pages; };

  Fp8KDma<DQK, VEC, BIGP> k8;
  Fp8VDma<DV, BIGP> v8d;
  Fp8Stager<DV, PAGED> v8r;
  Fp8VecV<DV> vv8;
  constexpr int kDmaPerTile = Fp8KDma<DQK, VEC, BIGP>::kPerWave + (VREG ? 0 : Fp8VDma<DV, BIGP>::kPerWave);
  k8.init(a.page_shift, wave, lane);
  if (!VREG) v8d.init(wave, lane);
  else if (!VEC) v8r.init(a.v_st, tid);
  auto stage_ptr = [&](int i) { return lds + i * T::kStage; };
  // K (and V unless VREG) by DMA straight into the stage, FP8 as E4M3
  // bytes; VREG: V into registers, converted when stored (fp8_store)
  auto issue = [&](int t, char FA_LDS* st) {
    const int k0 = t * BN;
    const bool fast = fast_tile(k0);
    k8.issue(a, sv, reinterpret_cast<const uint8_t*>(a.k), k0, fast, st, wave, lane);
    if (!VREG) v8d.issue(a, sv, reinterpret_cast<const uint8_t*>(a.v), k0, fast, st + T::kTileK, wave, lane);
    else if (VEC) vv8.load(a, sv, reinterpret_cast<const uint8_t*>(a.v), k0, fast, tid);
    else v8r.load(a, sv, reinterpret_cast<const uint8_t*>(a.v), a.v_st, a.v_sh, vpg, k0, fast, tid);
  };

  // VREG: the registers -> bf16 in the stage, then wait for the K copies
  auto fp8_store = [&](char FA_LDS* st) {
    if (VEC) vv8.store(st + T::kTileK, tid);
    else v8r.store(st + T::kTileK, tid);
    FA_WAIT_VMCNT(0);
  };

  // Tile pipeline: t (computed now, stage sc), t1 and t2 (the next two
  // active tiles).  A three-stage ring keeps t and t1 (and after the issue
  // below t2) in flight; a two-stage ring t and t1; VREG keeps t1's V in
  // registers.
  unsigned hb, hb1, hb2;
  int t = next_tile(t_begin, hb);
  int t1 = t <= t_end ? next_tile(t + 1, hb1) : t_end + 1;
  int t2 = (!VREG && t1 <= t_end) ? next_tile(t1 + 1, hb2) : t_end + 1;
  if (VREG) hb2 = 0;
  int sc = 0;
  if (t <= t_end) {
    issue(t, stage_ptr(0));
    if (VREG) {
      fp8_store(stage_ptr(0));
    } else if (T::kStages == 3 && t1 <= t_end) {
      issue(t1, stage_ptr(1));
      FA_WAIT_VMCNT(kDmaPerTile);
    } else {
      FA_WAIT_VMCNT(0);
    }
  }

  while (t <= t_end) {
    __syncthreads();   // tile t visible to all; everyone is done with the stage reused below
    if (T::kStages == 2) {
      if (t1 <= t_end) issue(t1, stage_ptr(sc ^ 1));   // VREG: K copies and V registers
    } else if (t2 <= t_end) {
      const int s2 = sc + 2 < T::kStages ? sc + 2 : sc + 2 - T::kStages;
      issue(t2, stage_ptr(s2));
    }
    const char FA_LDS* cur = stage_ptr(sc);
    const int k0 = t * BN;
    const bool wave_active = wave_rows && k0 <= wave_hi_max && k0 + BN - 1 >= wave_lo_min &&
                             ((hb >> my_half) & 1u);
    if (wave_active) {
      // ---------------- S^T = K Q^T ----------------
      // two independent accumulation chains (key blocks 0 and 1); the K
      // fragments of step s+1 are read while the products of step s run
      f32x16 sacc[2] = {f32x16{}, f32x16{}};
      {
        // K rows as E4M3: lane holds dims 64 s + 32 (lane/32) + [0, 32) of
        // key row lane%32 of each block, two 16-byte chunks
        const int r = lane & 31;                       // swz8(r) == swz8(r + 32)
        const char FA_LDS* rowp = cur + r * T::kRowK;
        const int sw = swz8<DQK>(r);
        const int c0 = 2 * (lane >> 5);
        auto kread = [&](int s, int kb) {
          const char FA_LDS* p = rowp + kb * 32 * T::kRowK;
          return cat8(*reinterpret_cast<const i32x4 FA_LDS*>(p + (((4 * s + c0) ^ sw) << 4)),
                      *reinterpret_cast<const i32x4 FA_LDS*>(p + (((4 * s + c0 + 1) ^ sw) << 4)));
        };
        // two K fragments live: the next step's fragment for a block is read
        // once that block's last product of this step has been issued
        constexpr int S = DQK / 64;
        i32x8 ka = kread(0, 0), kb = kread(0, 1);
  #pragma unroll
        for (int s = 0; s < S; ++s) {
          sacc[0] = mfma32_fp8(ka, qhi[s], sacc[0]);
          sacc[1] = mfma32_fp8(kb, qhi[s], sacc[1]);
          if (!Q8) {
            sacc[0] = mfma32_fp8(ka, qlo[s], sacc[0]);
            __builtin_amdgcn_sched_barrier(0);
            if (s + 1 < S) ka = kread(s + 1, 0);
            __builtin_amdgcn_sched_barrier(0);
            sacc[1] = mfma32_fp8(kb, qlo[s], sacc[1]);
            __builtin_amdgcn_sched_barrier(0);
            if (s + 1 < S) kb = kread(s + 1, 1);
          } else {
            __builtin_amdgcn_sched_barrier(0);
            if (s + 1 < S) {
              ka = kread(s + 1, 0);
              kb = kread(s + 1, 1);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }

      // ---------------- score mods (log2-domain logits) ----------------
      if (ANYMOD) {
        if (capped) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i)
              sacc[kb][i] = fmaf(rcp_hw(1.0f + exp2_hw(sacc[kb][i] * cap_k)), -2.0f * cap_c, cap_c);
        } else {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) sacc[kb][i] *= lin2;
        }
        // i' - j of register (kb, i) is d0 - (32 kb + 8 (i/4) + i%4), exact in
        // fp32 below 2^24 keys apart
        const float d0 = (float)(qrow + delta - k0 - lane_key);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            sacc[kb][i] = fmaf(-slope2, fabsf(d0 - (float)(kb * 32 + (i >> 2) * 8 + (i & 3))), sacc[kb][i]);
      }

      // ---------------- masks: only tiles that straddle a row's key interval ----------------
      const bool need_mask = !(k0 >= wave_lo_max && k0 + BN - 1 <= wave_hi_min);
      if (need_mask) {
        // keeps this a real branch: selects would otherwise be speculated onto every tile
        asm volatile("" ::);
        const int base = k0 + lane_key - my_lo;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const unsigned rel = (unsigned)(base + kb * 32 + (i >> 2) * 8 + (i & 3));
            sacc[kb][i] = rel < my_cnt ? sacc[kb][i] : -INFINITY;
          }
      }
      // ---------------- online softmax ----------------
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
      mx = max_pair32(mx);
      const float m_new = fmaxf(m_run, mx * C);
      if (__builtin_amdgcn_ballot_w64(m_new > m_run + kLazyTau) != 0) {
        const float alpha = exp2_hw(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int d = 0; d < DV / 32; ++d)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[d][i] *= alpha;
      }
      // P^T operand of key step u = registers 8 (u%2) .. +8 of key block u/2
      auto p_elem = [&](int u, int e) {
        const float p = exp2_hw(fmaf(sacc[u >> 1][(u & 1) * 8 + e], C, -m_run));
        l_run += p;
        return (bf16)p;
      };
      // O^T += V^T P^T, product n = u NDV + d.  For E4M3 V and vectorised
      // pages the exponentials of key step u + 1 run under the products of
      // step u (only step 0's are computed ahead of the products), with the
      // V fragments read four products ahead.  A = V^T: lane m + 32 h takes d = 32 blk + m and, of the 16
      // keys of step u, keys 4h..4h+3 and 8+4h..8+4h+3 (the order of P^T).
      bf16x8 pf[4];
      auto pv_loop = [&](auto vraw, auto vconv) {
        constexpr int NDV = DV / 32;
        constexpr int NV = 4 * NDV;
        constexpr int kAhead = 4;
        decltype(vraw(0)) vr[NV];
#pragma unroll
        for (int n = 0; n < kAhead && n < NV; ++n) vr[n] = vraw(n);
#pragma unroll
        for (int e = 0; e < 8; ++e) pf[0][e] = p_elem(0, e);
#pragma unroll
        for (int n = 0; n < NV; ++n) {
          const int u = n / NDV, d = n % NDV;
          if (n + kAhead < NV) vr[n + kAhead] = vraw(n + kAhead);
          oacc[d] = mfma32(vconv(vr[n]), pf[u], oacc[d]);
          if (u + 1 < 4) {
#pragma unroll
            for (int e = d * 8 / NDV; e < (d + 1) * 8 / NDV; ++e) pf[u + 1][e] = p_elem(u + 1, e);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      auto as_is = [](bf16x8 x) { return x; };
      if constexpr (FP8 && !VREG) {
        // E4M3 key-major rows: lanes 2t+q of a 16-lane group read half q of
        // row t of the group's eight keys; the transposing read gives lane i
        // byte column i of those rows, converted exactly to bf16
        const char FA_LDS* vt = cur + T::kTileK;
        const int h = lane >> 5;
        const int i16 = lane & 15, t8 = i16 >> 1, q = i16 & 1;
        const int key = (t8 < 4 ? t8 : 4 + t8) + 4 * h;   // key within the 16-key step
        const int cg = (lane >> 4) & 1;                    // 16-dim half of the 32-dim block
        pv_loop(
            [&](int n) {
              const int u = n / (DV / 32), d = n % (DV / 32);
              const int r = u * 16 + key;
              return lds_read_tr8(vt + r * DV + q * 8 + (((2 * d + cg) ^ swzv8<DV>(r)) << 4));
            },
            [](auto w) { return fp8x8_to_bf16(w); });
      } else if constexpr (VEC) {
        // V^T tile: row d = 32 blk + lane%32, chunk 2u + lane/32
        const char FA_LDS* vt = cur + T::kTileK + (lane & 31) * (BN * 2);
        const int sw = ((lane & 31) >> 1) & 7;
        pv_loop(
            [&](int n) {
              const int u = n / (DV / 32), d = n % (DV / 32);
              return lds_read_b128(vt + d * 32 * (BN * 2) + (((2 * u + (lane >> 5)) ^ sw) << 4));
            },
            as_is);
      } else {
        // bf16 V^T fragments read transposed (V staged through registers);
        // here every exponential first, then the products (interleaving
        // measured slower for this variant)
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int e = 0; e < 8; ++e) pf[u][e] = p_elem(u, e);
        const char FA_LDS* vt = cur + T::kTileK;
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
            const bf16x4 lo4 = lds_read_tr16(vt + r1 * T::kRowV + ((chunk ^ swz<T::kRowV>(r1)) << 4) + half * 8);
            const bf16x4 hi4 = lds_read_tr16(vt + r2 * T::kRowV + ((chunk ^ swz<T::kRowV>(r2)) << 4) + half * 8);
            bf16x8 vf;
            vf[0] = lo4[0]; vf[1] = lo4[1]; vf[2] = lo4[2]; vf[3] = lo4[3];
            vf[4] = hi4[0]; vf[5] = hi4[1]; vf[6] = hi4[2]; vf[7] = hi4[3];
            oacc[d] = mfma32(vf, pf[u], oacc[d]);
          }
        }
      }
    }

    // publish the next tile: wait for this wavefront's copies of t1 (t2 may
    // stay in flight)
    const int s1 = sc + 1 < T::kStages ? sc + 1 : 0;
    if (VREG) {
      if (t1 <= t_end) fp8_store(stage_ptr(s1));
    } else if (T::kStages == 3 && t2 <= t_end) {
      FA_WAIT_VMCNT(kDmaPerTile);
    } else {
      FA_WAIT_VMCNT(0);
    }
    sc = s1;
    t = t1;
    hb = hb1;
    if (VREG) {
      t1 = t1 <= t_end ? next_tile(t1 + 1, hb1) : t_end + 1;
    } else {
      t1 = t2;
      hb1 = hb2;
      t2 = t2 <= t_end ? next_tile(t2 + 1, hb2) : t_end + 1;
    }
  }

  // ---------------- epilogue ----------------
  const float l_tot = sum_pair32(l_run);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  const float osc = inv * vdesc;
  // every wavefront is done with the stages (and no copy is in flight)
  // after this barrier: O leaves through them
  static_assert(4 * 32 * DV * 2 <= T::kLds, "the output rows fit in the stages");
  __syncthreads();
  store_o_rows<DV>(oacc, osc, lds + wave * 32 * (DV * 2),
                   a.o + (sv.qstart + wq0) * a.o_st + (int64_t)sv.h * a.o_sh, a.o_st, sv.sq - wq0, lane);
  if (qvalid) {
    if (lane < 32) {
      const float lse = l_tot > 0.0f ? (m_run + log2_hw(l_tot)) * kLn2 : -INFINITY;
      int64_t li;
      if (a.cu_q) li = (int64_t)sv.h * a.lse_tq + sv.qstart + qrow;
      else li = ((int64_t)sv.b * a.Hq + sv.h) * a.Sq + qrow;
      a.lse[li] = lse;
    }
  }
}

template <int DQK, int DV, bool FP8, bool PAGED, bool VEC, int MODS>
static hipError_t launch_prefill(const PrefillArgs& a, int n_bh, int n_qtiles, hipStream_t stream) {
  dim3 grid((n_bh + 7) / 8 * 8, n_qtiles);
  const bool q8 = FP8 && a.q_descale, bigp = a.page_shift >= 6;
  if (q8 && bigp)
    hipLaunchKernelGGL((fa_prefill_kernel<DQK, DV, FP8, PAGED, VEC, FP8, MODS, true>), grid, dim3(NTHREADS), 0, stream, a);
  else if (q8)
    hipLaunchKernelGGL((fa_prefill_kernel<DQK, DV, FP8, PAGED, VEC, FP8, MODS, false>), grid, dim3(NTHREADS), 0, stream, a);
  else if (bigp)
    hipLaunchKernelGGL((fa_prefill_kernel<DQK, DV, FP8, PAGED, VEC, false, MODS, true>), grid, dim3(NTHREADS), 0, stream, a);
  else
    hipLaunchKernelGGL((fa_prefill_kernel<DQK, DV, FP8, PAGED, VEC, false, MODS, false>), grid, dim3(NTHREADS), 0, stream, a);
  return hipGetLastError();
}

// Instantiated shapes here: (192,128), (128,128) and (192,192) for FP8 E4M3
// paged caches, head-major or vectorised pages, without or with score mods.  bf16 K/V
// go to the software-pipelined kernel (fa_prefill_bf16.hip).
hipError_t prefill_dispatch(const PrefillArgs& a, int dqk, int dv, bool fp8, bool paged, bool vec, int mods,
                            int n_bh, int n_qtiles, hipStream_t stream, bool* supported) {
  *supported = true;
  if (!fp8) return prefill_bf16_dispatch(a, dqk == dv ? dqk : -1, paged, mods, n_bh, n_qtiles, stream, supported);
#define FA_CASE(DQ, DVV, F8, PG, VC, MD)                                                       \
  if (dqk == DQ && dv == DVV && fp8 == F8 && paged == PG && vec == VC && mods == MD)           \
    return launch_prefill<DQ, DVV, F8, PG, VC, MD>(a, n_bh, n_qtiles, stream);
  // every score mod goes to the one mods variant
  mods = mods ? (kModAlibi | kModSoftcap) : 0;
  FA_CASE(192, 128, true, true, false, 0) FA_CASE(192, 128, true, true, false, 3)
  FA_CASE(128, 128, true, true, false, 0) FA_CASE(128, 128, true, true, false, 3)
  FA_CASE(192, 128, true, true, true, 0) FA_CASE(192, 128, true, true, true, 3)
  FA_CASE(128, 128, true, true, true, 0) FA_CASE(128, 128, true, true, true, 3)
  FA_CASE(192, 192, true, true, false, 0) FA_CASE(192, 192, true, true, false, 3)
  FA_CASE(192, 192, true, true, true, 0) FA_CASE(192, 192, true, true, true, 3)
#undef FA_CASE
  *supported = false;
  return hipSuccess;
}

}  // namespace fa
