// Split-KV decode over a paged FP8 E4M3 cache, and the split combine, for gfx950.
//
// Decode is bound by HBM bandwidth: every cache byte is read once, and the
// q-heads that share a kv-head (GQA) are packed into the rows of one matrix
// product so that they share that read.
//
// Work split (stream-K style): the 32-key tiles of all units (sequence,
// kv-head) are laid end to end, and wavefront w of W takes tiles
// [w T / W, (w+1) T / W) of the T in total, so every wavefront streams the
// same number of cache bytes whatever the mix of context lengths.  A share
// may start or end inside a unit and may cover several short units; for each
// unit segment the wavefront writes a partial result (O normalised by its own
// denominator, and its natural-log LSE) to slot w + unit of the workspace.
// A unit's segments come from consecutive workers, so the combine kernel finds
// them from the unit's first and last tile and merges them by their LSE
// weights (LSE PR: split-K partials are finalised from per-split (m, l)).
// A one-workgroup plan kernel turns the per-sequence key counts into the
// tile prefix both kernels read, so the split needs no host round trip.
//
// Rows (query x q-head of the group, up to 16 per row block) are the N side
// of v_mfma_f32_16x16x32_bf16 products; one or two row blocks per wavefront:
//
//   S^T[32 keys x 16 rows] = K . Q^T     v_mfma_f32_16x16x32_fp8_fp8: A = the
//                                          E4M3 K bytes from LDS, B = Q as two
//                                          E4M3 parts (below), two products
//   O^T[Dv x 16 rows]    += V^T . P^T    bf16 MFMA: A = V read transposed from
//                                          LDS (ds_read_b64_tr_b8) and converted
//                                          exactly, B = P in bf16
//
// The K bytes enter the FP8 product as they are (no conversion instructions,
// the dominant vector cost of the loop otherwise).  Q (bf16) is scaled by 16
// (exact) and written as hi + lo with hi = E4M3(16 q), lo = E4M3(16 q - hi):
// the two 3-bit mantissas carry q to about 2^-8 relative, and the scaled
// values stay clear of the E4M3 subnormal range; the 1/16 is folded into the
// logit constant.  Each product is exact (3-bit x 3-bit mantissas) and
// accumulated in fp32, so the logits differ from the bf16-Q logits only by
// the split's rounding (about 1e-3 in natural-log units at the largest
// logits of N(0,1) data).  E4M3 queries (with their own descale) are the B
// operand as they are: one exact product per step, no split.
//
// The cache streams through registers with coalesced 16-byte loads (lane l
// of load i takes bytes [1024 i + 16 l, +16) of the tile, so every load
// instruction covers whole cache lines), one tile ahead; the wavefront then
// writes the tile into its own LDS buffer (16-byte chunks of K and V rows
// XOR-swizzled) and reads the matrix fragments back.  The wavefronts are
// independent (no barrier), and small register and LDS footprints let twelve
// of them share a CU, so plenty of cache lines are in flight.
//
// Page lookups are bounded to the sequence's own pages and every byte offset
// is 64-bit, so caches beyond 4 GiB are addressed correctly; keys past
// seqlen_k are clamped for the load and removed by select before the softmax.
//
// Vectorised pages (the 5-D layout of the paged FP8 PR review: K page
// [Hkv, D/16, page, 16], V page [Hkv, page/16, Dv, 16]) keep the cache's
// order in LDS.  A K load instruction covers two 16-byte columns c of the
// tile's 32 keys (lanes 0-31 column 2i, lanes 32-63 column 2i+1; each half
// is 512 contiguous bytes) and lands in a column-major K tile.  A V load
// covers 64 head dims of one 16-key block (1 KB contiguous): these are
// already V^T rows, so the tile is kept as V^T [Dv][32 keys] with each row's
// keys in the order the P^T operand enumerates them, and the A fragments
// are plain 8-byte reads.  Every 16-byte LDS store of these tiles is
// contiguous per 16 lanes: measured on the hardware, a 16-byte store whose
// 16-lane groups do not each write one contiguous 256 bytes takes twice the
// cycles, whatever its bank pattern.  Value bytes past the sequence's end
// share a 16-byte load with live ones and are cleared.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

constexpr int kDecWaves = 4;
constexpr int kDecKT = 32;       // keys per tile

// V tile rows are D_v bytes; chunk c (16 bytes) of row r is stored at
// c ^ dec_vswz<D_v>(r).  A transposed read instruction takes, per group of 16
// lanes g, rows {4g..4g+3, 16+4g..16+4g+3} at one chunk (two 8-byte halves).
// 128-byte rows: with this map the even rows of lanes 0-31 (and of lanes
// 32-63), and the odd rows, each cover all eight chunks, i.e. the 64 banks
// exactly once.  192-byte rows (12 chunks): a row starts 48 banks after the
// previous one, so rows 4 apart share banks; the map (inside the aligned
// group of four chunks) gives the four rows of a half wavefront that share a
// residue mod 4 four different chunks.
template <int DV>
__device__ __forceinline__ int dec_vswz(int r) {
  if (DV == 192) return ((r >> 2) & 1) | (((r >> 4) & 1) << 1);
  return ((r >> 1) & 3) | (((r >> 4) & 1) << 2);
}

// K tile rows are D_qk bytes (48 banks at 192); chunk c of row r is stored at
// c ^ dec_kswz(r), which stays inside the aligned group of four chunks.  A
// K fragment read takes 8 bytes of rows r..r+15 at one chunk: rows four apart
// start on the same bank and the map moves them to different chunks.
__device__ __forceinline__ int dec_kswz(int r) { return (r >> 2) & 3; }

__device__ __forceinline__ i32x2 lds_read_tr8(const char FA_LDS* __restrict__ p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((i32x2 FA_LDS*)(p));
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16_fp8(i32x2 a, i32x2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(__builtin_bit_cast(long, a), __builtin_bit_cast(long, b), c, 0, 0,
                                                    0);
}

// max / sum over the four lanes {l, l^16, l^32, l^48} (the four key groups
// that hold one row's scores)
__device__ __forceinline__ float max_quad16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  return max_pair32(x);
}
__device__ __forceinline__ float sum_quad16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  return sum_pair32(x);
}

template <int DQK, int DV>
struct DecTraits {
  static constexpr int kKTile = kDecKT * DQK;
  static constexpr int kVTile = kDecKT * DV;
  static constexpr int kWaveLds = kKTile + kVTile;
  static constexpr int kKLoads = kDecKT * DQK / 1024;   // 16-byte loads per lane per tile
  static constexpr int kVLoads = kDecKT * DV / 1024;
};

// Tiles per sequence, as an exclusive prefix: tiles[b] = sum over b' < b of
// ceil(keys_b' / 32) (0 for sequences with no query; keys capped at kv_cap), tiles[B] the total.
// One workgroup of 256 threads: each thread sums a contiguous run of
// sequences, thread 0 scans the 256 partial sums, each thread writes its run.
__global__ __launch_bounds__(256) void fa_decode_plan_kernel(const DecodePlanArgs a) {
  __shared__ int part[257];
  const int tid = threadIdx.x;
  const int per = (a.B + 255) / 256;
  const int b0 = min(a.B, tid * per), b1 = min(a.B, b0 + per);
  auto nt = [&](int b) {
    if (a.cu_q[b + 1] - a.cu_q[b] <= 0) return 0;
    const int kv = min(a.seqlen_k[b], a.kv_cap);
    return kv > 0 ? (kv + kDecKT - 1) / kDecKT : 0;
  };
  int sum = 0;
  for (int b = b0; b < b1; ++b) sum += nt(b);
  part[tid] = sum;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int i = 0; i < 256; ++i) {
      const int x = part[i];
      part[i] = run;
      run += x;
    }
    part[256] = run;
  }
  __syncthreads();
  int run = part[tid];
  for (int b = b0; b < b1; ++b) {
    a.tiles[b] = run;
    run += nt(b);
  }
  if (tid == 0) a.tiles[a.B] = part[256];
}

// worker that owns tile i of T in a split over W workers
__device__ __forceinline__ int worker_of(int64_t i, int64_t T, int W) { return (int)(((i + 1) * W - 1) / T); }

template <int DQK, int DV, int NRB, int NBUF, bool VEC, bool Q8, bool MODS>
__global__ __launch_bounds__(kDecWaves * 64)
__attribute__((amdgpu_waves_per_eu((NBUF >= 3 || DV > 128) ? 1 : (NRB == 1 && NBUF == 1 ? 3 : 2))))
void fa_decode_kernel(const DecodeArgs a) {
  static_assert(DQK % 32 == 0 && (DV == 128 || DV == 192) && (kDecKT * DQK) % 1024 == 0, "decode tile shapes");
  constexpr int kVPerBlk = DV / 64;                     // V loads per 16-key block (vectorised pages)
  using T = DecTraits<DQK, DV>;
  constexpr int kSteps = DQK / 32;                      // K.Q^T MFMA steps per 16-key half
  constexpr int kDB = DV / 16;                          // 16-wide blocks of the output
  __shared__ __attribute__((aligned(1024))) char lds_raw[kDecWaves * T::kWaveLds];

  // the wavefront index is uniform within a wavefront; readfirstlane lets the
  // compiler keep everything derived from it in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int w = blockIdx.x * kDecWaves + wave;
  if (w >= a.n_workers) return;
  // this worker's share [s0, s1) of the T tiles of all units
  const int64_t ntot = (int64_t)a.Hkv * load_uniform_i32(a.tiles, a.B);
  const int64_t s0 = (int64_t)w * ntot / a.n_workers, s1 = (int64_t)(w + 1) * ntot / a.n_workers;
  if (s0 >= s1) return;
  char FA_LDS* klds = (char FA_LDS*)(lds_raw) + wave * T::kWaveLds;
  char FA_LDS* vlds = klds + T::kKTile;
  const int kgrp = lane >> 4;                           // key group of this lane's scores

  // LDS byte of this lane's piece of each tile load (swizzled chunk)
  int kst[T::kKLoads], vst[T::kVLoads];
#pragma unroll
  for (int i = 0; i < T::kKLoads; ++i) {
    const int off = i * 1024 + lane * 16, row = off / DQK;
    // vectorised pages: column-major tile (column c of key r at 512 c + 16 r),
    // so each load's store is contiguous
    kst[i] = VEC ? off : row * DQK + ((((off % DQK) >> 4) ^ dec_kswz(row)) << 4);
  }
#pragma unroll
  for (int n = 0; n < T::kVLoads; ++n) {
    const int off = n * 1024 + lane * 16, row = off / DV;
    vst[n] = row * DV + ((((off % DV) >> 4) ^ dec_vswz<DV>(row)) << 4);
  }
  // transposed V reads: lanes 2t+q of key group kgrp take row vrow(t), half q
  const int t8 = (lane & 15) >> 1, vq = lane & 1;
  const int vrow = t8 < 4 ? 4 * kgrp + t8 : 16 + 4 * kgrp + (t8 - 4);
  const char FA_LDS* vrd = vlds + vrow * DV + vq * 8;
  const int vsw = dec_vswz<DV>(vrow);
  // V^T tile (vectorised pages): row d is 32 bytes, byte 8 kgrp + e holds key
  // (e / 4) * 16 + 4 kgrp + e % 4, so the lanes of key group kgrp read their
  // 8 bytes of row 16 blk + lane%16 at 8-byte unit kgrp.  The two 16-byte
  // halves of the rows are stored apart (half h of row d at h Dv 16 + 16 d):
  // a 16-lane group of a 16-byte store then writes one contiguous 256 bytes
  // (any other pattern measured twice the cycles), and a half wavefront's
  // reads cover the 64 banks once.
  const char FA_LDS* vtrd = vlds + (kgrp >> 1) * (DV * 16) + (lane & 15) * 16 + (kgrp & 1) * 8;
  const int vtst = lane * 16;                         // row d = lane (and 64 + lane, ...)
  // K fragment reads: row kh*16 + lane%16 (the swizzle of r and r+16 agree),
  // chunk 2 st + kgrp/2, half kgrp%2
  const int krow = lane & 15, kx = VEC ? 0 : dec_kswz(krow);
  const char FA_LDS* krd = klds + (VEC ? krow * 16 : krow * DQK) + (kgrp & 1) * 8;
  const float kdesc = *a.k_descale, vdesc = *a.v_descale;
  // E4M3 Q enters as it is, with its descale; bf16 Q scaled per row by the
  // power of two of its split (folded into that row's constant below)
  const float C0 = Q8 ? a.qk_scale * kLog2e * kdesc * *a.q_descale : a.qk_scale * kLog2e * kdesc;
  const int pmask = (1 << a.page_shift) - 1;

  // One unit segment: sequence b, kv-head g, tiles [t0, t1) -> partial slot.
  auto segment = [&](int b, int g, int t0, int t1, int64_t slot) {
    const int skv = min(a.seqlen_k[b], a.kv_cap);       // bounds the page-table lookups
    const int qs = a.cu_q[b];
    const int sq = a.cu_q[b + 1] - qs;
    const int R = sq * a.group;
    const int k_lo = t0 * kDecKT;
    const int k_hi = min(skv, t1 * kDecKT);
    const int delta = skv - sq;

    // rows of this lane: row block rb holds rows rb*16 + lane%16
    bool rvalid[NRB];
    int hq[NRB], my_lo[NRB], my_hi[NRB], ipos[NRB];
    int64_t tok[NRB];
    const uint8_t* bmrow[NRB];   // block-mask row of each row block (null: no mask)
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int r = rb * 16 + (lane & 15);
      rvalid[rb] = r < R;
      const int qi = rvalid[rb] ? r / a.group : 0;
      hq[rb] = g * a.group + (rvalid[rb] ? r % a.group : 0);
      tok[rb] = qs + qi;
      const int ip = qi + delta;
      ipos[rb] = ip;
      // (mask indices are clamped / bounded like the prefill's: a query or
      // key block past the mask's extent reads as inactive or as its last row)
      bmrow[rb] = (MODS && a.bmask) ? a.bmask + (((int64_t)b * a.Hq + hq[rb]) * a.bm_nqb + min(qi / a.bm_bq, a.bm_nqb - 1)) *
                                          a.bm_nkb
                          : nullptr;
      int hi = k_hi - 1, lo = k_lo;
      if (a.causal) hi = min(hi, ip);
      if (a.win_right >= 0) hi = min(hi, ip + a.win_right);
      if (a.win_left >= 0) lo = max(lo, ip - a.win_left);
      my_lo[rb] = lo;
      my_hi[rb] = hi;
    }
    // keys every row of this unit sees: tiles inside [all_lo, all_hi] skip
    // the per-score mask
    int all_hi = k_hi - 1, all_lo = k_lo;
    if (a.causal) all_hi = min(all_hi, delta);
    if (a.win_right >= 0) all_hi = min(all_hi, delta + a.win_right);
    if (a.win_left >= 0) all_lo = max(all_lo, (sq - 1) + delta - a.win_left);

    const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.k) + (int64_t)g * a.k_sh;
    const uint8_t* vbase = reinterpret_cast<const uint8_t*>(a.v) + (int64_t)g * a.v_sh;
    const int32_t* bt = a.block_table + (int64_t)b * a.max_pages;
    const int last = t1 - t0 - 1;

    // Coalesced tile loads: load i of this lane covers bytes [1024 i + 16
    // lane, +16) of the tile.  Page rows are contiguous (row stride = head
    // dim), so with pages of 32 keys or more a whole tile is one block of a
    // page: one wave-uniform scalar page lookup per tile, clamped to the
    // cache.  Smaller pages take a per-lane lookup of each row's page.  In the sequence's
    // last, partial tile the rows past the end re-read the last key (masked
    // before the softmax), so no stale bytes reach the products.
    using KBuf = i32x4[T::kKLoads];
    using VBuf = i32x4[T::kVLoads];
    KBuf kbuf[NBUF];
    VBuf vbuf[NBUF];
    auto load_tile = [&](int t, KBuf& kb, VBuf& vb) {
      const int k0 = k_lo + t * kDecKT;
      const int nv = skv - k0;                          // rows of the tile inside the sequence
      if (VEC) {
        // the tile's two 16-key blocks: one page when pages hold 32 keys or
        // more, else the pages of keys k0 and k0 + 16 (clamped to the sequence)
        const int64_t p0 = min(max(load_uniform_i32(bt, k0 >> a.page_shift), 0), a.num_pages - 1);
        const int64_t p1 = a.page_shift >= 5
                               ? p0
                               : min(max(load_uniform_i32(bt, (k0 + min(16, nv - 1)) >> a.page_shift), 0),
                                     a.num_pages - 1);
        // K: lane l of load i takes column 2i + l/32 of key row min(l%32, nv-1)
        const int r = min(lane & 31, nv - 1);
        const uint8_t* kp = kbase + (r >= 16 ? p1 : p0) * a.k_pg + ((k0 + r) & pmask) * 16 +
                            ((lane >> 5) << (a.page_shift + 4));
#pragma unroll
        for (int i = 0; i < T::kKLoads; ++i)
          kb[i] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(kp + ((2 * i) << (a.page_shift + 4))));
        // V: load n takes dims 64 (n % kVPerBlk) + l of block n / kVPerBlk
        const uint8_t* vt0 = vbase + p0 * a.v_pg + ((k0 & pmask) >> 4) * (DV * 16) + lane * 16;
        const uint8_t* vt1 = vbase + p1 * a.v_pg + (((k0 + 16) & pmask) >> 4) * (DV * 16) + lane * 16;
#pragma unroll
        for (int n = 0; n < T::kVLoads; ++n)
          vb[n] = __builtin_nontemporal_load(
              reinterpret_cast<const i32x4*>((n < kVPerBlk ? vt0 : vt1) + (n % kVPerBlk) * 1024));
        if (nv < kDecKT) {
#pragma unroll
          for (int n = 0; n < T::kVLoads; ++n) vb[n] = keep_bytes(vb[n], nv - 16 * (n / kVPerBlk));
        }
        return;
      }
      if (a.page_shift < 5) {
        // pages smaller than a tile: each lane looks up the page of the key
        // row its 16 bytes belong to (a chunk never straddles a row)
#pragma unroll
        for (int i = 0; i < T::kKLoads; ++i) {
          const int off = i * 1024 + lane * 16, key = k0 + min(off / DQK, nv - 1);
          const int64_t pg = min(max(bt[key >> a.page_shift], 0), a.num_pages - 1);
          kb[i] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(
              kbase + pg * a.k_pg + (int64_t)(key & pmask) * DQK + off % DQK));
        }
#pragma unroll
        for (int n = 0; n < T::kVLoads; ++n) {
          const int off = n * 1024 + lane * 16, key = k0 + min(off / DV, nv - 1);
          const int64_t pg = min(max(bt[key >> a.page_shift], 0), a.num_pages - 1);
          vb[n] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(
              vbase + pg * a.v_pg + (int64_t)(key & pmask) * DV + off % DV));
        }
        return;
      }
      const int64_t page = min(max(load_uniform_i32(bt, k0 >> a.page_shift), 0), a.num_pages - 1);
      const uint8_t* kt = kbase + page * a.k_pg + (int64_t)(k0 & pmask) * DQK;
      const uint8_t* vt = vbase + page * a.v_pg + (int64_t)(k0 & pmask) * DV;
      if (nv >= kDecKT) {
#pragma unroll
        for (int i = 0; i < T::kKLoads; ++i) kb[i] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(kt + i * 1024 + lane * 16));
#pragma unroll
        for (int n = 0; n < T::kVLoads; ++n) vb[n] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(vt + n * 1024 + lane * 16));
      } else {
#pragma unroll
        for (int i = 0; i < T::kKLoads; ++i) {
          const int off = i * 1024 + lane * 16, row = off / DQK;
          kb[i] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(kt + min(row, nv - 1) * DQK + off % DQK));
        }
#pragma unroll
        for (int n = 0; n < T::kVLoads; ++n) {
          const int off = n * 1024 + lane * 16, row = off / DV;
          vb[n] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(vt + min(row, nv - 1) * DV + off % DV));
        }
      }
    };

    // Q fragments (B operand): step s of row block rb holds the E4M3 parts
    // of 16 Q[row rb*16 + lane%16][d = 32 s + 8 (lane/16) + e]; read before
    // the first tile is requested, so waiting for them never waits for the
    // cache loads
    i32x2 qhi[NRB][kSteps], qlo[NRB][kSteps];
    float C[NRB];        // per row block: raw dot product -> log2-domain scaled logit
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int64_t qoff = tok[rb] * a.q_st + (int64_t)hq[rb] * a.q_sh + kgrp * 8;
      C[rb] = C0;
      if (Q8) {
#pragma unroll
        for (int st = 0; st < kSteps; ++st) {
          // E4M3 queries are the B operand as they are (one product per step)
          i32x2 x = *reinterpret_cast<const i32x2*>(reinterpret_cast<const uint8_t*>(a.q) + qoff + 32 * st);
          qhi[rb][st] = rvalid[rb] ? x : i32x2{};
          qlo[rb][st] = i32x2{};
        }
      } else {
        // the row's power-of-two split scale from its largest magnitude (its
        // dims are spread over the four lanes with this lane % 16)
        const bf16* qp = reinterpret_cast<const bf16*>(a.q) + qoff;
        float amax = 0.0f;
#pragma unroll
        for (int st = 0; st < kSteps; ++st) {
          bf16x8 x = *reinterpret_cast<const bf16x8*>(qp + 32 * st);
          if (!rvalid[rb]) x = bf16x8{};
          amax = amax8(x, amax);
        }
        float qinv;
        const float qscale = split_scale(max_quad16(amax), &qinv);
        C[rb] = C0 * qinv;
        // read the row again (cached) rather than keep it in registers
        asm volatile("" ::: "memory");
#pragma unroll
        for (int st = 0; st < kSteps; ++st) {
          bf16x8 x = *reinterpret_cast<const bf16x8*>(qp + 32 * st);
          if (!rvalid[rb]) x = bf16x8{};
          split_e4m3(x, qscale, qhi[rb][st], qlo[rb][st]);
        }
      }
    }
    // Score mods (the MODS variant; which ones is a runtime, uniform choice):
    // the scores are converted to log2-domain logits explicitly and C
    // becomes 1.  Soft-cap: c tanh(u / c) log2(e) =
    // c' - 2 c' / (1 + 2^(k s)) for the raw dot product s (u = s C / log2(e),
    // k = 2 C / c, c' = c log2(e)); ALiBi: - slope log2(e) |i' - j|.
    const bool mods_on = MODS && (a.alibi_slope != 0.0f || a.softcap > 0.0f);
    const bool capped = MODS && a.softcap > 0.0f;
    const float cap_c = capped ? a.softcap * kLog2e : 0.0f, slope2 = a.alibi_slope * kLog2e;
    float lin[NRB], cap_k[NRB];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      lin[rb] = C[rb];
      cap_k[rb] = capped ? 2.0f * C[rb] / a.softcap : 0.0f;
      if (mods_on) C[rb] = 1.0f;
    }
#pragma unroll
    for (int j = 0; j < NBUF; ++j) load_tile(min(j, last), kbuf[j], vbuf[j]);

    f32x4 oacc[NRB][kDB];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
      for (int d = 0; d < kDB; ++d) oacc[rb][d] = f32x4{};
    float m_run[NRB], l_run[NRB];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      m_run[rb] = kMaxFloor;
      l_run[rb] = 0.0f;
    }

    // One tile: registers -> this wavefront's LDS buffer (the fragment reads
    // of the previous tile were consumed, hence complete, before this
    // point), refill the registers with the tile NBUF ahead, then the
    // products from LDS.
    auto step = [&](int t, KBuf& kb, VBuf& vb, bool refill) {
#pragma unroll
      for (int i = 0; i < T::kKLoads; ++i) *reinterpret_cast<i32x4 FA_LDS*>(klds + kst[i]) = kb[i];
      if (VEC) {
        // row d = 64 hr + lane from loads hr (block 0) and kVPerBlk + hr
        // (block 1): dword j of block b goes to dword 2 j + b
#pragma unroll
        for (int hr = 0; hr < kVPerBlk; ++hr) {
          const i32x4 b0 = vb[hr], b1 = vb[kVPerBlk + hr];
          char FA_LDS* row = vlds + vtst + hr * 64 * 16;
          *reinterpret_cast<i32x4 FA_LDS*>(row) = i32x4{b0[0], b1[0], b0[1], b1[1]};
          *reinterpret_cast<i32x4 FA_LDS*>(row + DV * 16) = i32x4{b0[2], b1[2], b0[3], b1[3]};
        }
      } else {
#pragma unroll
        for (int n = 0; n < T::kVLoads; ++n) *reinterpret_cast<i32x4 FA_LDS*>(vlds + vst[n]) = vb[n];
      }
      if (refill) load_tile(min(t + NBUF, last), kb, vb);

      // block-mask activity of this tile for each row block (a 32-key tile
      // lies in one mask block); read before the products so that they
      // cover the load
      const int k0 = k_lo + t * kDecKT;
      bool act[NRB];
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) act[rb] = true;
      if (MODS && a.bmask) {
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
          const int kb = k0 / a.bm_bk;
          act[rb] = kb < a.bm_nkb && bmrow[rb][kb] != 0;
        }
      }

      // ---- S^T = K Q^T ----  (fragment n = (kh, st); each read runs two
      // fragments ahead of its products, one chunk per fragment)
      constexpr int kNK = 2 * kSteps;
      auto kread = [&](int n) {
        const int kh = n / kSteps, st = n % kSteps;
        const int c = (2 * st + (kgrp >> 1)) ^ kx;
        if (VEC) return *reinterpret_cast<const i32x2 FA_LDS*>(krd + kh * 16 * 16 + c * 512);
        return *reinterpret_cast<const i32x2 FA_LDS*>(krd + kh * 16 * DQK + c * 16);
      };
      f32x4 sacc[NRB][2];
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) sacc[rb][0] = sacc[rb][1] = f32x4{};
      i32x2 kraw[kNK];
      kraw[0] = kread(0);
      kraw[1] = kread(1);
#pragma unroll
      for (int n = 0; n < kNK; ++n) {
        if (n + 2 < kNK) kraw[n + 2] = kread(n + 2);
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
          sacc[rb][n / kSteps] = mfma16_fp8(kraw[n], qhi[rb][n % kSteps], sacc[rb][n / kSteps]);
          if (!Q8) sacc[rb][n / kSteps] = mfma16_fp8(kraw[n], qlo[rb][n % kSteps], sacc[rb][n / kSteps]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }

      // ---- score mods, masks and online softmax, per row block ----
      bf16x8 pf[NRB];
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        if (mods_on) {
          // i' - j of register (kh, i) is d0 - (16 kh + i), exact in fp32
          // below 2^24 keys apart
          const float d0 = (float)(ipos[rb] - k0 - 4 * kgrp);
#pragma unroll
          for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              float x = sacc[rb][kh][i];
              x = capped ? fmaf(rcp_hw(1.0f + exp2_hw(x * cap_k[rb])), -2.0f * cap_c, cap_c) : x * lin[rb];
              sacc[rb][kh][i] = fmaf(-slope2, fabsf(d0 - (float)(kh * 16 + i)), x);
            }
        }
        if (MODS && a.bmask) {
#pragma unroll
          for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int i = 0; i < 4; ++i) sacc[rb][kh][i] = act[rb] ? sacc[rb][kh][i] : -INFINITY;
        }
        if (k0 < all_lo || k0 + kDecKT - 1 > all_hi) {
          // keeps this a real branch: selects would otherwise be speculated onto every tile
          asm volatile("" ::);
#pragma unroll
          for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int j = k0 + kh * 16 + 4 * kgrp + i;
              sacc[rb][kh][i] = (j >= my_lo[rb] && j <= my_hi[rb]) ? sacc[rb][kh][i] : -INFINITY;
            }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sacc[rb][kh][i]);
        mx = max_quad16(mx);
        const float m_new = fmaxf(m_run[rb], mx * C[rb]);
        if (__builtin_amdgcn_ballot_w64(m_new > m_run[rb] + 8.0f) != 0) {
          const float alpha = exp2_hw(m_run[rb] - m_new);
          m_run[rb] = m_new;
          l_run[rb] *= alpha;
#pragma unroll
          for (int d = 0; d < kDB; ++d) oacc[rb][d] *= alpha;
        }
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p = exp2_hw(fmaf(sacc[rb][kh][i], C[rb], -m_run[rb]));
            l_run[rb] += p;
            pf[rb][kh * 4 + i] = (bf16)p;
          }
      }

      // ---- O^T += V^T P^T ----  (same two-ahead chunking)
      auto vread = [&](int d) {
        if (VEC) return *reinterpret_cast<const i32x2 FA_LDS*>(vtrd + d * 16 * 16);
        return lds_read_tr8(vrd + ((d ^ vsw) << 4));
      };
      i32x2 vraw[kDB];
      vraw[0] = vread(0);
      vraw[1] = vread(1);
#pragma unroll
      for (int d = 0; d < kDB; ++d) {
        if (d + 2 < kDB) vraw[d + 2] = vread(d + 2);
        const bf16x8 vf = fp8x8_to_bf16(vraw[d]);
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) oacc[rb][d] = mfma16(vf, pf[rb], oacc[rb][d]);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // Unrolled by NBUF so that each register buffer has a fixed name and the
    // wait for a tile leaves the later tiles' loads in flight.  The refills
    // are unconditional (clamped to the last tile, so the final round
    // re-reads it): conditional ones make the compiler merge the buffers
    // through copies that wait for every load.
    int t = 0;
    for (; t + NBUF - 1 <= last; t += NBUF) {
#pragma unroll
      for (int j = 0; j < NBUF; ++j) step(t + j, kbuf[j], vbuf[j], true);
    }
#pragma unroll
    for (int j = 0; j < NBUF - 1; ++j)
      if (t + j <= last) step(t + j, kbuf[j], vbuf[j], false);

    // ---- partial result: lane l holds O^T[16 d + 4 (l/16) + i][row l%16] ----
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const float l_tot = sum_quad16(l_run[rb]);
      const int r = rb * 16 + (lane & 15);
      if (rvalid[rb]) {
        const float inv = l_tot > 0.0f ? vdesc / l_tot : 0.0f;
        float* po = a.part_o + (slot * a.slot_rows + r) * DV + kgrp * 4;
#pragma unroll
        for (int d = 0; d < kDB; ++d) {
          f32x4 w4;
          w4[0] = oacc[rb][d][0] * inv;
          w4[1] = oacc[rb][d][1] * inv;
          w4[2] = oacc[rb][d][2] * inv;
          w4[3] = oacc[rb][d][3] * inv;
          *reinterpret_cast<f32x4*>(po + d * 16) = w4;
        }
        if (lane < 16)
          a.part_lse[slot * a.slot_rows + r] = l_tot > 0.0f ? (m_run[rb] + log2_hw(l_tot)) * kLn2 : -INFINITY;
      }
    }
  };

  // first sequence of the share: the largest b with Hkv*tiles[b] <= s0
  int lo = 0, hi = a.B;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if ((int64_t)a.Hkv * load_uniform_i32(a.tiles, mid) <= s0) lo = mid;
    else hi = mid;
  }
  int b = lo;
  int64_t pos = s0;
  for (;;) {
    const int tb = load_uniform_i32(a.tiles, b);
    const int nt = load_uniform_i32(a.tiles, b + 1) - tb;
    const int64_t base = (int64_t)a.Hkv * tb;
    const int g = (int)((pos - base) / nt);
    const int t0 = (int)(pos - base - (int64_t)g * nt);
    const int t1 = (int)min((int64_t)nt, t0 + (s1 - pos));
    segment(b, g, t0, t1, (int64_t)w + (int64_t)b * a.Hkv + g);
    pos += t1 - t0;
    if (pos >= s1) break;
    if (pos >= base + (int64_t)a.Hkv * nt) {
      // next sequence with tiles
      do {
        ++b;
      } while (load_uniform_i32(a.tiles, b + 1) == load_uniform_i32(a.tiles, b));
    }
  }
}

// Merge the partials of a unit's rows: one wavefront per (sequence, kv-head,
// row), lanes over the head dimension.  The workers that touched unit u are
// those with a non-empty share from the owner of its first tile through the
// owner of its last; their partials sit in slots w + u.  A unit with no tile
// (no keys) gives O = 0 and LSE = -inf.
template <int DV>
__global__ __launch_bounds__(256) void fa_combine_kernel(const CombineArgs a) {
  constexpr int kPer = DV / 64;
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= (int64_t)a.B * a.Hkv * a.slot_rows) return;
  const int r = (int)(item % a.slot_rows);
  const int u = (int)(item / a.slot_rows);
  const int g = u % a.Hkv, b = u / a.Hkv;
  const int qs = a.cu_q[b];
  if (r >= (a.cu_q[b + 1] - qs) * a.group) return;
  const int64_t tok = qs + r / a.group;
  const int h = g * a.group + r % a.group;
  const int tb = a.tiles[b], nt = a.tiles[b + 1] - tb;
  float acc[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) acc[e] = 0.0f;
  float lse = -INFINITY, inv = 0.0f;
  if (nt > 0) {
    const int64_t ntot = (int64_t)a.Hkv * a.tiles[a.B];
    const int64_t first = (int64_t)a.Hkv * tb + (int64_t)g * nt;
    const int w0 = worker_of(first, ntot, a.n_workers), w1 = worker_of(first + nt - 1, ntot, a.n_workers);
    // workers with an empty share (more workers than tiles) wrote nothing
    auto busy = [&](int w) { return (int64_t)w * ntot / a.n_workers < (int64_t)(w + 1) * ntot / a.n_workers; };
    float m = -INFINITY;
    for (int w = w0; w <= w1; ++w)
      if (busy(w)) m = fmaxf(m, a.part_lse[((int64_t)w + u) * a.slot_rows + r]);
    if (m > -INFINITY) {
      float sum = 0.0f;
      for (int w = w0; w <= w1; ++w) {
        const int64_t slot = (int64_t)w + u;
        const float ls = busy(w) ? a.part_lse[slot * a.slot_rows + r] : -INFINITY;
        if (ls > -INFINITY) {
          const float wt = exp2_hw((ls - m) * kLog2e);
          sum += wt;
          const float* po = a.part_o + (slot * a.slot_rows + r) * DV + lane * kPer;
#pragma unroll
          for (int e = 0; e < kPer; ++e) acc[e] += wt * po[e];
        }
      }
      inv = 1.0f / sum;
      lse = m + log2_hw(sum) * kLn2;
    }
  }
  bf16* op = a.o + tok * a.o_st + (int64_t)h * a.o_sh + lane * kPer;
#pragma unroll
  for (int e = 0; e < kPer; ++e) op[e] = (bf16)(acc[e] * inv);
  if (lane == 0) a.lse[(int64_t)h * a.total_q + tok] = lse;
}

hipError_t decode_dispatch(const DecodePlanArgs& plan, const DecodeArgs& a, int dqk, int dv, bool fp8, bool vec,
                           bool q8, hipStream_t stream, bool* supported) {
  *supported = fp8 && ((dv == 128 && (dqk == 192 || dqk == 128)) || (dv == 192 && dqk == 192));
  if (!*supported) return hipSuccess;
  hipLaunchKernelGGL(fa_decode_plan_kernel, dim3(1), dim3(256), 0, stream, plan);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid((a.n_workers + kDecWaves - 1) / kDecWaves);
  const bool two = a.slot_rows > 16;
  // score mods and block masks: one variant, with two row blocks (any unit)
  const bool mods = a.alibi_slope != 0.0f || a.softcap > 0.0f || a.bmask;
#define FA_DEC(DQ, DVV, VC, Q)                                                                           \
  if (dqk == DQ && dv == DVV && vec == VC && q8 == Q) {                                                    \
    if (mods)                                                                                              \
      hipLaunchKernelGGL((fa_decode_kernel<DQ, DVV, 2, (DVV > 128 ? 2 : 1), VC, Q, true>), grid,           \
                         dim3(kDecWaves * 64), 0, stream, a);                                              \
    else if (two)                                                                                          \
      hipLaunchKernelGGL((fa_decode_kernel<DQ, DVV, 2, (DVV > 128 ? 2 : 1), VC, Q, false>), grid,          \
                         dim3(kDecWaves * 64), 0, stream, a);                                              \
    else                                                                                                   \
      hipLaunchKernelGGL((fa_decode_kernel<DQ, DVV, 1, 2, VC, Q, false>), grid, dim3(kDecWaves * 64), 0,   \
                         stream, a);                                                                       \
    return hipGetLastError();                                                                              \
  }
#define FA_DEC2(DQ, DVV, VC) FA_DEC(DQ, DVV, VC, false) FA_DEC(DQ, DVV, VC, true)
  FA_DEC2(192, 128, false)
  FA_DEC2(128, 128, false)
  FA_DEC2(192, 128, true)
  FA_DEC2(128, 128, true)
  FA_DEC2(192, 192, false)
  FA_DEC2(192, 192, true)
#undef FA_DEC2
#undef FA_DEC
  *supported = false;
  return hipSuccess;
}

hipError_t combine_dispatch(const CombineArgs& a, int dv, hipStream_t stream, bool* supported) {
  *supported = true;
  const int64_t items = (int64_t)a.B * a.Hkv * a.slot_rows;
  const dim3 grid((unsigned)((items + 3) / 4));
  if (dv == 128) {
    hipLaunchKernelGGL((fa_combine_kernel<128>), grid, dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  if (dv == 192) {
    hipLaunchKernelGGL((fa_combine_kernel<192>), grid, dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  *supported = false;
  return hipSuccess;
}

}  // namespace fa
