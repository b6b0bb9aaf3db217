// Pieces shared by the prefill kernels: the sequence view of a workgroup,
// the LDS row swizzle and the K/V row addressing.
#pragma once
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

constexpr int NWAVES = 4;
constexpr int BM = 32 * NWAVES;
constexpr int BN = 64;
constexpr int NTHREADS = 64 * NWAVES;
constexpr int kMaskRows = 128;          // block-mask query tiles are multiples of this
constexpr int kHalves = BM / kMaskRows; // mask rows one workgroup can span
constexpr float kLazyTau = 8.0f;

struct SeqView {
  int b, h, g;
  int sq, skv;            // lengths of this sequence
  int64_t qstart, kstart; // first token row (packed Q/O; contiguous K/V)
};

// Lengths and token offsets of the (sequence, q-head) that workgroup row bh
// works on: dense batches (b*Sq, b*Skv), packed sequences (cu_seqlens) or a
// paged cache (seqlen_k, bounded by the pages the block table can name).
__device__ __forceinline__ void seq_view(const PrefillArgs& a, int bh, bool paged, SeqView& sv) {
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
  if (paged) {
    sv.kstart = 0;
    sv.skv = (int)min((int64_t)a.seqlen_k[sv.b], (int64_t)a.max_pages << a.page_shift);
  } else if (a.cu_k) {
    const int s0 = a.cu_k[sv.b], s1 = a.cu_k[sv.b + 1];
    sv.kstart = s0;
    sv.skv = s1 - s0;
  } else {
    sv.kstart = (int64_t)sv.b * a.Skv;
    sv.skv = a.Skv;
  }
}

// LDS row swizzle: 16-byte chunk c of tile row r is stored at c ^ swz(r).
// The LDS behaves as 64 four-byte banks (256 bytes per conflict-free cycle).
// K reads (ds_read_b128) touch rows r..r+15 at one chunk per 16 lanes; the
// transposed V reads (ds_read_b64_tr_b16) touch 4 rows x 4 adjacent chunks
// per 32 lanes.  256-byte rows: a 4-bit map that is a bijection on r mod 16
// and sends the 4 rows of a V group to distinct quarters of the bank space.
// 128- and 384-byte rows alternate bank halves by themselves: a 3-bit map on
// r >> 1 that also keeps rows 2 apart in different 4-chunk groups.  The XOR
// stays inside aligned groups of 16 (8) chunks, i.e. inside the row.
template <int kRow>
__device__ __forceinline__ int swz(int r) {
  if (kRow == 256) return ((r & 3) << 2) | ((r >> 2) & 3);
  return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// FP8 K tile rows of D bytes (kept as E4M3 bytes): chunk c of row r at
// c ^ swz8<D>(r).  192-byte rows start 48 banks apart, so rows four apart
// share banks: the map (inside the aligned group of four chunks) sends them
// elsewhere; 128-byte rows alternate bank halves and the map runs over the
// whole row.  Either way the 16 rows that 16 lanes read at one chunk fall in
// 16 different 16-byte bank slots.
template <int D>
__device__ __forceinline__ int swz8(int r) {
  if (D == 128) return (r >> 1) & 7;
  return (r >> 2) & 3;
}

// FP8 V tile rows of D bytes (key-major E4M3): chunk c of row r at
// c ^ swzv8<D>(r).  A transposing byte read of half a wavefront takes the
// keys {0-3, 8-11} of a 16-key step (the other half: +4) at two adjacent
// chunks.  128-byte rows alternate bank halves: the map gives the four rows
// of each parity four different even chunk offsets, so the 16 pieces fill
// all 64 banks.  192-byte rows repeat their bank offset every four rows:
// the map moves rows 8..11 (and 12..15) to the other chunk pair of their
// aligned group of four.
template <int D>
__device__ __forceinline__ int swzv8(int r) {
  if (D == 128) return (((r >> 1) & 1) << 1) | (((r >> 3) & 1) << 2);
  return ((r >> 3) & 1) << 1;
}

// Element offset of key row j in the slow path (tail tiles, pages smaller
// than a tile): clamped row, per-row page lookup.
__device__ __forceinline__ int64_t key_row_offset(const PrefillArgs& a, const SeqView& sv, int j,
                                                  int64_t st, int64_t sh, int64_t pg, bool paged) {
  j = j < sv.skv ? j : sv.skv - 1;                  // tail rows are masked anyway
  if (paged) {
    int page = a.block_table[(int64_t)sv.b * a.max_pages + (j >> a.page_shift)];
    page = min(max(page, 0), a.num_pages - 1);      // never read outside the cache
    const int slot = j & ((1 << a.page_shift) - 1);
    return (int64_t)page * pg + (int64_t)sv.g * sh + (int64_t)slot * st;
  }
  return (sv.kstart + j) * st + (int64_t)sv.g * sh;
}

// Element offset of row 0 of tile k0 in the fast path (whole tile inside the
// sequence and, for paged caches, inside one page: one scalar page lookup).
__device__ __forceinline__ int64_t tile_base(const PrefillArgs& a, const SeqView& sv, int k0,
                                             int64_t st, int64_t sh, int64_t pg, bool paged) {
  if (paged) {
    int page = load_uniform_i32(a.block_table, (int64_t)sv.b * a.max_pages + (k0 >> a.page_shift));
    page = min(max(page, 0), a.num_pages - 1);
    return (int64_t)page * pg + (int64_t)sv.g * sh + (int64_t)(k0 & ((1 << a.page_shift) - 1)) * st;
  }
  return (sv.kstart + k0) * st + (int64_t)sv.g * sh;
}

// Workgroup -> (sequence*head, query tile).  The grid is (B*Hq rounded up
// to a multiple of 8) x (query tiles); workgroups are dispatched in linear
// order i and dealt round-robin to the 8 XCDs, so XCD x = i mod 8 takes the
// heads bh = 8 s + x (head slots s) whatever the order below.
//  - causal (query tiles of unequal cost): an XCD takes its head slots in
//    groups of 8 and, within a group, query-tile levels longest first, so
//    the costliest tiles start first (the tail is short) while only a group's
//    heads stream their K/V through the XCD's L2: the 8 longest tiles of a
//    head start together and read its K/V in step.  On the varlen causal
//    batch this fetches 39 % fewer bytes than levels over all heads (+1.2 %);
//    the balance cost is under 1 % on most batch shapes.  Workgroups are
//    dealt to SEs and CUs round-robin in dispatch order whatever their cost,
//    so the head of each slot rotates per level.
//  - otherwise (equal cost): head major, all query tiles of one head in a
//    row, so the workgroups that read the same K/V share one XCD's L2.
// G is the group size: 8 for the forward kernels; the backward's smaller
// units balance in groups of 4.
template <int G = 8>
__device__ __forceinline__ void wg_tile(bool causal, int& bh, int& qt) {
  const int gx = (int)gridDim.x, gy = (int)gridDim.y;
  if (causal) {
    // k-th workgroup of XCD x: group g of (up to) G head slots, level y
    // within it, and the slot rotated by one per level (without the rotation
    // a CU would meet the same (sequence, head) at every level it serves and
    // inherit that sequence's length as its load)
    const int i = (int)blockIdx.y * gx + (int)blockIdx.x;
    const int x = i & 7, k = i >> 3;
    const int g = k / (G * gy);
    const int gs = min(G, (gx >> 3) - g * G);
    const int rem = k - g * G * gy;
    const int y = rem / gs;
    bh = (g * G + (rem % gs + y) % gs) * 8 + x;
    qt = gy - 1 - y;
    return;
  }
  const int i = (int)blockIdx.y * gx + (int)blockIdx.x;
  const int p = i >> 3;
  bh = (p / gy) * 8 + (i & 7);
  qt = gy - 1 - p % gy;
}

// bf16 tile of D columns: global -> LDS with one 1 KB global_load_lds per
// wave instruction.  Instruction n covers LDS bytes [n*1024, n*1024+1024);
// lane l fills 16 bytes at n*1024 + 16*l, i.e. tile row r, stored chunk pos,
// which holds source chunk pos ^ swz(r).
template <int D, bool PAGED>
struct Bf16Stager {
  static constexpr int kRow = D * 2;
  static constexpr int kPerWave = BN * kRow / 1024 / NWAVES;
  static_assert(kPerWave >= 1, "a bf16 tile must give every wavefront a 1 KB piece");
  unsigned off[kPerWave];   // byte offset of this lane's 16 bytes from tile row 0
  __device__ __forceinline__ static void place(int i, int wave, int lane, int& row, int& chunk) {
    const int byte = (wave * kPerWave + i) * 1024 + lane * 16;
    row = byte / kRow;
    chunk = ((byte % kRow) >> 4) ^ swz<kRow>(row);
  }
  __device__ __forceinline__ void init(int64_t st, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      int row, chunk;
      place(i, wave, lane, row, chunk);
      off[i] = (unsigned)(row * (int)st + chunk * 8) * 2u;
    }
  }
  // Whole tiles and the sequence tail of contiguous K/V: buffer loads into
  // LDS from a descriptor based at the tile's first row (32-bit per-lane
  // offsets; the tail re-reads the last row).  Paged tails and pages smaller
  // than a tile: per-row page lookups and 64-bit addresses.
  __device__ __forceinline__ void issue(const PrefillArgs& a, const SeqView& sv, const bf16* base, int64_t st,
                                        int64_t sh, int64_t pg, char FA_LDS* tile, int k0, bool fast, int wave,
                                        int lane) {
    if (fast || !PAGED) {
      const bf16* tb = base + tile_base(a, sv, k0, st, sh, pg, PAGED);
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(tb);
      if (fast) {
#pragma unroll
        for (int i = 0; i < kPerWave; ++i) buffer_to_lds16(rs, off[i], tile + (wave * kPerWave + i) * 1024);
      } else {
        // the lane index goes through an opaque copy so that the per-row
        // offsets are computed here, not kept live across the tile loop
        int l = lane;
        asm volatile("" : "+v"(l));
        const int last = sv.skv - 1 - k0;
#pragma unroll
        for (int i = 0; i < kPerWave; ++i) {
          int row, chunk;
          place(i, wave, l, row, chunk);
          const unsigned o = (unsigned)(min(row, last) * (int)st + chunk * 8) * 2u;
          buffer_to_lds16(rs, o, tile + (wave * kPerWave + i) * 1024);
        }
      }
    } else {
      int l = lane;
      asm volatile("" : "+v"(l));
#pragma unroll
      for (int i = 0; i < kPerWave; ++i) {
        int row, chunk;
        place(i, wave, l, row, chunk);
        global_to_lds16(base + key_row_offset(a, sv, k0 + row, st, sh, pg, PAGED) + chunk * 8,
                        tile + (wave * kPerWave + i) * 1024);
      }
    }
  }
};

// Active-tile bits of the block-mask rows that a workgroup spans (one per
// 128-query half), 64 mask key-blocks at a time: one vector load and a ballot
// per row and 64 blocks; the per-tile tests are scalar.  tile_bits(t) has bit
// h set when half h has tile t active.
struct MaskBits {
  const uint8_t* row[kHalves];
  int nkb, bk;
  int chunk;
  uint64_t bits[kHalves];
  __device__ __forceinline__ void init(const PrefillArgs& a, const SeqView& sv, int q0) {
    nkb = a.bm_nkb;
    bk = a.bm_bk;
    chunk = -1;
#pragma unroll
    for (int h = 0; h < kHalves; ++h) {
      const int qh = min(q0 + h * kMaskRows, sv.sq - 1);   // halves past the end reuse the last row
      row[h] = a.bmask ? a.bmask + (((int64_t)sv.b * a.Hq + sv.h) * a.bm_nqb + qh / a.bm_bq) * a.bm_nkb : nullptr;
      bits[h] = ~0ull;
    }
  }
  __device__ __forceinline__ unsigned tile_bits(int t) {
    if (!row[0]) return (1u << kHalves) - 1;
    const int kb = (t * BN) / bk;
    const int c = kb >> 6;
    if (c != chunk) {
      const int idx = c * 64 + __lane_id();
#pragma unroll
      for (int h = 0; h < kHalves; ++h) bits[h] = __builtin_amdgcn_ballot_w64(idx < nkb && row[h][idx] != 0);
      chunk = c;
    }
    unsigned r = 0;
#pragma unroll
    for (int h = 0; h < kHalves; ++h) r |= (unsigned)((bits[h] >> (kb & 63)) & 1ull) << h;
    return r;
  }
};

// Output rows of one wavefront: the 32 x D tile held as O^T accumulators
// (lane l: row l % 32, columns 32 d + 8 g + 4 (l / 32) + [0, 4)) is scaled,
// rounded to bf16 and written row-major into this wavefront's 32 x 2D bytes
// of free LDS at ot, then read back 16 bytes per lane so that every global
// store writes whole rows (non-temporal: O is not read again here, and the
// stores retire sooner).  Chunk c of row r sits at c ^ osw(r) (inside its
// aligned group of eight or sixteen chunks); rows 16-31 also swap the two
// 8-byte halves of each chunk, so that the 32 rows that half a wavefront
// writes at one chunk fill all 64 banks.  Rows >= nrows are not stored.
template <int D>
__device__ __forceinline__ void store_o_rows(const f32x16 (&oacc)[D / 32], float scale, char FA_LDS* ot,
                                             bf16* o_row0, int64_t o_st, int nrows, int lane) {
  constexpr int kRow = D * 2;
  constexpr int kChunks = D / 8;               // 16-byte chunks per row
  static_assert(kChunks == 8 || kChunks == 16 || kChunks == 24, "row widths of 64, 128 or 192 elements");
  auto osw = [](int r) { return kChunks == 16 ? (r & 15) : ((r >> 1) & 7); };
  {
    const int r = lane & 31;
    char FA_LDS* rowp = ot + r * kRow + (((lane >> 5) ^ (r >> 4)) << 3);
#pragma unroll
    for (int d = 0; d < D / 32; ++d)
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        bf16x4 w;
        w[0] = (bf16)(oacc[d][gi * 4 + 0] * scale);
        w[1] = (bf16)(oacc[d][gi * 4 + 1] * scale);
        w[2] = (bf16)(oacc[d][gi * 4 + 2] * scale);
        w[3] = (bf16)(oacc[d][gi * 4 + 3] * scale);
        *reinterpret_cast<bf16x4 FA_LDS*>(rowp + (((d * 4 + gi) ^ osw(r)) << 4)) = w;
      }
  }
#pragma unroll
  for (int i = 0; i < 32 * kChunks / 64; ++i) {
    const int f = i * 64 + lane;
    const int r = f / kChunks, c = f % kChunks;
    bf16x8 v = *reinterpret_cast<const bf16x8 FA_LDS*>(ot + r * kRow + ((c ^ osw(r)) << 4));
    const bf16x8 sw = __builtin_shufflevector(v, v, 4, 5, 6, 7, 0, 1, 2, 3);
    if constexpr (64 % kChunks == 0) {
      if (i * (64 / kChunks) >= 16) v = sw;    // the rows of one read are all on one side
    } else {
      if (r >= 16) v = sw;
    }
    if (r < nrows) __builtin_nontemporal_store(v, reinterpret_cast<bf16x8*>(o_row0 + r * o_st + c * 8));
  }
}

}  // namespace fa
