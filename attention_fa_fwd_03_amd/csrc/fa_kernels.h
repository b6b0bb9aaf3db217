// Kernel argument blocks and launch entry points shared by the host library
// and the kernel translation units.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

constexpr int kModAlibi = 1;
constexpr int kModSoftcap = 2;

// Strides are in elements.  Contiguous K/V: element (token t, kv-head g, d) at
// t*k_st + g*k_sh + d.  Paged K/V: element (page p, kv-head g, slot s, d) at
// p*k_pg + g*k_sh + s*k_st + d.  Vectorised FP8 pages (kernels built with the
// vec flag): the (p, g) block starts at p*k_pg + g*k_sh as well, and inside
// it K byte (s, d) sits at (d/16)*page*16 + s*16 + d%16 and V byte (s, d) at
// (s/16)*Dv*16 + d*16 + s%16; k_st / v_st are not used.
struct PrefillArgs {
  const void* q;               // bf16, or OCP E4M3 codes when q_descale is set
  const float* q_descale;      // FP8 queries: per-tensor descale (device scalar); else null
  const void* k;
  const void* v;
  __bf16* o;
  float* lse;
  const int32_t* cu_q;         // packed query starts [B+1]; null: dense (b*Sq)
  const int32_t* cu_k;         // packed key starts [B+1]; null: dense or paged
  const int32_t* seqlen_k;     // paged: keys per sequence [B]
  const int32_t* block_table;  // paged: [B, max_pages]
  const float* k_descale;      // FP8 caches: per-tensor descales (device scalars)
  const float* v_descale;
  int64_t q_st, q_sh, k_st, k_sh, v_st, v_sh, o_st, o_sh;
  int64_t k_pg, v_pg;
  int64_t lse_tq;              // packed layouts: LSE is [Hq, lse_tq]
  int Sq, Skv;                 // dense lengths
  int Hq, group;               // group = Hq / Hkv
  int n_bh;                    // B * Hq (the grid's x extent is this rounded up to 8)
  int max_pages;
  int page_shift;
  int num_pages;               // paged: page ids are clamped to [0, num_pages)
  float qk_scale;
  float alibi_slope;
  float softcap;
  int causal;
  int win_left, win_right;     // < 0: unbounded
  const uint8_t* bmask;        // [B*Hq, bm_nqb, bm_nkb] or null
  int bm_bq, bm_bk, bm_nqb, bm_nkb;
};

// Decode over a paged cache, balanced over a fixed number of workers.  The
// key tiles (32 keys) of all (sequence, kv-head) units form one list, unit
// u = b*Hkv + g holding tiles[b+1] - tiles[b] tiles; worker w (one wavefront)
// takes the tiles [w*T/W, (w+1)*T/W) of that list and writes one partial
// result per unit it touches, into slot w + u.  A unit's rows are
// (query i, q-head h in the kv-head's group), rows <= 32.
struct DecodeArgs {
  const void* q;               // bf16, or OCP E4M3 codes (kernels built with the q8 flag)
  const float* q_descale;      // FP8 queries: per-tensor descale (device scalar)
  const void* k;
  const void* v;
  float* part_o;               // [n_slots, slot_rows, Dv] fp32 (normalised by own l)
  float* part_lse;             // [n_slots, slot_rows] fp32 natural-log LSE
  const int32_t* cu_q;
  const int32_t* seqlen_k;
  const int32_t* block_table;
  const float* k_descale;
  const float* v_descale;
  const int32_t* tiles;        // [B+1] exclusive prefix of per-sequence tile counts
  int64_t q_st, q_sh, k_st, k_sh, v_st, v_sh, k_pg, v_pg;
  int B, Hq, Hkv, group;
  int max_pages, page_shift;
  int kv_cap;                  // keys read per sequence at most: min(seqlen_k, kv_cap)
  int num_pages;
  int n_workers;               // W
  int slot_rows;               // max_seqlen_q * group
  float qk_scale;
  int causal;
  int win_left, win_right;
  float alibi_slope;           // 0: none
  float softcap;               // <= 0: none
  const uint8_t* bmask;        // [B*Hq, bm_nqb, bm_nkb] or null (bm_bk is a multiple of 64)
  int bm_bq, bm_bk, bm_nqb, bm_nkb;
};

struct DecodePlanArgs {
  const int32_t* cu_q;
  const int32_t* seqlen_k;
  int32_t* tiles;
  int B;
  int kv_cap;
};

struct CombineArgs {
  const float* part_o;
  const float* part_lse;
  __bf16* o;
  float* lse;
  const int32_t* cu_q;
  const int32_t* tiles;
  int64_t o_st, o_sh;
  int64_t total_q;
  int B, Hq, Hkv, group;
  int n_workers, slot_rows;
};

// Backward pass (fa_backward.hip).  Rows of Q, O, dO, dQ: token t, head h at
// t*q_st + h*q_sh (O and dO with o_st / o_sh); K, V, dK, dV rows with
// k_st / k_sh (v_st / v_sh).  Dense batches are packed rows with sequence b
// starting at b*Sq (b*Skv); LSE and Delta share the forward's LSE layout.
struct BwdArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const __bf16* o;
  const __bf16* dout;
  const float* lse;
  float* delta;
  __bf16* dq;
  __bf16* dk;
  __bf16* dv;
  const int32_t* cu_q;         // null: dense
  const int32_t* cu_k;
  int64_t q_st, q_sh, k_st, k_sh, v_st, v_sh, o_st, o_sh;
  int64_t lse_tq;              // packed layouts: LSE is [Hq, lse_tq]
  int64_t total_rows;          // query rows over all sequences
  int Sq, Skv;                 // dense lengths
  int B, Hq, Hkv, group;
  float qk_scale;
  int causal;
  int win_left, win_right;     // < 0: unbounded
};

hipError_t bwd_dispatch(const BwdArgs& a, int d, int max_sq, int max_skv, hipStream_t stream, bool* supported);

// FP8 KV-cache write (fa_kvcache.hip).
struct KvAmaxArgs {
  const __bf16* k;
  const __bf16* v;
  int64_t n_k, n_v;            // elements of k and v (multiples of 16)
  int nb_k, nb_v;              // reduction blocks per tensor
  float* partial;              // [nb_k + nb_v] per-block maxima
  float* k_descale;            // outputs: max(amax / 448, 2^-126)
  float* v_descale;
};

struct KvWriteArgs {
  const __bf16* k;             // [T, Hkv, d_qk] token-major
  const __bf16* v;             // [T, Hkv, d_v]
  const int64_t* slot_mapping; // [T]: page * page_size + slot, < 0 skips
  void* k_cache;
  void* v_cache;
  const float* k_descale;
  const float* v_descale;
  int64_t T, Hkv;
  int d_qk, d_v;
  int64_t num_pages;
  int page_shift;
  int heads_per_pass;          // kv-heads per workgroup (16 tokens of them fit in LDS)
};

hipError_t kv_amax_dispatch(const KvAmaxArgs& a, hipStream_t stream);
hipError_t kv_write_dispatch(const KvWriteArgs& a, bool vec, hipStream_t stream);

hipError_t prefill_dispatch(const PrefillArgs& a, int dqk, int dv, bool fp8, bool paged, bool vec, int mods,
                            int n_bh, int n_qtiles, hipStream_t stream, bool* supported);
hipError_t prefill_bf16_dispatch(const PrefillArgs& a, int d, bool paged, int mods, int n_bh, int n_qtiles,
                                 hipStream_t stream, bool* supported);
hipError_t decode_dispatch(const DecodePlanArgs& plan, const DecodeArgs& a, int dqk, int dv, bool fp8, bool vec,
                           bool q8, hipStream_t stream, bool* supported);
hipError_t combine_dispatch(const CombineArgs& a, int dv, hipStream_t stream, bool* supported);

}  // namespace fa
