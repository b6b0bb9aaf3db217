/*
 * fa.h - C ABI of the MI355X (gfx950) FlashAttention forward library, libfa.so.
 *
 * The library computes, in one fused pass per (sequence, q-head) and query
 * tile, the attention output O = softmax(scale * Q K^T [+ score mods, masks]) V
 * together with the per-row log-sum-exp LSE = m + ln(l) of the scaled logits
 * (running max m, denominator l).  Sources: "Add forward LSE output to FlyDSL
 * flash attention kernels" (FlyDSL PR 844, Summary and Changes: LSE is the
 * per-row normalisation statistic, fully masked rows get -inf, split-K
 * partials merge from (m, l)); "SM90 TMA + mma.sync FlashAttention ..."
 * (RL-Kernel PR 237, description: packed varlen [total_tokens, H, D] with
 * cu_seqlens, attention-domain LSE, zero-length sequences valid); "Support
 * paged FP8 Flash attention with asymmetric K/V head dim on gfx950" (FlyDSL
 * PR 1066, overview and review: paged OCP E4M3 K/V with single-value
 * descales, Q/K width 192 with V/O width 128, int32 block_table and seqlen_k,
 * native-width bf16 output, 64-bit cache offsets past 4 GiB, int32 overflow
 * guards, no host work inside graph capture); "flash_attention: prologue
 * fusion, mma tensor cores, fp8 KV cache, flex attention + block sparsity"
 * (fkl_python PR 7, part 4: ALiBi, SoftCap, SlidingWindow score mods whose
 * values are runtime parameters, and a (bh, nQB, nKB) uint8 tile mask whose
 * inactive tiles are skipped).
 *
 * Conventions for every entry point
 *  - All tensor pointers are DEVICE pointers owned by the caller; the library
 *    never allocates, frees or keeps them.  Tensors are contiguous in the
 *    layouts stated per function; bf16 means IEEE bfloat16, FP8 means OCP
 *    E4M3 (e4m3fn, max 448, 0x7F/0xFF NaN).
 *  - Tensor and workspace pointers must be 16-byte aligned (the kernels
 *    move 16 bytes at a time), fp32 and int32 arrays 4-byte aligned and the
 *    int64 slot mapping 8-byte aligned; otherwise FA_ERR_INVALID.
 *  - Sizes are int64_t host values.  Token counts, page counts and every
 *    flattened tensor extent must stay below 2^31 elements (FA_ERR_LIMIT);
 *    byte offsets inside the kernels are 64-bit.
 *  - `stream` is a hipStream_t (NULL: the default stream).  Work is only
 *    enqueued on it; nothing synchronises with the host and no host-device
 *    copy happens, so calls can be captured in a HIP graph.
 *  - Return 0 (FA_OK) on success.  Every argument check runs on the host
 *    before any HIP call; on failure nothing is enqueued and fa_last_error()
 *    returns a message (thread-local).  Device-resident metadata
 *    (cu_seqlens, seqlen_k, block_table, block_mask) cannot be checked
 *    without a synchronisation; it must be consistent with the host sizes.
 *  - Rows that see no key (causal with fewer keys than queries, windows,
 *    inactive block-mask tiles, empty key sequences) produce O = 0 and
 *    LSE = -inf.  Zero-length query sequences write nothing.
 *  - Query row i of a sequence with Sq queries and Skv keys is aligned to key
 *    position i' = i + Skv - Sq (bottom-right); causal means key j <= i'.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_OK 0
#define FA_ERR_INVALID (-1)     /* null / aliasing / misaligned pointers, inconsistent sizes */
#define FA_ERR_UNSUPPORTED (-2) /* head-dim pair, dtype, page size or mod combination not built */
#define FA_ERR_LIMIT (-3)       /* a count or flattened extent >= 2^31 */
#define FA_ERR_WORKSPACE (-4)   /* workspace missing or too small */
#define FA_ERR_HIP (-5)         /* the HIP runtime rejected a launch */

typedef enum fa_dtype { FA_BF16 = 0, FA_FP8_E4M3 = 1 } fa_dtype;

/* fa_mods.flags */
#define FA_CAUSAL 1u     /* key j visible to row i only if j <= i' */
#define FA_WINDOW 2u     /* i' - window_left <= j <= i' + window_right (negative: unbounded side) */
#define FA_ALIBI 4u      /* logit -= alibi_slope * |i' - j| (same slope for every head) */
#define FA_SOFTCAP 8u    /* logit = softcap * tanh(logit / softcap), applied before ALiBi */
#define FA_BLOCK_MASK 16u /* tile mask: key j visible to row i only if
                             block_mask[(b*Hq + h)][i / mask_block_q][j / mask_block_k] != 0 */

/* Score modifications and masks.  A NULL fa_mods* means: no flags, default scale. */
typedef struct fa_mods {
  uint32_t flags;
  float softmax_scale;      /* <= 0: 1/sqrt(d_qk) */
  float alibi_slope;        /* FA_ALIBI */
  float softcap;            /* FA_SOFTCAP, > 0 */
  int64_t window_left;      /* FA_WINDOW */
  int64_t window_right;
  const uint8_t* block_mask; /* FA_BLOCK_MASK: device uint8 [B*Hq, mask_nqb, mask_nkb] */
  int64_t mask_block_q;     /* must be a multiple of 128 */
  int64_t mask_block_k;     /* must be a multiple of 64 */
  int64_t mask_nqb;         /* >= ceil(max_seqlen_q / mask_block_q) */
  int64_t mask_nkb;         /* >= ceil(max_seqlen_k / mask_block_k) */
} fa_mods;

/*
 * Dense batch.  Q [B, Sq, Hq, d_qk], K [B, Skv, Hkv, d_qk], V [B, Skv, Hkv, d_v]
 * and O [B, Sq, Hq, d_v] are bf16; LSE [B, Hq, Sq] is fp32.  Hq % Hkv == 0;
 * q-head h reads kv-head h / (Hq / Hkv).  Built head dims: (64, 64), (128, 128).
 * All mods are supported.  O and LSE must not overlap each other or the inputs.
 */
int fa_fwd_dense(const void* q, const void* k, const void* v, void* o, float* lse,
                 int64_t B, int64_t Sq, int64_t Skv, int64_t Hq, int64_t Hkv,
                 int64_t d_qk, int64_t d_v, const fa_mods* mods, void* stream);

/*
 * Packed variable-length batch.  Sequence b owns query rows
 * [cu_seqlens_q[b], cu_seqlens_q[b+1]) and key rows [cu_seqlens_k[b],
 * cu_seqlens_k[b+1]) (device int32 [B+1], non-decreasing, starting at 0).
 * Q [total_q, Hq, d_qk], K [total_k, Hkv, d_qk], V [total_k, Hkv, d_v],
 * O [total_q, Hq, d_v] bf16; LSE [Hq, total_q] fp32.  max_seqlen_q/k bound
 * every sequence's lengths (host scalars, so no device read-back is needed).
 * Built head dims and mods as for fa_fwd_dense.
 */
int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                  const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int64_t B,
                  int64_t total_q, int64_t total_k, int64_t max_seqlen_q, int64_t max_seqlen_k,
                  int64_t Hq, int64_t Hkv, int64_t d_qk, int64_t d_v,
                  const fa_mods* mods, void* stream);

/*
 * Paged KV cache.  Q [total_q, Hq, d_qk] bf16 packed by cu_seqlens_q (device
 * int32 [B+1]); O [total_q, Hq, d_v] bf16; LSE [Hq, total_q] fp32.
 * Caches are head-major pages: K [num_pages, Hkv, page_size, d_qk] and
 * V [num_pages, Hkv, page_size, d_v], elements FP8 E4M3 (kv_dtype =
 * FA_FP8_E4M3, real value = code * descale with k_descale / v_descale device
 * fp32 scalars) or bf16 (FA_BF16, descales ignored, may be NULL).
 * Key j of sequence b is slot j % page_size of page
 * block_table[b * max_pages_per_seq + j / page_size] (device int32
 * [B, max_pages_per_seq]); seqlen_k (device int32 [B]) is its key count.
 * Only the first ceil(seqlen_k[b] / page_size) entries of a block-table row
 * are read, and bytes past seqlen_k in a page never influence the result.
 * page_size: a power of two in [1, 1024].
 * Built: FP8 (d_qk, d_v) in {(192, 128), (128, 128), (192, 192)} (192/192:
 * the V192 variant of the paged FP8 PR); bf16 (64, 64), (128, 128).
 * Mods: every mod, as for fa_fwd_dense, with either cache type and on the
 * decode path too (the flex page, part 4, applies its score mods and block
 * sparsity to the forward in general).  A block mask's query blocks index
 * the query's row i within its sequence, its key blocks the key index j.
 * bf16 queries against an FP8 cache enter the FP8 products as two E4M3
 * parts of 2^e q, e chosen per query row from its largest magnitude
 * (2^e amax in [128, 256)): any finite bf16 query row is representable, each
 * element to about 2^-8 of itself or 2^-17 of the row's maximum.
 * When max_seqlen_q * (Hq / Hkv) <= 32 (decode) and kv_dtype is FP8, the
 * keys are split and partial results merged; that path needs a device
 * workspace of fa_fwd_paged_workspace_size(...) bytes (else
 * FA_ERR_WORKSPACE).  The workspace is scratch, overwritten by the call; it
 * may overlap no argument array (q, caches, o, lse, cu_seqlens_q, seqlen_k,
 * block_table, descales: FA_ERR_INVALID).
 */
int fa_fwd_paged(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                 const int32_t* cu_seqlens_q, const int32_t* seqlen_k, const int32_t* block_table,
                 int64_t B, int64_t total_q, int64_t max_seqlen_q, int64_t max_seqlen_k,
                 int64_t num_pages, int64_t page_size, int64_t max_pages_per_seq,
                 int64_t Hq, int64_t Hkv, int64_t d_qk, int64_t d_v, fa_dtype kv_dtype,
                 const float* k_descale, const float* v_descale,
                 void* workspace, size_t workspace_bytes,
                 const fa_mods* mods, void* stream);

/*
 * fa_fwd_paged without a workspace argument, for callers that cannot
 * allocate device memory per call: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  Arguments, results and
 * errors are fa_fwd_paged's (bitwise the same outputs).  The decode path's
 * scratch (tile prefix and split-KV partials) lives in a static device
 * array of 64 MiB that every GPU running the library holds until the
 * process ends; a call whose decode path would need more returns
 * FA_ERR_LIMIT (fa_fwd_paged_workspace_size gives the need).  Nothing is
 * allocated and no part of the array needs clearing (each call writes what
 * it reads).  Every call on one GPU shares that GPU's array: calls that
 * overlap in time on one GPU (other streams, other threads) race.
 */
int fa_fwd_paged_noalloc(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                         const int32_t* cu_seqlens_q, const int32_t* seqlen_k, const int32_t* block_table,
                         int64_t B, int64_t total_q, int64_t max_seqlen_q, int64_t max_seqlen_k,
                         int64_t num_pages, int64_t page_size, int64_t max_pages_per_seq,
                         int64_t Hq, int64_t Hkv, int64_t d_qk, int64_t d_v, fa_dtype kv_dtype,
                         const float* k_descale, const float* v_descale,
                         const fa_mods* mods, void* stream);

/*
 * Paged KV cache in the vectorised 5-D page format (review of "Support paged
 * FP8 Flash attention with asymmetric K/V head dim on gfx950", which gives
 * the two cache shapes and the permutes that take them back to token-major):
 *   K [num_pages, Hkv, d_qk / 16, page_size, 16]  byte (page, g, c, s, x) is
 *     element d = 16 c + x of key slot s;
 *   V [num_pages, Hkv, page_size / 16, d_v, 16]   byte (page, g, j, d, x) is
 *     element d of key slot 16 j + x.
 * Elements are FP8 E4M3 only (kv_dtype must be FA_FP8_E4M3; FA_BF16 gives
 * FA_ERR_UNSUPPORTED), page_size a power of two in [16, 1024].  Every other
 * argument, the built head dims, the mods, the workspace (same size rule:
 * fa_fwd_paged_workspace_size) and the error behaviour are those of
 * fa_fwd_paged, and for the same logical cache the result is bitwise the one
 * fa_fwd_paged gives with head-major pages.
 */
int fa_fwd_paged_vec(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                     const int32_t* cu_seqlens_q, const int32_t* seqlen_k, const int32_t* block_table,
                     int64_t B, int64_t total_q, int64_t max_seqlen_q, int64_t max_seqlen_k,
                     int64_t num_pages, int64_t page_size, int64_t max_pages_per_seq,
                     int64_t Hq, int64_t Hkv, int64_t d_qk, int64_t d_v, fa_dtype kv_dtype,
                     const float* k_descale, const float* v_descale,
                     void* workspace, size_t workspace_bytes,
                     const fa_mods* mods, void* stream);

/* fa_paged_opts.page_layout */
#define FA_PAGES_HEAD_MAJOR 0  /* fa_fwd_paged's pages */
#define FA_PAGES_VECTORIZED 1  /* fa_fwd_paged_vec's pages */

/* Query type and page format of fa_fwd_paged_ex.  A NULL fa_paged_opts*
 * means bf16 queries and head-major pages (fa_fwd_paged). */
typedef struct fa_paged_opts {
  fa_dtype q_dtype;         /* FA_BF16, or FA_FP8_E4M3 (FP8 caches only) */
  const float* q_descale;   /* FA_FP8_E4M3 queries: device fp32 scalar, real q = code * q_descale */
  int32_t page_layout;      /* FA_PAGES_HEAD_MAJOR or FA_PAGES_VECTORIZED */
} fa_paged_opts;

/*
 * fa_fwd_paged with a choice of query type and page format.  E4M3 queries
 * follow the description of "Support paged FP8 Flash attention with
 * asymmetric K/V head dim on gfx950" (OCP E4M3 Q/K/V with scalar descales):
 * Q is [total_q, Hq, d_qk] E4M3 codes (1 byte each) and every logit carries
 * q_descale * k_descale; they need kv_dtype FA_FP8_E4M3 (else
 * FA_ERR_UNSUPPORTED) and a non-NULL q_descale (else FA_ERR_INVALID).  O
 * stays bf16.  Everything else is fa_fwd_paged's (or, for vectorised pages,
 * fa_fwd_paged_vec's), the workspace rule included.
 */
int fa_fwd_paged_ex(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                    const int32_t* cu_seqlens_q, const int32_t* seqlen_k, const int32_t* block_table,
                    int64_t B, int64_t total_q, int64_t max_seqlen_q, int64_t max_seqlen_k,
                    int64_t num_pages, int64_t page_size, int64_t max_pages_per_seq,
                    int64_t Hq, int64_t Hkv, int64_t d_qk, int64_t d_v, fa_dtype kv_dtype,
                    const float* k_descale, const float* v_descale,
                    void* workspace, size_t workspace_bytes,
                    const fa_paged_opts* opts, const fa_mods* mods, void* stream);

/* Workspace bytes the paged entry points need for these sizes (0 when they
 * need none). */
size_t fa_fwd_paged_workspace_size(int64_t B, int64_t total_q, int64_t max_seqlen_q,
                                   int64_t max_seqlen_k, int64_t Hq, int64_t Hkv, int64_t d_qk,
                                   int64_t d_v, int64_t page_size, fa_dtype kv_dtype);

/*
 * Backward pass of the dense / varlen forward: dQ, dK, dV from Q, K, V, the
 * forward's O and LSE and the upstream gradient dO (method: "SM90 TMA +
 * mma.sync FlashAttention, forward + backward (causal, varlen, LSE)",
 * backward commit — a Delta = rowsum(dO * O) preprocess, then dQ/dK/dV
 * recomputing P from the saved LSE).  Layouts are the forward's: dense Q,
 * O, dO, dQ [B, Sq, Hq, d], K, V, dK, dV [B, Skv, Hkv, d], LSE [B, Hq, Sq];
 * varlen rows packed by cu_seqlens_q / cu_seqlens_k, LSE [Hq, total_q].
 * All tensors bf16 except LSE (fp32).  GQA: dK / dV of a kv-head sum over
 * its q-heads.  Built: d_qk = d_v in {64, 128}.  Mods: FA_CAUSAL and
 * FA_WINDOW (and softmax_scale) — the masks the forward used must be passed
 * again.  Rows with no visible key contribute nothing; every element of dQ,
 * dK and dV is written (zeros where no gradient flows).  Needs a device
 * workspace of fa_bwd_workspace_size(...) bytes (Delta, fp32), else
 * FA_ERR_WORKSPACE; outputs must not overlap the inputs or each other.
 * Hq * d must stay below 2^24 (FA_ERR_LIMIT).
 * Deterministic: every output element is summed in a fixed order.
 */
int fa_bwd_dense(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                 void* dq, void* dk, void* dv, int64_t B, int64_t Sq, int64_t Skv, int64_t Hq, int64_t Hkv,
                 int64_t d_qk, int64_t d_v, const fa_mods* mods, void* workspace, size_t workspace_bytes,
                 void* stream);
int fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                  void* dq, void* dk, void* dv, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                  int64_t B, int64_t total_q, int64_t total_k, int64_t max_seqlen_q, int64_t max_seqlen_k,
                  int64_t Hq, int64_t Hkv, int64_t d_qk, int64_t d_v, const fa_mods* mods,
                  void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes of the backward entry points (total_q = B * Sq for dense). */
size_t fa_bwd_workspace_size(int64_t total_q, int64_t Hq);

/* fa_kv_cache_write_fp8 scale_mode */
#define FA_SCALE_GIVEN 0  /* quantise with the descales already in *k_descale / *v_descale */
#define FA_SCALE_AMAX 1   /* first set *k_descale = max(max|k| / 448, 2^-126), same for v */

/*
 * Quantise new K/V rows to OCP E4M3 and write them into paged caches (the
 * step before the FP8 paged entry points).  Method: the GPU quantisation of
 * the fp8 KV-cache page ("flash_attention: prologue fusion, mma tensor
 * cores, fp8 KV cache, flex attention + block sparsity", part 3: scale from
 * the largest magnitude over 448) with the per-tensor descales of the paged
 * FP8 PR.
 * k [T, Hkv, d_qk] and v [T, Hkv, d_v] are bf16, token-major; d_qk and d_v
 * are multiples of 16 (else FA_ERR_UNSUPPORTED).  slot_mapping (device
 * int64 [T]) sends token t to page slot_mapping[t] / page_size, slot
 * slot_mapping[t] % page_size; a negative entry, or one at or past
 * num_pages * page_size, skips the token.  Caches are uint8 in page_layout
 * (FA_PAGES_HEAD_MAJOR: [num_pages, Hkv, page_size, d]; FA_PAGES_VECTORIZED:
 * K [num_pages, Hkv, d_qk/16, page_size, 16], V [num_pages, Hkv,
 * page_size/16, d_v, 16], page_size >= 16); page_size a power of two <= 1024.
 * Each element becomes E4M3(x * (1 / descale)), fp32 steps with a correctly
 * rounded division, nearest with ties to even, saturating at +-448.
 * k_descale / v_descale are device fp32 scalars: read (FA_SCALE_GIVEN; they
 * must be positive and finite) or written first (FA_SCALE_AMAX, which needs
 * a device workspace of fa_kv_cache_write_fp8_workspace_size(...) bytes,
 * else FA_ERR_WORKSPACE).  Inputs must be finite.  Bytes of slots not
 * written keep their values; two tokens mapped to one slot race.  T = 0
 * writes nothing, descales included.
 */
int fa_kv_cache_write_fp8(const void* k, const void* v, const int64_t* slot_mapping,
                          int64_t T, int64_t Hkv, int64_t d_qk, int64_t d_v,
                          void* k_cache, void* v_cache, int64_t num_pages, int64_t page_size,
                          int32_t page_layout, float* k_descale, float* v_descale, int32_t scale_mode,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes fa_kv_cache_write_fp8 needs in FA_SCALE_AMAX mode. */
size_t fa_kv_cache_write_fp8_workspace_size(int64_t T, int64_t Hkv, int64_t d_qk, int64_t d_v);

/* Message describing the last non-zero return on this thread ("" if none). */
const char* fa_last_error(void);

/* ABI version of this header (increments on any signature change). */
int fa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
