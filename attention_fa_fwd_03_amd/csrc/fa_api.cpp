// Host side of libfa: argument validation, shape specialisation and launch.
//
// Every check here runs before the first HIP call so that a rejected call
// enqueues nothing (and the checks can be exercised without a GPU).  Nothing
// in this file allocates memory, synchronises, or copies between host and
// device: all metadata is consumed on the device, with the host-side maxima
// passed by the caller.  The one static device array (the decode scratch of
// fa_fwd_paged_noalloc) is part of the code object, not an allocation.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <mutex>
#include <string>

#include "fa.h"
#include "fa_kernels.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

constexpr int64_t kI32 = (int64_t)1 << 31;
constexpr int kBM = 128;           // prefill query rows per workgroup
constexpr int kMaskBQ = 128;       // block-mask query tiles: multiples of a workgroup's rows
constexpr int kBN = 64;            // prefill keys per tile
constexpr int kKvLdsBytes = 24576;  // KV-cache writer: LDS for 16 tokens' codes per workgroup
constexpr int kDecodeRows = 32;    // decode rows (query x q-head-in-group) per wavefront

// Decode scratch of fa_fwd_paged_noalloc (see below): at most this many bytes.
constexpr size_t kScratchBytes = (size_t)64 << 20;

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

struct Mods {
  uint32_t flags = 0;
  float scale = 0.f;
  float slope = 0.f;
  float cap = 0.f;
  int64_t wl = -1, wr = -1;
  const uint8_t* bm = nullptr;
  int64_t bq = 0, bk = 0, nqb = 0, nkb = 0;
};

int read_mods(const fa_mods* m, int64_t d_qk, int64_t max_sq, int64_t max_sk, Mods* out) {
  Mods r;
  if (m) {
    const uint32_t known = FA_CAUSAL | FA_WINDOW | FA_ALIBI | FA_SOFTCAP | FA_BLOCK_MASK;
    if (m->flags & ~known) return fail(FA_ERR_INVALID, "unknown fa_mods flag bits 0x%x", m->flags & ~known);
    r.flags = m->flags;
    r.scale = m->softmax_scale;
    if (!(r.scale == r.scale)) return fail(FA_ERR_INVALID, "softmax_scale is NaN");
    if (r.flags & FA_ALIBI) {
      r.slope = m->alibi_slope;
      if (!std::isfinite(r.slope)) return fail(FA_ERR_INVALID, "alibi_slope must be finite");
    }
    if (r.flags & FA_SOFTCAP) {
      r.cap = m->softcap;
      if (!(r.cap > 0.f) || !std::isfinite(r.cap)) return fail(FA_ERR_INVALID, "softcap must be finite and > 0");
    }
    if (r.flags & FA_WINDOW) {
      r.wl = m->window_left;
      r.wr = m->window_right;
    }
    if (r.flags & FA_BLOCK_MASK) {
      r.bm = m->block_mask;
      r.bq = m->mask_block_q;
      r.bk = m->mask_block_k;
      r.nqb = m->mask_nqb;
      r.nkb = m->mask_nkb;
      if (!r.bm) return fail(FA_ERR_INVALID, "FA_BLOCK_MASK set but block_mask is NULL");
      if (r.bq <= 0 || r.bk <= 0 || r.bq % kMaskBQ != 0 || r.bk % kBN != 0)
        return fail(FA_ERR_UNSUPPORTED, "block mask tiles must be multiples of %d (query) and %d (key), got %lld x %lld",
                    kMaskBQ, kBN, (long long)r.bq, (long long)r.bk);
      if (r.nqb < (max_sq + r.bq - 1) / r.bq || r.nkb < (max_sk + r.bk - 1) / r.bk)
        return fail(FA_ERR_INVALID, "block mask geometry %lld x %lld does not cover %lld x %lld tokens",
                    (long long)r.nqb, (long long)r.nkb, (long long)max_sq, (long long)max_sk);
      if (r.nqb >= kI32 || r.nkb >= kI32 || r.bq >= kI32 || r.bk >= kI32)
        return fail(FA_ERR_LIMIT, "block mask geometry exceeds int32");
    }
  }
  if (!(r.scale > 0.f)) r.scale = 1.0f / std::sqrt((float)d_qk);
  if (!std::isfinite(r.scale)) return fail(FA_ERR_INVALID, "softmax_scale must be finite");
  *out = r;
  return FA_OK;
}

// The kernels move tensors 16 bytes at a time (vector loads, LDS DMA):
// tensor bases must be 16-byte aligned, and every row then is (head dims are
// multiples of 8 elements); fp32 and int32 arrays 4-byte, int64 8-byte.
bool misaligned(uintptr_t align, std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (p && (reinterpret_cast<uintptr_t>(p) % align) != 0) return true;
  return false;
}

int clamp_i32(int64_t w) {
  if (w < 0) return -1;
  return w >= INT_MAX / 2 ? INT_MAX / 2 : (int)w;
}

bool prefill_dims_built(int64_t dqk, int64_t dv, bool fp8, bool paged) {
  if (fp8) return paged && ((dqk == 192 && dv == 128) || (dqk == 128 && dv == 128) || (dqk == 192 && dv == 192));
  return (dqk == 64 && dv == 64) || (dqk == 128 && dv == 128);
}

void fill_mods(fa::PrefillArgs& a, const Mods& m) {
  a.qk_scale = m.scale;
  a.alibi_slope = m.slope;
  a.softcap = m.cap;
  a.causal = (m.flags & FA_CAUSAL) ? 1 : 0;
  a.win_left = (m.flags & FA_WINDOW) ? clamp_i32(m.wl) : -1;
  a.win_right = (m.flags & FA_WINDOW) ? clamp_i32(m.wr) : -1;
  a.bmask = (m.flags & FA_BLOCK_MASK) ? m.bm : nullptr;
  a.bm_bq = (int)m.bq;
  a.bm_bk = (int)m.bk;
  a.bm_nqb = (int)m.nqb;
  a.bm_nkb = (int)m.nkb;
}

int mod_bits(const Mods& m) {
  return ((m.flags & FA_ALIBI) ? fa::kModAlibi : 0) | ((m.flags & FA_SOFTCAP) ? fa::kModSoftcap : 0);
}

int launch_prefill(const fa::PrefillArgs& a_in, int64_t dqk, int64_t dv, bool fp8, bool paged, bool vec, int mods,
                   int64_t B, int64_t Hq, int64_t max_sq, hipStream_t stream) {
  const int64_t n_bh = B * Hq;
  const int64_t n_qt = (max_sq + kBM - 1) / kBM;
  // grid: x = B*Hq rounded up to 8, y = query tiles
  if (n_bh + 7 >= kI32) return fail(FA_ERR_LIMIT, "B*Hq = %lld exceeds the grid limit", (long long)n_bh);
  if (n_qt > 65535) return fail(FA_ERR_LIMIT, "max_seqlen_q = %lld exceeds %d", (long long)max_sq, 65535 * kBM);
  if (n_bh == 0 || n_qt == 0) return FA_OK;
  fa::PrefillArgs a = a_in;
  a.n_bh = (int)n_bh;
  bool supported = false;
  hipError_t e = fa::prefill_dispatch(a, (int)dqk, (int)dv, fp8, paged, vec, mods, (int)n_bh, (int)n_qt, stream,
                                       &supported);
  if (!supported) return fail(FA_ERR_UNSUPPORTED, "no kernel built for d_qk=%lld d_v=%lld fp8=%d paged=%d mods=%d",
                              (long long)dqk, (long long)dv, (int)fp8, (int)paged, mods);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return FA_OK;
}

int check_common(int64_t B, int64_t Hq, int64_t Hkv, int64_t d_qk, int64_t d_v) {
  if (B < 0) return fail(FA_ERR_INVALID, "B must be >= 0");
  if (Hq <= 0 || Hkv <= 0) return fail(FA_ERR_INVALID, "head counts must be positive (Hq=%lld Hkv=%lld)", (long long)Hq, (long long)Hkv);
  if (Hq % Hkv != 0) return fail(FA_ERR_INVALID, "Hq (%lld) must be a multiple of Hkv (%lld)", (long long)Hq, (long long)Hkv);
  if (d_qk <= 0 || d_v <= 0) return fail(FA_ERR_INVALID, "head dims must be positive");
  if (B >= kI32 || Hq >= kI32) return fail(FA_ERR_LIMIT, "B or Hq exceeds int32");
  return FA_OK;
}

// Decode workers: one wavefront each.  With one 16-row block per wavefront
// the kernel keeps two tiles in flight per wavefront and runs one wavefront
// per SIMD (256 CUs x 4), which measured faster than two; with two row
// blocks it keeps one tile in flight and runs two per SIMD.  Value width 192
// needs the register file of one wavefront per SIMD: 1024 workers, two
// tiles in flight.  Capped by the tile count so small calls keep small
// workspaces.
// Stream-K workers of the decode (one wavefront each).  Measured on the
// 64-sequence decode batch: head-major pages stream best with 768 (3 % over
// 1024; 512 and 1536 lose 6-11 %), vectorised pages with 1024 (768: -5 %);
// two query-row blocks (slot_rows > 16) with 2048.
int64_t decode_workers(int64_t B, int64_t Hkv, int64_t slot_rows, int64_t kv_cap, int64_t d_v, bool vec) {
  const int64_t wmax = (slot_rows > 16 && d_v <= 128) ? 2048 : (vec ? 1024 : 768);
  const int64_t tiles = B * Hkv * ((kv_cap + 31) / 32);
  return std::max<int64_t>(1, std::min(wmax, tiles));
}

bool uses_decode(int64_t max_sq, int64_t Hq, int64_t Hkv, int64_t d_qk, int64_t d_v, fa_dtype kv, int64_t page_size) {
  if (kv != FA_FP8_E4M3) return false;
  if (!((d_v == 128 && (d_qk == 192 || d_qk == 128)) || (d_v == 192 && d_qk == 192))) return false;
  return max_sq >= 1 && max_sq * (Hq / Hkv) <= kDecodeRows;
}

// Workspace of the decode path: the tile prefix ([B+1] int32, padded to 256
// bytes), then the partial O [slots, slot_rows, d_v] and LSE [slots,
// slot_rows] in fp32, slots = workers + B * Hkv.
struct DecodeLayout {
  int64_t workers = 0, slots = 0, slot_rows = 0, kv_cap = 0;
  size_t tiles_bytes = 0, o_bytes = 0, total = 0;
};

DecodeLayout decode_layout(int64_t B, int64_t max_sq, int64_t max_sk, int64_t Hq, int64_t Hkv, int64_t d_v,
                           int64_t kv_cap, bool vec) {
  DecodeLayout L;
  L.slot_rows = max_sq * (Hq / Hkv);
  L.kv_cap = std::min(kv_cap, max_sk);
  L.workers = decode_workers(B, Hkv, L.slot_rows, L.kv_cap, d_v, vec);
  L.slots = L.workers + B * Hkv;
  L.tiles_bytes = (size_t)((B + 1) * 4 + 255) / 256 * 256;
  L.o_bytes = (size_t)(L.slots * L.slot_rows * d_v) * sizeof(float);
  L.total = L.tiles_bytes + L.o_bytes + (size_t)(L.slots * L.slot_rows) * sizeof(float);
  return L;
}

// Reduction blocks of the KV-cache writer's per-tensor maximum: enough to
// fill the chip, at least 32 elements per thread.
int kv_amax_blocks(int64_t n) {
  const int64_t b = (n + 256 * 8 * 4 - 1) / (256 * 8 * 4);
  return (int)std::max<int64_t>(1, std::min<int64_t>(b, 2048));
}

size_t workspace_bytes(int64_t B, int64_t total_q, int64_t max_sq, int64_t max_sk, int64_t Hq, int64_t Hkv,
                       int64_t d_qk, int64_t d_v, fa_dtype kv, int64_t page_size) {
  (void)total_q;
  if (B < 0 || max_sq < 0 || max_sk < 0 || Hkv <= 0 || Hq <= 0 || Hq % Hkv != 0) return 0;
  if (!uses_decode(max_sq, Hq, Hkv, d_qk, d_v, kv, page_size)) return 0;
  // the larger of the two page formats' worker counts: enough for either
  return decode_layout(B, max_sq, max_sk, Hq, Hkv, d_v, max_sk, true).total;
}

}  // namespace

extern "C" {

const char* fa_last_error(void) { return g_err.c_str(); }

int fa_abi_version(void) { return 1; }

int fa_fwd_dense(const void* q, const void* k, const void* v, void* o, float* lse,
                 int64_t B, int64_t Sq, int64_t Skv, int64_t Hq, int64_t Hkv,
                 int64_t d_qk, int64_t d_v, const fa_mods* mods, void* stream) {
  g_err.clear();
  int rc = check_common(B, Hq, Hkv, d_qk, d_v);
  if (rc) return rc;
  if (Sq < 0 || Skv < 0) return fail(FA_ERR_INVALID, "sequence lengths must be >= 0");
  if (Sq >= kI32 || Skv >= kI32 || B * Sq >= kI32 || B * Skv >= kI32)
    return fail(FA_ERR_LIMIT, "token counts must stay below 2^31");
  Mods m;
  if ((rc = read_mods(mods, d_qk, Sq, Skv, &m))) return rc;
  if (!prefill_dims_built(d_qk, d_v, false, false))
    return fail(FA_ERR_UNSUPPORTED, "dense bf16 head dims (%lld, %lld) not built; built: (64,64), (128,128)",
                (long long)d_qk, (long long)d_v);
  if (B == 0 || Sq == 0) return FA_OK;
  if (!q || !o || !lse) return fail(FA_ERR_INVALID, "q, o and lse must be non-NULL");
  if (Skv > 0 && (!k || !v)) return fail(FA_ERR_INVALID, "k and v must be non-NULL");
  if (misaligned(16, {q, k, v, o}) || misaligned(4, {lse}))
    return fail(FA_ERR_INVALID, "q, k, v and o must be 16-byte aligned, lse 4-byte aligned");
  const size_t nq = (size_t)(B * Sq * Hq * d_qk) * 2, no = (size_t)(B * Sq * Hq * d_v) * 2;
  const size_t nk = (size_t)(B * Skv * Hkv * d_qk) * 2, nv = (size_t)(B * Skv * Hkv * d_v) * 2;
  const size_t nl = (size_t)(B * Hq * Sq) * 4;
  if (overlaps(o, no, lse, nl)) return fail(FA_ERR_INVALID, "lse must not overlap o");
  if (overlaps(o, no, q, nq) || overlaps(o, no, k, nk) || overlaps(o, no, v, nv) ||
      overlaps(lse, nl, q, nq) || overlaps(lse, nl, k, nk) || overlaps(lse, nl, v, nv))
    return fail(FA_ERR_INVALID, "outputs must not overlap inputs");
  fa::PrefillArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = (__bf16*)o;
  a.lse = lse;
  a.q_st = Hq * d_qk; a.q_sh = d_qk;
  a.k_st = Hkv * d_qk; a.k_sh = d_qk;
  a.v_st = Hkv * d_v; a.v_sh = d_v;
  a.o_st = Hq * d_v; a.o_sh = d_v;
  a.Sq = (int)Sq; a.Skv = (int)Skv;
  a.Hq = (int)Hq; a.group = (int)(Hq / Hkv);
  fill_mods(a, m);
  return launch_prefill(a, d_qk, d_v, false, false, false, mod_bits(m), B, Hq, Sq, (hipStream_t)stream);
}

int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                  const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int64_t B,
                  int64_t total_q, int64_t total_k, int64_t max_seqlen_q, int64_t max_seqlen_k,
                  int64_t Hq, int64_t Hkv, int64_t d_qk, int64_t d_v,
                  const fa_mods* mods, void* stream) {
  g_err.clear();
  int rc = check_common(B, Hq, Hkv, d_qk, d_v);
  if (rc) return rc;
  if (total_q < 0 || total_k < 0 || max_seqlen_q < 0 || max_seqlen_k < 0)
    return fail(FA_ERR_INVALID, "token counts must be >= 0");
  if (max_seqlen_q > total_q || max_seqlen_k > total_k)
    return fail(FA_ERR_INVALID, "max_seqlen exceeds the packed token count");
  if (total_q >= kI32 || total_k >= kI32) return fail(FA_ERR_LIMIT, "token counts must stay below 2^31");
  Mods m;
  if ((rc = read_mods(mods, d_qk, max_seqlen_q, max_seqlen_k, &m))) return rc;
  if (!prefill_dims_built(d_qk, d_v, false, false))
    return fail(FA_ERR_UNSUPPORTED, "varlen bf16 head dims (%lld, %lld) not built; built: (64,64), (128,128)",
                (long long)d_qk, (long long)d_v);
  if (B == 0 || total_q == 0) return FA_OK;
  if (!q || !o || !lse || !cu_seqlens_q || !cu_seqlens_k) return fail(FA_ERR_INVALID, "q, o, lse and cu_seqlens must be non-NULL");
  if (total_k > 0 && (!k || !v)) return fail(FA_ERR_INVALID, "k and v must be non-NULL");
  if (misaligned(16, {q, k, v, o}) || misaligned(4, {lse, cu_seqlens_q, cu_seqlens_k}))
    return fail(FA_ERR_INVALID, "q, k, v and o must be 16-byte aligned, lse and cu_seqlens 4-byte aligned");
  const size_t nq = (size_t)(total_q * Hq * d_qk) * 2, no = (size_t)(total_q * Hq * d_v) * 2;
  const size_t nk = (size_t)(total_k * Hkv * d_qk) * 2, nv = (size_t)(total_k * Hkv * d_v) * 2;
  const size_t nl = (size_t)(Hq * total_q) * 4;
  if (overlaps(o, no, lse, nl)) return fail(FA_ERR_INVALID, "lse must not overlap o");
  if (overlaps(o, no, q, nq) || overlaps(o, no, k, nk) || overlaps(o, no, v, nv) ||
      overlaps(lse, nl, q, nq) || overlaps(lse, nl, k, nk) || overlaps(lse, nl, v, nv))
    return fail(FA_ERR_INVALID, "outputs must not overlap inputs");
  fa::PrefillArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = (__bf16*)o;
  a.lse = lse;
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.q_st = Hq * d_qk; a.q_sh = d_qk;
  a.k_st = Hkv * d_qk; a.k_sh = d_qk;
  a.v_st = Hkv * d_v; a.v_sh = d_v;
  a.o_st = Hq * d_v; a.o_sh = d_v;
  a.lse_tq = total_q;
  a.Hq = (int)Hq; a.group = (int)(Hq / Hkv);
  fill_mods(a, m);
  return launch_prefill(a, d_qk, d_v, false, false, false, mod_bits(m), B, Hq, max_seqlen_q, (hipStream_t)stream);
}

size_t fa_fwd_paged_workspace_size(int64_t B, int64_t total_q, int64_t max_seqlen_q, int64_t max_seqlen_k,
                                   int64_t Hq, int64_t Hkv, int64_t d_qk, int64_t d_v, int64_t page_size,
                                   fa_dtype kv_dtype) {
  return workspace_bytes(B, total_q, max_seqlen_q, max_seqlen_k, Hq, Hkv, d_qk, d_v, kv_dtype, page_size);
}

}  // extern "C"

// Decode scratch of fa_fwd_paged_noalloc: the tile prefix and the split-KV
// partials of one call, in a static device array (each GPU that runs the
// library holds its own copy until the process ends).  Host code never uses
// the array's name as an address: its device address is looked up once per
// device with hipGetSymbolAddress and kept in g_scratch_ptr.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address (looked up on its first use).
int scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(FA_ERR_LIMIT, "device %d beyond the %d the library tracks", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(FA_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FA_OK;
}

// The paged entry points.
int paged_impl(const fa_paged_opts* opts, const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
               const int32_t* cu_seqlens_q, const int32_t* seqlen_k, const int32_t* block_table,
               int64_t B, int64_t total_q, int64_t max_seqlen_q, int64_t max_seqlen_k,
               int64_t num_pages, int64_t page_size, int64_t max_pages_per_seq,
               int64_t Hq, int64_t Hkv, int64_t d_qk, int64_t d_v, fa_dtype kv_dtype,
               const float* k_descale, const float* v_descale,
               void* workspace, size_t workspace_bytes_in,
               const fa_mods* mods, void* stream, bool use_scratch = false) {
  g_err.clear();
  int rc = check_common(B, Hq, Hkv, d_qk, d_v);
  if (rc) return rc;
  if (kv_dtype != FA_BF16 && kv_dtype != FA_FP8_E4M3) return fail(FA_ERR_INVALID, "unknown kv_dtype %d", (int)kv_dtype);
  const fa_paged_opts def{FA_BF16, nullptr, FA_PAGES_HEAD_MAJOR};
  if (!opts) opts = &def;
  if (opts->q_dtype != FA_BF16 && opts->q_dtype != FA_FP8_E4M3)
    return fail(FA_ERR_INVALID, "unknown q_dtype %d", (int)opts->q_dtype);
  if (opts->page_layout != FA_PAGES_HEAD_MAJOR && opts->page_layout != FA_PAGES_VECTORIZED)
    return fail(FA_ERR_INVALID, "unknown page_layout %d", (int)opts->page_layout);
  const bool vec = opts->page_layout == FA_PAGES_VECTORIZED;
  const bool q8 = opts->q_dtype == FA_FP8_E4M3;
  if (vec && kv_dtype != FA_FP8_E4M3) return fail(FA_ERR_UNSUPPORTED, "vectorised pages hold FP8 E4M3 K/V only");
  if (q8 && kv_dtype != FA_FP8_E4M3) return fail(FA_ERR_UNSUPPORTED, "E4M3 queries need an FP8 E4M3 cache");
  if (q8 && !opts->q_descale) return fail(FA_ERR_INVALID, "E4M3 queries need q_descale");
  if (total_q < 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || num_pages < 0 || max_pages_per_seq < 0)
    return fail(FA_ERR_INVALID, "sizes must be >= 0");
  if (max_seqlen_q > total_q) return fail(FA_ERR_INVALID, "max_seqlen_q exceeds total_q");
  if (page_size < 1 || page_size > 1024 || (page_size & (page_size - 1)))
    return fail(FA_ERR_UNSUPPORTED, "page_size must be a power of two in [1, 1024], got %lld", (long long)page_size);
  if (vec && page_size < 16)
    return fail(FA_ERR_UNSUPPORTED, "vectorised pages hold whole 16-key blocks: page_size >= 16, got %lld",
                (long long)page_size);
  if (total_q >= kI32 || max_seqlen_k >= kI32 || num_pages >= kI32 || max_pages_per_seq >= kI32)
    return fail(FA_ERR_LIMIT, "token and page counts must stay below 2^31");
  if (B * max_pages_per_seq >= kI32) return fail(FA_ERR_LIMIT, "block_table extent exceeds 2^31");
  if (max_pages_per_seq * page_size < max_seqlen_k)
    return fail(FA_ERR_INVALID, "max_pages_per_seq * page_size (%lld) < max_seqlen_k (%lld)",
                (long long)(max_pages_per_seq * page_size), (long long)max_seqlen_k);
  Mods m;
  if ((rc = read_mods(mods, d_qk, max_seqlen_q, max_seqlen_k, &m))) return rc;
  const bool fp8 = kv_dtype == FA_FP8_E4M3;
  const bool decode = uses_decode(max_seqlen_q, Hq, Hkv, d_qk, d_v, kv_dtype, page_size);
  if (!decode && !prefill_dims_built(d_qk, d_v, fp8, true))
    return fail(FA_ERR_UNSUPPORTED, "paged head dims (%lld, %lld) with kv_dtype %d not built", (long long)d_qk,
                (long long)d_v, (int)kv_dtype);
  if (B == 0 || total_q == 0) return FA_OK;
  if (!q || !o || !lse || !cu_seqlens_q || !seqlen_k || !block_table)
    return fail(FA_ERR_INVALID, "q, o, lse, cu_seqlens_q, seqlen_k and block_table must be non-NULL");
  if (num_pages > 0 && (!k_cache || !v_cache)) return fail(FA_ERR_INVALID, "caches must be non-NULL");
  if (max_seqlen_k > 0 && num_pages == 0) return fail(FA_ERR_INVALID, "num_pages is 0 but max_seqlen_k > 0");
  if (fp8 && (!k_descale || !v_descale)) return fail(FA_ERR_INVALID, "FP8 caches need k_descale and v_descale");
  if (misaligned(16, {q, k_cache, v_cache, o, workspace}) ||
      misaligned(4, {lse, cu_seqlens_q, seqlen_k, block_table, k_descale, v_descale}))
    return fail(FA_ERR_INVALID, "q, the caches, o and workspace must be 16-byte aligned, the other arrays 4-byte aligned");
  const size_t es = fp8 ? 1 : 2;
  const size_t nq = (size_t)(total_q * Hq * d_qk) * (q8 ? 1 : 2), no = (size_t)(total_q * Hq * d_v) * 2;
  const size_t nk = (size_t)num_pages * Hkv * page_size * d_qk * es, nv = (size_t)num_pages * Hkv * page_size * d_v * es;
  const size_t nl = (size_t)(Hq * total_q) * 4;
  if (overlaps(o, no, lse, nl)) return fail(FA_ERR_INVALID, "lse must not overlap o");
  if (overlaps(o, no, q, nq) || overlaps(o, no, k_cache, nk) || overlaps(o, no, v_cache, nv) ||
      overlaps(lse, nl, q, nq) || overlaps(lse, nl, k_cache, nk) || overlaps(lse, nl, v_cache, nv))
    return fail(FA_ERR_INVALID, "outputs must not overlap inputs");
  int shift = 0;
  while ((1ll << shift) < page_size) ++shift;
  const hipStream_t st = (hipStream_t)stream;

  if (decode) {
    const size_t need = workspace_bytes(B, total_q, max_seqlen_q, max_seqlen_k, Hq, Hkv, d_qk, d_v, kv_dtype, page_size);
    if (use_scratch) {
      if (need > kScratchBytes)
        return fail(FA_ERR_LIMIT, "this decode call needs %zu bytes of scratch; fa_fwd_paged_noalloc holds %zu "
                    "(fa_fwd_paged with a workspace has no such limit)", need, kScratchBytes);
    } else {
      if (!workspace || workspace_bytes_in < need)
        return fail(FA_ERR_WORKSPACE, "decode path needs a workspace of %zu bytes (got %zu)", need, workspace_bytes_in);
      // the plan kernel writes the workspace while the same call reads the
      // metadata, the caches and the descales: it may overlap none of them
      if (overlaps(workspace, need, o, no) || overlaps(workspace, need, lse, nl) || overlaps(workspace, need, q, nq))
        return fail(FA_ERR_INVALID, "workspace must not overlap q, o or lse");
      if (overlaps(workspace, need, cu_seqlens_q, (size_t)(B + 1) * 4) ||
          overlaps(workspace, need, seqlen_k, (size_t)B * 4) ||
          overlaps(workspace, need, block_table, (size_t)(B * max_pages_per_seq) * 4))
        return fail(FA_ERR_INVALID, "workspace must not overlap cu_seqlens_q, seqlen_k or block_table");
      if (overlaps(workspace, need, k_cache, nk) || overlaps(workspace, need, v_cache, nv) ||
          overlaps(workspace, need, k_descale, 4) || overlaps(workspace, need, v_descale, 4) ||
          (q8 && overlaps(workspace, need, opts->q_descale, 4)))
        return fail(FA_ERR_INVALID, "workspace must not overlap the caches or the descales");
    }
    if (B * Hkv * ((max_seqlen_k + 31) / 32) >= kI32) return fail(FA_ERR_LIMIT, "decode tile count exceeds 2^31");
    const DecodeLayout L = decode_layout(B, max_seqlen_q, max_seqlen_k, Hq, Hkv, d_v,
                                         std::min<int64_t>(max_pages_per_seq * page_size, kI32 - 1), vec);
    // every host check is done: the first HIP call of the no-allocation path
    // looks up this device's copy of the scratch array
    if (use_scratch && (rc = scratch_for_current_device(&workspace))) return rc;
    int32_t* tiles = (int32_t*)workspace;
    float* part_o = (float*)((char*)workspace + L.tiles_bytes);
    float* part_lse = (float*)((char*)part_o + L.o_bytes);
    fa::DecodePlanArgs pl{};
    pl.cu_q = cu_seqlens_q;
    pl.seqlen_k = seqlen_k;
    pl.tiles = tiles;
    pl.B = (int)B;
    pl.kv_cap = (int)L.kv_cap;
    fa::DecodeArgs d{};
    d.q = q;
    d.q_descale = q8 ? opts->q_descale : nullptr;
    d.k = k_cache;
    d.v = v_cache;
    d.part_o = part_o;
    d.part_lse = part_lse;
    d.cu_q = cu_seqlens_q;
    d.seqlen_k = seqlen_k;
    d.block_table = block_table;
    d.k_descale = k_descale;
    d.v_descale = v_descale;
    d.tiles = tiles;
    d.q_st = Hq * d_qk; d.q_sh = d_qk;
    d.k_st = d_qk; d.k_sh = page_size * d_qk; d.k_pg = Hkv * page_size * d_qk;
    d.v_st = d_v; d.v_sh = page_size * d_v; d.v_pg = Hkv * page_size * d_v;
    d.B = (int)B; d.Hq = (int)Hq; d.Hkv = (int)Hkv; d.group = (int)(Hq / Hkv);
    d.max_pages = (int)max_pages_per_seq;
    d.page_shift = shift;
    d.kv_cap = (int)L.kv_cap;
    d.num_pages = (int)num_pages;
    d.n_workers = (int)L.workers;
    d.slot_rows = (int)L.slot_rows;
    d.qk_scale = m.scale;
    d.causal = (m.flags & FA_CAUSAL) ? 1 : 0;
    d.win_left = (m.flags & FA_WINDOW) ? clamp_i32(m.wl) : -1;
    d.win_right = (m.flags & FA_WINDOW) ? clamp_i32(m.wr) : -1;
    d.alibi_slope = (m.flags & FA_ALIBI) ? m.slope : 0.0f;
    d.softcap = (m.flags & FA_SOFTCAP) ? m.cap : 0.0f;
    d.bmask = (m.flags & FA_BLOCK_MASK) ? m.bm : nullptr;
    d.bm_bq = (int)m.bq;
    d.bm_bk = (int)m.bk;
    d.bm_nqb = (int)m.nqb;
    d.bm_nkb = (int)m.nkb;
    bool supported = false;
    hipError_t e = fa::decode_dispatch(pl, d, (int)d_qk, (int)d_v, fp8, vec, q8, st, &supported);
    if (!supported) return fail(FA_ERR_UNSUPPORTED, "no decode kernel for (%lld, %lld)", (long long)d_qk, (long long)d_v);
    if (e != hipSuccess) return fail(FA_ERR_HIP, "decode launch failed: %s", hipGetErrorString(e));
    fa::CombineArgs c{};
    c.part_o = part_o;
    c.part_lse = part_lse;
    c.o = (__bf16*)o;
    c.lse = lse;
    c.cu_q = cu_seqlens_q;
    c.tiles = tiles;
    c.o_st = Hq * d_v; c.o_sh = d_v;
    c.total_q = total_q;
    c.B = (int)B; c.Hq = (int)Hq; c.Hkv = (int)Hkv; c.group = (int)(Hq / Hkv);
    c.n_workers = (int)L.workers;
    c.slot_rows = (int)L.slot_rows;
    e = fa::combine_dispatch(c, (int)d_v, st, &supported);
    if (!supported) return fail(FA_ERR_UNSUPPORTED, "no combine kernel for d_v=%lld", (long long)d_v);
    if (e != hipSuccess) return fail(FA_ERR_HIP, "combine launch failed: %s", hipGetErrorString(e));
    return FA_OK;
  }

  fa::PrefillArgs a{};
  a.q = q;
  a.q_descale = q8 ? opts->q_descale : nullptr;
  a.k = k_cache;
  a.v = v_cache;
  a.o = (__bf16*)o;
  a.lse = lse;
  a.cu_q = cu_seqlens_q;
  a.seqlen_k = seqlen_k;
  a.block_table = block_table;
  a.k_descale = k_descale;
  a.v_descale = v_descale;
  a.q_st = Hq * d_qk; a.q_sh = d_qk;
  a.k_st = d_qk; a.k_sh = page_size * d_qk; a.k_pg = Hkv * page_size * d_qk;
  a.v_st = d_v; a.v_sh = page_size * d_v; a.v_pg = Hkv * page_size * d_v;
  a.o_st = Hq * d_v; a.o_sh = d_v;
  a.lse_tq = total_q;
  a.Hq = (int)Hq; a.group = (int)(Hq / Hkv);
  a.max_pages = (int)max_pages_per_seq;
  a.page_shift = shift;
  a.num_pages = (int)num_pages;
  fill_mods(a, m);
  return launch_prefill(a, d_qk, d_v, fp8, true, vec, mod_bits(m), B, Hq, max_seqlen_q, st);
}

}  // namespace

extern "C" {

int fa_fwd_paged(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                 const int32_t* cu_seqlens_q, const int32_t* seqlen_k, const int32_t* block_table,
                 int64_t B, int64_t total_q, int64_t max_seqlen_q, int64_t max_seqlen_k,
                 int64_t num_pages, int64_t page_size, int64_t max_pages_per_seq,
                 int64_t Hq, int64_t Hkv, int64_t d_qk, int64_t d_v, fa_dtype kv_dtype,
                 const float* k_descale, const float* v_descale,
                 void* workspace, size_t workspace_bytes_in,
                 const fa_mods* mods, void* stream) {
  return paged_impl(nullptr, q, k_cache, v_cache, o, lse, cu_seqlens_q, seqlen_k, block_table, B, total_q,
                    max_seqlen_q, max_seqlen_k, num_pages, page_size, max_pages_per_seq, Hq, Hkv, d_qk, d_v,
                    kv_dtype, k_descale, v_descale, workspace, workspace_bytes_in, mods, stream);
}

int fa_fwd_paged_noalloc(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                         const int32_t* cu_seqlens_q, const int32_t* seqlen_k, const int32_t* block_table,
                         int64_t B, int64_t total_q, int64_t max_seqlen_q, int64_t max_seqlen_k,
                         int64_t num_pages, int64_t page_size, int64_t max_pages_per_seq,
                         int64_t Hq, int64_t Hkv, int64_t d_qk, int64_t d_v, fa_dtype kv_dtype,
                         const float* k_descale, const float* v_descale,
                         const fa_mods* mods, void* stream) {
  return paged_impl(nullptr, q, k_cache, v_cache, o, lse, cu_seqlens_q, seqlen_k, block_table, B, total_q,
                    max_seqlen_q, max_seqlen_k, num_pages, page_size, max_pages_per_seq, Hq, Hkv, d_qk, d_v,
                    kv_dtype, k_descale, v_descale, nullptr, 0, mods, stream, true);
}

int fa_fwd_paged_vec(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                     const int32_t* cu_seqlens_q, const int32_t* seqlen_k, const int32_t* block_table,
                     int64_t B, int64_t total_q, int64_t max_seqlen_q, int64_t max_seqlen_k,
                     int64_t num_pages, int64_t page_size, int64_t max_pages_per_seq,
                     int64_t Hq, int64_t Hkv, int64_t d_qk, int64_t d_v, fa_dtype kv_dtype,
                     const float* k_descale, const float* v_descale,
                     void* workspace, size_t workspace_bytes_in,
                     const fa_mods* mods, void* stream) {
  const fa_paged_opts vec{FA_BF16, nullptr, FA_PAGES_VECTORIZED};
  return paged_impl(&vec, q, k_cache, v_cache, o, lse, cu_seqlens_q, seqlen_k, block_table, B, total_q,
                    max_seqlen_q, max_seqlen_k, num_pages, page_size, max_pages_per_seq, Hq, Hkv, d_qk, d_v,
                    kv_dtype, k_descale, v_descale, workspace, workspace_bytes_in, mods, stream);
}

int fa_fwd_paged_ex(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                    const int32_t* cu_seqlens_q, const int32_t* seqlen_k, const int32_t* block_table,
                    int64_t B, int64_t total_q, int64_t max_seqlen_q, int64_t max_seqlen_k,
                    int64_t num_pages, int64_t page_size, int64_t max_pages_per_seq,
                    int64_t Hq, int64_t Hkv, int64_t d_qk, int64_t d_v, fa_dtype kv_dtype,
                    const float* k_descale, const float* v_descale,
                    void* workspace, size_t workspace_bytes_in,
                    const fa_paged_opts* opts, const fa_mods* mods, void* stream) {
  return paged_impl(opts, q, k_cache, v_cache, o, lse, cu_seqlens_q, seqlen_k, block_table, B, total_q,
                    max_seqlen_q, max_seqlen_k, num_pages, page_size, max_pages_per_seq, Hq, Hkv, d_qk, d_v,
                    kv_dtype, k_descale, v_descale, workspace, workspace_bytes_in, mods, stream);
}

size_t fa_kv_cache_write_fp8_workspace_size(int64_t T, int64_t Hkv, int64_t d_qk, int64_t d_v) {
  if (T <= 0 || Hkv <= 0 || d_qk <= 0 || d_v <= 0) return 0;
  return (size_t)(kv_amax_blocks(T * Hkv * d_qk) + kv_amax_blocks(T * Hkv * d_v)) * sizeof(float);
}

int fa_kv_cache_write_fp8(const void* k, const void* v, const int64_t* slot_mapping,
                          int64_t T, int64_t Hkv, int64_t d_qk, int64_t d_v,
                          void* k_cache, void* v_cache, int64_t num_pages, int64_t page_size,
                          int32_t page_layout, float* k_descale, float* v_descale, int32_t scale_mode,
                          void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  if (T < 0 || num_pages < 0) return fail(FA_ERR_INVALID, "T and num_pages must be >= 0");
  if (Hkv <= 0 || d_qk <= 0 || d_v <= 0) return fail(FA_ERR_INVALID, "Hkv and head dims must be positive");
  if (d_qk % 16 || d_v % 16) return fail(FA_ERR_UNSUPPORTED, "head dims must be multiples of 16");
  if (page_layout != FA_PAGES_HEAD_MAJOR && page_layout != FA_PAGES_VECTORIZED)
    return fail(FA_ERR_INVALID, "unknown page_layout %d", (int)page_layout);
  if (scale_mode != FA_SCALE_GIVEN && scale_mode != FA_SCALE_AMAX)
    return fail(FA_ERR_INVALID, "unknown scale_mode %d", (int)scale_mode);
  const bool vec = page_layout == FA_PAGES_VECTORIZED;
  if (page_size < (vec ? 16 : 1) || page_size > 1024 || (page_size & (page_size - 1)))
    return fail(FA_ERR_UNSUPPORTED, "page_size must be a power of two in [%d, 1024], got %lld", vec ? 16 : 1,
                (long long)page_size);
  if (T >= kI32 || Hkv >= kI32) return fail(FA_ERR_LIMIT, "T and Hkv must stay below 2^31");
  if (d_qk + d_v > kKvLdsBytes / 16)
    return fail(FA_ERR_UNSUPPORTED, "d_qk + d_v must be at most %d", kKvLdsBytes / 16);
  if (T == 0) return FA_OK;
  if (!k || !v || !slot_mapping || !k_descale || !v_descale)
    return fail(FA_ERR_INVALID, "k, v, slot_mapping and the descales must be non-NULL");
  if (num_pages > 0 && (!k_cache || !v_cache)) return fail(FA_ERR_INVALID, "caches must be non-NULL");
  if (misaligned(16, {k, v, k_cache, v_cache, workspace}) || misaligned(8, {slot_mapping}) ||
      misaligned(4, {k_descale, v_descale}))
    return fail(FA_ERR_INVALID, "k, v, the caches and workspace must be 16-byte aligned, slot_mapping 8-byte, "
                "the descales 4-byte");
  const size_t nk = (size_t)(T * Hkv * d_qk) * 2, nv = (size_t)(T * Hkv * d_v) * 2;
  const size_t ck = (size_t)num_pages * Hkv * page_size * d_qk, cv = (size_t)num_pages * Hkv * page_size * d_v;
  if (overlaps(k_cache, ck, v_cache, cv) || overlaps(k_cache, ck, k, nk) || overlaps(k_cache, ck, v, nv) ||
      overlaps(v_cache, cv, k, nk) || overlaps(v_cache, cv, v, nv))
    return fail(FA_ERR_INVALID, "caches must not overlap each other or the rows");
  if (overlaps(k_descale, 4, v_descale, 4)) return fail(FA_ERR_INVALID, "k_descale and v_descale must differ");
  int shift = 0;
  while ((1ll << shift) < page_size) ++shift;
  const hipStream_t st = (hipStream_t)stream;
  if (scale_mode == FA_SCALE_AMAX) {
    const size_t need = fa_kv_cache_write_fp8_workspace_size(T, Hkv, d_qk, d_v);
    if (!workspace || workspace_bytes < need)
      return fail(FA_ERR_WORKSPACE, "FA_SCALE_AMAX needs a workspace of %zu bytes (got %zu)", need, workspace_bytes);
    fa::KvAmaxArgs m{};
    m.k = (const __bf16*)k;
    m.v = (const __bf16*)v;
    m.n_k = T * Hkv * d_qk;
    m.n_v = T * Hkv * d_v;
    m.nb_k = kv_amax_blocks(m.n_k);
    m.nb_v = kv_amax_blocks(m.n_v);
    m.partial = (float*)workspace;
    m.k_descale = k_descale;
    m.v_descale = v_descale;
    hipError_t e = fa::kv_amax_dispatch(m, st);
    if (e != hipSuccess) return fail(FA_ERR_HIP, "amax launch failed: %s", hipGetErrorString(e));
  }
  if (num_pages == 0) return FA_OK;
  fa::KvWriteArgs w{};
  w.k = (const __bf16*)k;
  w.v = (const __bf16*)v;
  w.slot_mapping = slot_mapping;
  w.k_cache = k_cache;
  w.v_cache = v_cache;
  w.k_descale = k_descale;
  w.v_descale = v_descale;
  w.T = T;
  w.Hkv = Hkv;
  w.d_qk = (int)d_qk;
  w.d_v = (int)d_v;
  w.num_pages = num_pages;
  w.page_shift = shift;
  w.heads_per_pass = (int)std::min<int64_t>(Hkv, kKvLdsBytes / (16 * (d_qk + d_v)));
  hipError_t e = fa::kv_write_dispatch(w, vec, st);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "cache write launch failed: %s", hipGetErrorString(e));
  return FA_OK;
}

size_t fa_bwd_workspace_size(int64_t total_q, int64_t Hq) {
  if (total_q <= 0 || Hq <= 0) return 0;
  return (size_t)(total_q * Hq) * sizeof(float);
}

}  // extern "C"

namespace {

// Shared checks and launch of the two backward entry points (cu_q null: dense).
int bwd_impl(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
             void* dq, void* dk, void* dv, const int32_t* cu_q, const int32_t* cu_k, int64_t B, int64_t Sq,
             int64_t Skv, int64_t total_q, int64_t total_k, int64_t max_sq, int64_t max_sk, int64_t Hq, int64_t Hkv,
             int64_t d_qk, int64_t d_v, const fa_mods* mods, void* workspace, size_t workspace_bytes,
             void* stream) {
  int rc = check_common(B, Hq, Hkv, d_qk, d_v);
  if (rc) return rc;
  if (total_q < 0 || total_k < 0 || max_sq < 0 || max_sk < 0) return fail(FA_ERR_INVALID, "token counts must be >= 0");
  if (max_sq > total_q || max_sk > total_k) return fail(FA_ERR_INVALID, "max_seqlen exceeds the packed token count");
  if (total_q >= kI32 || total_k >= kI32) return fail(FA_ERR_LIMIT, "token counts must stay below 2^31");
  if (B * Hq >= kI32 || B * Hkv >= 65536 * 16384) return fail(FA_ERR_LIMIT, "B*H exceeds the grid limit");
  if (max_sq / 128 >= 65535 || max_sk / 64 >= 65535) return fail(FA_ERR_LIMIT, "sequence length exceeds the grid limit");
  // the kernels' tile copies take 32-bit offsets of up to 63 rows
  if (Hq * std::max(d_qk, d_v) >= (1 << 24))
    return fail(FA_ERR_LIMIT, "Hq * head dim must stay below 2^24 for the backward");
  Mods m;
  if ((rc = read_mods(mods, d_qk, max_sq, max_sk, &m))) return rc;
  if (m.flags & (FA_ALIBI | FA_SOFTCAP | FA_BLOCK_MASK))
    return fail(FA_ERR_UNSUPPORTED, "the backward supports FA_CAUSAL and FA_WINDOW only");
  if (d_qk != d_v || (d_qk != 64 && d_qk != 128))
    return fail(FA_ERR_UNSUPPORTED, "backward head dims (%lld, %lld) not built; built: (64,64), (128,128)",
                (long long)d_qk, (long long)d_v);
  if (B == 0 || (total_q == 0 && total_k == 0)) return FA_OK;
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || (cu_q && !cu_k))
    return fail(FA_ERR_INVALID, "tensor pointers must be non-NULL");
  if (misaligned(16, {q, k, v, o, dout, dq, dk, dv, workspace}) || misaligned(4, {lse, cu_q, cu_k}))
    return fail(FA_ERR_INVALID, "tensors and workspace must be 16-byte aligned, lse and cu_seqlens 4-byte aligned");
  const size_t need = fa_bwd_workspace_size(total_q, Hq);
  if (need && (!workspace || workspace_bytes < need))
    return fail(FA_ERR_WORKSPACE, "the backward needs a workspace of %zu bytes (got %zu)", need, workspace_bytes);
  const size_t nq = (size_t)(total_q * Hq * d_qk) * 2, nk = (size_t)(total_k * Hkv * d_qk) * 2;
  const size_t nv = (size_t)(total_k * Hkv * d_v) * 2, no = (size_t)(total_q * Hq * d_v) * 2;
  const size_t nl = (size_t)(total_q * Hq) * 4;
  const void* ins[] = {q, k, v, o, dout, lse};
  const size_t in_n[] = {nq, nk, nv, no, no, nl};
  void* outs[] = {dq, dk, dv, workspace};
  const size_t out_n[] = {nq, nk, nv, need};
  for (int x = 0; x < 4; ++x) {
    for (int y = 0; y < 6; ++y)
      if (overlaps(outs[x], out_n[x], ins[y], in_n[y])) return fail(FA_ERR_INVALID, "outputs must not overlap inputs");
    for (int y = x + 1; y < 4; ++y)
      if (overlaps(outs[x], out_n[x], outs[y], out_n[y])) return fail(FA_ERR_INVALID, "outputs must not overlap");
  }
  fa::BwdArgs a{};
  a.q = (const __bf16*)q;
  a.k = (const __bf16*)k;
  a.v = (const __bf16*)v;
  a.o = (const __bf16*)o;
  a.dout = (const __bf16*)dout;
  a.lse = lse;
  a.delta = (float*)workspace;
  a.dq = (__bf16*)dq;
  a.dk = (__bf16*)dk;
  a.dv = (__bf16*)dv;
  a.cu_q = cu_q;
  a.cu_k = cu_k;
  a.q_st = Hq * d_qk; a.q_sh = d_qk;
  a.k_st = Hkv * d_qk; a.k_sh = d_qk;
  a.v_st = Hkv * d_v; a.v_sh = d_v;
  a.o_st = Hq * d_v; a.o_sh = d_v;
  a.lse_tq = total_q;
  a.total_rows = total_q;
  a.Sq = (int)Sq; a.Skv = (int)Skv;
  a.B = (int)B; a.Hq = (int)Hq; a.Hkv = (int)Hkv; a.group = (int)(Hq / Hkv);
  a.qk_scale = m.scale;
  a.causal = (m.flags & FA_CAUSAL) ? 1 : 0;
  a.win_left = (m.flags & FA_WINDOW) ? clamp_i32(m.wl) : -1;
  a.win_right = (m.flags & FA_WINDOW) ? clamp_i32(m.wr) : -1;
  bool supported = false;
  hipError_t e = fa::bwd_dispatch(a, (int)d_qk, (int)max_sq, (int)max_sk, (hipStream_t)stream, &supported);
  if (!supported) return fail(FA_ERR_UNSUPPORTED, "no backward kernel for d=%lld", (long long)d_qk);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "backward launch failed: %s", hipGetErrorString(e));
  return FA_OK;
}

}  // namespace

extern "C" {

int fa_bwd_dense(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                 void* dq, void* dk, void* dv, int64_t B, int64_t Sq, int64_t Skv, int64_t Hq, int64_t Hkv,
                 int64_t d_qk, int64_t d_v, const fa_mods* mods, void* workspace, size_t workspace_bytes,
                 void* stream) {
  g_err.clear();
  if (B < 0 || Sq < 0 || Skv < 0) return fail(FA_ERR_INVALID, "sizes must be >= 0");
  if (Sq >= kI32 || Skv >= kI32 || B * Sq >= kI32 || B * Skv >= kI32)
    return fail(FA_ERR_LIMIT, "token counts must stay below 2^31");
  return bwd_impl(q, k, v, o, dout, lse, dq, dk, dv, nullptr, nullptr, B, Sq, Skv, B * Sq, B * Skv, Sq, Skv, Hq, Hkv,
                  d_qk, d_v, mods, workspace, workspace_bytes, stream);
}

int fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                  void* dq, void* dk, void* dv, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                  int64_t B, int64_t total_q, int64_t total_k, int64_t max_seqlen_q, int64_t max_seqlen_k,
                  int64_t Hq, int64_t Hkv, int64_t d_qk, int64_t d_v, const fa_mods* mods,
                  void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  if (!cu_seqlens_q || !cu_seqlens_k) {
    if (B > 0 && (total_q > 0 || total_k > 0)) return fail(FA_ERR_INVALID, "cu_seqlens must be non-NULL");
  }
  return bwd_impl(q, k, v, o, dout, lse, dq, dk, dv, cu_seqlens_q, cu_seqlens_k, B, 0, 0, total_q, total_k,
                  max_seqlen_q, max_seqlen_k, Hq, Hkv, d_qk, d_v, mods, workspace, workspace_bytes, stream);
}

}  // extern "C"
