// C ABI of libfa: argument validation (host only, before any HIP call) and
// dispatch to the gfx950 kernel instantiations. See include/fa.h for the
// contract of each entry point.
#include "fa.h"

#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>

#include "fa_params.h"
#include "fa_noalloc.h"

static_assert(fa::NOALLOC_SCRATCH_BYTES == FA_NOALLOC_SCRATCH_BYTES,
              "the header states the static buffer's size");

namespace {

constexpr int kMaxSeq = 1 << 28;
constexpr int64_t kMaxGroups = (int64_t(1) << 31) - 1;

using Launcher = int (*)(const fa::FwdParams&, void*);

template <int MODE>
Launcher pick_bf16(int head_dim, bool softcap, bool alibi) {
#define FA_PICK(D)                                                      \
  if (softcap && alibi) return &fa::launch_fwd_bf16<D, true, true, MODE>; \
  if (softcap) return &fa::launch_fwd_bf16<D, true, false, MODE>;        \
  if (alibi) return &fa::launch_fwd_bf16<D, false, true, MODE>;          \
  return &fa::launch_fwd_bf16<D, false, false, MODE>;
  if (head_dim == 64) { FA_PICK(64) }
  FA_PICK(128)
#undef FA_PICK
}

template <bool PAGED>
Launcher pick_f32(int head_dim, bool softcap, bool alibi) {
#define FA_PICK(D)                                                       \
  if (softcap && alibi) return &fa::launch_fwd_f32<D, true, true, PAGED>;  \
  if (softcap) return &fa::launch_fwd_f32<D, true, false, PAGED>;         \
  if (alibi) return &fa::launch_fwd_f32<D, false, true, PAGED>;           \
  return &fa::launch_fwd_f32<D, false, false, PAGED>;
  if (head_dim == 64) { FA_PICK(64) }
  FA_PICK(128)
#undef FA_PICK
}

// One query row per (batch, head) over an E4M3 cache.
Launcher pick_decode_fp8(int head_dim, bool softcap, bool alibi) {
#define FA_PICK_DEC8(D)                                                 \
  if (softcap && alibi) return &fa::launch_decode_fp8<D, true, true>;   \
  if (softcap) return &fa::launch_decode_fp8<D, true, false>;           \
  if (alibi) return &fa::launch_decode_fp8<D, false, true>;             \
  return &fa::launch_decode_fp8<D, false, false>;
  if (head_dim == 64) { FA_PICK_DEC8(64) }
  FA_PICK_DEC8(128)
#undef FA_PICK_DEC8
}

// One query row per (batch, head): the split pass streams the cache with the
// dedicated decode kernel.
template <bool APPEND>
Launcher pick_decode(int head_dim, bool softcap, bool alibi) {
#define FA_PICK_DEC(D)                                                          \
  if (softcap && alibi) return &fa::launch_decode_bf16<D, true, true, APPEND>;  \
  if (softcap) return &fa::launch_decode_bf16<D, true, false, APPEND>;          \
  if (alibi) return &fa::launch_decode_bf16<D, false, true, APPEND>;            \
  return &fa::launch_decode_bf16<D, false, false, APPEND>;
  if (head_dim == 64) { FA_PICK_DEC(64) }
  FA_PICK_DEC(128)
#undef FA_PICK_DEC
}

int check_sizes(int batch, int heads, int seqlen_q, int seqlen_k) {
  if (batch <= 0 || heads <= 0 || seqlen_q <= 0 || seqlen_k <= 0) return FA_ERR_SHAPE;
  if (seqlen_q > kMaxSeq || seqlen_k > kMaxSeq || heads > (1 << 16) || batch > (1 << 24))
    return FA_ERR_SHAPE;
  return FA_OK;
}

int check_kind(int in_dtype, int head_dim) {
  if (in_dtype != FA_FP32 && in_dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

int check_mask_and_values(int causal, int window_left, int window_right, float scale,
                          float softcap) {
  if (window_left < -1 || window_right < -1) return FA_ERR_MASK;
  if (causal && window_right > 0) return FA_ERR_MASK;
  if (!(scale > 0.0f) || !isfinite(scale)) return FA_ERR_VALUE;
  if (!(softcap >= 0.0f) || !isfinite(softcap)) return FA_ERR_VALUE;
  return FA_OK;
}

// Fill the fields common to both forward entry points. A window wider than
// both sequences is no constraint, so it is folded to -1 (keeps index
// arithmetic inside 32 bits); causal is the right window 0.
void fill_common(fa::FwdParams& p, int batch, int heads, int seqlen_q, int seqlen_k,
                 float scale, int causal, int window_left, int window_right,
                 const float* alibi_slopes, float softcap, int tile_rows) {
  p.B = batch;
  p.H = heads;
  p.Nq = seqlen_q;
  p.Nk = seqlen_k;
  const int span = seqlen_q + seqlen_k;
  p.window_left = window_left > span ? -1 : window_left;
  int wr = window_right > span ? -1 : window_right;
  if (causal) wr = 0;
  p.window_right = wr;
  p.alibi = alibi_slopes;
  const float log2e = 1.4426950408889634f;
  p.scale_log2 = scale * log2e;
  p.softcap_log2 = softcap * log2e;
  p.scale_over_cap2 = softcap > 0.0f ? 2.0f * scale / softcap * log2e : 0.0f;
  p.num_q_tiles = (seqlen_q + tile_rows - 1) / tile_rows;
}

int64_t split_len(int seqlen_k, int num_splits, int page_size) {
  int64_t c = (seqlen_k + (int64_t)num_splits - 1) / num_splits;
  return (c + page_size - 1) / page_size * page_size;
}

// fa_fwd_splitkv, fa_fwd_splitkv_seqlens and fa_fwd_splitkv_append
// (seqlens_k = nullptr: every sequence holds seqlen_k keys; k_new = nullptr: no
// append).
// fp8_cache: k_cache / v_cache hold E4M3 codes valued k_descale / v_descale
// times their decoded value (bf16 queries, one query row).
int splitkv(const void* q, const void* k_cache, const void* v_cache, const void* k_new,
            const void* v_new, int in_dtype, const int* block_table, int max_pages_per_seq,
            int page_size, const int* seqlens_k,
            float* o_part, float* lse_part, int num_splits, int batch, int heads, int seqlen_q,
            int seqlen_k, int head_dim, float softmax_scale, int causal, int window_left,
            int window_right, const float* alibi_slopes, float softcap, void* stream,
            bool fp8_cache = false, float k_descale = 1.0f, float v_descale = 1.0f) {
  if (!q || !k_cache || !v_cache || !block_table || !o_part || !lse_part) return FA_ERR_NULL;
  int st = check_sizes(batch, heads, seqlen_q, seqlen_k);
  if (st) return st;
  if (num_splits <= 0 || num_splits > (1 << 16) || max_pages_per_seq <= 0 || page_size <= 0)
    return FA_ERR_SHAPE;
  if ((int64_t)max_pages_per_seq * page_size < seqlen_k) return FA_ERR_SHAPE;
  if ((int64_t)page_size * heads * head_dim >= (int64_t(1) << 31)) return FA_ERR_SHAPE;
  if ((st = check_kind(in_dtype, head_dim))) return st;
  if ((st = check_mask_and_values(causal, window_left, window_right, softmax_scale, softcap)))
    return st;
  if (fp8_cache) {
    if (in_dtype != FA_BF16 || seqlen_q != 1 || k_new) return FA_ERR_UNSUPPORTED;
    for (float d : {k_descale, v_descale})
      if (!(d > 0.0f) || !isfinite(d)) return FA_ERR_VALUE;
    // K's descale scales every score, so it joins softmax_scale.
    softmax_scale *= k_descale;
    if (!(softmax_scale > 0.0f) || !isfinite(softmax_scale)) return FA_ERR_VALUE;
  }

  fa::FwdParams p = {};
  p.q = q;
  p.k = k_cache;
  p.v = v_cache;
  p.v_descale = v_descale;
  p.o_part = o_part;
  p.lse_part = lse_part;
  p.block_table = block_table;
  p.max_pages = max_pages_per_seq;
  p.page_size = page_size;
  p.page_shift = -1;
  if ((page_size & (page_size - 1)) == 0)
    for (int sh = 0; sh < 31; ++sh)
      if ((1 << sh) == page_size) p.page_shift = sh;
  p.num_splits = num_splits;
  p.row_stride = heads * head_dim;
  p.page_stride = (int64_t)page_size * heads * head_dim;
  p.seqlens_k = seqlens_k;
  p.k_new = k_new;
  p.v_new = v_new;
  const int tile = in_dtype == FA_BF16 ? fa::BF16_BM : fa::F32_BM;
  fill_common(p, batch, heads, seqlen_q, seqlen_k, softmax_scale, causal, window_left,
              window_right, alibi_slopes, softcap, tile);
  if (split_len(seqlen_k, num_splits, page_size) > kMaxSeq) return FA_ERR_SHAPE;
  p.split_align = page_size;
  if ((int64_t)p.num_q_tiles * heads * batch * num_splits > kMaxGroups) return FA_ERR_SHAPE;

  const bool sc = softcap > 0.0f, al = alibi_slopes != nullptr;
  if (k_new && in_dtype == FA_BF16 && seqlen_q != 1 && page_size % 16 == 0) {
    // Several appended rows: the append runs as a launch of its own, then the
    // split pass reads every key from the cache in page slabs (the fused form
    // would gather the rows one by one).
    const int head = head_dim == 64 ? fa::launch_append_bf16<64>(p, stream)
                                    : fa::launch_append_bf16<128>(p, stream);
    if (head) return FA_ERR_HIP;
    fa::FwdParams q2 = p;
    q2.k_new = q2.v_new = nullptr;
    q2.appended = seqlen_q;
    return pick_bf16<fa::FWD_PAGED_TILES>(head_dim, sc, al)(q2, stream) ? FA_ERR_HIP : FA_OK;
  }
  Launcher fn = fp8_cache             ? pick_decode_fp8(head_dim, sc, al)
                : in_dtype != FA_BF16 ? pick_f32<true>(head_dim, sc, al)
                : seqlen_q != 1 && !k_new && page_size % 16 == 0
                    ? pick_bf16<fa::FWD_PAGED_TILES>(head_dim, sc, al)
                : seqlen_q != 1       ? pick_bf16<fa::FWD_PAGED_SPLIT>(head_dim, sc, al)
                : k_new               ? pick_decode<true>(head_dim, sc, al)
                                      : pick_decode<false>(head_dim, sc, al);
  return fn(p, stream) ? FA_ERR_HIP : FA_OK;
}

// fa_bwd and fa_bwd_varlen (cu_seqlens_q = nullptr: the batched layout; seqlen_q,
// seqlen_k are then the lengths, else the maxima). Sizes are checked by the callers.
int bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
        const float* lse, int in_dtype, int o_dtype, void* dq, void* dk, void* dv, int grad_dtype,
        float* workspace, const int* cu_seqlens_q, const int* cu_seqlens_k, int batch, int heads,
        int total_q, int total_k, int seqlen_q, int seqlen_k, int head_dim, float softmax_scale,
        int causal, int window_left, int window_right, const float* alibi_slopes, float softcap,
        void* stream, bool noalloc = false) {
  int st = check_kind(in_dtype, head_dim);
  if (st) return st;
  if (in_dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (o_dtype != FA_FP32 && o_dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (grad_dtype != FA_FP32 && grad_dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if ((st = check_mask_and_values(causal, window_left, window_right, softmax_scale, softcap)))
    return st;
  if (cu_seqlens_q && total_q == 0 && total_k == 0) return FA_OK;  // an empty pack

  // Reuse the forward's mask folding (a window wider than both sequences is no
  // constraint; causal is the right window 0).
  fa::FwdParams f = {};
  fill_common(f, batch, heads, seqlen_q, seqlen_k, softmax_scale, causal, window_left,
              window_right, alibi_slopes, softcap, fa::BWD_BM);
  fa::BwdParams p = {};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.dout = dout;
  p.lse = lse;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.rowterms = workspace;
  p.nblk = (seqlen_q + fa::BWD_RB - 1) / fa::BWD_RB;
  p.alibi = alibi_slopes;
  p.cu_seqlens_q = cu_seqlens_q;
  p.cu_seqlens_k = cu_seqlens_k;
  p.total_q = total_q;
  p.total_k = total_k;
  p.B = batch;
  p.H = heads;
  p.Nq = seqlen_q;
  p.Nk = seqlen_k;
  p.window_left = f.window_left;
  p.window_right = f.window_right;
  p.o_bf16 = o_dtype == FA_BF16;
  p.g_bf16 = grad_dtype == FA_BF16;
  p.num_q_tiles = (seqlen_q + fa::BWD_BM - 1) / fa::BWD_BM;
  p.num_k_tiles = (seqlen_k + fa::BWD_BK - 1) / fa::BWD_BK;
  p.scale = softmax_scale;
  p.scale_log2 = f.scale_log2;
  p.softcap_log2 = f.softcap_log2;
  p.scale_over_cap2 = f.scale_over_cap2;
  // (dK/dV and dQ share one grid at head_dim 128: two key-tile workgroups per
  // BWD_BK keys, then the query tiles.)
  if ((2 * (int64_t)p.num_k_tiles + p.num_q_tiles) * heads * batch > kMaxGroups ||
      (int64_t)p.nblk * fa::BWD_RB * heads * batch / 8 > kMaxGroups)
    return FA_ERR_SHAPE;
  // Everything is validated: only now the static buffer's address (a HIP call).
  if (noalloc && fa::noalloc_scratch(&p.rowterms)) return FA_ERR_HIP;

  const bool sc = softcap > 0.0f, al = alibi_slopes != nullptr;
  int rc;
#define FA_BWD(D)                                                       \
  if (sc && al) rc = fa::launch_bwd_bf16<D, true, true>(p, stream);     \
  else if (sc) rc = fa::launch_bwd_bf16<D, true, false>(p, stream);     \
  else if (al) rc = fa::launch_bwd_bf16<D, false, true>(p, stream);     \
  else rc = fa::launch_bwd_bf16<D, false, false>(p, stream);
  if (head_dim == 64) {
    FA_BWD(64)
  } else {
    FA_BWD(128)
  }
#undef FA_BWD
  return rc ? FA_ERR_HIP : FA_OK;
}

}  // namespace

extern "C" {

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE:
      return "bad sizes: every size must be >= 1, seqlens <= 2^28, heads <= 2^16, "
             "batch <= 2^24, the launch below 2^31 workgroups, "
             "max_pages_per_seq * page_size >= seqlen_k, and page_size * heads * head_dim < 2^31";
    case FA_ERR_UNSUPPORTED: return "unsupported dtype or head_dim (head_dim 64 or 128; FP32 or BF16)";
    case FA_ERR_MASK: return "bad mask: windows must be >= -1 and causal needs window_right <= 0";
    case FA_ERR_HIP: return "the HIP runtime rejected a kernel launch";
    case FA_ERR_VALUE: return "bad value: softmax_scale must be finite and > 0, softcap finite and >= 0";
    case FA_ERR_SCRATCH:
      return "the problem needs more than the allocation-free backward's static buffer: "
             "fa_bwd_workspace_bytes(batch, heads, seqlen_q) must be <= FA_NOALLOC_SCRATCH_BYTES "
             "(16 MiB per GPU); call fa_bwd with a workspace instead";
    default: return "unknown status";
  }
}

int fa_split_chunk_len(int seqlen_k, int num_splits, int page_size) {
  if (seqlen_k <= 0 || num_splits <= 0 || page_size <= 0) return -1;
  const int64_t c = split_len(seqlen_k, num_splits, page_size);
  return c > kMaxSeq ? -1 : (int)c;
}

int fa_num_splits(int batch, int heads, int seqlen_q, int seqlen_k, int head_dim, int page_size,
                  int fp8_cache, int num_cus) {
  if (batch <= 0 || heads <= 0 || seqlen_q <= 0 || seqlen_k <= 0 || page_size <= 0) return -1;
  if (head_dim != 64 && head_dim != 128) return -1;
  if (num_cus <= 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&num_cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        num_cus <= 0)
      return -1;
  }
  int64_t per_split, target;
  if (seqlen_q == 1) {
    // The decode kernel: one workgroup per (head group, batch, split); a head
    // group is the heads whose rows of one key make 256 bytes, twice that at
    // head_dim 128 on launches large enough for wide groups. Two workgroups per
    // compute unit, counted at the wide size, was the best split count on every
    // decode shape measured (one per unit left the E4M3 cache up to 17% slower).
    const int row_bytes = head_dim * (fp8_cache ? 1 : 2);
    const int g = (row_bytes >= 256 ? 1 : 256 / row_bytes) * (head_dim == 128 ? 2 : 1);
    per_split = (int64_t)batch * ((heads + g - 1) / g);
    target = 2 * (int64_t)num_cus;
  } else {
    // The tiled kernel: one workgroup per (128-row query tile, head, batch,
    // split), two resident per compute unit.
    per_split = (int64_t)batch * heads * ((seqlen_q + fa::BF16_BM - 1) / fa::BF16_BM);
    target = 2 * (int64_t)num_cus;
  }
  const int64_t chunks = (seqlen_k + (int64_t)page_size - 1) / page_size;
  const int64_t s = std::min<int64_t>({(target + per_split - 1) / per_split, chunks, 64});
  return (int)std::max<int64_t>(s, 1);
}

int fa_fwd(const void* q, const void* k, const void* v, int in_dtype, void* o, int o_dtype,
           float* lse, int batch, int heads, int seqlen_q, int seqlen_k, int head_dim,
           float softmax_scale, int causal, int window_left, int window_right,
           const float* alibi_slopes, float softcap, void* stream) {
  if (!q || !k || !v || !o) return FA_ERR_NULL;
  int st = check_sizes(batch, heads, seqlen_q, seqlen_k);
  if (st) return st;
  if ((st = check_kind(in_dtype, head_dim))) return st;
  if (o_dtype != FA_FP32 && o_dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if ((st = check_mask_and_values(causal, window_left, window_right, softmax_scale, softcap)))
    return st;

  fa::FwdParams p = {};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.o_bf16 = o_dtype == FA_BF16;
  p.num_splits = 1;
  const int tile = in_dtype == FA_BF16 ? fa::BF16_BM : fa::F32_BM;
  fill_common(p, batch, heads, seqlen_q, seqlen_k, softmax_scale, causal, window_left,
              window_right, alibi_slopes, softcap, tile);
  if ((int64_t)p.num_q_tiles * heads * batch > kMaxGroups) return FA_ERR_SHAPE;

  const bool sc = softcap > 0.0f, al = alibi_slopes != nullptr;
  Launcher fn = in_dtype == FA_BF16 ? pick_bf16<fa::FWD_CONTIG>(head_dim, sc, al)
                                    : pick_f32<false>(head_dim, sc, al);
  return fn(p, stream) ? FA_ERR_HIP : FA_OK;
}

int fa_fwd_split(const void* q, const void* k, const void* v, int in_dtype, float* o_part,
                 float* lse_part, int num_splits, int batch, int heads, int seqlen_q,
                 int seqlen_k, int head_dim, float softmax_scale, int causal, int window_left,
                 int window_right, const float* alibi_slopes, float softcap, void* stream) {
  if (!q || !k || !v || !o_part || !lse_part) return FA_ERR_NULL;
  int st = check_sizes(batch, heads, seqlen_q, seqlen_k);
  if (st) return st;
  if (num_splits <= 0 || num_splits > (1 << 16)) return FA_ERR_SHAPE;
  if ((st = check_kind(in_dtype, head_dim))) return st;
  if (in_dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if ((st = check_mask_and_values(causal, window_left, window_right, softmax_scale, softcap)))
    return st;

  fa::FwdParams p = {};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o_part = o_part;
  p.lse_part = lse_part;
  p.num_splits = num_splits;
  fill_common(p, batch, heads, seqlen_q, seqlen_k, softmax_scale, causal, window_left,
              window_right, alibi_slopes, softcap, fa::BF16_BM);
  if (split_len(seqlen_k, num_splits, fa::SPLIT_ALIGN) > kMaxSeq) return FA_ERR_SHAPE;
  p.split_align = fa::SPLIT_ALIGN;
  if ((int64_t)p.num_q_tiles * heads * batch * num_splits > kMaxGroups) return FA_ERR_SHAPE;

  Launcher fn = pick_bf16<fa::FWD_CONTIG_SPLIT>(head_dim, softcap > 0.0f, alibi_slopes != nullptr);
  return fn(p, stream) ? FA_ERR_HIP : FA_OK;
}

int fa_fwd_splitkv(const void* q, const void* k_cache, const void* v_cache, int in_dtype,
                   const int* block_table, int max_pages_per_seq, int page_size,
                   float* o_part, float* lse_part, int num_splits, int batch, int heads,
                   int seqlen_q, int seqlen_k, int head_dim, float softmax_scale, int causal,
                   int window_left, int window_right, const float* alibi_slopes, float softcap,
                   void* stream) {
  return splitkv(q, k_cache, v_cache, nullptr, nullptr, in_dtype, block_table,
                 max_pages_per_seq, page_size, nullptr, o_part, lse_part, num_splits, batch,
                 heads, seqlen_q, seqlen_k, head_dim, softmax_scale, causal, window_left,
                 window_right, alibi_slopes,
                 softcap, stream);
}

int fa_fwd_splitkv_fp8(const void* q, const void* k_cache, const void* v_cache,
                       float k_descale, float v_descale, const int* block_table,
                       int max_pages_per_seq, int page_size, const int* cache_seqlens,
                       float* o_part, float* lse_part, int num_splits, int batch, int heads,
                       int seqlen_q, int seqlen_k, int head_dim, float softmax_scale, int causal,
                       int window_left, int window_right, const float* alibi_slopes,
                       float softcap, void* stream) {
  return splitkv(q, k_cache, v_cache, nullptr, nullptr, FA_BF16, block_table, max_pages_per_seq,
                 page_size, cache_seqlens, o_part, lse_part, num_splits, batch, heads, seqlen_q,
                 seqlen_k, head_dim, softmax_scale, causal, window_left, window_right,
                 alibi_slopes, softcap, stream, true, k_descale, v_descale);
}

int fa_fwd_splitkv_seqlens(const void* q, const void* k_cache, const void* v_cache, int in_dtype,
                           const int* block_table, int max_pages_per_seq, int page_size,
                           const int* cache_seqlens, float* o_part, float* lse_part,
                           int num_splits, int batch, int heads, int seqlen_q, int max_seqlen_k,
                           int head_dim, float softmax_scale, int causal, int window_left,
                           int window_right, const float* alibi_slopes, float softcap,
                           void* stream) {
  if (!cache_seqlens) return FA_ERR_NULL;
  return splitkv(q, k_cache, v_cache, nullptr, nullptr, in_dtype, block_table,
                 max_pages_per_seq, page_size, cache_seqlens, o_part, lse_part, num_splits,
                 batch, heads, seqlen_q, max_seqlen_k, head_dim, softmax_scale, causal,
                 window_left, window_right, alibi_slopes, softcap, stream);
}

int fa_fwd_splitkv_append(const void* q, const void* k_new, const void* v_new, void* k_cache,
                          void* v_cache, int in_dtype, const int* block_table,
                          int max_pages_per_seq, int page_size, const int* cache_seqlens,
                          float* o_part, float* lse_part, int num_splits, int batch, int heads,
                          int seqlen_q, int max_seqlen_k, int head_dim, float softmax_scale,
                          int causal, int window_left, int window_right,
                          const float* alibi_slopes, float softcap, void* stream) {
  if (!cache_seqlens || !k_new || !v_new) return FA_ERR_NULL;
  if (seqlen_q > 0 && max_seqlen_k < seqlen_q) return FA_ERR_SHAPE;
  return splitkv(q, k_cache, v_cache, k_new, v_new, in_dtype, block_table, max_pages_per_seq,
                 page_size, cache_seqlens, o_part, lse_part, num_splits, batch, heads, seqlen_q,
                 max_seqlen_k, head_dim, softmax_scale, causal, window_left, window_right,
                 alibi_slopes, softcap, stream);
}

int fa_fwd_varlen(const void* q, const void* k, const void* v, int in_dtype, void* o,
                  int o_dtype, float* lse, const int* cu_seqlens_q, const int* cu_seqlens_k,
                  int batch, int heads, int total_q, int total_k, int max_seqlen_q,
                  int max_seqlen_k, int head_dim, float softmax_scale, int causal,
                  int window_left, int window_right, const float* alibi_slopes, float softcap,
                  void* stream) {
  if (!cu_seqlens_q || !cu_seqlens_k) return FA_ERR_NULL;
  if ((total_q > 0 && (!q || !o)) || (total_k > 0 && (!k || !v))) return FA_ERR_NULL;
  if (batch <= 0 || batch > (1 << 24) || heads <= 0 || heads > (1 << 16)) return FA_ERR_SHAPE;
  if (total_q < 0 || total_k < 0 || max_seqlen_q <= 0 || max_seqlen_k < 0) return FA_ERR_SHAPE;
  if (max_seqlen_q > kMaxSeq || max_seqlen_k > kMaxSeq) return FA_ERR_SHAPE;
  int st = check_kind(in_dtype, head_dim);
  if (st) return st;
  if (o_dtype != FA_FP32 && o_dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if ((st = check_mask_and_values(causal, window_left, window_right, softmax_scale, softcap)))
    return st;
  if (total_q == 0) return FA_OK;  // no query row: nothing to compute

  fa::FwdParams p = {};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.o_bf16 = o_dtype == FA_BF16;
  p.num_splits = 1;
  p.cu_seqlens_q = cu_seqlens_q;
  p.cu_seqlens_k = cu_seqlens_k;
  p.total_q = total_q;
  p.total_k = total_k;
  const int tile = in_dtype == FA_BF16 ? fa::BF16_BM : fa::F32_BM;
  fill_common(p, batch, heads, max_seqlen_q, max_seqlen_k, softmax_scale, causal, window_left,
              window_right, alibi_slopes, softcap, tile);
  if ((int64_t)p.num_q_tiles * heads * batch > kMaxGroups) return FA_ERR_SHAPE;

  const bool sc = softcap > 0.0f, al = alibi_slopes != nullptr;
  Launcher fn = in_dtype == FA_BF16 ? pick_bf16<fa::FWD_CONTIG>(head_dim, sc, al)
                                    : pick_f32<false>(head_dim, sc, al);
  return fn(p, stream) ? FA_ERR_HIP : FA_OK;
}

namespace {
// The FP8 forward instantiation for head_dim, score transforms and mode
// (fa::FWD_CONTIG, fa::FWD_CONTIG_SPLIT, fa::FWD_PAGED_TILES or fa::FWD_PAGED_SPLIT).
int launch_fp8(const fa::FwdParams& p, int head_dim, bool sc, bool al, int mode, void* stream) {
#define FA_FP8(D, M)                                              \
  (sc && al ? fa::launch_fwd_fp8<D, true, true, M>(p, stream)     \
   : sc     ? fa::launch_fwd_fp8<D, true, false, M>(p, stream)    \
   : al     ? fa::launch_fwd_fp8<D, false, true, M>(p, stream)    \
            : fa::launch_fwd_fp8<D, false, false, M>(p, stream))
#define FA_FP8_D(D)                                                    \
  (mode == fa::FWD_CONTIG         ? FA_FP8(D, fa::FWD_CONTIG)          \
   : mode == fa::FWD_CONTIG_SPLIT ? FA_FP8(D, fa::FWD_CONTIG_SPLIT)    \
   : mode == fa::FWD_PAGED_TILES  ? FA_FP8(D, fa::FWD_PAGED_TILES)     \
                                  : FA_FP8(D, fa::FWD_PAGED_SPLIT))
  const int rc = head_dim == 64 ? FA_FP8_D(64) : FA_FP8_D(128);
#undef FA_FP8_D
#undef FA_FP8
  return rc ? FA_ERR_HIP : FA_OK;
}
}  // namespace

int fa_fwd_fp8(const void* q, const void* k, const void* v, float q_descale, float k_descale,
               float v_descale, void* o, int o_dtype, float* lse, int batch, int heads,
               int seqlen_q, int seqlen_k, int head_dim, float softmax_scale, int causal,
               int window_left, int window_right, const float* alibi_slopes, float softcap,
               void* stream) {
  if (!q || !k || !v || !o) return FA_ERR_NULL;
  int st = check_sizes(batch, heads, seqlen_q, seqlen_k);
  if (st) return st;
  if (head_dim != 64 && head_dim != 128) return FA_ERR_UNSUPPORTED;
  if (o_dtype != FA_FP32 && o_dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if ((st = check_mask_and_values(causal, window_left, window_right, softmax_scale, softcap)))
    return st;
  for (float d : {q_descale, k_descale, v_descale})
    if (!(d > 0.0f) || !isfinite(d)) return FA_ERR_VALUE;
  const float qk = softmax_scale * q_descale * k_descale;
  if (!(qk > 0.0f) || !isfinite(qk)) return FA_ERR_VALUE;

  fa::FwdParams p = {};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.o_bf16 = o_dtype == FA_BF16;
  p.num_splits = 1;
  p.v_descale = v_descale;
  // The descales of Q and K scale every score, so they join softmax_scale.
  fill_common(p, batch, heads, seqlen_q, seqlen_k, qk, causal, window_left, window_right,
              alibi_slopes, softcap, fa::FP8_BM);
  if ((int64_t)p.num_q_tiles * heads * batch > kMaxGroups) return FA_ERR_SHAPE;
  return launch_fp8(p, head_dim, softcap > 0.0f, alibi_slopes != nullptr, fa::FWD_CONTIG, stream);
}

int fa_fwd_split_fp8(const void* q, const void* k, const void* v, float q_descale,
                     float k_descale, float v_descale, float* o_part, float* lse_part,
                     int num_splits, int batch, int heads, int seqlen_q, int seqlen_k,
                     int head_dim, float softmax_scale, int causal, int window_left,
                     int window_right, const float* alibi_slopes, float softcap, void* stream) {
  if (!q || !k || !v || !o_part || !lse_part) return FA_ERR_NULL;
  int st = check_sizes(batch, heads, seqlen_q, seqlen_k);
  if (st) return st;
  if (num_splits <= 0 || num_splits > (1 << 16)) return FA_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128) return FA_ERR_UNSUPPORTED;
  if ((st = check_mask_and_values(causal, window_left, window_right, softmax_scale, softcap)))
    return st;
  for (float d : {q_descale, k_descale, v_descale})
    if (!(d > 0.0f) || !isfinite(d)) return FA_ERR_VALUE;
  const float qk = softmax_scale * q_descale * k_descale;
  if (!(qk > 0.0f) || !isfinite(qk)) return FA_ERR_VALUE;

  fa::FwdParams p = {};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o_part = o_part;
  p.lse_part = lse_part;
  p.num_splits = num_splits;
  p.v_descale = v_descale;
  fill_common(p, batch, heads, seqlen_q, seqlen_k, qk, causal, window_left, window_right,
              alibi_slopes, softcap, fa::FP8_BM);
  if (split_len(seqlen_k, num_splits, fa::FP8_SPLIT_ALIGN) > kMaxSeq) return FA_ERR_SHAPE;
  p.split_align = fa::FP8_SPLIT_ALIGN;
  if ((int64_t)p.num_q_tiles * heads * batch * num_splits > kMaxGroups) return FA_ERR_SHAPE;
  return launch_fp8(p, head_dim, softcap > 0.0f, alibi_slopes != nullptr, fa::FWD_CONTIG_SPLIT,
                    stream);
}

int fa_fwd_paged_fp8(const void* q, const void* k_cache, const void* v_cache, float q_descale,
                     float k_descale, float v_descale, const int* block_table,
                     int max_pages_per_seq, int page_size, const int* cache_seqlens,
                     float* o_part, float* lse_part, int num_splits, int batch, int heads,
                     int seqlen_q, int seqlen_k, int head_dim, float softmax_scale, int causal,
                     int window_left, int window_right, const float* alibi_slopes, float softcap,
                     void* stream) {
  if (!q || !k_cache || !v_cache || !block_table || !o_part || !lse_part) return FA_ERR_NULL;
  int st = check_sizes(batch, heads, seqlen_q, seqlen_k);
  if (st) return st;
  if (num_splits <= 0 || num_splits > (1 << 16) || max_pages_per_seq <= 0 || page_size <= 0)
    return FA_ERR_SHAPE;
  if ((int64_t)max_pages_per_seq * page_size < seqlen_k) return FA_ERR_SHAPE;
  if ((int64_t)page_size * heads * head_dim >= (int64_t(1) << 31)) return FA_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128) return FA_ERR_UNSUPPORTED;
  if ((st = check_mask_and_values(causal, window_left, window_right, softmax_scale, softcap)))
    return st;
  for (float d : {q_descale, k_descale, v_descale})
    if (!(d > 0.0f) || !isfinite(d)) return FA_ERR_VALUE;
  const float qk = softmax_scale * q_descale * k_descale;
  if (!(qk > 0.0f) || !isfinite(qk)) return FA_ERR_VALUE;

  fa::FwdParams p = {};
  p.q = q;
  p.k = k_cache;
  p.v = v_cache;
  p.o_part = o_part;
  p.lse_part = lse_part;
  p.block_table = block_table;
  p.max_pages = max_pages_per_seq;
  p.page_size = page_size;
  p.page_shift = -1;
  if ((page_size & (page_size - 1)) == 0)
    for (int sh = 0; sh < 31; ++sh)
      if ((1 << sh) == page_size) p.page_shift = sh;
  p.row_stride = heads * head_dim;
  p.page_stride = (int64_t)page_size * heads * head_dim;
  p.seqlens_k = cache_seqlens;
  p.num_splits = num_splits;
  p.v_descale = v_descale;
  fill_common(p, batch, heads, seqlen_q, seqlen_k, qk, causal, window_left, window_right,
              alibi_slopes, softcap, fa::FP8_BM);
  if (split_len(seqlen_k, num_splits, page_size) > kMaxSeq) return FA_ERR_SHAPE;
  p.split_align = page_size;
  if ((int64_t)p.num_q_tiles * heads * batch * num_splits > kMaxGroups) return FA_ERR_SHAPE;
  // Pages of a multiple of 32 keys travel as per-wavefront slabs of the 128-key
  // tiles; other page sizes row by row.
  const int mode = page_size % 32 == 0 ? fa::FWD_PAGED_TILES : fa::FWD_PAGED_SPLIT;
  return launch_fp8(p, head_dim, softcap > 0.0f, alibi_slopes != nullptr, mode, stream);
}

long long fa_bwd_workspace_bytes(int batch, int heads, int seqlen_q) {
  if (batch <= 0 || heads <= 0 || seqlen_q <= 0) return -1;
  const long long nblk = (seqlen_q + fa::BWD_RB - 1) / fa::BWD_RB;
  return 2LL * fa::BWD_RB * nblk * batch * heads * (long long)sizeof(float);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, int in_dtype, int o_dtype, void* dq, void* dk, void* dv,
           int grad_dtype, float* workspace, int batch, int heads, int seqlen_q, int seqlen_k,
           int head_dim, float softmax_scale, int causal, int window_left, int window_right,
           const float* alibi_slopes, float softcap, void* stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !workspace) return FA_ERR_NULL;
  const int st = check_sizes(batch, heads, seqlen_q, seqlen_k);
  if (st) return st;
  return bwd(q, k, v, o, dout, lse, in_dtype, o_dtype, dq, dk, dv, grad_dtype, workspace, nullptr,
             nullptr, batch, heads, 0, 0, seqlen_q, seqlen_k, head_dim, softmax_scale, causal,
             window_left, window_right, alibi_slopes, softcap, stream);
}

int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, int in_dtype, int o_dtype, void* dq, void* dk, void* dv,
                   int grad_dtype, int batch, int heads, int seqlen_q, int seqlen_k,
                   int head_dim, float softmax_scale, int causal, int window_left,
                   int window_right, const float* alibi_slopes, float softcap, void* stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return FA_ERR_NULL;
  const int st = check_sizes(batch, heads, seqlen_q, seqlen_k);
  if (st) return st;
  if (fa_bwd_workspace_bytes(batch, heads, seqlen_q) > fa::NOALLOC_SCRATCH_BYTES)
    return FA_ERR_SCRATCH;
  return bwd(q, k, v, o, dout, lse, in_dtype, o_dtype, dq, dk, dv, grad_dtype, nullptr, nullptr,
             nullptr, batch, heads, 0, 0, seqlen_q, seqlen_k, head_dim, softmax_scale, causal,
             window_left, window_right, alibi_slopes, softcap, stream, /*noalloc=*/true);
}

int fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const void* dout,
                  const float* lse, int in_dtype, int o_dtype, void* dq, void* dk, void* dv,
                  int grad_dtype, float* workspace, const int* cu_seqlens_q,
                  const int* cu_seqlens_k, int batch, int heads, int total_q, int total_k,
                  int max_seqlen_q, int max_seqlen_k, int head_dim, float softmax_scale,
                  int causal, int window_left, int window_right, const float* alibi_slopes,
                  float softcap, void* stream) {
  if (!cu_seqlens_q || !cu_seqlens_k || !workspace) return FA_ERR_NULL;
  if (total_q > 0 && (!q || !o || !dout || !lse || !dq)) return FA_ERR_NULL;
  if (total_k > 0 && (!k || !v || !dk || !dv)) return FA_ERR_NULL;
  if (batch <= 0 || batch > (1 << 24) || heads <= 0 || heads > (1 << 16)) return FA_ERR_SHAPE;
  if (total_q < 0 || total_k < 0 || max_seqlen_q <= 0 || max_seqlen_k < 0) return FA_ERR_SHAPE;
  if (max_seqlen_q > kMaxSeq || max_seqlen_k > kMaxSeq) return FA_ERR_SHAPE;
  return bwd(q, k, v, o, dout, lse, in_dtype, o_dtype, dq, dk, dv, grad_dtype, workspace,
             cu_seqlens_q, cu_seqlens_k, batch, heads, total_q, total_k, max_seqlen_q,
             std::max(max_seqlen_k, 1), head_dim, softmax_scale, causal, window_left, window_right,
             alibi_slopes, softcap, stream);
}

int fa_splitkv_combine(const float* o_part, const float* lse_part, int num_splits, int batch,
                       int heads, int seqlen_q, int head_dim, void* o, int o_dtype, float* lse,
                       void* stream) {
  if (!o_part || !lse_part || !o) return FA_ERR_NULL;
  if (num_splits <= 0 || num_splits > (1 << 16)) return FA_ERR_SHAPE;
  int st = check_sizes(batch, heads, seqlen_q, 1);
  if (st) return st;
  if (head_dim != 64 && head_dim != 128) return FA_ERR_UNSUPPORTED;
  if (o_dtype != FA_FP32 && o_dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (((int64_t)batch * heads * seqlen_q + 3) / 4 > kMaxGroups) return FA_ERR_SHAPE;
  fa::CombineParams p = {};
  p.o_part = o_part;
  p.lse_part = lse_part;
  p.o = o;
  p.lse = lse;
  p.S = num_splits;
  p.B = batch;
  p.H = heads;
  p.Nq = seqlen_q;
  p.o_bf16 = o_dtype == FA_BF16;
  const int rc = head_dim == 64 ? fa::launch_combine<64>(p, stream) : fa::launch_combine<128>(p, stream);
  return rc ? FA_ERR_HIP : FA_OK;
}

}  // extern "C"
