// Parameters shared by the host dispatcher and the gfx950 kernels.
#pragma once
#include <stdint.h>

namespace fa {

// One forward launch: contiguous (fa_fwd, fa_fwd_split), packed variable-length
// (fa_fwd_varlen) or paged + split (fa_fwd_splitkv, fa_fwd_splitkv_seqlens).
struct FwdParams {
  const void* q;            // [B, Nq, H, D], or packed [total_q, H, D]
  const void* k;            // contiguous [B, Nk, H, D], packed [total_k, H, D] or page pool [P, ps, H, D]
  const void* v;
  void* o;                  // like q (o_bf16 selects bf16 vs fp32)
  float* lse;               // [B, H, Nq], packed [H, total_q], or nullptr
  float* o_part;            // [S, B, H, Nq, D] (split launches)
  float* lse_part;          // [S, B, H, Nq]
  const int* block_table;   // [B, max_pages] (paged launches)
  const float* alibi;       // [H] ALiBi slopes (natural-log units); nullptr = off
  const int* cu_seqlens_q;  // [B + 1] packed batch offsets, or nullptr (batched layout)
  const int* cu_seqlens_k;  // [B + 1]
  const int* seqlens_k;     // [B] per-sequence key counts of a batched layout, or nullptr
  int appended;             // rows already appended behind every seqlens_k count (the
                            //   pass after a separate append): key counts seqlens_k + appended
  const void* k_new;        // [B, Nq, H, D] keys appended to the paged cache before attending
  const void* v_new;        //   (fa_fwd_splitkv_append), or nullptr
  int B, H;
  int Nq, Nk;               // query rows and keys per sequence (packed: the maxima)
  int total_q, total_k;     // rows of the packed tensors
  int max_pages, page_size;
  int page_shift;           // log2(page_size) when it is a power of two, else -1
  int row_stride;           // H * D: elements between consecutive keys of one page
  int64_t page_stride;      // page_size * H * D: elements per page
  int num_splits;
  int split_align;          // split chunks are whole multiples of this many keys
  int num_q_tiles;          // query tiles of the longest sequence
  int window_left;          // -1 = unbounded
  int window_right;         // -1 = unbounded; causal arrives here as 0
  int o_bf16;
  float scale_log2;         // softmax_scale * log2(e)
  float softcap_log2;       // softcap * log2(e) (softcap launches)
  float scale_over_cap2;    // 2 * softmax_scale / softcap * log2(e)  (tanh via exp2)
  float v_descale;          // fp8 launches: the value of V's code 1.0
};

struct CombineParams {
  const float* o_part;
  const float* lse_part;
  void* o;
  float* lse;
  int S, B, H, Nq;
  int o_bf16;
};

// One backward launch (fa_bwd, fa_bwd_varlen): gradients of the forward over a
// batched or a packed variable-length layout.
struct BwdParams {
  const void* q;            // [B, Nq, H, D] bf16, or packed [total_q, H, D]
  const void* k;            // [B, Nk, H, D] bf16, or packed [total_k, H, D]
  const void* v;
  const void* o;            // like q, fp32 or bf16 (o_bf16): the forward's output
  const void* dout;         // like q, bf16
  const float* lse;         // [B, H, Nq] or packed [H, total_q]: the forward's log-sum-exp
  void* dq;                 // [B, Nq, H, D], fp32 or bf16 (g_bf16)
  void* dk;                 // [B, Nk, H, D]
  void* dv;
  float* rowterms;          // workspace [B, H, nblk, 64]: per block of 32 query rows, LSE*log2(e)
                            // (32, +inf for a row with no key or past Nq) then D = rowsum(dO*O)
                            // (32, 0 past Nq)
  int nblk;                 // ceil(Nq / 32)
  const float* alibi;       // [H] or nullptr
  const int* cu_seqlens_q;  // [B + 1] packed batch offsets (fa_bwd_varlen), or nullptr
  const int* cu_seqlens_k;  // [B + 1]
  int B, H, Nq, Nk;         // packed: Nq, Nk are the maxima
  int total_q, total_k;     // rows of the packed tensors
  int window_left, window_right;
  int o_bf16, g_bf16;
  int num_q_tiles, num_k_tiles;
  float scale;              // softmax_scale
  float scale_log2;         // softmax_scale * log2(e)
  float softcap_log2;       // softcap * log2(e)
  float scale_over_cap2;    // 2 * softmax_scale / softcap * log2(e)
};

// Modes of the bf16 tiled forward.
enum FwdMode {
  FWD_CONTIG = 0,        // contiguous K/V, whole key range -> O, LSE
  FWD_CONTIG_SPLIT = 1,  // contiguous K/V, one key split per workgroup -> o_part, lse_part
  FWD_PAGED_SPLIT = 2,   // paged K/V through the block table, per split -> o_part, lse_part
                         //   (rows gathered one by one: any page size, appended keys in
                         //   the bf16 forward)
  FWD_PAGED_TILES = 3,   // the same with page_size a multiple of 16 and no append:
                         //   each wavefront's 16-row slab of a 64-key tile from one
                         //   page (FP8 forward: a multiple of 128, its key tile)
};

// Launchers (defined in the .hip files). Return hipError_t as int.
template <int D, bool SOFTCAP, bool ALIBI, int MODE>
int launch_fwd_bf16(const FwdParams& p, void* stream);
template <int D, bool SOFTCAP, bool ALIBI, bool PAGED>
int launch_fwd_f32(const FwdParams& p, void* stream);
template <int D, bool SOFTCAP, bool ALIBI, int MODE>
int launch_fwd_fp8(const FwdParams& p, void* stream);  // head_dim 64 or 128; any mode
template <int D, bool SOFTCAP, bool ALIBI, bool APPEND>
int launch_decode_bf16(const FwdParams& p, void* stream);
template <int D>
int launch_append_bf16(const FwdParams& p, void* stream);  // k_new/v_new rows into their pages
template <int D, bool SOFTCAP, bool ALIBI>
int launch_decode_fp8(const FwdParams& p, void* stream);  // E4M3 paged cache, one query row
template <int D>
int launch_combine(const CombineParams& p, void* stream);
template <int D, bool SOFTCAP, bool ALIBI>
int launch_bwd_bf16(const BwdParams& p, void* stream);  // preprocess, dK/dV, dQ

// Tile geometry the host needs for grid sizing.
constexpr int BF16_BM = 128;
// fa_fwd_split chunks are multiples of the key tile width.
constexpr int SPLIT_ALIGN = 64;
constexpr int F32_BM = 32;
constexpr int FP8_BM = 128;
constexpr int FP8_SPLIT_ALIGN = 128;  // key tile of the FP8 forward: fa_fwd_split_fp8 chunks are multiples
// Backward tiles: keys per dK/dV workgroup, query rows per dQ workgroup, and
// the query-row block of the row-term workspace.
constexpr int BWD_BK = 128;
constexpr int BWD_BM = 128;
constexpr int BWD_RB = 32;

}  // namespace fa
