// FP8 (E4M3) tiled attention forward for gfx950 (MI355X), head_dim 64 or 128.
//
// Q, K and V arrive as E4M3 codes with one descale factor per tensor
// (FlashAttention-3's FP8 forward, "IO感知技术革命: FlashAttention如何重塑大模型训练
// 的经济学", the section on H100 and FP8; the deep-analysis page lists FP8
// forward support on its roadmap). The method is the bf16 kernel's: one
// workgroup of 4 wavefronts per 128-row query tile of one (batch, head), each
// wavefront holding 32 query rows, 128-key tiles of K and V staged in LDS by
// copies that write LDS directly, S^T = K Q^T, an online softmax per lane pair
// and O^T += V^T P^T. The products run on the gfx950 FP8 matrix instruction
// v_mfma_scale_f32_32x32x64_f8f6f4 (K = 64 per instruction, unit block
// scales), so a 128-key tile takes 8 MFMAs for S and 8 for the output instead
// of 32 + 32 in bf16 at head_dim 128 (4 + 4 at head_dim 64). The FP8 operands need fewer registers than bf16 ones,
// which leaves room for the 128-key score block (64 fp32 per lane) at two
// wavefronts per SIMD; 64 KB of LDS per workgroup still lets two share a CU.
//
// P: with the exact running maximum the largest probability of a row is 1;
// it is scaled by 2^8 (folded into the exponent) so that the E4M3 grid reaches
// down to 2^-17 of the row maximum, then rounded to E4M3 (nearest even) as the
// operand of the output product. O and LSE are normalised by the unrounded
// fp32 row sum. V's operand is gathered transposed with ds_read_b64_tr_b8:
// within 16 lanes, lane i receives byte i % 8 of the 8-byte pieces addressed
// by lanes i / 8 + 2k (k = 0..7); pairs of addressing lanes name the same key
// and neighbouring 8-column pieces, so byte 8t + k of every lane of a half-wave
// holds the same key, matching the byte order of the P operand.
//
// MODE FWD_CONTIG_SPLIT: one workgroup per (query tile, head, batch, key
// split); the split's keys [s C, (s + 1) C) (C a multiple of the 128-key tile)
// bound the key range like a window, and the epilogue writes normalised
// partials for the combine kernel (the update article's split-KV entries,
// applied to the FP8 forward). MODE FWD_PAGED_TILES: the same over a paged
// cache (the article's paged KV entry) whose pages hold a multiple of 32 keys:
// each wavefront copies a slab of 32 consecutive rows of every 128-key tile,
// which then lies inside one page with the row stride of a contiguous tensor
// and travels from a per-wavefront base address. MODE FWD_PAGED_SPLIT: any
// page size; each lane gathers its 16-byte pieces of key rows from their pages,
// with the workgroup's page ids staged in LDS.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "fa_device.h"
#include "fa_lds.h"

namespace fa {

namespace {

constexpr int kBM = FP8_BM;    // query rows per workgroup
constexpr int kBN = 128;       // keys per tile
constexpr int kThreads = 256;  // 4 wavefronts
constexpr int kNB = kBN / 32;  // 32-key blocks of S^T per tile
constexpr int kNH = kBN / 64;  // 64-key halves: one output MFMA each per 32 head_dim rows

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));

// Chunk swizzle of an LDS row of D bytes (D / 16 chunks): the 16 rows read
// together by a K operand load land on 16 distinct 16-byte slots of a bank
// sweep, and so do the rows of the transposed V reads. 128-byte rows (two per
// sweep) take three row bits; 64-byte rows (four per sweep) take rows 4 apart
// onto the four chunks of their slot group.
template <int D>
__device__ __forceinline__ int swz_fp8(int r) {
  if constexpr (D == 128) return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  else return (r >> 2) & 3;
}
template <int D>
__device__ __forceinline__ int tile_byte(int row, int chunk) {
  return row * D + 16 * (chunk ^ swz_fp8<D>(row));
}

__device__ __forceinline__ i32x8_t mfma_operand(u32x4_t a, u32x4_t b) {
  return i32x8_t{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
}

__device__ __forceinline__ f32x16_t mfma_fp8(i32x8_t a, i32x8_t b, f32x16_t c) {
  // Formats 0/0 = E4M3 for both operands; block scales 127 = 2^0.
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ i32x2_t ds_read_tr8(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2_t*)p);
}

// Wavefronts per SIMD the register budget is sized for: two at head_dim 128,
// three at 64 (half the output accumulators and Q operand).
template <int D>
struct Fp8Waves {
  static constexpr int kWaves = D == 128 ? 2 : 3;
};

template <int D, bool SOFTCAP, bool ALIBI, int MODE>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(Fp8Waves<D>::kWaves, Fp8Waves<D>::kWaves)))
void fwd_fp8_kernel(FwdParams p) {
  constexpr bool SPLIT = MODE != FWD_CONTIG;        // one key split per workgroup, partial outputs
  constexpr bool PTILES = MODE == FWD_PAGED_TILES;  // each wavefront's slab of a tile from one page
  constexpr bool PGATHER = MODE == FWD_PAGED_SPLIT; // K/V rows gathered from their pages
  constexpr int kD = D;             // head_dim (bytes per K/V row of one head)
  constexpr int kTile = kBN * kD;   // bytes per K or V tile
  constexpr int kCPR = kD / 16;     // 16-byte chunks per row
  constexpr int kRPL = 64 / kCPR;   // rows per wavefront-wide copy
  constexpr int kLoads = kBN / kRPL / 4;  // copies per wavefront per tensor per tile
  constexpr int KS = kD / 64;       // k-steps of the score product (64 bytes each)
  constexpr int NDB = kD / 32;      // 32-row blocks of O^T
  __shared__ __attribute__((aligned(1024))) uint8_t sK0[kTile];
  __shared__ __attribute__((aligned(1024))) uint8_t sK1[kTile];
  __shared__ __attribute__((aligned(1024))) uint8_t sV0[kTile];
  __shared__ __attribute__((aligned(1024))) uint8_t sV1[kTile];
  // Page ids of the workgroup's keys (row gathers): 8 KB, which covers 2048 pages.
  constexpr int kTablePages = PGATHER ? 2048 : 1;
  __shared__ int s_pt[kTablePages];

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, r = lane & 31, h2 = lane >> 5;
  const WorkItem wi = decode_work<SPLIT>(p);
  const int b = wi.b, h = wi.h, s = wi.s;
  const SeqInfo si = seq_info(p, b, h);
  const int nq = si.nq, nk = si.nk;
  const int qt = query_tile(p, wi, nq, kBM);
  if (qt < 0) return;
  const int off = nk - nq;
  int slo = 0, shi = nk;
  if constexpr (SPLIT) split_range(p, nk, s, slo, shi);
  const int q0 = qt * kBM, q1 = min(nq, q0 + kBM);
  const KeyBounds wg = key_bounds(q0, q1, off, slo, shi, p.window_left, p.window_right);
  if (wg.hi <= wg.lo) {
    write_empty_rows<SPLIT>(p, si, b, h, s, q0, q1, kD, tid, kThreads);
    return;
  }
  const int wq0 = q0 + 32 * w, wq1 = min(nq, wq0 + 32);
  const bool wave_live = wq0 < nq;
  const KeyBounds wk = key_bounds(wq0, max(wq1, wq0 + 1), off, slo, shi, p.window_left,
                                  p.window_right);
  const int row = wq0 + r;
  const KeyBounds rk = key_bounds(row, row + 1, off, slo, shi, p.window_left, p.window_right);

  float slope_log2 = 0.0f;
  if constexpr (ALIBI) slope_log2 = p.alibi[h] * kLog2e;
  const float c = exponent_scale<SOFTCAP, ALIBI>(p);

  // Q of this lane's row: bytes 64ks + 32h2 .. +31 (B operand of S^T = K Q^T).
  i32x8_t qf[KS];
  {
    const uint8_t* qp = (const uint8_t*)p.q + ((si.q_row0 + min(row, nq - 1)) * p.H + h) * kD + 32 * h2;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4_t x0 = *(const u32x4_t*)(qp + 64 * ks);
      u32x4_t x1 = *(const u32x4_t*)(qp + 64 * ks + 16);
      if (row >= nq) x0 = x1 = u32x4_t{0, 0, 0, 0};
      qf[ks] = mfma_operand(x0, x1);
    }
  }

  // Contiguous K/V copies: descriptors rebased per tile and bounded by the
  // last key, so rows past it arrive as zeros.
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int64_t row_bytes = (int64_t)p.H * kD;
  const int64_t bh_bytes = (si.k_row0 * p.H + h) * kD;
  const int64_t end_bytes = (int64_t)(nk - 1) * row_bytes + kD;
  const char* kbh = (const char*)p.k + bh_bytes;
  const char* vbh = (const char*)p.v + bh_bytes;
  unsigned lane_bytes[kLoads];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int trow = kRPL * (kLoads * wu + i) + lane / kCPR;
    lane_bytes[i] = (unsigned)(trow * row_bytes + 16 * ((lane % kCPR) ^ swz_fp8<kD>(trow)));
  }
  // One tile of K and V whose first rows start `koff` bytes into the K and V
  // tensors (or page pools), `left` bytes of it in range.
  auto copy_at = [&](const char* kb, const char* vb, int64_t left, uint8_t* kd, uint8_t* vd)
                     __attribute__((always_inline)) {
    const int n = left <= 0 ? 0 : (left >= 0x7FFFFFFF ? 0x7FFFFFFF : (int)left);
    const __amdgpu_buffer_rsrc_t rk_ = make_rsrc(kb, n);
    const __amdgpu_buffer_rsrc_t rv_ = make_rsrc(vb, n);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      buffer_load_lds16(rk_, (uint16_t*)(kd + 1024 * (kLoads * wu + i)), lane_bytes[i]);
      buffer_load_lds16(rv_, (uint16_t*)(vd + 1024 * (kLoads * wu + i)), lane_bytes[i]);
    }
  };
  auto copy_tiles = [&](uint8_t* kd, uint8_t* vd, int j0) __attribute__((always_inline)) {
    const int64_t tb = (int64_t)j0 * row_bytes;
    copy_at(kbh + tb, vbh + tb, end_bytes - tb, kd, vd);
  };
  // Paged cache (PTILES): this wavefront's slab of tile j0 (rows kSlab wu ..
  // +kSlab-1) from page `page`, whose slot for the slab is a multiple of kSlab.
  // The descriptors are based kSlab wu rows before the slab, so the per-lane
  // offsets of the contiguous path apply unchanged; only the slab's rows are
  // read, and rows past the sequence's last key read as zeros.
  constexpr int kSlab = kRPL * kLoads;
  static_assert(kSlab == 32, "slab rows");
  auto copy_page_tiles = [&](int page, uint8_t* kd, uint8_t* vd, int j0) __attribute__((always_inline)) {
    const int js = j0 + kSlab * wu;
    const int slot = p.page_shift >= 0 ? js & (p.page_size - 1) : js % p.page_size;
    const int64_t pb = (((int64_t)page * p.page_size + slot) * p.H + h) * kD - (int64_t)kSlab * wu * row_bytes;
    copy_at((const char*)p.k + pb, (const char*)p.v + pb, (int64_t)(nk - 1 - j0) * row_bytes + kD,
            kd, vd);
  };
  // Block-table entry of this wavefront's slab of tile j0 (clamped into the
  // workgroup's keys, so the index stays in the table), read by a vector load:
  // the caller makes it uniform once the load has been waited for, so the load
  // never stalls the copies issued beside it.
  auto page_entry = [&](int j0) __attribute__((always_inline)) {
    const int kk = min(j0 + kSlab * wu, wg.hi - 1);
    const int idx = p.page_shift >= 0 ? kk >> p.page_shift : kk / p.page_size;
    return p.block_table[(int64_t)b * p.max_pages + idx + (lane >> 6)];
  };
  // Row gathers (PGATHER): the page ids of keys [j_first, wg.hi) are staged in
  // LDS when they fit, so a copy needs no dependent global load; lane L of copy
  // i fetches physical chunk L % kCPR of tile row kRPL (kLoads w + i) + L / kCPR.
  // Rows past the workgroup's keys re-read its last key (finite data, masked).
  const int j_first = (wg.lo / kBN) * kBN;
  int pt0 = 0;
  bool pt_lds = false;
  if constexpr (PGATHER) {
    pt0 = p.page_shift >= 0 ? j_first >> p.page_shift : j_first / p.page_size;
    const int pt1 = p.page_shift >= 0 ? (wg.hi - 1) >> p.page_shift : (wg.hi - 1) / p.page_size;
    pt_lds = pt1 - pt0 < kTablePages;
    if (pt_lds) {
      const int* bt_row = p.block_table + (int64_t)b * p.max_pages;
      for (int i = tid; i <= pt1 - pt0; i += kThreads) s_pt[i] = bt_row[pt0 + i];
    }
    __syncthreads();
  }
  auto copy_gather = [&](uint8_t* kd, uint8_t* vd, int j0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int ld = kLoads * wu + i;
      const int trow = kRPL * ld + lane / kCPR;
      const int key = min(j0 + trow, wg.hi - 1);
      int idx, slot;
      if (p.page_shift >= 0) {
        idx = key >> p.page_shift;
        slot = key & (p.page_size - 1);
      } else {
        idx = key / p.page_size;
        slot = key - idx * p.page_size;
      }
      const int page = pt_lds ? s_pt[idx - pt0] : p.block_table[(int64_t)b * p.max_pages + idx];
      const int64_t o = (((int64_t)page * p.page_size + slot) * p.H + h) * kD +
                        16 * ((lane % kCPR) ^ swz_fp8<kD>(trow));
      __builtin_amdgcn_global_load_lds((gbl_ptr_t)((const uint8_t*)p.k + o), (lds_ptr_t)(kd + 1024 * ld),
                                       16, 0, 0);
      __builtin_amdgcn_global_load_lds((gbl_ptr_t)((const uint8_t*)p.v + o), (lds_ptr_t)(vd + 1024 * ld),
                                       16, 0, 0);
    }
  };

  f32x16_t oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16_t{};
  float m_run = kNegInf, l_run = 0.0f;  // l_run: sum of the unrounded (2^8-scaled) P
  const int a16 = lane & 15, grp = lane >> 4;

  auto compute = [&](auto masked_t, const uint8_t* kt, const uint8_t* vt, int j0)
                     __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_t)::value;
    // S^T for the tile's 32-key blocks: A = K row 32j + r, bytes 64ks + 32h2 .. +31.
    f32x16_t sacc[kNB];
#pragma unroll
    for (int j = 0; j < kNB; ++j) {
      sacc[j] = f32x16_t{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int kr = 32 * j + r, ch = 4 * ks + 2 * h2;
        const u32x4_t a0 = *(const u32x4_t*)(kt + tile_byte<kD>(kr, ch));
        const u32x4_t a1 = *(const u32x4_t*)(kt + tile_byte<kD>(kr, ch + 1));
        sacc[j] = mfma_fp8(mfma_operand(a0, a1), qf[ks], sacc[j]);
      }
    }
    float t[kNB][16];
#pragma unroll
    for (int j = 0; j < kNB; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) t[j][v] = sacc[j][v];
    // ALiBi distances are measured from the row's anchor (its diagonal position
    // clamped into its visible keys), which only differs from the diagonal in
    // a key split far from the row.
    const float rel = (float)(ALIBI ? alibi_anchor(row + off, rk) : row + off) - (float)(j0 + 4 * h2);
    transform_scores<kNB, SOFTCAP, ALIBI>(t, p, slope_log2, rel, MASKED, j0, rk.lo, rk.hi, h2);
    bool any_rescale;
    float mc;
    const float alpha = online_max<kNB>(t, c, m_run, l_run, any_rescale, mc, 0.0f);
    if (any_rescale) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
    }
    // P * 2^8 (exponent shifted by 8), its fp32 row sum, and its E4M3 codes:
    // operand pq[hb] holds this lane's 32 keys of the 64-key half hb in byte
    // order 16(j - 2hb) + v (the P^T operand).
    const float mc8 = mc - 8.0f;
    i32x8_t pq[kNH];
    float ls[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int wd = 0; wd < 8 * kNH; ++wd) {
      const int j = wd >> 2, v0 = 4 * (wd & 3);
      float e[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        e[u] = fast_exp2(__builtin_fmaf(t[j][v0 + u], c, -mc8));
        ls[u] += e[u];
      }
      int x = __builtin_amdgcn_cvt_pk_fp8_f32(e[0], e[1], 0, false);
      x = __builtin_amdgcn_cvt_pk_fp8_f32(e[2], e[3], x, true);
      pq[wd >> 3][wd & 7] = x;
    }
    l_run += (ls[0] + ls[1]) + (ls[2] + ls[3]);
    // O^T += V^T P^T, one MFMA per 64-key half and 32 head_dim rows: byte
    // 8tr + k of lane l's operand is V[64hb + key(h2, tr, k)][32db + l % 32],
    // gathered with 4 transposed reads.
#pragma unroll
    for (int hb = 0; hb < kNH; ++hb) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        i32x8_t a;
#pragma unroll
        for (int tr = 0; tr < 4; ++tr) {
          const int k = a16 >> 1, pc = a16 & 1;
          const int jj = tr >> 1, g = 2 * (tr & 1) + (k >> 2), e = k & 3;
          const int key = 64 * hb + 32 * jj + 8 * g + 4 * h2 + e;
          const int ch = 2 * db + (grp & 1);
          const i32x2_t x = ds_read_tr8(vt + tile_byte<kD>(key, ch) + 8 * pc);
          a[2 * tr] = x[0];
          a[2 * tr + 1] = x[1];
        }
        oacc[db] = mfma_fp8(a, pq[hb], oacc[db]);
      }
    }
  };

  auto live = [&](int j0) __attribute__((always_inline)) {
    return wave_live && j0 < wk.hi && j0 + kBN > wk.lo;
  };
  const int ntiles = (wg.hi - j_first + kBN - 1) / kBN;
#ifdef FA_SERIAL_COPIES
  // Verification build: one buffer per tensor, each tile copied, waited for and
  // fenced by barriers on both sides; the results must match the two-stage
  // loop bit for bit.
  for (int it = 0; it < ntiles; ++it) {
    const int j0 = j_first + it * kBN;
    if constexpr (PTILES) {
      const int pe = page_entry(j0);
      wait_vmem();
      copy_page_tiles(__builtin_amdgcn_readfirstlane(pe), sK0, sV0, j0);
    } else if constexpr (PGATHER) {
      copy_gather(sK0, sV0, j0);
    } else {
      copy_tiles(sK0, sV0, j0);
    }
    wait_vmem_barrier<0>();
    if (live(j0)) {
      if (j0 >= wk.flo && j0 + kBN <= wk.fhi)
        compute(std::false_type{}, sK0, sV0, j0);
      else
        compute(std::true_type{}, sK0, sV0, j0);
    }
    __syncthreads();
  }
#else
  // Paged cache: step t copies tile t + 1 from the page whose id step t - 1
  // loaded, then loads the id of tile t + 2's page; the step's closing wait
  // covers that load too.
  int pg_next = 0;
  if constexpr (PTILES) {
    const int pe0 = page_entry(j_first);
    wait_vmem();
    copy_page_tiles(__builtin_amdgcn_readfirstlane(pe0), sK0, sV0, j_first);
    pg_next = page_entry(j_first + kBN);
  } else if constexpr (PGATHER) {
    copy_gather(sK0, sV0, j_first);
  } else {
    copy_tiles(sK0, sV0, j_first);
  }
  wait_vmem_barrier<0>();
  auto step = [&](auto par, int it) __attribute__((always_inline)) {
    constexpr bool ODD = decltype(par)::value;
    const int j0 = j_first + it * kBN;
    if constexpr (PTILES) {
      if (it + 1 < ntiles) {
        copy_page_tiles(__builtin_amdgcn_readfirstlane(pg_next), ODD ? sK0 : sK1, ODD ? sV0 : sV1,
                        j0 + kBN);
        if (it + 2 < ntiles) pg_next = page_entry(j0 + 2 * kBN);
      }
    } else if constexpr (PGATHER) {
      if (it + 1 < ntiles) copy_gather(ODD ? sK0 : sK1, ODD ? sV0 : sV1, j0 + kBN);
    } else {
      if (it + 1 < ntiles) copy_tiles(ODD ? sK0 : sK1, ODD ? sV0 : sV1, j0 + kBN);
    }
    if (live(j0)) {
      if (j0 >= wk.flo && j0 + kBN <= wk.fhi)
        compute(std::false_type{}, ODD ? sK1 : sK0, ODD ? sV1 : sV0, j0);
      else
        compute(std::true_type{}, ODD ? sK1 : sK0, ODD ? sV1 : sV0, j0);
    }
    wait_vmem_barrier<0>();
  };
  for (int it = 0; it < ntiles; it += 2) {
    step(std::false_type{}, it);
    if (it + 1 < ntiles) step(std::true_type{}, it + 1);
  }
#endif

  // Epilogue: O = v_descale * O~ / l, LSE = (c m + log2 l - 8) ln 2, with the
  // anchor's dropped ALiBi constant subtracted (zero without a key split).
  if (!wave_live) return;
  const float l_tot = half_sum(l_run);
  if (row >= nq) return;
  const float inv = l_tot > 0.0f ? p.v_descale / l_tot : 0.0f;
  float mref = m_run * c;
  if constexpr (ALIBI) mref -= slope_log2 * (float)abs(row + off - alibi_anchor(row + off, rk));
  const float lse = l_tot > 0.0f ? (mref + __log2f(l_tot) - 8.0f) * kLn2 : kNegInf;
  if constexpr (SPLIT) {
    const int64_t ro = (((int64_t)s * p.B + b) * p.H + h) * p.Nq + row;
    float* op = p.o_part + ro * kD;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4_t x = {oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv, oacc[db][4 * g + 2] * inv,
                     oacc[db][4 * g + 3] * inv};
        *(f32x4_t*)(op + 32 * db + 8 * g + 4 * h2) = x;
      }
    if (h2 == 0) p.lse_part[ro] = lse;
  } else {
    const int64_t ob = q_offset(p, si, row, h, kD);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        store_out4(p, ob + 32 * db + 8 * g + 4 * h2, oacc[db][4 * g] * inv,
                   oacc[db][4 * g + 1] * inv, oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
    if (h2 == 0 && p.lse) p.lse[si.lse0 + row] = lse;
  }
}

}  // namespace

template <int D, bool SOFTCAP, bool ALIBI, int MODE>
int launch_fwd_fp8(const FwdParams& p, void* stream) {
  const int64_t groups =
      (int64_t)p.num_q_tiles * p.H * p.B * (MODE != FWD_CONTIG ? p.num_splits : 1);
  hipLaunchKernelGGL((fwd_fp8_kernel<D, SOFTCAP, ALIBI, MODE>), dim3((unsigned)groups),
                     dim3(kThreads), 0, (hipStream_t)stream, p);
  return (int)hipGetLastError();
}

#define FA_INST(D, SC, AL)                                                          \
  template int launch_fwd_fp8<D, SC, AL, FWD_CONTIG>(const FwdParams&, void*);       \
  template int launch_fwd_fp8<D, SC, AL, FWD_CONTIG_SPLIT>(const FwdParams&, void*); \
  template int launch_fwd_fp8<D, SC, AL, FWD_PAGED_TILES>(const FwdParams&, void*);    \
  template int launch_fwd_fp8<D, SC, AL, FWD_PAGED_SPLIT>(const FwdParams&, void*);
FA_INST(64, false, false)
FA_INST(64, false, true)
FA_INST(64, true, false)
FA_INST(64, true, true)
FA_INST(128, false, false)
FA_INST(128, false, true)
FA_INST(128, true, false)
FA_INST(128, true, true)
#undef FA_INST

}  // namespace fa
