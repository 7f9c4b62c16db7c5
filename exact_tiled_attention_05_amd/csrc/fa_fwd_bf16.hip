// bf16 tiled attention forward for gfx950 (MI355X).
//
// One workgroup of 4 wavefronts owns a 128-row query tile of one (batch, head)
// [and one key split in the split modes]. Each wavefront keeps its 32 query rows in
// registers and walks the key range its rows can see in 64-key tiles:
//   S^T = K Q^T     on v_mfma_f32_32x32x16_bf16 (K from LDS, Q from VGPRs)
//   score transform, mask, online softmax in VGPRs (row = lane pair l, l^32)
//   O^T += V^T P^T  on v_mfma_f32_32x32x16_bf16 (V read transposed from LDS
//                   with ds_read_b64_tr_b16, P from VGPRs)
// K and V tiles travel HBM -> LDS with loads that write LDS directly (no
// staging registers), in their natural [key][d] layout with the 16-byte chunks
// of each row XOR-swizzled so that both the K operand reads and the
// transposed V reads are free of bank conflicts. Contiguous K/V use buffer
// loads whose descriptor moves by whole tiles (scalar arithmetic only) and
// whose range check turns keys past the end into zero rows; K sits in a
// three-stage ring and V in two buffers, so step t copies V(t+1) as it starts
// and K(t+2) after its score MFMAs (spreading the copies of a step over time)
// and ends with K(t+2) still in flight. Paged K/V whose pages hold a multiple
// of 16 keys run the same loop, each wavefront's 16-row slab of a tile taken
// from its page; other page sizes and appended keys gather rows through the
// block table with global loads into two buffers each. Inside a tile the LDS
// reads run several MFMAs ahead of their use (pinned with scheduling groups).
// Tiles inside every row's key range take a path with no per-element mask.
// A workgroup uses 80 KiB of LDS at head_dim 128, so two fit on a CU.
// (Tiled IO-aware forward with online softmax: "IO感知技术革命: FlashAttention如何
// 重塑大模型训练的经济学", sections on block tiling, online softmax and overlap of
// copies with compute; mask and score variants: flash-attn v2.0-v2.7 update
// article, v2.1-v2.6 entries; split + paged form: its v2.2 and v2.5 entries.)
#include <hip/hip_runtime.h>

#include <type_traits>

#include "fa_device.h"
#include "fa_lds.h"

namespace fa {

namespace {

constexpr int kBM = BF16_BM;   // query rows per workgroup
constexpr int kBN = 64;        // keys per tile
constexpr int kThreads = 256;  // 4 wavefronts

// Wavefronts per SIMD the register budget is sized for: two at head_dim 128
// (and for the tanh cap at 64, whose transform needs the extra registers),
// three otherwise.
template <int D, bool SOFTCAP>
struct Tuning {
  static constexpr int kWaves = (D == 128 || SOFTCAP) ? 2 : 3;
};

// MODE: FWD_CONTIG (contiguous K/V -> O, LSE), FWD_CONTIG_SPLIT (contiguous K/V,
// one key split per workgroup -> normalised partials), FWD_PAGED_TILES (paged
// K/V in pages of a multiple of 16 keys -> partials) or FWD_PAGED_SPLIT (paged
// K/V through the block table -> partials).
template <int D, bool SOFTCAP, bool ALIBI, int MODE>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(Tuning<D, SOFTCAP>::kWaves, Tuning<D, SOFTCAP>::kWaves)))
void fwd_bf16_kernel(FwdParams p) {
  constexpr bool PAGED = MODE == FWD_PAGED_SPLIT;  // K/V rows gathered through the block table
  constexpr bool PTILES = MODE == FWD_PAGED_TILES; // each wavefront's slab of a tile from one page
  constexpr bool SPLIT = MODE != FWD_CONTIG;       // one key split per workgroup, partial outputs
  constexpr int KS = D / 16;                 // MFMA k-steps of Q K^T
  constexpr int NDB = D / 32;                // 32-row blocks of O^T
  constexpr int CPR = D / 8;                 // 16-byte chunks per K/V row
  constexpr int ROWS_PER_LOAD = 64 / CPR;    // rows one wavefront-wide LDS copy fills
  constexpr int LOADS = kBN / ROWS_PER_LOAD / 4;  // copies per wavefront per tensor per tile
  constexpr int TILE = kBN * D;              // elements per tile
  // LDS reads issued ahead of the MFMA that consumes them: K fragments in the
  // score product, transposed V reads (in MFMAs) in the PV product. The score
  // transforms need registers, so their PV product reads less far ahead. For
  // plain scores two K fragments ahead (the rest one per MFMA) timed fastest
  // (causal prefill 3% faster than eight ahead); with a cap or ALiBi, eight.
  constexpr int kQkReadAhead = (SOFTCAP || ALIBI) ? (8 < 2 * KS ? 8 : 2 * KS) : 2;
  constexpr int kPvReadAhead = (SOFTCAP || ALIBI) ? 4 : 6;
  // Plain scores at head_dim 128 also spell the read-ahead out in source order
  // (the other variants keep it from the schedule alone and would spill with it).
  constexpr bool kPvRingInSource = D == 128 && !SOFTCAP && !ALIBI;

  __shared__ __attribute__((aligned(1024))) uint16_t sK0[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t sK1[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t sV0[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t sV1[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t sK2[TILE];  // third K stage (contiguous K/V)

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, r = lane & 31, h2 = lane >> 5;
  const WorkItem wi = decode_work<SPLIT>(p);
  const int b = wi.b, h = wi.h, s = wi.s;
  const SeqInfo si = seq_info(p, b, h);
  const int nq = si.nq, nk = si.nk;
  if constexpr (PAGED) {
    // Append: one workgroup per (b, h) copies the new keys into their pages.
    if (p.k_new && s == 0 && wi.rank == 0) append_rows<uint16_t>(p, si, b, h, D, tid, kThreads);
  }
  const int qt = query_tile(p, wi, nq, kBM);
  if (qt < 0) return;  // a packed sequence shorter than the longest

  const int off = nk - nq;
  int slo = 0, shi = nk;
  if constexpr (SPLIT) split_range(p, nk, s, slo, shi);

  const int q0 = qt * kBM;
  const int q1 = min(nq, q0 + kBM);
  const KeyBounds wg = key_bounds(q0, q1, off, slo, shi, p.window_left, p.window_right);
  if (wg.hi <= wg.lo) {
    write_empty_rows<SPLIT>(p, si, b, h, s, q0, q1, D, tid, kThreads);
    return;
  }

  // This wavefront's rows and keys.
  const int wq0 = q0 + 32 * w;
  const int wq1 = min(nq, wq0 + 32);
  const bool wave_live = wq0 < nq;
  const KeyBounds wk = key_bounds(wq0, max(wq1, wq0 + 1), off, slo, shi, p.window_left,
                                  p.window_right);
  const int row = wq0 + r;
  const KeyBounds rk = key_bounds(row, row + 1, off, slo, shi, p.window_left, p.window_right);

  float slope_log2 = 0.0f;
  if constexpr (ALIBI) slope_log2 = p.alibi[h] * kLog2e;
  const float c = exponent_scale<SOFTCAP, ALIBI>(p);

  // Q fragment: row `row`, columns 16*ks + 8*h2 .. +7 (the B operand of S^T = K Q^T).
  bf16x8_t qf[KS];
  {
    const uint16_t* qp = (const uint16_t*)p.q + q_offset(p, si, min(row, nq - 1), h, D) + 8 * h2;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4_t x = *(const u32x4_t*)(qp + 16 * ks);
      if (row >= nq) x = u32x4_t{0, 0, 0, 0};
      qf[ks] = __builtin_bit_cast(bf16x8_t, x);
    }
  }

  const int j_first = (wg.lo / kBN) * kBN;
  const int ntiles = (wg.hi - j_first + kBN - 1) / kBN;

  // Paged K/V. Each wavefront copies a slab of kSlab consecutive rows of every
  // tile; with pages of a multiple of kSlab keys and no appended key (PTILES)
  // every slab lies inside one page with the row stride of a contiguous tensor,
  // so it travels as in the contiguous path from a per-wavefront base address
  // (pages of a multiple of the 64-key tile give every wavefront of a tile the
  // same page). Otherwise (PAGED) rows are gathered one by one,
  // with the page ids of the workgroup's keys [j_first, wg.hi) staged in LDS
  // (in the third K buffer, which that path does not use) so that a copy needs
  // no dependent block-table load.
  constexpr int kTablePages = TILE / 2;  // ints in one K buffer
  int* const s_pt = (int*)sK2;
  int pt0 = 0;
  bool pt_lds = false;
  if constexpr (PAGED) {
    pt0 = p.page_shift >= 0 ? j_first >> p.page_shift : j_first / p.page_size;
    const int pt1 = p.page_shift >= 0 ? (wg.hi - 1) >> p.page_shift : (wg.hi - 1) / p.page_size;
    pt_lds = pt1 - pt0 < kTablePages;
    if (pt_lds) {
      const int* bt_row = p.block_table + (int64_t)b * p.max_pages;
      for (int i = tid; i <= pt1 - pt0; i += kThreads) s_pt[i] = bt_row[pt0 + i];
    }
    __syncthreads();
  }
  // Element offset of key `key` (in [j_first, wg.hi)) of this (b, h) in the page pool.
  auto paged_offset = [&](int key) __attribute__((always_inline)) {
    int idx, slot;
    if (p.page_shift >= 0) {
      idx = key >> p.page_shift;
      slot = key & (p.page_size - 1);
    } else {
      idx = key / p.page_size;
      slot = key - idx * p.page_size;
    }
    const int page = pt_lds ? s_pt[idx - pt0] : p.block_table[(int64_t)b * p.max_pages + idx];
    return (((int64_t)page * p.page_size + slot) * p.H + h) * D;
  };

  // ---- HBM -> LDS copies of one tile of K and V. Copy i of this wavefront
  // fills tile rows [ROWS_PER_LOAD * (LOADS*w + i), +ROWS_PER_LOAD); lane L
  // writes physical chunk L % CPR of its row, i.e. logical chunk
  // (L % CPR) ^ swz(row). K and V share the layout, hence one offset per copy.
  const int wu = __builtin_amdgcn_readfirstlane(w);
  // Contiguous K/V: per-(batch, head) buffer descriptors rebased on the tile's
  // first key and bounded by the end of the last key, so rows past the end
  // arrive as zeros; the per-lane byte offsets are fixed.
  const int64_t row_bytes = 2 * (int64_t)p.H * D;
  const int64_t bh_bytes = 2 * ((si.k_row0 * p.H + h) * D);
  const int64_t end_bytes = (int64_t)(nk - 1) * row_bytes + 2 * D;
  const char* kbh = (const char*)p.k + bh_bytes;
  const char* vbh = (const char*)p.v + bh_bytes;
  unsigned lane_bytes[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int trow = ROWS_PER_LOAD * (LOADS * wu + i) + lane / CPR;
    const int chunk = (lane % CPR) ^ swz<D>(trow);
    lane_bytes[i] = (unsigned)(trow * row_bytes + 16 * chunk);
  }
  // Paged K/V: rows past the workgroup's key range re-read its last key (finite
  // data; masked later); appended keys come from k_new / v_new.
  const uint16_t* kg = (const uint16_t*)p.k;
  const uint16_t* vg = (const uint16_t*)p.v;
  const uint16_t* kn = (const uint16_t*)p.k_new;
  const uint16_t* vn = (const uint16_t*)p.v_new;
  // One tile from `base` (its first row), `left` bytes of it in range.
  auto copy_rows = [&](const char* base, int64_t left, uint16_t* dst) __attribute__((always_inline)) {
    const int n = left <= 0 ? 0 : (left >= 0x7FFFFFFF ? 0x7FFFFFFF : (int)left);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(base, n);
#pragma unroll
    for (int i = 0; i < LOADS; ++i) buffer_load_lds16(rs, dst + 512 * (LOADS * wu + i), lane_bytes[i]);
  };
  auto copy_one = [&](const char* bh, uint16_t* dst, int j0) __attribute__((always_inline)) {
    const int64_t tb = (int64_t)j0 * row_bytes;
    copy_rows(bh + tb, end_bytes - tb, dst);
  };
  // This wavefront's slab of tile j0 (rows kSlab wu .. +kSlab-1) from page
  // `page` of a pool whose pages hold a multiple of kSlab keys (PTILES). The
  // descriptor is based kSlab wu rows before the slab, so the per-lane offsets
  // of the contiguous path apply unchanged; only the slab's rows are read, and
  // rows past the sequence's last key read as zeros.
  constexpr int kSlab = ROWS_PER_LOAD * LOADS;
  static_assert(kSlab == 16, "slab rows");
  auto copy_page_tile = [&](const void* pool, int page, uint16_t* dst, int j0) __attribute__((always_inline)) {
    const int js = j0 + kSlab * wu;
    const int slot = p.page_shift >= 0 ? js & (p.page_size - 1) : js % p.page_size;
    const char* base = (const char*)pool + 2 * ((((int64_t)page * p.page_size + slot) * p.H + h) * D) -
                       (int64_t)kSlab * wu * row_bytes;
    copy_rows(base, (int64_t)(nk - 1 - j0) * row_bytes + 2 * D, dst);
  };
  // Page of this wavefront's slab of tile j0 (slabs past the key range, which
  // read nothing, take the range's last page so the index stays in the table).
  // The id is read with a vector load (the address is written per lane:
  // lane >> 6 is 0) and made uniform afterwards: a scalar load would be waited
  // for with the counter that also tracks LDS reads, stalling the products'
  // operand reads.
  auto page_of = [&](int j0) __attribute__((always_inline)) {
    const int kk = min(j0 + kSlab * wu, wg.hi - 1);
    const int idx = p.page_shift >= 0 ? kk >> p.page_shift : kk / p.page_size;
    return __builtin_amdgcn_readfirstlane(p.block_table[(int64_t)b * p.max_pages + idx + (lane >> 6)]);
  };
  auto copy_tiles = [&](uint16_t* kdst, uint16_t* vdst, int j0) __attribute__((always_inline)) {
    if constexpr (!PAGED) {
      copy_one(kbh, kdst, j0);
      copy_one(vbh, vdst, j0);
    } else {
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int ld = LOADS * wu + i;
        const int trow = ROWS_PER_LOAD * ld + lane / CPR;
        const int chunk = (lane % CPR) ^ swz<D>(trow);
        const int key = min(j0 + trow, wg.hi - 1);
        const bool fresh = key >= si.n_cached;
        const int64_t o = (fresh ? new_key_offset(p, si, b, key, h, D) : paged_offset(key)) + 8 * chunk;
        __builtin_amdgcn_global_load_lds((gbl_ptr_t)((fresh ? kn : kg) + o),
                                         (lds_ptr_t)(kdst + 512 * ld), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((gbl_ptr_t)((fresh ? vn : vg) + o),
                                         (lds_ptr_t)(vdst + 512 * ld), 16, 0, 0);
      }
    }
  };

  // ---- S^T = K Q^T for one 64-key tile (two 32-key blocks).
  auto qk = [&](const uint16_t* kt, f32x16_t (&sacc)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const bf16x8_t a = __builtin_bit_cast(
            bf16x8_t, *(const u32x4_t*)(kt + tile_off<D>(32 * j + r, 2 * ks + h2)));
        sacc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], ks == 0 ? f32x16_t{} : sacc[j],
                                                          0, 0, 0);
      }
    }
    // Schedule: kQkReadAhead K reads, then alternate one MFMA and one read.
    static_assert(kQkReadAhead <= 2 * KS, "read-ahead");
    __builtin_amdgcn_sched_group_barrier(0x100, kQkReadAhead, 0);  // DS reads
#pragma unroll
    for (int i = 0; i < 2 * KS - kQkReadAhead; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kQkReadAhead, 0);
  };

  f32x16_t oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16_t{};
  // m_run: running max (score units). l_run: row sum of the bf16-rounded P that
  // feeds the PV product (normalises O). l_exact: row sum of the unrounded P
  // (gives the log-sum-exp).
  float m_run = kNegInf, l_run = 0.0f, l_exact = 0.0f;

  const int gl = lane & 15, sub = (lane >> 4) & 1;

  // ---- softmax of tile j0 (scores in sacc) and O^T += V^T P^T.
  // MASKED: the tile crosses some row's key range boundary, so scores are
  // masked element by element; full tiles skip that code entirely.
  auto softmax_pv = [&](auto masked, const f32x16_t (&sacc)[2], const uint16_t* vt, int j0)
                        __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked)::value;
    float t[2][16];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) t[j][v] = sacc[j][v];
    const float rel = (float)(ALIBI ? alibi_anchor(row + off, rk) : row + off) - (float)(j0 + 4 * h2);
    transform_scores<2, SOFTCAP, ALIBI>(t, p, slope_log2, rel, MASKED, j0, rk.lo, rk.hi, h2);
    bool any_rescale;
    float mc;
    const float alpha = online_max<2>(t, c, m_run, l_run, any_rescale, mc, 0.0f);
    l_exact *= alpha;
    if (any_rescale) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
    }

    // P (bf16, rounded to nearest even) and its row sums, each summed in
    // independent partials (short dependency chains).
    bf16x8_t pf[4];
    float le[4] = {0.0f, 0.0f, 0.0f, 0.0f}, lr[2] = {0.0f, 0.0f};
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      f32x8_t x;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[e] = fast_exp2(__builtin_fmaf(t[tt >> 1][(tt & 1) * 8 + e], c, -mc));
        le[e & 3] += x[e];
      }
      pf[tt] = __builtin_convertvector(x, bf16x8_t);
      lr[tt & 1] = sum_bf16x8(pf[tt], lr[tt & 1]);
    }
    l_exact += (le[0] + le[1]) + (le[2] + le[3]);
    l_run += lr[0] + lr[1];

    // k-step tt covers keys 16*tt .. 16*tt+15. The A operand (lane: d-row
    // m = lane % 32, keys 16tt + 4*h2 + {0..3, 8..11}) comes from two transposed
    // reads: in each 16-lane group, lanes 4k..4k+3 address the four 4-column
    // pieces of key k, and lane i receives column i of those 4 keys.
    auto v_operand = [&](int tt, int db) __attribute__((always_inline)) {
      const int vrow = 16 * tt + 4 * h2 + (gl >> 2);
      const int col = 32 * db + 16 * sub + 4 * (gl & 3);
      const s16x4_t lo = ds_read_tr16(vt + tile_off<D>(vrow, col >> 3) + (col & 7));
      const s16x4_t hi = ds_read_tr16(vt + tile_off<D>(vrow + 8, col >> 3) + (col & 7));
      return s16x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
    if constexpr (kPvRingInSource) {
      // MFMA i = (i / NDB, i % NDB); its operand is read kPvReadAhead MFMAs
      // ahead in source order as well, which the scheduler keeps when it falls
      // back to source order under register pressure (the masked tiles).
      s16x8_t vring[kPvReadAhead];
#pragma unroll
      for (int i = 0; i < kPvReadAhead; ++i) vring[i] = v_operand(i / NDB, i % NDB);
#pragma unroll
      for (int i = 0; i < 4 * NDB; ++i) {
        const s16x8_t x = vring[i % kPvReadAhead];
        if (i + kPvReadAhead < 4 * NDB)
          vring[i % kPvReadAhead] = v_operand((i + kPvReadAhead) / NDB, (i + kPvReadAhead) % NDB);
        oacc[i % NDB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8_t, x), pf[i / NDB], oacc[i % NDB], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8_t, v_operand(tt, db)), pf[tt], oacc[db], 0, 0, 0);
      }
    }
    // Schedule: the reads of kPvReadAhead MFMAs first, then one MFMA and the
    // two reads of a later one, alternately.
    static_assert(kPvReadAhead <= 4 * NDB, "read-ahead");
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * kPvReadAhead, 1);  // DS reads
#pragma unroll
    for (int i = 0; i < 4 * NDB - kPvReadAhead; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kPvReadAhead, 1);
  };

  auto live = [&](int j0) __attribute__((always_inline)) { return wave_live && j0 < wk.hi && j0 + kBN > wk.lo; };

  // ---- tile loop: K(t) in stage t % 3, V(t) in buffer t & 1. Step t copies
  // V(t+1) over V(t-1) and K(t+2) over K(t-1) (both last read in step t-1,
  // ended by a barrier), computes tile t, then waits for all but the K(t+2)
  // copies. Copies past the key range read nothing and write zeros. kcopy /
  // vcopy (dst, j0) copy the K / V tile of key j0.
  auto tile_loop = [&](auto kcopy, auto vcopy) __attribute__((always_inline)) {
#ifdef FA_SERIAL_COPIES
    // Verification build: one buffer per tensor, each tile copied, waited for
    // and fenced by barriers on both sides (no copy overlaps any compute). The
    // arithmetic is the pipelined loop's, so the results must agree bit for bit.
    f32x16_t sacc_s[2];
    for (int it = 0; it < ntiles; ++it) {
      const int j0 = j_first + it * kBN;
      kcopy(sK0, j0);
      vcopy(sV0, j0);
      wait_vmem_barrier<0>();
      if (live(j0)) {
        qk(sK0, sacc_s);
        if (j0 >= wk.flo && j0 + kBN <= wk.fhi)
          softmax_pv(std::false_type{}, sacc_s, sV0, j0);
        else
          softmax_pv(std::true_type{}, sacc_s, sV0, j0);
      }
      __syncthreads();
    }
    return;
#endif
    constexpr int kKC = LOADS;  // vector-memory ops of one K tile copy
    kcopy(sK0, j_first);
    vcopy(sV0, j_first);
    kcopy(sK1, j_first + kBN);
    wait_vmem_barrier<kKC>();
    f32x16_t sacc[2];
    auto step3 = [&](auto kst, auto vpar, int it) __attribute__((always_inline)) {
      constexpr int KSt = decltype(kst)::value;
      constexpr bool VODD = decltype(vpar)::value;
      const uint16_t* k_cur = KSt == 0 ? sK0 : KSt == 1 ? sK1 : sK2;
      uint16_t* k_nn = KSt == 0 ? sK2 : KSt == 1 ? sK0 : sK1;
      const uint16_t* v_cur = VODD ? sV1 : sV0;
      uint16_t* v_nxt = VODD ? sV0 : sV1;
      const int j0 = j_first + it * kBN;
      vcopy(v_nxt, j0 + kBN);
      const bool lv = live(j0);
      if (lv) qk(k_cur, sacc);
      kcopy(k_nn, j0 + 2 * kBN);
      if (lv) {
        if (j0 >= wk.flo && j0 + kBN <= wk.fhi)
          softmax_pv(std::false_type{}, sacc, v_cur, j0);
        else
          softmax_pv(std::true_type{}, sacc, v_cur, j0);
      }
      wait_vmem_barrier<kKC>();
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    for (int it = 0; it < ntiles; it += 6) {
      step3(I0{}, std::false_type{}, it);
      if (it + 1 < ntiles) step3(I1{}, std::true_type{}, it + 1);
      if (it + 2 < ntiles) step3(I2{}, std::false_type{}, it + 2);
      if (it + 3 < ntiles) step3(I0{}, std::true_type{}, it + 3);
      if (it + 4 < ntiles) step3(I1{}, std::false_type{}, it + 4);
      if (it + 5 < ntiles) step3(I2{}, std::true_type{}, it + 5);
    }
    wait_vmem_barrier<0>();  // no copy may still be writing LDS at exit
  };

  if constexpr (PTILES) {
    // The loop copies K(t+2) and V(t+1) in step t: each K copy also loads the
    // page of the next tile, one step before the next K copy needs it, and
    // leaves its own page for the V copy of the next step.
    int pk_j = -1, pk = 0, pv_j = -1, pv = 0;
    tile_loop(
        [&](uint16_t* dst, int j0) __attribute__((always_inline)) {
          const int pg = j0 == pk_j ? pk : page_of(j0);
          copy_page_tile(p.k, pg, dst, j0);
          pv = pg;
          pv_j = j0;
          pk = page_of(j0 + kBN);
          pk_j = j0 + kBN;
        },
        [&](uint16_t* dst, int j0) __attribute__((always_inline)) {
          copy_page_tile(p.v, j0 == pv_j ? pv : page_of(j0), dst, j0);
        });
  } else if constexpr (!PAGED) {
    tile_loop([&](uint16_t* dst, int j0) __attribute__((always_inline)) { copy_one(kbh, dst, j0); },
              [&](uint16_t* dst, int j0) __attribute__((always_inline)) { copy_one(vbh, dst, j0); });
  } else {
    // ---- paged K/V gathered row by row: two buffers each; step t copies tile
    // t+1 and waits for it.
#ifdef FA_SERIAL_COPIES
    {  // verification build: one buffer, no overlap (see tile_loop)
      f32x16_t sacc[2];
      for (int it = 0; it < ntiles; ++it) {
        const int j0 = j_first + it * kBN;
        copy_tiles(sK0, sV0, j0);
        wait_vmem();
        __syncthreads();
        if (live(j0)) {
          qk(sK0, sacc);
          if (j0 >= wk.flo && j0 + kBN <= wk.fhi)
            softmax_pv(std::false_type{}, sacc, sV0, j0);
          else
            softmax_pv(std::true_type{}, sacc, sV0, j0);
        }
        __syncthreads();
      }
    }
#else
    copy_tiles(sK0, sV0, j_first);
    wait_vmem();
    __syncthreads();

    // Step t: copy K(t+1), V(t+1) into buffers (t+1)&1 (free since the
    // barrier that ended step t-1), then S(t), softmax(t), PV(t) from buffers t&1.
    f32x16_t sacc[2];
    auto step = [&](auto par, int it) __attribute__((always_inline)) {
      constexpr bool ODD = decltype(par)::value;
      const uint16_t* k_cur = ODD ? sK1 : sK0;
      const uint16_t* v_cur = ODD ? sV1 : sV0;
      uint16_t* k_nxt = ODD ? sK0 : sK1;
      uint16_t* v_nxt = ODD ? sV0 : sV1;
      const int j0 = j_first + it * kBN;
      if (it + 1 < ntiles) copy_tiles(k_nxt, v_nxt, j0 + kBN);
      if (live(j0)) {
        qk(k_cur, sacc);
        if (j0 >= wk.flo && j0 + kBN <= wk.fhi)
          softmax_pv(std::false_type{}, sacc, v_cur, j0);
        else
          softmax_pv(std::true_type{}, sacc, v_cur, j0);
      }
      wait_vmem();
      __syncthreads();
    };

    for (int it = 0; it < ntiles; it += 2) {
      step(std::false_type{}, it);
      if (it + 1 < ntiles) step(std::true_type{}, it + 1);
    }
#endif
  }

  // ---- epilogue: O = O / l, LSE = (c m + log2 l) ln 2
  if (!wave_live) return;
  const float l_tot = half_sum(l_run);
  const float l_ex = half_sum(l_exact);
  if (row >= nq) return;
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  float mref = m_run * c;  // the maximum in units of the unshifted ALiBi bias
  if constexpr (ALIBI) mref -= slope_log2 * (float)abs(row + off - alibi_anchor(row + off, rk));
  const float lse = l_ex > 0.0f ? (mref + __log2f(l_ex)) * kLn2 : kNegInf;
  if constexpr (SPLIT) {
    const int64_t ro = (((int64_t)s * p.B + b) * p.H + h) * p.Nq + row;
    float* op = p.o_part + ro * D;
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
    const int64_t ob = q_offset(p, si, row, h, D);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        store_out4(p, ob + 32 * db + 8 * g + 4 * h2, oacc[db][4 * g] * inv,
                   oacc[db][4 * g + 1] * inv, oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
    if (h2 == 0 && p.lse) p.lse[si.lse0 + row] = lse;
  }
}

// The append of a multi-row split pass as a launch of its own (one workgroup
// per (batch, head) copies its k_new / v_new rows into their cache pages), so
// that the pass after it can read every key from the cache in page slabs.
template <int D>
__global__ __launch_bounds__(kThreads) void append_kernel(FwdParams p) {
  const int h = blockIdx.x % p.H, b = blockIdx.x / p.H;
  const SeqInfo si = seq_info(p, b, h);
  append_rows<uint16_t>(p, si, b, h, D, threadIdx.x, kThreads);
}

}  // namespace

template <int D>
int launch_append_bf16(const FwdParams& p, void* stream) {
  hipLaunchKernelGGL((append_kernel<D>), dim3((unsigned)((int64_t)p.B * p.H)), dim3(kThreads), 0,
                     (hipStream_t)stream, p);
  return (int)hipGetLastError();
}
template int launch_append_bf16<64>(const FwdParams&, void*);
template int launch_append_bf16<128>(const FwdParams&, void*);

template <int D, bool SOFTCAP, bool ALIBI, int MODE>
int launch_fwd_bf16(const FwdParams& p, void* stream) {
  const int64_t groups =
      (int64_t)p.num_q_tiles * p.H * p.B * (MODE != FWD_CONTIG ? p.num_splits : 1);
  hipLaunchKernelGGL((fwd_bf16_kernel<D, SOFTCAP, ALIBI, MODE>), dim3((unsigned)groups),
                     dim3(kThreads), 0, (hipStream_t)stream, p);
  return (int)hipGetLastError();
}

#define FA_INST(D, SC, AL, M) template int launch_fwd_bf16<D, SC, AL, M>(const FwdParams&, void*);
#define FA_INST_M(D, M) \
  FA_INST(D, false, false, M) FA_INST(D, false, true, M) FA_INST(D, true, false, M) FA_INST(D, true, true, M)
#define FA_INST_D(D) FA_INST_M(D, FWD_CONTIG) FA_INST_M(D, FWD_CONTIG_SPLIT) \
  FA_INST_M(D, FWD_PAGED_SPLIT) FA_INST_M(D, FWD_PAGED_TILES)
FA_INST_D(64)
FA_INST_D(128)
#undef FA_INST_D
#undef FA_INST_M
#undef FA_INST

}  // namespace fa
