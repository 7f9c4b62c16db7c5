// Split-KV pass for one query row per (batch, head): the decode step, run as
// an HBM stream over the paged KV cache (flash-attn v2.0-v2.7 update article:
// v2.2 entry for cutting the cache along the sequence across workgroups, v2.5
// for pages addressed through block_table; the inference article's point that
// decode time goes to loading the cache when the query is one token).
//
// One workgroup of 4 wavefronts per (split, head group, batch), head group
// fastest: the adjacent heads whose rows of one key form a 256-byte segment of
// the page (512 bytes on large launches). Each lane owns a 16-byte chunk of a
// key row (8 bf16 or 16 E4M3 columns), so D / 8 (bf16) or D / 16 (E4M3) lanes
// share a row and a wavefront-wide load reads several whole segments. A lane keeps 8 K and 8 V loads in flight per
// batch. Scores are reduced across the row's lanes with DPP, and each lane
// runs an fp32 online softmax over its group's keys for its output columns.
// Groups, then wavefronts, are merged by log-sum-exp at the end. With an
// append, this step's new keys are read from k_new / v_new and written into
// their pages by one workgroup per (batch, head) (the inference article's
// key-value cache, which keeps each processed key for later steps). An E4M3
// cache (the FP8 forward support of the roadmap in "FlashAttention深度解析：
// 从算法创新到产业变革的全面影响", applied to the stored keys and values) halves
// the bytes per key; its codes are widened to fp32 in registers, K's descale
// is folded into the score scale and V's into the output.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "fa_device.h"

namespace fa {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
#ifndef FA_DECODE_LOADS
#define FA_DECODE_LOADS 8
#endif
constexpr int kU = FA_DECODE_LOADS;  // loads in flight per lane, per tensor
// Block-table entries staged in LDS per workgroup (the pages its key range
// touches); longer ranges read the table from global memory instead.
constexpr int kTablePages = 1024;

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                                0xf, 0xf, false));
}

// Sum over each group of CH consecutive lanes (CH = 4, 8 or 16); every lane of
// the group receives the sum.
template <int CH>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp<0xB1>(x);   // quad_perm(1,0,3,2): swap neighbours
  x += dpp<0x4E>(x);   // quad_perm(2,3,0,1): swap pairs
  if constexpr (CH >= 8) x += dpp<0x141>(x);   // row_half_mirror: lane i <-> 7 - i within 8
  if constexpr (CH == 16) x += dpp<0x140>(x);  // row_mirror: lane i <-> 15 - i within 16
  return x;
}

__device__ __forceinline__ float lo_bf16(unsigned w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float hi_bf16(unsigned w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// The four E4M3 codes of a 32-bit word (byte i = column i) as floats; every
// code converts exactly.
__device__ __forceinline__ void e4m3x4_to_f32(unsigned w, float (&f)[4]) {
  const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  f[0] = lo[0];
  f[1] = lo[1];
  f[2] = hi[0];
  f[3] = hi[1];
}

// Heads per workgroup: a key's rows of G adjacent heads are contiguous in a
// page, so G heads together make a 256-byte segment per key (one head when its
// row alone is 256 bytes). WIDE doubles the group to 512-byte segments.
template <int D, int ESIZE, bool WIDE>
struct DecodeGroup {
  static constexpr int EPL = 16 / ESIZE;  // columns per lane: one 16-byte chunk
  static constexpr int CH = D / EPL;      // lanes per head row
  static constexpr int G = (CH >= 16 ? 1 : 16 / CH) * (WIDE ? 2 : 1);
};

// APPEND: keys [n_cached, nk) are this step's new keys, read from k_new / v_new;
// the split-0 workgroup of each (b, head group) also copies them into their
// cache pages. FP8: the cache holds E4M3 codes (no append).
template <int D, bool SOFTCAP, bool ALIBI, bool APPEND, bool FP8, bool WIDE>
__device__ __forceinline__ void decode_body(const FwdParams& p) {
  static_assert(!(FP8 && APPEND), "no append into an E4M3 cache");
  using E = std::conditional_t<FP8, uint8_t, uint16_t>;  // cache element
  using DG = DecodeGroup<D, (int)sizeof(E), WIDE>;
  constexpr int EPL = DG::EPL;
  constexpr int CH = DG::CH;      // lanes per head row
  constexpr int G = DG::G;        // heads per workgroup
  constexpr int LPK = CH * G;     // lanes per key (its G head rows)
  constexpr int KPI = 64 / LPK;   // keys per wavefront-wide load
  constexpr int KPB = KPI * kU;   // keys per wavefront batch
  __shared__ float s_m[kWaves][G], s_l[kWaves][G];
  __shared__ float s_o[kWaves][G * D];
  __shared__ int s_bt[kTablePages];

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int ck = lane % LPK, g = lane / LPK;  // chunk of the key's segment, key group
  const int hg = ck / CH, c = ck % CH;        // head in the group, chunk of its row
  // Workgroup id: head group fastest, then batch, then split.
  int wid = blockIdx.x;
  const int HG = (p.H + G - 1) / G;
  const int h0 = G * (wid % HG);  // first head of the group
  wid /= HG;
  const int b = wid % p.B, s = wid / p.B;
  // A group past the last head repeats the last head and writes nothing for it.
  const int h = min(h0 + hg, p.H - 1);
  const SeqInfo si = seq_info(p, b, h0);
  const int nk = si.nk;
  if constexpr (APPEND) {
    if (s == 0)
      for (int j = 0; j < G && h0 + j < p.H; ++j)
        append_rows<uint16_t>(p, si, b, h0 + j, D, tid, kThreads);
  }

  int slo, shi;
  split_range(p, nk, s, slo, shi);
  const int ip = nk - 1;  // the single query row, aligned to the sequence's last key
  int lo = slo, hi = shi;
  if (p.window_left >= 0) lo = max(lo, ip - p.window_left);
  if (p.window_right >= 0) hi = min(hi, ip + p.window_right + 1);
  if (hi <= lo) {
    for (int j = 0; j < G && h0 + j < p.H; ++j)
      write_empty_rows<true>(p, si, b, h0 + j, s, 0, 1, D, tid, kThreads);
    return;
  }

  // Pages [p0, p0 + np) hold this workgroup's keys; stage their ids in LDS.
  const int p0 = p.page_shift >= 0 ? lo >> p.page_shift : lo / p.page_size;
  const int p1 = p.page_shift >= 0 ? (hi - 1) >> p.page_shift : (hi - 1) / p.page_size;
  const int np = p1 - p0 + 1;
  const bool table_in_lds = np <= kTablePages;
  const int* bt_row = p.block_table + (int64_t)b * p.max_pages;
  if (table_in_lds)
    for (int i = tid; i < np; i += kThreads) s_bt[i] = bt_row[p0 + i];
  __syncthreads();

  // The lane's EPL query columns: bf16 pairs for the dot2 products with a bf16
  // cache, floats for an E4M3 cache.
  const uint16_t* qrow = (const uint16_t*)p.q + q_offset(p, si, 0, h, D) + EPL * c;
  bf16x2_t qp[4];
  float qx[FP8 ? EPL : 1];
  if constexpr (FP8) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const u32x4_t qv = *(const u32x4_t*)(qrow + 8 * half);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qx[8 * half + 2 * e] = lo_bf16(qv[e]);
        qx[8 * half + 2 * e + 1] = hi_bf16(qv[e]);
      }
    }
  } else {
    const u32x4_t qv = *(const u32x4_t*)qrow;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const unsigned wq = qv[e];
      qp[e] = as_bf16x2(wq);
    }
  }
  // ALiBi distances are taken from the workgroup's last key (kref), not from the
  // query: for a split far from the query the bias is then small for the keys
  // that carry its weight, instead of thousands of log2 units that fp32 holds
  // to ~1e-4. The dropped constant slope * (ip - kref) is the same for every key
  // of the workgroup, so it leaves the normalised partial unchanged and is
  // subtracted from its log-sum-exp at the end.
  const int kref = hi - 1;
  float slope_log2 = 0.0f;
  if constexpr (ALIBI) slope_log2 = p.alibi[h] * kLog2e;

  float m = kNegInf, l = 0.0f, o[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) o[e] = 0.0f;

  const int lane_col = h * D + EPL * c;  // the lane's 16 bytes of a key's row
  const E* kbase = (const E*)p.k + lane_col;
  const E* vbase = (const E*)p.v + lane_col;
  const E* knew = (const E*)p.k_new + lane_col;
  const E* vnew = (const E*)p.v_new + lane_col;
  for (int base = lo + w * KPB; base < hi; base += kWaves * KPB) {
    // Row offsets first, then every load back to back (no branches between
    // them). A key past the end re-reads key `lo`, whose page is real, and its
    // score is masked below, so its finite V row gets weight 0.
    int64_t off[kU];
    bool fresh[kU];  // an appended key (APPEND only)
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int t = min(base + g + KPI * u, hi - 1);
      const int tt = base + g + KPI * u < hi ? t : lo;
      int idx, slot;
      if (p.page_shift >= 0) {
        idx = tt >> p.page_shift;
        slot = tt & (p.page_size - 1);
      } else {
        idx = tt / p.page_size;
        slot = tt - idx * p.page_size;
      }
      const int page = table_in_lds ? s_bt[idx - p0] : bt_row[idx];
      off[u] = (int64_t)page * p.page_stride + slot * p.row_stride;
      fresh[u] = false;
      if constexpr (APPEND) {
        fresh[u] = tt >= si.n_cached;
        if (fresh[u]) off[u] = new_key_offset(p, si, b, tt, 0, D);
      }
    }
    // Every cache row is read once per launch: non-temporal loads keep the
    // stream from displacing other lines (5.95 -> 6.65 TB/s on the 32768-key
    // decode shape; a plain streaming read probe shows the same gap).
    u32x4_t kx[kU], vx[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      kx[u] = __builtin_nontemporal_load((const u32x4_t*)((fresh[u] ? knew : kbase) + off[u]));
      vx[u] = __builtin_nontemporal_load((const u32x4_t*)((fresh[u] ? vnew : vbase) + off[u]));
    }
    float sc[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      float a = 0.0f;
      if constexpr (FP8) {
        float a2[2] = {0.0f, 0.0f};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float f[4];
          e4m3x4_to_f32(kx[u][e], f);
#pragma unroll
          for (int i = 0; i < 4; ++i) a2[i & 1] = __builtin_fmaf(f[i], qx[4 * e + i], a2[i & 1]);
        }
        a = a2[0] + a2[1];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const unsigned wk = kx[u][e];
          a = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(wk), qp[e], a, false);
        }
      }
      a = group_sum<CH>(a);
      if constexpr (SOFTCAP) {
        const float ex = fast_exp2(a * p.scale_over_cap2);
        a = p.softcap_log2 - 2.0f * p.softcap_log2 * __builtin_amdgcn_rcpf(ex + 1.0f);
      } else {
        a *= p.scale_log2;
      }
      const int t = base + g + KPI * u;
      if constexpr (ALIBI) a -= slope_log2 * (float)(kref - t);
      sc[u] = t < hi ? a : kNegInf;
    }
    float mb = sc[0];
#pragma unroll
    for (int u = 1; u < kU; ++u) mb = fmaxf(mb, sc[u]);
    const float m_new = fmaxf(m, mb);
    if (m_new > m + kLazyRescaleThreshold) {
      const float alpha = fast_exp2(m - m_new);
      l *= alpha;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[e] *= alpha;
      m = m_new;
    }
    const float bse = m == kNegInf ? 0.0f : m;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const float pu = fast_exp2(sc[u] - bse);
      l += pu;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (FP8) {
          float f[4];
          e4m3x4_to_f32(vx[u][e], f);
#pragma unroll
          for (int i = 0; i < 4; ++i) o[4 * e + i] += pu * f[i];
        } else {
          o[2 * e] += pu * lo_bf16(vx[u][e]);
          o[2 * e + 1] += pu * hi_bf16(vx[u][e]);
        }
      }
    }
  }

  // Merge the KPI lane groups of this wavefront (same columns, different keys).
#pragma unroll
  for (int msk = LPK; msk < 64; msk <<= 1) {
    const float m2 = __shfl_xor(m, msk);
    const float l2 = __shfl_xor(l, msk);
    const float mn = fmaxf(m, m2);
    const float a1 = m == kNegInf ? 0.0f : fast_exp2(m - mn);
    const float a2 = m2 == kNegInf ? 0.0f : fast_exp2(m2 - mn);
    l = l * a1 + l2 * a2;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] = o[e] * a1 + __shfl_xor(o[e], msk) * a2;
    m = mn;
  }
  if (g == 0) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) s_o[w][D * hg + EPL * c + e] = o[e];
    if (c == 0) {
      s_m[w][hg] = m;
      s_l[w][hg] = l;
    }
  }
  __syncthreads();
  for (int t = tid; t < G * D; t += kThreads) {
    const int oh = t / D, col = t % D;  // head in the group, column
    if (h0 + oh >= p.H) continue;
    float M = kNegInf;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) M = fmaxf(M, s_m[i][oh]);
    float L = 0.0f, acc = 0.0f;
    if (M != kNegInf) {
#pragma unroll
      for (int i = 0; i < kWaves; ++i) {
        const float a = s_m[i][oh] == kNegInf ? 0.0f : fast_exp2(s_m[i][oh] - M);
        L += a * s_l[i][oh];
        acc += a * s_o[i][t];
      }
    }
    const int64_t ro = (((int64_t)s * p.B + b) * p.H + h0 + oh) * p.Nq;
    float out = L > 0.0f ? acc / L : 0.0f;
    if constexpr (FP8) out *= p.v_descale;
    p.o_part[ro * D + col] = out;
    if (col == 0) {
      float mref = M;  // the maximum in query-relative units
      if constexpr (ALIBI) mref -= p.alibi[h0 + oh] * kLog2e * (float)(ip - kref);
      p.lse_part[ro] = L > 0.0f ? (mref + __log2f(L)) * kLn2 : kNegInf;
    }
  }
}

template <int D, bool SOFTCAP, bool ALIBI, bool APPEND, bool WIDE>
__global__ __launch_bounds__(kThreads) void decode_bf16_kernel(FwdParams p) {
  decode_body<D, SOFTCAP, ALIBI, APPEND, false, WIDE>(p);
}

template <int D, bool SOFTCAP, bool ALIBI, bool WIDE>
__global__ __launch_bounds__(kThreads) void decode_fp8_kernel(FwdParams p) {
  decode_body<D, SOFTCAP, ALIBI, false, true, WIDE>(p);
}

// Workgroups of a decode launch: (head group, batch, split).
template <int D, int ESIZE, bool WIDE>
int64_t decode_groups(const FwdParams& p) {
  constexpr int G = DecodeGroup<D, ESIZE, WIDE>::G;
  return (int64_t)((p.H + G - 1) / G) * p.B * p.num_splits;
}

// Wide groups (twice the heads per workgroup: 512-byte segments of a key's
// rows) stream the cache 2-6% faster on MI355X at head_dim 128, but halve the
// workgroup count: they are used when the launch still has a workgroup per
// compute unit (256) and each split holds at least 1024 keys; smaller launches
// are latency-bound and keep 256-byte segments.
constexpr int64_t kWideMinGroups = 256;
constexpr int64_t kWideMinSplitKeys = 1024;
template <int D, int ESIZE>
bool decode_wide(const FwdParams& p) {
  if (D != 128) return false;
  const int64_t a = p.split_align;
  const int64_t chunk = ((p.Nk + (int64_t)p.num_splits - 1) / p.num_splits + a - 1) / a * a;
  return decode_groups<D, ESIZE, true>(p) >= kWideMinGroups && chunk >= kWideMinSplitKeys;
}

}  // namespace

template <int D, bool SOFTCAP, bool ALIBI>
int launch_decode_fp8(const FwdParams& p, void* stream) {
  if constexpr (D == 128) {
    if (decode_wide<D, 1>(p)) {
      const int64_t groups = decode_groups<D, 1, true>(p);
      hipLaunchKernelGGL((decode_fp8_kernel<D, SOFTCAP, ALIBI, true>), dim3((unsigned)groups),
                         dim3(kThreads), 0, (hipStream_t)stream, p);
      return (int)hipGetLastError();
    }
  }
  const int64_t groups = decode_groups<D, 1, false>(p);
  hipLaunchKernelGGL((decode_fp8_kernel<D, SOFTCAP, ALIBI, false>), dim3((unsigned)groups),
                     dim3(kThreads), 0, (hipStream_t)stream, p);
  return (int)hipGetLastError();
}

template <int D, bool SOFTCAP, bool ALIBI, bool APPEND>
int launch_decode_bf16(const FwdParams& p, void* stream) {
  if constexpr (D == 128) {
    if (decode_wide<D, 2>(p)) {
      const int64_t groups = decode_groups<D, 2, true>(p);
      hipLaunchKernelGGL((decode_bf16_kernel<D, SOFTCAP, ALIBI, APPEND, true>),
                         dim3((unsigned)groups), dim3(kThreads), 0, (hipStream_t)stream, p);
      return (int)hipGetLastError();
    }
  }
  const int64_t groups = decode_groups<D, 2, false>(p);
  hipLaunchKernelGGL((decode_bf16_kernel<D, SOFTCAP, ALIBI, APPEND, false>),
                     dim3((unsigned)groups), dim3(kThreads), 0, (hipStream_t)stream, p);
  return (int)hipGetLastError();
}

#define FA_INST(D, SC, AL) \
  template int launch_decode_bf16<D, SC, AL, false>(const FwdParams&, void*); \
  template int launch_decode_bf16<D, SC, AL, true>(const FwdParams&, void*); \
  template int launch_decode_fp8<D, SC, AL>(const FwdParams&, void*);
FA_INST(64, false, false)
FA_INST(64, false, true)
FA_INST(64, true, false)
FA_INST(64, true, true)
FA_INST(128, false, false)
FA_INST(128, false, true)
FA_INST(128, true, false)
FA_INST(128, true, true)

}  // namespace fa
