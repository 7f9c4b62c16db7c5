// Device helpers shared by the gfx950 attention kernels.
//
// Register layout used throughout: the score tile is computed transposed,
// S^T = K Q^T, with the 32x32 MFMA output layout of CDNA: lane l owns output
// column l % 32 (one query row) and, in its 16 accumulator slots v = 0..15,
// the rows (keys) 8*(v/4) + 4*(l/32) + (v%4). A query row therefore lives in
// two lanes (l and l ^ 32), so every softmax reduction is in-lane except one
// exchange between the two wave halves.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_params.h"

namespace fa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));

// Reinterpret one 32-bit word as two bf16. Takes the word by value: applying
// __builtin_bit_cast directly to a vector subscript (v[e]) inside an unrolled
// loop was seen to read element 0 for every e with this toolchain.
__device__ __forceinline__ bf16x2_t as_bf16x2(unsigned w) { return __builtin_bit_cast(bf16x2_t, w); }

// ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives element
// i % 4 of the 8-byte chunks addressed by lanes i/4, i/4 + 4, i/4 + 8, i/4 + 12.
__device__ __forceinline__ s16x4_t ds_read_tr16(const uint16_t* lds_ptr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4_t*)(lds_ptr));
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// Lazy running maximum: the exponent base is only moved when a tile's maximum
// exceeds it by more than this many powers of two, so most tiles skip
// rescaling the output accumulator. Used where P stays fp32. Where P is rounded
// to bf16 the base must be the exact running maximum (threshold 0): then the
// largest probability of a row is exactly 1 and rounds without error, which
// keeps the bf16 rounding error of O well inside its bound.
constexpr float kLazyRescaleThreshold = 8.0f;

// Key offset (within a 32-key block) held in accumulator slot v of a lane in half h2.
__device__ __forceinline__ constexpr int acc_key(int v, int h2) {
  return 8 * (v >> 2) + 4 * h2 + (v & 3);
}

// Reductions over the lane pair (l, l ^ 32) that holds one query row, on the
// VALU lane-swap (v_permlane32_swap) rather than the LDS crossbar: with both
// operands = x it returns {x[l & 31], x[(l & 31) + 32]} in every lane.
__device__ __forceinline__ float half_max(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Keys that rows [r0, r1) may see, as the union [lo, hi) and the
// intersection [flo, fhi) over the rows (bottom-right aligned: i' = i + off).
struct KeyBounds {
  int lo, hi, flo, fhi;
};

__device__ __forceinline__ KeyBounds key_bounds(int r0, int r1, int off, int slo, int shi,
                                                int wl, int wr) {
  KeyBounds kb;
  kb.lo = slo;
  kb.hi = shi;
  kb.flo = slo;
  kb.fhi = shi;
  if (wl >= 0) {
    kb.lo = max(kb.lo, r0 + off - wl);
    kb.flo = max(kb.flo, r1 - 1 + off - wl);
  }
  if (wr >= 0) {
    kb.hi = min(kb.hi, r1 - 1 + off + wr + 1);
    kb.fhi = min(kb.fhi, r0 + off + wr + 1);
  }
  return kb;
}

// ALiBi anchor of a row: its diagonal position i' clamped into its visible keys
// [lo, hi). For every visible key j, |i' - j| = |i' - a| + |a - j|, so biases
// measured from the anchor give the same softmax over the row's keys, and the
// dropped constant slope * |i' - a| is subtracted from the row's log-sum-exp.
// In a key split far from the row, the keys that carry the split's weight then
// keep small biases instead of thousands of log2 units (where fp32 resolves
// only ~1e-4).
__device__ __forceinline__ int alibi_anchor(int ip, const KeyBounds& rk) {
  return rk.hi > rk.lo ? min(max(ip, rk.lo), rk.hi - 1) : ip;
}

// Score units. Without a softcap or ALiBi the kernels keep the raw dot product
// q.k and fold softmax_scale * log2(e) into the exponent (one FMA per score);
// with either transform the transform itself yields log2-domain scores and the
// exponent factor is 1. Probabilities are exp2(c * (t - m)).
template <bool SOFTCAP, bool ALIBI>
__device__ __forceinline__ float exponent_scale(const FwdParams& p) {
  return (SOFTCAP || ALIBI) ? 1.0f : p.scale_log2;
}

// Score transform for one tile held as NB 32-key blocks of accumulators:
// optional tanh cap (on the scaled score), optional ALiBi distance penalty,
// optional mask to [row_lo, row_hi).
template <int NB, bool SOFTCAP, bool ALIBI>
__device__ __forceinline__ void transform_scores(float (&t)[NB][16], const FwdParams& p,
                                                 float slope_log2, float rel_pos,
                                                 bool need_mask, int key0, int row_lo,
                                                 int row_hi, int h2) {
  if constexpr (SOFTCAP) {
    // tanh(y) = 1 - 2 / (exp(2y) + 1), evaluated with exp2 and a reciprocal in
    // three passes over the tile. Each pass holds NB * 16 independent operations,
    // so no instruction waits for a transcendental issued just before it (taken
    // score by score, the schedule keeps two scores in flight and stalls on every
    // exponential and reciprocal). Same operations per score, same results.
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) t[j][v] = fast_exp2(t[j][v] * p.scale_over_cap2);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) t[j][v] = __builtin_amdgcn_rcpf(t[j][v] + 1.0f);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < NB; ++j) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float x = p.softcap_log2 - 2.0f * p.softcap_log2 * t[j][v];
        if constexpr (ALIBI) {
          // rel_pos = (i + off) - (key0 + 4*h2): distance to the key = rel_pos - offset.
          const float dist = rel_pos - (float)(32 * j + 8 * (v >> 2) + (v & 3));
          x -= slope_log2 * __builtin_fabsf(dist);
        }
        t[j][v] = x;
      }
    }
  } else if constexpr (ALIBI) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        // rel_pos = (i + off) - (key0 + 4*h2): distance to the key = rel_pos - offset.
        const float dist = rel_pos - (float)(32 * j + 8 * (v >> 2) + (v & 3));
        float x = t[j][v] * p.scale_log2;
        x -= slope_log2 * __builtin_fabsf(dist);
        t[j][v] = x;
      }
    }
  }
  if (need_mask) {
    // key = key0 + 4*h2 + kk with kk a compile-time offset per slot: compare kk
    // against this lane's bounds shifted by key0 + 4*h2.
    const int lo_rel = row_lo - key0 - 4 * h2;
    const int hi_rel = row_hi - key0 - 4 * h2;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int kk = 32 * j + 8 * (v >> 2) + (v & 3);
        if (kk < lo_rel || kk >= hi_rel) t[j][v] = kNegInf;
      }
    }
  }
}

// Online softmax step for this lane's row. m_run is the running max in score
// units; it moves when the tile max exceeds it by more than `threshold`
// (score units). Returns the factor for the output accumulator and sets
// `mc` = c * m_run (0 while the row has seen no key) for the exponent FMA.
template <int NB>
__device__ __forceinline__ float online_max(const float (&t)[NB][16], float c, float& m_run,
                                            float& l_run, bool& any_rescale, float& mc,
                                            float threshold) {
  // Four independent partial maxima keep the dependent chain short.
  float m4[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) m4[v & 3] = fmaxf(m4[v & 3], t[j][v]);
  float mt = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
  mt = half_max(mt);
  const float m_new = fmaxf(m_run, mt);
  const bool need = m_new > m_run + threshold;
  float alpha = 1.0f;
  if (need) {
    alpha = fast_exp2((m_run - m_new) * c);  // 0 when m_run is still -inf
    m_run = m_new;
  }
  l_run *= alpha;
  any_rescale = __any(need);
  mc = (m_run == kNegInf) ? 0.0f : m_run * c;
  return alpha;
}

// Row-sum of 8 bf16 values (the rounded probabilities fed to the PV product).
__device__ __forceinline__ float sum_bf16x8(bf16x8_t v, float acc) {
  const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    bf16x2_t pr = {v[2 * e], v[2 * e + 1]};
    acc = __builtin_amdgcn_fdot2_f32_bf16(pr, one, acc, false);
  }
  return acc;
}

// The sequence a workgroup works on: its lengths and where its rows sit.
struct SeqInfo {
  int nq, nk;       // query rows and keys of this sequence
  int n_cached;     // keys [0, n_cached) come from k/v, keys [n_cached, nk) from k_new/v_new
  int64_t q_row0;   // row (of H * D elements) of query 0 in q and o
  int64_t k_row0;   // row of key 0 in contiguous or packed k and v
  int64_t lse0;     // lse index of (this head, query 0); the sequence's rows follow
};

// Packed batches read their offsets from cu_seqlens_q/k, clamped into the
// tensors and to the stated maxima, so that any contents keep every access in
// bounds. A batched layout may carry per-sequence key counts (clamped to Nk).
__device__ __forceinline__ SeqInfo seq_info(const FwdParams& p, int b, int h) {
  SeqInfo si;
  if (p.cu_seqlens_q) {
    const int q0 = min(max(p.cu_seqlens_q[b], 0), p.total_q);
    const int q1 = min(max(p.cu_seqlens_q[b + 1], q0), p.total_q);
    const int k0 = min(max(p.cu_seqlens_k[b], 0), p.total_k);
    const int k1 = min(max(p.cu_seqlens_k[b + 1], k0), p.total_k);
    si.nq = min(q1 - q0, p.Nq);
    si.nk = min(k1 - k0, p.Nk);
    si.n_cached = si.nk;
    si.q_row0 = q0;
    si.k_row0 = k0;
    si.lse0 = (int64_t)h * p.total_q + q0;
  } else {
    si.nq = p.Nq;
    int n = p.seqlens_k ? min(max(p.seqlens_k[b], 0), p.Nk) : p.Nk;
    if (p.k_new) {
      // Append: the Nq new keys follow the cached ones and must fit in Nk.
      n = min(n, p.Nk - p.Nq);
      si.n_cached = n;
      n += p.Nq;
    } else if (p.appended) {
      // After a separate append of `appended` rows: the same counts, every key
      // now in the cache.
      n = min(n, p.Nk - p.appended) + p.appended;
      si.n_cached = n;
    } else {
      si.n_cached = n;
    }
    si.nk = n;
    si.q_row0 = (int64_t)b * p.Nq;
    si.k_row0 = (int64_t)b * p.Nk;
    si.lse0 = ((int64_t)b * p.H + h) * p.Nq;
  }
  return si;
}

__device__ __forceinline__ int64_t q_offset(const FwdParams& p, const SeqInfo& si, int row, int h,
                                            int D) {
  return ((si.q_row0 + row) * p.H + h) * D;
}

// Physical element offset of logical key `key` of sequence b, head h, in a page pool.
__device__ __forceinline__ int64_t page_offset(const FwdParams& p, int b, int key, int h, int D) {
  int idx, slot;
  if (p.page_shift >= 0) {
    idx = key >> p.page_shift;
    slot = key & (p.page_size - 1);
  } else {
    idx = key / p.page_size;
    slot = key - idx * p.page_size;
  }
  const int page = p.block_table[(int64_t)b * p.max_pages + idx];
  return (((int64_t)page * p.page_size + slot) * p.H + h) * D;
}

template <bool PAGED>
__device__ __forceinline__ int64_t kv_offset(const FwdParams& p, int b, const SeqInfo& si, int key,
                                             int h, int D) {
  if constexpr (PAGED) {
    return page_offset(p, b, key, h, D);
  } else {
    return ((si.k_row0 + key) * p.H + h) * D;
  }
}

// Append: copy the Nq new key and value rows of (b, h) into their cache pages,
// logical keys [n_cached, n_cached + Nq), in 16-byte pieces (T: element type).
// Within the launch no workgroup reads those cache rows (new keys are read from
// k_new / v_new), so exactly one workgroup per (b, h) may write them at any time.
template <typename T>
__device__ void append_rows(const FwdParams& p, const SeqInfo& si, int b, int h, int D, int tid,
                            int nthreads) {
  constexpr int EPC = 16 / sizeof(T);
  const int cpr = D / EPC;
  for (int idx = tid; idx < p.Nq * cpr; idx += nthreads) {
    const int i = idx / cpr, c = idx - (idx / cpr) * cpr;
    const int64_t dst = page_offset(p, b, si.n_cached + i, h, D) + c * EPC;
    const int64_t src = (((int64_t)b * p.Nq + i) * p.H + h) * D + c * EPC;
    *(u32x4_t*)((T*)const_cast<void*>(p.k) + dst) = *(const u32x4_t*)((const T*)p.k_new + src);
    *(u32x4_t*)((T*)const_cast<void*>(p.v) + dst) = *(const u32x4_t*)((const T*)p.v_new + src);
  }
}

// Element offset of appended key `key` (>= n_cached) of (b, h) in k_new / v_new.
__device__ __forceinline__ int64_t new_key_offset(const FwdParams& p, const SeqInfo& si, int b,
                                                  int key, int h, int D) {
  return (((int64_t)b * p.Nq + (key - si.n_cached)) * p.H + h) * D;
}

// Keys [slo, shi) of split s of a sequence with nk keys: chunks of
// ceil(nk / num_splits) keys rounded up to a multiple of split_align.
__device__ __forceinline__ void split_range(const FwdParams& p, int nk, int s, int& slo, int& shi) {
  const int64_t a = p.split_align;
  const int64_t c = ((nk + (int64_t)p.num_splits - 1) / p.num_splits + a - 1) / a * a;
  const int64_t lo = (int64_t)s * c;
  slo = (int)min<int64_t>(nk, lo);
  shi = (int)min<int64_t>(nk, lo + c);
}

// Store one lane's 4 consecutive output values of a row (normalised).
__device__ __forceinline__ void store_out4(const FwdParams& p, int64_t off, float a, float b,
                                           float c, float d) {
  if (p.o_bf16) {
    f32x4_t x = {a, b, c, d};
    typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
    bf16x4_t y = __builtin_convertvector(x, bf16x4_t);
    *(bf16x4_t*)((__bf16*)p.o + off) = y;
  } else {
    f32x4_t x = {a, b, c, d};
    *(f32x4_t*)((float*)p.o + off) = x;
  }
}

// Output of a workgroup whose rows see no key at all: O = 0, LSE = -inf.
template <bool PAGED>
__device__ void write_empty_rows(const FwdParams& p, const SeqInfo& si, int b, int h, int s,
                                 int q0, int q1, int D, int tid, int nthreads) {
  const int n = (q1 - q0) * D;
  for (int idx = tid; idx < n; idx += nthreads) {
    const int row = q0 + idx / D, d = idx % D;
    if constexpr (PAGED) {
      p.o_part[((((int64_t)s * p.B + b) * p.H + h) * p.Nq + row) * D + d] = 0.0f;
    } else {
      const int64_t o = q_offset(p, si, row, h, D) + d;
      if (p.o_bf16)
        ((__bf16*)p.o)[o] = (__bf16)0.0f;
      else
        ((float*)p.o)[o] = 0.0f;
    }
  }
  for (int row = q0 + tid; row < q1; row += nthreads) {
    if constexpr (PAGED) {
      p.lse_part[(((int64_t)s * p.B + b) * p.H + h) * p.Nq + row] = kNegInf;
    } else if (p.lse) {
      p.lse[si.lse0 + row] = kNegInf;
    }
  }
}

// Decode the flat workgroup id: head fastest, then batch, then split, then the
// query tile counted from the sequence's last (heaviest) tile.
struct WorkItem {
  int h, b, s, rank;
};
template <bool PAGED>
__device__ __forceinline__ WorkItem decode_work(const FwdParams& p) {
  WorkItem w;
  int L = blockIdx.x;
  w.h = L % p.H;
  L /= p.H;
  w.b = L % p.B;
  L /= p.B;
  w.s = 0;
  if constexpr (PAGED) {
    w.s = L % p.num_splits;
    L /= p.num_splits;
  }
  w.rank = L;
  return w;
}

// Query tile of a work item in a sequence of nq rows, counted from the last
// tile: of the sequence in a batched layout, of the longest sequence
// (num_q_tiles - 1 - rank) in a packed one, so that a packed batch runs its
// tiles in one order of absolute position (under a causal mask, heaviest
// first across the whole pack). Negative when the sequence has no such tile.
__device__ __forceinline__ int query_tile(const FwdParams& p, const WorkItem& w, int nq,
                                          int tile_rows) {
  const int qt = p.cu_seqlens_q ? p.num_q_tiles - 1 - w.rank
                                : (nq + tile_rows - 1) / tile_rows - 1 - w.rank;
  return qt * tile_rows < nq ? qt : -1;
}

}  // namespace fa
