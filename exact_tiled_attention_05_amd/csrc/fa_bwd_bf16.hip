// Backward pass of the bf16 tiled attention for gfx950 (MI355X).
//
// The probabilities are recomputed from the forward's per-row log-sum-exp
// instead of being stored, so no Nq x Nk matrix reaches device memory in this
// direction either ("IO感知技术革命: FlashAttention如何重塑大模型训练的经济学", the
// sections on tiling and on O(N) memory; the backward is what its training
// figures run on). Three launches, none with atomics: every gradient element
// is produced by one workgroup in one fixed order, so the pass is
// deterministic by construction (the update article lists a deterministic
// backward under v2.4).
//
//   1. prep:  D_i = dO_i . O_i and the LSE in log2 units (+inf for a row with
//             no key, so that its probabilities come out 0).
//   2. dK/dV: one workgroup per (key tile, head, batch), keys in lanes (32 per
//             wavefront): K as the B operand of S = Q K^T in registers, V as the
//             B operand of dP = dO V^T (in registers at head_dim 128, in LDS at
//             64), walking the 32-row query blocks that see the keys:
//               P = exp2(S' - LSE2), dS = P (dP - D), dZ = dS (1 - tanh^2) with a cap,
//               dV^T += dO^T P and dK^T += Q^T dZ, the transposed dO and Q read
//               from LDS with ds_read_b64_tr_b16. At head_dim 128 (64-key tiles)
//               two wavefronts share each 32-key group (one for S, P, dV; one for
//               dP, dZ, dK); at head_dim 64 (128-key tiles) one wavefront does all of it.
//   3. dQ:    one workgroup per (128-row query tile, head, batch), laid out as
//             the forward (a query row per lane pair): S^T = K Q^T and
//             dP^T = V dO^T with Q and dO in registers, dQ^T += K^T dZ^T with K
//             read transposed from LDS.
// All products run on v_mfma_f32_32x32x16_bf16 with fp32 accumulation; P and
// dZ are rounded to bf16 (nearest even) as MFMA operands. K/V (dQ) and Q/dO
// (dK/dV) tiles travel HBM -> LDS with buffer loads that write LDS directly,
// two stages deep, in the forward's swizzled layout.
#include <hip/hip_runtime.h>

#include <mutex>
#include <type_traits>

#include "fa_device.h"
#include "fa_lds.h"
#include "fa_noalloc.h"

namespace fa {

namespace {

constexpr int kThreads = 256;  // 4 wavefronts
constexpr int kBQ = 32;        // query rows per dK/dV step
constexpr int kBN = 64;        // keys per dQ step
constexpr int kBK = BWD_BK;    // keys per dK/dV workgroup (32 per wavefront)
constexpr int kBM = BWD_BM;    // query rows per dQ workgroup (32 per wavefront)
constexpr float kInf = __builtin_inff();

// The sequence of (b, h): its lengths and where its rows sit. A packed batch
// reads its offsets from cu_seqlens_q/k, clamped into the tensors and to the
// maxima so that any contents keep every access in bounds.
struct BwdSeq {
  int nq, nk;
  int64_t q_row0, k_row0;  // rows (of H * D elements) of query 0 and key 0
  int64_t lse0;            // lse index of (h, query 0)
};
__device__ __forceinline__ BwdSeq bwd_seq(const BwdParams& p, int b, int h) {
  BwdSeq s;
  if (p.cu_seqlens_q) {
    const int q0 = min(max(p.cu_seqlens_q[b], 0), p.total_q);
    const int q1 = min(max(p.cu_seqlens_q[b + 1], q0), p.total_q);
    const int k0 = min(max(p.cu_seqlens_k[b], 0), p.total_k);
    const int k1 = min(max(p.cu_seqlens_k[b + 1], k0), p.total_k);
    s.nq = min(q1 - q0, p.Nq);
    s.nk = min(k1 - k0, p.Nk);
    s.q_row0 = q0;
    s.k_row0 = k0;
    s.lse0 = (int64_t)h * p.total_q + q0;
  } else {
    s.nq = p.Nq;
    s.nk = p.Nk;
    s.q_row0 = (int64_t)b * p.Nq;
    s.k_row0 = (int64_t)b * p.Nk;
    s.lse0 = ((int64_t)b * p.H + h) * p.Nq;
  }
  return s;
}

__device__ __forceinline__ float bf16_lo(unsigned w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// ---------------------------------------------------------------------------
// 1. Row terms: per (b, h) and block of 32 query rows, LSE * log2(e) for the 32
//    rows (+inf for a row with no key, so its probabilities come out 0, and for
//    rows past Nq) and then D = rowsum(dO * O) (0 past Nq). LPR lanes per row,
//    8 elements each; rows run fastest within a (b, h).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_prep_kernel(BwdParams p) {
  constexpr int LPR = D / 8;
  constexpr int RPB = kThreads / LPR;
  const int tid = threadIdx.x, c = tid % LPR;
  const int nqp = p.nblk * BWD_RB;
  const int64_t slot = (int64_t)blockIdx.x * RPB + tid / LPR;  // (b * H + h) * nqp + i
  const bool ok = slot < (int64_t)p.B * p.H * nqp;
  const int i = (int)(slot % nqp);
  const int64_t bh = slot / nqp;
  const int h = (int)(bh % p.H), b = (int)(bh / p.H);
  const BwdSeq sq = bwd_seq(p, ok ? b : 0, h);
  const bool live = ok && i < sq.nq;
  float acc = 0.0f;
  if (live) {
    const int64_t e = ((sq.q_row0 + i) * p.H + h) * D + 8 * c;
    const u32x4_t g = *(const u32x4_t*)((const uint16_t*)p.dout + e);
    float o[8];
    if (p.o_bf16) {
      const u32x4_t x = *(const u32x4_t*)((const uint16_t*)p.o + e);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        o[2 * k] = bf16_lo(x[k]);
        o[2 * k + 1] = bf16_hi(x[k]);
      }
    } else {
      const f32x4_t x0 = *(const f32x4_t*)((const float*)p.o + e);
      const f32x4_t x1 = *(const f32x4_t*)((const float*)p.o + e + 4);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        o[k] = x0[k];
        o[4 + k] = x1[k];
      }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) acc += bf16_lo(g[k]) * o[2 * k] + bf16_hi(g[k]) * o[2 * k + 1];
  }
#pragma unroll
  for (int m = 1; m < LPR; m <<= 1) acc += __shfl_xor(acc, m);
  if (ok && c == 0) {
    float l2 = kInf;
    if (live) {
      const float l = p.lse[sq.lse0 + i];
      l2 = l == kNegInf ? kInf : l * kLog2e;
    }
    float* rt = p.rowterms + (bh * p.nblk + i / BWD_RB) * (2 * BWD_RB) + i % BWD_RB;
    rt[0] = l2;
    rt[BWD_RB] = acc;
  }
}

// Score in log2 units for a raw product s = q.k: scaled, capped (th = the tanh
// value, for the cap's derivative), ALiBi-shifted by dist = |i + off - j|.
template <bool SOFTCAP, bool ALIBI>
__device__ __forceinline__ float bwd_score(const BwdParams& p, float s, float slope_log2,
                                           float dist, float& th) {
  float x;
  if constexpr (SOFTCAP) {
    const float e = fast_exp2(s * p.scale_over_cap2);
    th = 1.0f - 2.0f * __builtin_amdgcn_rcpf(e + 1.0f);
    x = p.softcap_log2 * th;
  } else {
    th = 0.0f;
    x = s * p.scale_log2;
  }
  if constexpr (ALIBI) x -= slope_log2 * dist;
  return x;
}

// Queries that may see key j: [lo, hi), bottom-right aligned (off = Nk - Nq).
__device__ __forceinline__ void query_range(int j, int off, int nq, int wl, int wr, int& lo,
                                            int& hi) {
  lo = wr >= 0 ? max(0, j - off - wr) : 0;
  hi = wl >= 0 ? min(nq, j - off + wl + 1) : nq;
  hi = max(hi, lo);
}

// Store 4 consecutive gradient values (scaled) as fp32 or bf16.
__device__ __forceinline__ void store_grad4(void* base, int bf16, int64_t off, float a, float b,
                                            float c, float d) {
  f32x4_t x = {a, b, c, d};
  if (bf16) {
    typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
    *(bf16x4_t*)((__bf16*)base + off) = __builtin_convertvector(x, bf16x4_t);
  } else {
    *(f32x4_t*)((float*)base + off) = x;
  }
}

// Zero rows [r0, r1) of a [B, N, H, D] gradient for (b, h), NT threads.
template <int NT>
__device__ void zero_rows(void* base, int bf16, int64_t row0, int h, int H, int D, int r0, int r1,
                          int tid) {
  const int n = (r1 - r0) * D / 4;
  for (int idx = tid; idx < n; idx += NT) {
    const int row = r0 + idx / (D / 4), c = idx % (D / 4);
    store_grad4(base, bf16, ((row0 + row) * H + h) * D + 4 * c, 0.f, 0.f, 0.f, 0.f);
  }
}

// ---------------------------------------------------------------------------
// 2. dK and dV (head_dim 128)
//
// Four wavefronts: two key groups of 32 keys (the workgroup's 64 keys) times
// two roles. Role 0 (S, P, dV): S = Q K^T with K in registers, P = exp2(S' -
// LSE2) under the mask, dV^T += dO^T P; it also publishes P' = P (1 - tanh^2
// with a cap, 1 without) in fp32 through LDS. Role 1 (dP, dZ, dK): dP = dO V^T
// with V in registers, and one block behind, dZ = P' (dP - D) and dK^T += Q^T
// dZ. The 32-row query blocks (Q, dO, row terms) cycle through three LDS
// stages, the copy of block t+1 issued in step t, so block t-1 is still
// resident while role 1 finishes it. 65 KiB of LDS and 256 registers per lane
// let two workgroups share a CU: each SIMD then runs one wavefront of each, and
// the two workgroups' barriers are independent of each other.
// ---------------------------------------------------------------------------
constexpr int kDkdvThreads = 256;
constexpr int kDkdvGroups = 2;                   // key groups of 32 per workgroup
constexpr int kDkdvKeys = 32 * kDkdvGroups;      // keys per workgroup (head_dim 128)

// LDS of the head_dim-128 dK/dV workgroup: three Q and three dO stages, two P'
// buffers and three row-term stages, in that order.
constexpr int kDkdvLdsBytes = 6 * (BWD_RB * 128 * 2) + 2 * (kDkdvGroups * 16 * 64 * 4) + 3 * (2 * BWD_RB * 4);

// dK/dV of key tile `block` (flat index, head fastest) with its LDS at `lds`.
template <int D, bool SOFTCAP, bool ALIBI>
__device__ __forceinline__ void bwd_dkdv_body(const BwdParams& p, int block, char* lds) {
  constexpr int KS = D / 16;               // k-steps over head_dim
  constexpr int NDB = D / 32;              // 32-row blocks of dK^T / dV^T
  constexpr int CPR = D / 8;               // 16-byte chunks per row
  constexpr int RPL = 64 / CPR;            // rows per wavefront-wide copy
  constexpr int QL = kBQ / RPL / kDkdvGroups;  // copies per wavefront of its role's tensor per block
  static_assert(QL >= 1 && kBQ == BWD_RB, "tile shape");
  constexpr int QT = kBQ * D;
  constexpr int kSReadAhead = 3;           // k-steps of dO operands read ahead in dP
  constexpr int kReadAhead = 8;            // transposed-read MFMAs in flight (all of a product's)
  static_assert(kReadAhead <= 2 * (D / 32), "read-ahead");
  constexpr int XG = 16 * 64;              // floats of P' per key group

  static_assert(D == 128, "layout of kDkdvLdsBytes");
  uint16_t* const sQ0 = (uint16_t*)lds;  // 1024-byte aligned, as every stage below
  uint16_t* const sQ1 = sQ0 + QT;
  uint16_t* const sQ2 = sQ1 + QT;
  uint16_t* const sG0 = sQ2 + QT;  // dO
  uint16_t* const sG1 = sG0 + QT;
  uint16_t* const sG2 = sG1 + QT;
  float* const sX0 = (float*)(sG2 + QT);      // P' of even blocks
  float* const sX1 = sX0 + kDkdvGroups * XG;  // P' of odd blocks
  float* const sR0 = sX1 + kDkdvGroups * XG;  // LSE2 | D
  float* const sR1 = sR0 + 2 * kBQ;
  float* const sR2 = sR1 + 2 * kBQ;

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, r = lane & 31, h2 = lane >> 5;
  const int grp = w & (kDkdvGroups - 1);
  const int role = __builtin_amdgcn_readfirstlane(w / kDkdvGroups);
  int L = block;
  const int h = L % p.H;
  L /= p.H;
  const int b = L % p.B;
  const int kt = L / p.B;  // ascending: under causal the first key tile is seen by the most rows
  const BwdSeq sq = bwd_seq(p, b, h);
  const int nq = sq.nq, nk = sq.nk, off = nk - nq;
  const int wl = p.window_left, wr = p.window_right;
  const int k0 = kt * kDkdvKeys, k1 = min(nk, k0 + kDkdvKeys);
  if (k0 >= nk) return;  // past the keys (a packed sequence shorter than the longest)

  // Query rows the workgroup's keys are seen by (union over its keys).
  int ulo, uhi, tmp;
  query_range(k0, off, nq, wl, wr, ulo, tmp);
  query_range(k1 - 1, off, nq, wl, wr, tmp, uhi);
  uhi = max(uhi, ulo);
  if (uhi <= ulo) {
    zero_rows<kDkdvThreads>(p.dk, p.g_bf16, sq.k_row0, h, p.H, D, k0, k1, tid);
    zero_rows<kDkdvThreads>(p.dv, p.g_bf16, sq.k_row0, h, p.H, D, k0, k1, tid);
    return;
  }

  // This group's keys: the union [wlo, whi) and intersection [wflo, wfhi) of
  // their query ranges; this lane's key and its own range [rlo, rhi).
  const int kw0 = k0 + 32 * grp, kw1 = min(k1, kw0 + 32);
  const bool group_live = kw0 < k1;
  int wlo = 0, whi = 0, wflo = 0, wfhi = 0;
  if (group_live) {
    query_range(kw0, off, nq, wl, wr, wlo, wfhi);
    query_range(kw1 - 1, off, nq, wl, wr, wflo, whi);
  }
  const bool group_full = kw1 - kw0 == 32;
  const int key = kw0 + r;
  int rlo = 0, rhi = 0;
  if (key < k1) query_range(key, off, nq, wl, wr, rlo, rhi);
  auto live = [&](int qb) __attribute__((always_inline)) {
    return group_live && qb < whi && qb + kBQ > wlo;
  };

  // This lane's key row of K (role 0) or V (role 1), columns 16ks + 8h2 .. +7:
  // the B operand of S = Q K^T and of dP = dO V^T (zero past Nk).
  bf16x8_t kvf[KS];
  {
    const uint16_t* kp = (const uint16_t*)(role == 0 ? p.k : p.v) +
                         ((sq.k_row0 + min(key, nk - 1)) * p.H + h) * D + 8 * h2;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4_t x = *(const u32x4_t*)(kp + 16 * ks);
      if (key >= k1) x = u32x4_t{0, 0, 0, 0};
      kvf[ks] = __builtin_bit_cast(bf16x8_t, x);
    }
  }

  // HBM -> LDS copies. Copy i of a wavefront with copy slot c fills rows
  // RPL*(QL*c + i) + lane/CPR, lane L the physical chunk L % CPR. Role 0 copies
  // Q, role 1 copies dO (two wavefronts each); every wavefront copies the
  // block's 64 row terms (identical values). Blocks past the range are not copied.
  const int64_t row_bytes = 2 * (int64_t)p.H * D;
  auto lane_off = [&](int ld) __attribute__((always_inline)) {
    const int trow = RPL * ld + lane / CPR;
    const int chunk = (lane % CPR) ^ swz<D>(trow);
    return (unsigned)(trow * row_bytes + 16 * chunk);
  };
  const int cs = __builtin_amdgcn_readfirstlane(grp);
  const char* tbh = (const char*)(role == 0 ? p.q : p.dout) + 2 * ((sq.q_row0 * p.H + h) * D);
  const int64_t qend = (int64_t)(nq - 1) * row_bytes + 2 * D;
  const float* rbh = p.rowterms + ((int64_t)b * p.H + h) * p.nblk * (2 * kBQ);
  const int qb_first = (ulo / kBQ) * kBQ;
  const int nblocks = (uhi - qb_first + kBQ - 1) / kBQ;
  auto copy_block = [&](uint16_t* dq_, uint16_t* dg_, float* dr_, int qb) __attribute__((always_inline)) {
    const int64_t tb = (int64_t)qb * row_bytes;
    const int64_t left = qend - tb;
    const int n = left <= 0 ? 0 : (left >= 0x7FFFFFFF ? 0x7FFFFFFF : (int)left);
    const __amdgpu_buffer_rsrc_t rt = make_rsrc(tbh + tb, n);
    uint16_t* dst = role == 0 ? dq_ : dg_;
#pragma unroll
    for (int i = 0; i < QL; ++i) buffer_load_lds16(rt, dst + 512 * (QL * cs + i), lane_off(QL * cs + i));
    const __amdgpu_buffer_rsrc_t rr = make_rsrc((const char*)(rbh + (int64_t)(qb / kBQ) * (2 * kBQ)), 8 * kBQ);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, (lds_ptr_t)dr_, 4, 4 * lane, 0, 0, 0);
  };

  const int gl = lane & 15, sub = (lane >> 4) & 1;
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  auto stq = [&](auto st) __attribute__((always_inline)) {
    constexpr int S = decltype(st)::value;
    return S == 0 ? sQ0 : S == 1 ? sQ1 : sQ2;
  };
  auto stg = [&](auto st) __attribute__((always_inline)) {
    constexpr int S = decltype(st)::value;
    return S == 0 ? sG0 : S == 1 ? sG1 : sG2;
  };
  auto str = [&](auto st) __attribute__((always_inline)) {
    constexpr int S = decltype(st)::value;
    return S == 0 ? sR0 : S == 1 ? sR1 : sR2;
  };
  // Issue the copies of block it + 1 into stage (S + 1) % 3 (held block it - 2).
  auto prefetch = [&](auto st, int it) __attribute__((always_inline)) {
    constexpr int S = decltype(st)::value;
    using N = std::integral_constant<int, (S + 1) % 3>;
    if (it + 1 < nblocks) copy_block(stq(N{}), stg(N{}), str(N{}), qb_first + (it + 1) * kBQ);
  };
  // Transposed head_dim x 16-row operand of k-step tt from a 32-row tile.
  auto tr_operand = [&](const uint16_t* t, int tt, int db) __attribute__((always_inline)) {
    const int vrow = 16 * tt + 4 * h2 + (gl >> 2);
    const int col = 32 * db + 16 * sub + 4 * (gl & 3);
    const s16x4_t lo = ds_read_tr16(t + tile_off<D>(vrow, col >> 3) + (col & 7));
    const s16x4_t hi = ds_read_tr16(t + tile_off<D>(vrow + 8, col >> 3) + (col & 7));
    const s16x8_t x = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8_t, x);
  };

  copy_block(sQ0, sG0, sR0, qb_first);
  wait_vmem_barrier<0>();  // K or V and block 0 have landed

  f32x16_t acc[NDB];  // dV^T (role 0) or dK^T (role 1)
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16_t{};

  if (role == 0) {
    // ---- role 0: S, P, dV
    float slope_log2 = 0.0f;
    if constexpr (ALIBI) slope_log2 = p.alibi[h] * kLog2e;
    auto compute = [&](auto masked_t, const uint16_t* sq, const uint16_t* sg, const float* sr,
                       float* sx, int qb) __attribute__((always_inline)) {
      constexpr bool MASKED = decltype(masked_t)::value;
      f32x16_t sacc = f32x16_t{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8_t aq =
            __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(sq + tile_off<D>(r, 2 * ks + h2)));
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, kvf[ks], sacc, 0, 0, 0);
      }
      // Slot v holds query qb + 8*(v/4) + 4*h2 + v%4 of this lane's key.
      const int lo_rel = rlo - qb - 4 * h2, hi_rel = rhi - qb - 4 * h2;
      const float rel = (float)(key - off - qb - 4 * h2);
      bf16x8_t pb[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        f32x8_t pa;
#pragma unroll
        for (int gg = 0; gg < 2; ++gg) {
          const int g = 2 * tt + gg;
          const f32x4_t l4 = *(const f32x4_t*)(sr + 8 * g + 4 * h2);
          f32x4_t px;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int v = 4 * g + e, kk = 8 * g + e;
            float th;
            const float x = bwd_score<SOFTCAP, ALIBI>(p, sacc[v], slope_log2,
                                                      __builtin_fabsf(rel - (float)kk), th);
            float pr = fast_exp2(x - l4[e]);
            if (MASKED && (kk < lo_rel || kk >= hi_rel)) pr = 0.0f;
            pa[4 * gg + e] = pr;
            px[e] = SOFTCAP ? pr * (1.0f - th * th) : pr;
          }
          *(f32x4_t*)(sx + 4 * (g * 64 + lane)) = px;
        }
        pb[tt] = __builtin_convertvector(pa, bf16x8_t);
      }
      // dV^T += dO^T P: k-step tt covers the block's queries 16tt + 4h2 + {0..3, 8..11}.
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand(sg, tt, db), pb[tt], acc[db], 0,
                                                            0, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * kReadAhead, 1);
#pragma unroll
      for (int i = 0; i < 2 * NDB - kReadAhead; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, kReadAhead, 1);
    };
    auto step = [&](auto st, int it) __attribute__((always_inline)) {
      const int qb = qb_first + it * kBQ;
      prefetch(st, it);
      if (live(qb)) {
        float* sx = (it & 1) ? sX1 : sX0;
        sx += grp * XG;
        if (group_full && qb >= wflo && qb + kBQ <= wfhi)
          compute(std::false_type{}, stq(st), stg(st), str(st), sx, qb);
        else
          compute(std::true_type{}, stq(st), stg(st), str(st), sx, qb);
      }
      wait_vmem_barrier<0>();  // block it + 1 has landed; P' of block it is visible
    };
#ifdef FA_SERIAL_COPIES
    // Verification build: one stage, each block copied, waited for and fenced by
    // barriers; role 1 finishes the block before the next copy. Three barriers per
    // block, as in role 1's loop below. The arithmetic and its order are unchanged.
    for (int it = 0; it < nblocks; ++it) {
      const int qb = qb_first + it * kBQ;
      copy_block(sQ0, sG0, sR0, qb);
      wait_vmem_barrier<0>();
      if (live(qb)) {
        if (group_full && qb >= wflo && qb + kBQ <= wfhi)
          compute(std::false_type{}, sQ0, sG0, sR0, sX0 + grp * XG, qb);
        else
          compute(std::true_type{}, sQ0, sG0, sR0, sX0 + grp * XG, qb);
      }
      __syncthreads();  // P' of the block is visible to role 1
      __syncthreads();  // role 1 is done with the block
    }
#else
    for (int it = 0; it < nblocks; it += 3) {
      step(I0{}, it);
      if (it + 1 < nblocks) step(I1{}, it + 1);
      if (it + 2 < nblocks) step(I2{}, it + 2);
    }
#endif
  } else {
    // ---- role 1: dP, then dZ and dK one block behind
    f32x16_t pprev = f32x16_t{};
    auto dp_block = [&](const uint16_t* sg) __attribute__((always_inline)) {
      f32x16_t pacc = f32x16_t{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8_t ag =
            __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(sg + tile_off<D>(r, 2 * ks + h2)));
        pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ag, kvf[ks], pacc, 0, 0, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, kSReadAhead, 2);
#pragma unroll
      for (int i = 0; i < KS - kSReadAhead; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 2);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 2);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, kSReadAhead, 2);
      return pacc;
    };
    // dZ = P' (dP - D) of a finished block and dK^T += Q^T dZ.
    auto dk_block = [&](const uint16_t* sq, const float* sr, const float* sx,
                        const f32x16_t& pacc) __attribute__((always_inline)) {
      bf16x8_t zb[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        f32x8_t za;
#pragma unroll
        for (int gg = 0; gg < 2; ++gg) {
          const int g = 2 * tt + gg;
          const f32x4_t d4 = *(const f32x4_t*)(sr + kBQ + 8 * g + 4 * h2);
          const f32x4_t px = *(const f32x4_t*)(sx + 4 * (g * 64 + lane));
#pragma unroll
          for (int e = 0; e < 4; ++e) za[4 * gg + e] = px[e] * (pacc[4 * g + e] - d4[e]);
        }
        zb[tt] = __builtin_convertvector(za, bf16x8_t);
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand(sq, tt, db), zb[tt], acc[db], 0,
                                                            0, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * kReadAhead, 3);
#pragma unroll
      for (int i = 0; i < 2 * NDB - kReadAhead; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 3);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 3);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, kReadAhead, 3);
    };
    auto step = [&](auto st, int it) __attribute__((always_inline)) {
      constexpr int S = decltype(st)::value;
      using P1 = std::integral_constant<int, (S + 2) % 3>;  // stage of block it - 1
      const int qb = qb_first + it * kBQ;
      prefetch(st, it);
      f32x16_t pcur = f32x16_t{};
      if (live(qb)) pcur = dp_block(stg(st));
      if (it > 0 && live(qb - kBQ)) {
        const float* sx = ((it - 1) & 1) ? sX1 : sX0;
        dk_block(stq(P1{}), str(P1{}), sx + grp * XG, pprev);
      }
      pprev = pcur;
      wait_vmem_barrier<0>();
    };
#ifdef FA_SERIAL_COPIES
    (void)pprev;
    for (int it = 0; it < nblocks; ++it) {
      const int qb = qb_first + it * kBQ;
      copy_block(sQ0, sG0, sR0, qb);
      wait_vmem_barrier<0>();
      f32x16_t pcur = f32x16_t{};
      if (live(qb)) pcur = dp_block(sG0);
      __syncthreads();  // role 0's P' of the block is visible
      if (live(qb)) dk_block(sQ0, sR0, sX0 + grp * XG, pcur);
      __syncthreads();
    }
#else
    for (int it = 0; it < nblocks; it += 3) {
      step(I0{}, it);
      if (it + 1 < nblocks) step(I1{}, it + 1);
      if (it + 2 < nblocks) step(I2{}, it + 2);
    }
    // The last block: its stage, row terms and P' are still resident.
    const int last = nblocks - 1;
    if (live(qb_first + last * kBQ)) {
      const int sl = last % 3;
      const uint16_t* sq = sl == 0 ? sQ0 : sl == 1 ? sQ1 : sQ2;
      const float* sr = sl == 0 ? sR0 : sl == 1 ? sR1 : sR2;
      const float* sx = (last & 1) ? sX1 : sX0;
      dk_block(sq, sr, sx + grp * XG, pprev);
    }
#endif
  }

  // Epilogue: lane = key, slots = head_dim rows 32db + 8g + 4h2 + {0..3}.
  if (key >= k1) return;
  const int64_t base = ((sq.k_row0 + key) * p.H + h) * D;
  void* dst = role == 0 ? p.dv : p.dk;
  const float sc = role == 0 ? 1.0f : p.scale;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      store_grad4(dst, p.g_bf16, base + 32 * db + 8 * g + 4 * h2, acc[db][4 * g] * sc,
                  acc[db][4 * g + 1] * sc, acc[db][4 * g + 2] * sc, acc[db][4 * g + 3] * sc);
}

// ---------------------------------------------------------------------------
// 2b. dK and dV with four wavefronts (head_dim 64)
//
// Each wavefront owns 32 keys and does both roles of the kernel above for them:
// S, dP, dV and dK per 32-row block, with the Q / dO / row-term blocks in a
// four-stage ring prefetched three blocks ahead. At head_dim 64 it needs no
// P' exchange, so its 50 KiB of LDS let two workgroups share a CU, which the
// split kernel's larger footprint does not.
// ---------------------------------------------------------------------------
// LDS of the head_dim-64 dK/dV workgroup: the V tile, four Q and four dO
// stages and four row-term stages, in that order.
constexpr int kW4LdsBytes = BWD_BK * 64 * 2 + 8 * (BWD_RB * 64 * 2) + 4 * (2 * BWD_RB * 4);

// dK/dV of key tile `block` (flat index, head fastest) with its LDS at `lds`.
template <int D, bool SOFTCAP, bool ALIBI>
__device__ __forceinline__ void bwd_dkdv_w4_body(const BwdParams& p, int block, char* lds) {
  constexpr int KS = D / 16;               // k-steps over head_dim
  constexpr int NDB = D / 32;              // 32-row blocks of dK^T / dV^T
  constexpr int CPR = D / 8;               // 16-byte chunks per row
  constexpr int RPL = 64 / CPR;            // rows per wavefront-wide copy
  constexpr int QLOADS = kBQ / RPL / 4;    // copies per wavefront per tensor per block
  constexpr int VLOADS = kBK / RPL / 4;    // copies per wavefront for the V tile
  static_assert(QLOADS >= 1 && VLOADS >= 1 && kBQ == BWD_RB, "tile shape");
  constexpr int QT = kBQ * D;
  // Vector-memory operations per wavefront per block: Q, dO and the row terms.
  constexpr int kCopies = 2 * QLOADS + 1;
  constexpr int kSReadAhead = 2;           // k-steps of S / dP operands read ahead
  constexpr int kReadAhead = 4;            // transposed-read MFMAs in flight

  // Q / dO / row-term blocks cycle through four stages: the copy of block t+3
  // is issued while block t is computed, so three blocks of copies are in flight.
  static_assert(D == 64, "layout of kW4LdsBytes");
  uint16_t* const sV = (uint16_t*)lds;  // 1024-byte aligned, as every stage below
  uint16_t* const sQ0 = sV + kBK * D;
  uint16_t* const sQ1 = sQ0 + QT;
  uint16_t* const sQ2 = sQ1 + QT;
  uint16_t* const sQ3 = sQ2 + QT;
  uint16_t* const sG0 = sQ3 + QT;  // dO
  uint16_t* const sG1 = sG0 + QT;
  uint16_t* const sG2 = sG1 + QT;
  uint16_t* const sG3 = sG2 + QT;
  float* const sR0 = (float*)(sG3 + QT);  // LSE2 | D
  float* const sR1 = sR0 + 2 * kBQ;
  float* const sR2 = sR1 + 2 * kBQ;
  float* const sR3 = sR2 + 2 * kBQ;

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, r = lane & 31, h2 = lane >> 5;
  int L = block;
  const int h = L % p.H;
  L /= p.H;
  const int b = L % p.B;
  const int kt = L / p.B;  // ascending: under causal the first key tile is seen by the most rows
  const BwdSeq sq = bwd_seq(p, b, h);
  const int nq = sq.nq, nk = sq.nk, off = nk - nq;
  const int wl = p.window_left, wr = p.window_right;
  const int k0 = kt * kBK, k1 = min(nk, k0 + kBK);
  if (k0 >= nk) return;  // a packed sequence shorter than the longest

  // Query rows the workgroup's keys are seen by (union over its keys).
  int ulo, uhi, tmp;
  query_range(k0, off, nq, wl, wr, ulo, tmp);
  query_range(k1 - 1, off, nq, wl, wr, tmp, uhi);
  uhi = max(uhi, ulo);
  if (uhi <= ulo) {
    zero_rows<kThreads>(p.dk, p.g_bf16, sq.k_row0, h, p.H, D, k0, k1, tid);
    zero_rows<kThreads>(p.dv, p.g_bf16, sq.k_row0, h, p.H, D, k0, k1, tid);
    return;
  }

  // This wavefront's keys: the union [wlo, whi) and intersection [wflo, wfhi)
  // of their query ranges; this lane's key and its own range [rlo, rhi).
  const int kw0 = k0 + 32 * w, kw1 = min(k1, kw0 + 32);
  const bool wave_live = kw0 < k1;
  int wlo = 0, whi = 0, wflo = 0, wfhi = 0;
  if (wave_live) {
    query_range(kw0, off, nq, wl, wr, wlo, wfhi);
    query_range(kw1 - 1, off, nq, wl, wr, wflo, whi);
  }
  const bool wave_full = kw1 - kw0 == 32;
  const int key = kw0 + r;
  int rlo = 0, rhi = 0;
  if (key < k1) query_range(key, off, nq, wl, wr, rlo, rhi);

  float slope_log2 = 0.0f;
  if constexpr (ALIBI) slope_log2 = p.alibi[h] * kLog2e;

  // K of this lane's key: columns 16ks + 8h2 .. +7 (B operand of S = Q K^T).
  bf16x8_t kf[KS];
  {
    const uint16_t* kp =
        (const uint16_t*)p.k + ((sq.k_row0 + min(key, nk - 1)) * p.H + h) * D + 8 * h2;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4_t x = *(const u32x4_t*)(kp + 16 * ks);
      if (key >= k1) x = u32x4_t{0, 0, 0, 0};
      kf[ks] = __builtin_bit_cast(bf16x8_t, x);
    }
  }

  // HBM -> LDS copies. Copy i of wavefront w fills rows RPL*(n*w + i) + lane/CPR
  // (n copies per wavefront), lane L the physical chunk L % CPR of its row.
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int64_t row_bytes = 2 * (int64_t)p.H * D;
  auto lane_off = [&](int ld) __attribute__((always_inline)) {
    const int trow = RPL * ld + lane / CPR;
    const int chunk = (lane % CPR) ^ swz<D>(trow);
    return (unsigned)(trow * row_bytes + 16 * chunk);
  };
  {
    // V tile of the workgroup's keys (rows past Nk arrive as zeros).
    const char* vb = (const char*)p.v + 2 * (((sq.k_row0 + k0) * p.H + h) * D);
    const int64_t left = (int64_t)(nk - 1 - k0) * row_bytes + 2 * D;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(vb, left >= 0x7FFFFFFF ? 0x7FFFFFFF : (int)left);
#pragma unroll
    for (int i = 0; i < VLOADS; ++i)
      buffer_load_lds16(rs, sV + 512 * (VLOADS * wu + i), lane_off(VLOADS * wu + i));
  }
  const char* qbh = (const char*)p.q + 2 * ((sq.q_row0 * p.H + h) * D);
  const char* gbh = (const char*)p.dout + 2 * ((sq.q_row0 * p.H + h) * D);
  const int64_t qend = (int64_t)(nq - 1) * row_bytes + 2 * D;
  const float* rbh = p.rowterms + ((int64_t)b * p.H + h) * p.nblk * (2 * kBQ);
  const int qb_first = (ulo / kBQ) * kBQ;
  const int nblocks = (uhi - qb_first + kBQ - 1) / kBQ;
  const int qb_end = qb_first + nblocks * kBQ;
  // Block starting at row qb into one stage. Every wavefront issues the same
  // number of operations for every block; blocks past the range read nothing
  // and write zeros (range-checked descriptors), which keeps the wait counts fixed.
  auto copy_block = [&](uint16_t* dq_, uint16_t* dg_, float* dr_, int qb) __attribute__((always_inline)) {
    const int64_t tb = (int64_t)qb * row_bytes;
    const int64_t left = qb < qb_end ? qend - tb : 0;
    const int n = left <= 0 ? 0 : (left >= 0x7FFFFFFF ? 0x7FFFFFFF : (int)left);
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(qbh + tb, n);
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(gbh + tb, n);
#pragma unroll
    for (int i = 0; i < QLOADS; ++i) {
      buffer_load_lds16(rq, dq_ + 512 * (QLOADS * wu + i), lane_off(QLOADS * wu + i));
      buffer_load_lds16(rg, dg_ + 512 * (QLOADS * wu + i), lane_off(QLOADS * wu + i));
    }
    // The block's 64 row terms, 4 bytes per lane (every wavefront writes the same values).
    const __amdgpu_buffer_rsrc_t rr =
        make_rsrc((const char*)(rbh + (int64_t)(qb / kBQ) * (2 * kBQ)), qb < qb_end ? 8 * kBQ : 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, (lds_ptr_t)dr_, 4, 4 * lane, 0, 0, 0);
  };

  f32x16_t dkacc[NDB], dvacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dkacc[db] = f32x16_t{};
    dvacc[db] = f32x16_t{};
  }
  const int gl = lane & 15, sub = (lane >> 4) & 1;

  auto compute = [&](auto masked_t, const uint16_t* sq, const uint16_t* sg, const float* sr,
                     int qb) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_t)::value;
    // S = Q K^T and dP = dO V^T for 32 queries x this wavefront's 32 keys.
    f32x16_t sacc = f32x16_t{}, pacc = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8_t aq = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(sq + tile_off<D>(r, 2 * ks + h2)));
      const bf16x8_t ag = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(sg + tile_off<D>(r, 2 * ks + h2)));
      const bf16x8_t bv =
          __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(sV + tile_off<D>(32 * w + r, 2 * ks + h2)));
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, kf[ks], sacc, 0, 0, 0);
      pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ag, bv, pacc, 0, 0, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 3 * kSReadAhead, 0);  // DS reads
#pragma unroll
    for (int i = 0; i < KS - kSReadAhead; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * kSReadAhead, 0);

    // Slot v holds query qb + 8*(v/4) + 4*h2 + v%4 of this lane's key.
    const int lo_rel = rlo - qb - 4 * h2, hi_rel = rhi - qb - 4 * h2;
    const float rel = (float)(key - off - qb - 4 * h2);
    bf16x8_t pb[2], zb[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      f32x8_t pa, za;
#pragma unroll
      for (int gg = 0; gg < 2; ++gg) {
        const int g = 2 * tt + gg;
        const f32x4_t l4 = *(const f32x4_t*)(sr + 8 * g + 4 * h2);
        const f32x4_t d4 = *(const f32x4_t*)(sr + kBQ + 8 * g + 4 * h2);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int v = 4 * g + e, kk = 8 * g + e;
          float th;
          const float x = bwd_score<SOFTCAP, ALIBI>(p, sacc[v], slope_log2,
                                                    __builtin_fabsf(rel - (float)kk), th);
          float pr = fast_exp2(x - l4[e]);
          float dz = pr * (pacc[v] - d4[e]);
          if constexpr (SOFTCAP) dz *= 1.0f - th * th;
          if (MASKED && (kk < lo_rel || kk >= hi_rel)) {
            pr = 0.0f;
            dz = 0.0f;
          }
          pa[4 * gg + e] = pr;
          za[4 * gg + e] = dz;
        }
      }
      pb[tt] = __builtin_convertvector(pa, bf16x8_t);
      zb[tt] = __builtin_convertvector(za, bf16x8_t);
    }
    // dV^T += dO^T P and dK^T += Q^T dZ: k-step tt covers the block's queries
    // 16tt + 4h2 + {0..3, 8..11}, read transposed from the dO and Q tiles.
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int vrow = 16 * tt + 4 * h2 + (gl >> 2);
        const int col = 32 * db + 16 * sub + 4 * (gl & 3);
        const int o_lo = tile_off<D>(vrow, col >> 3) + (col & 7);
        const int o_hi = tile_off<D>(vrow + 8, col >> 3) + (col & 7);
        const s16x4_t g_lo = ds_read_tr16(sg + o_lo), g_hi = ds_read_tr16(sg + o_hi);
        const s16x4_t q_lo = ds_read_tr16(sq + o_lo), q_hi = ds_read_tr16(sq + o_hi);
        const s16x8_t ga = {g_lo[0], g_lo[1], g_lo[2], g_lo[3], g_hi[0], g_hi[1], g_hi[2], g_hi[3]};
        const s16x8_t qa = {q_lo[0], q_lo[1], q_lo[2], q_lo[3], q_hi[0], q_hi[1], q_hi[2], q_hi[3]};
        dvacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, ga), pb[tt],
                                                            dvacc[db], 0, 0, 0);
        dkacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, qa), zb[tt],
                                                            dkacc[db], 0, 0, 0);
      }
    }
    // Schedule: the transposed reads of kReadAhead MFMAs first, then one MFMA
    // and the two reads of a later one, alternately (bounds the live operands).
    constexpr int kMf = 4 * NDB;  // MFMAs of the two products
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * kReadAhead, 1);
#pragma unroll
    for (int i = 0; i < kMf - kReadAhead; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kReadAhead, 1);
  };

#ifdef FA_SERIAL_COPIES
  // Verification build: one stage, each block copied, waited for and fenced by
  // barriers on both sides (the arithmetic and its order are unchanged).
  for (int it = 0; it < nblocks; ++it) {
    const int qb = qb_first + it * kBQ;
    copy_block(sQ0, sG0, sR0, qb);
    wait_vmem_barrier<0>();
    if (wave_live && qb < whi && qb + kBQ > wlo) {
      if (wave_full && qb >= wflo && qb + kBQ <= wfhi)
        compute(std::false_type{}, sQ0, sG0, sR0, qb);
      else
        compute(std::true_type{}, sQ0, sG0, sR0, qb);
    }
    __syncthreads();
  }
#else
  copy_block(sQ0, sG0, sR0, qb_first);
  copy_block(sQ1, sG1, sR1, qb_first + kBQ);
  copy_block(sQ2, sG2, sR2, qb_first + 2 * kBQ);
  wait_vmem_barrier<2 * kCopies>();  // V and block 0 have landed
  auto step = [&](auto st, int it) __attribute__((always_inline)) {
    constexpr int S = decltype(st)::value;
    uint16_t* sq = S == 0 ? sQ0 : S == 1 ? sQ1 : S == 2 ? sQ2 : sQ3;
    uint16_t* sg = S == 0 ? sG0 : S == 1 ? sG1 : S == 2 ? sG2 : sG3;
    float* sr = S == 0 ? sR0 : S == 1 ? sR1 : S == 2 ? sR2 : sR3;
    // Stage (S + 3) % 4 held block it - 1, finished before the last barrier.
    uint16_t* nq_ = S == 0 ? sQ3 : S == 1 ? sQ0 : S == 2 ? sQ1 : sQ2;
    uint16_t* ng_ = S == 0 ? sG3 : S == 1 ? sG0 : S == 2 ? sG1 : sG2;
    float* nr_ = S == 0 ? sR3 : S == 1 ? sR0 : S == 2 ? sR1 : sR2;
    const int qb = qb_first + it * kBQ;
    copy_block(nq_, ng_, nr_, qb + 3 * kBQ);
    if (wave_live && qb < whi && qb + kBQ > wlo) {
      if (wave_full && qb >= wflo && qb + kBQ <= wfhi)
        compute(std::false_type{}, sq, sg, sr, qb);
      else
        compute(std::true_type{}, sq, sg, sr, qb);
    }
    wait_vmem_barrier<2 * kCopies>();  // block it + 1 has landed
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  for (int it = 0; it < nblocks; it += 4) {
    step(I0{}, it);
    if (it + 1 < nblocks) step(I1{}, it + 1);
    if (it + 2 < nblocks) step(I2{}, it + 2);
    if (it + 3 < nblocks) step(I3{}, it + 3);
  }
  wait_vmem_barrier<0>();  // no copy may still be writing LDS at exit
#endif

  // Epilogue: lane = key, slots = head_dim rows 32db + 8g + 4h2 + {0..3}.
  if (key >= k1) return;
  const int64_t base = ((sq.k_row0 + key) * p.H + h) * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int64_t o = base + 32 * db + 8 * g + 4 * h2;
      store_grad4(p.dk, p.g_bf16, o, dkacc[db][4 * g] * p.scale, dkacc[db][4 * g + 1] * p.scale,
                  dkacc[db][4 * g + 2] * p.scale, dkacc[db][4 * g + 3] * p.scale);
      store_grad4(p.dv, p.g_bf16, o, dvacc[db][4 * g], dvacc[db][4 * g + 1], dvacc[db][4 * g + 2],
                  dvacc[db][4 * g + 3]);
    }
}

// ---------------------------------------------------------------------------
// 3. dQ
// ---------------------------------------------------------------------------
// dQ of query tile `block` (flat index, head fastest) with its LDS at `lds`.
template <int D, bool SOFTCAP, bool ALIBI>
__device__ __forceinline__ void bwd_dq_body(const BwdParams& p, int block, char* lds) {
  constexpr int KS = D / 16;
  constexpr int NDB = D / 32;
  constexpr int CPR = D / 8;
  constexpr int RPL = 64 / CPR;
  constexpr int LOADS = kBN / RPL / 4;
  constexpr int TILE = kBN * D;
  // Operands of the score and dP products (K, then V) read this many MFMAs ahead.
  constexpr int kDqReadAhead = 4;

  // The four stages in one array: a K read and the V read of the same k-step
  // differ by a constant, so they share an address register (immediate offset).
  uint16_t* const smem = (uint16_t*)lds;  // 1024-byte aligned
  uint16_t* const sK0 = smem;
  uint16_t* const sK1 = smem + TILE;
  uint16_t* const sV0 = smem + 2 * TILE;
  uint16_t* const sV1 = smem + 3 * TILE;

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, r = lane & 31, h2 = lane >> 5;
  int L = block;
  const int h = L % p.H;
  L /= p.H;
  const int b = L % p.B;
  const BwdSeq sq = bwd_seq(p, b, h);
  const int nq = sq.nq, nk = sq.nk, off = nk - nq;
  // Heaviest (last) tile first: of the sequence in a batched layout, of the
  // longest sequence in a packed one (one order of absolute tile position
  // across the pack, as in the forward).
  const int qt = p.cu_seqlens_q ? p.num_q_tiles - 1 - L / p.B : (nq + kBM - 1) / kBM - 1 - L / p.B;
  if (qt < 0 || qt * kBM >= nq) return;  // a packed sequence without this tile
  const int q0 = qt * kBM, q1 = min(nq, q0 + kBM);
  const KeyBounds wg = key_bounds(q0, q1, off, 0, nk, p.window_left, p.window_right);
  if (wg.hi <= wg.lo) {
    zero_rows<kThreads>(p.dq, p.g_bf16, sq.q_row0, h, p.H, D, q0, q1, tid);
    return;
  }
  const int wq0 = q0 + 32 * w, wq1 = min(nq, wq0 + 32);
  const bool wave_live = wq0 < nq;
  const KeyBounds wk = key_bounds(wq0, max(wq1, wq0 + 1), off, 0, nk, p.window_left, p.window_right);
  const int row = wq0 + r;
  const KeyBounds rk = key_bounds(row, row + 1, off, 0, nk, p.window_left, p.window_right);

  float slope_log2 = 0.0f;
  if constexpr (ALIBI) slope_log2 = p.alibi[h] * kLog2e;

  // Q and dO of this lane's row: columns 16ks + 8h2 .. +7 (B operands).
  bf16x8_t qf[KS], gf[KS];
  {
    const int64_t ro = ((sq.q_row0 + min(row, nq - 1)) * p.H + h) * D + 8 * h2;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4_t x = *(const u32x4_t*)((const uint16_t*)p.q + ro + 16 * ks);
      u32x4_t y = *(const u32x4_t*)((const uint16_t*)p.dout + ro + 16 * ks);
      if (row >= nq) x = y = u32x4_t{0, 0, 0, 0};
      qf[ks] = __builtin_bit_cast(bf16x8_t, x);
      gf[ks] = __builtin_bit_cast(bf16x8_t, y);
    }
  }
  const int rc = min(row, nq - 1);
  const float* rt = p.rowterms + (((int64_t)b * p.H + h) * p.nblk + rc / BWD_RB) * (2 * BWD_RB) +
                    rc % BWD_RB;
  const float lse2 = row < nq ? rt[0] : kInf;
  const float drow = row < nq ? rt[BWD_RB] : 0.0f;

  // Contiguous K/V copies, as in the forward.
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int64_t row_bytes = 2 * (int64_t)p.H * D;
  const int64_t bh_bytes = 2 * ((sq.k_row0 * p.H + h) * D);
  const int64_t end_bytes = (int64_t)(nk - 1) * row_bytes + 2 * D;
  const char* kbh = (const char*)p.k + bh_bytes;
  const char* vbh = (const char*)p.v + bh_bytes;
  unsigned lane_bytes[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int trow = RPL * (LOADS * wu + i) + lane / CPR;
    const int chunk = (lane % CPR) ^ swz<D>(trow);
    lane_bytes[i] = (unsigned)(trow * row_bytes + 16 * chunk);
  }
  auto copy_tiles = [&](uint16_t* kd, uint16_t* vd, int j0) __attribute__((always_inline)) {
    const int64_t tb = (int64_t)j0 * row_bytes;
    const int64_t left = end_bytes - tb;
    const int n = left <= 0 ? 0 : (left >= 0x7FFFFFFF ? 0x7FFFFFFF : (int)left);
    const __amdgpu_buffer_rsrc_t rk_ = make_rsrc(kbh + tb, n);
    const __amdgpu_buffer_rsrc_t rv_ = make_rsrc(vbh + tb, n);
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      buffer_load_lds16(rk_, kd + 512 * (LOADS * wu + i), lane_bytes[i]);
      buffer_load_lds16(rv_, vd + 512 * (LOADS * wu + i), lane_bytes[i]);
    }
  };

  f32x16_t dqacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dqacc[db] = f32x16_t{};
  const int gl = lane & 15, sub = (lane >> 4) & 1;

  auto compute = [&](const uint16_t* kt, const uint16_t* vt, int j0) __attribute__((always_inline)) {
    // S^T = K Q^T and dP^T = V dO^T for 64 keys x this wavefront's 32 rows:
    // MFMA i (k-step (i / 2) % KS, 32-key block i % 2) takes K for i < 2 KS and
    // V after. Each operand is read kDqReadAhead MFMAs ahead, in source order as
    // well, since under this register pressure the scheduler keeps source order.
    constexpr int NOP = 4 * KS;
    f32x16_t sacc[2], pacc[2];
    auto sp_operand = [&](int i) __attribute__((always_inline)) {
      const uint16_t* t = i < 2 * KS ? kt : vt;
      return *(const u32x4_t*)(t + tile_off<D>(32 * (i & 1) + r, 2 * ((i >> 1) % KS) + h2));
    };
    u32x4_t ring[kDqReadAhead];
#pragma unroll
    for (int i = 0; i < kDqReadAhead; ++i) ring[i] = sp_operand(i);
#pragma unroll
    for (int i = 0; i < NOP; ++i) {
      const bf16x8_t a = __builtin_bit_cast(bf16x8_t, ring[i % kDqReadAhead]);
      if (i + kDqReadAhead < NOP) ring[i % kDqReadAhead] = sp_operand(i + kDqReadAhead);
      const int ks = (i >> 1) % KS, j = i & 1;
      if (i < 2 * KS)
        sacc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], ks == 0 ? f32x16_t{} : sacc[j], 0, 0, 0);
      else
        pacc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, gf[ks], ks == 0 ? f32x16_t{} : pacc[j], 0, 0, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, kDqReadAhead, 4);  // DS reads
#pragma unroll
    for (int i = 0; i < NOP - kDqReadAhead; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 4);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 4);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kDqReadAhead, 4);
    // Slot v of block j holds key j0 + 32j + 8*(v/4) + 4*h2 + v%4 of this lane's row.
    const bool masked = __builtin_amdgcn_readfirstlane(!(j0 >= wk.flo && j0 + kBN <= wk.fhi));
    const int lo_rel = rk.lo - j0 - 4 * h2, hi_rel = rk.hi - j0 - 4 * h2;
    const float rel = (float)(row + off - j0 - 4 * h2);
    float zv[2][16];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int kk = 32 * j + 8 * (v >> 2) + (v & 3);
        float th;
        const float x = bwd_score<SOFTCAP, ALIBI>(p, sacc[j][v], slope_log2,
                                                  __builtin_fabsf(rel - (float)kk), th);
        float pr = fast_exp2(x - lse2);
        float dz = pr * (pacc[j][v] - drow);
        if constexpr (SOFTCAP) dz *= 1.0f - th * th;
        zv[j][v] = dz;
      }
    // Only tiles that cross a row's key range (or Nk) take the per-element mask:
    // a wave-uniform branch, so the other tiles skip the compares.
    if (masked) {
      asm volatile("");  // keeps the branch (not if-converted into every tile)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int kk = 32 * j + 8 * (v >> 2) + (v & 3);
          if (kk < lo_rel || kk >= hi_rel) zv[j][v] = 0.0f;
        }
    }
    // dQ^T += K^T dZ^T: k-step tt covers keys 16tt + 4h2 + {0..3, 8..11},
    // K read transposed from LDS.
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      f32x8_t z;
#pragma unroll
      for (int e = 0; e < 8; ++e) z[e] = zv[tt >> 1][(tt & 1) * 8 + e];
      const bf16x8_t zb = __builtin_convertvector(z, bf16x8_t);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int krow = 16 * tt + 4 * h2 + (gl >> 2);
        const int col = 32 * db + 16 * sub + 4 * (gl & 3);
        const s16x4_t lo = ds_read_tr16(kt + tile_off<D>(krow, col >> 3) + (col & 7));
        const s16x4_t hi = ds_read_tr16(kt + tile_off<D>(krow + 8, col >> 3) + (col & 7));
        const s16x8_t x = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        dqacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, x), zb,
                                                            dqacc[db], 0, 0, 0);
      }
    }
  };

  const int j_first = (wg.lo / kBN) * kBN;
  const int ntiles = (wg.hi - j_first + kBN - 1) / kBN;
#ifdef FA_SERIAL_COPIES
  // Verification build: one buffer per tensor, each tile copied, waited for and
  // fenced by barriers on both sides (the arithmetic and its order are unchanged).
  for (int it = 0; it < ntiles; ++it) {
    const int j0 = j_first + it * kBN;
    copy_tiles(sK0, sV0, j0);
    wait_vmem_barrier<0>();
    if (wave_live && j0 < wk.hi && j0 + kBN > wk.lo) compute(sK0, sV0, j0);
    __syncthreads();
  }
#else
  copy_tiles(sK0, sV0, j_first);
  wait_vmem_barrier<0>();
  auto step = [&](auto par, int it) __attribute__((always_inline)) {
    constexpr bool ODD = decltype(par)::value;
    const int j0 = j_first + it * kBN;
    if (it + 1 < ntiles) copy_tiles(ODD ? sK0 : sK1, ODD ? sV0 : sV1, j0 + kBN);
    if (wave_live && j0 < wk.hi && j0 + kBN > wk.lo) compute(ODD ? sK1 : sK0, ODD ? sV1 : sV0, j0);
    wait_vmem_barrier<0>();
  };
  for (int it = 0; it < ntiles; it += 2) {
    step(std::false_type{}, it);
    if (it + 1 < ntiles) step(std::true_type{}, it + 1);
  }
#endif

  if (row >= nq) return;
  const int64_t base = ((sq.q_row0 + row) * p.H + h) * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      store_grad4(p.dq, p.g_bf16, base + 32 * db + 8 * g + 4 * h2, dqacc[db][4 * g] * p.scale,
                  dqacc[db][4 * g + 1] * p.scale, dqacc[db][4 * g + 2] * p.scale,
                  dqacc[db][4 * g + 3] * p.scale);
}

// dK/dV and dQ in one launch: workgroups [0, n_dkdv) are dK/dV's key tiles,
// the rest dQ's query tiles. Both only read the row terms, so the dQ
// workgroups start as soon as CUs free up and fill the slots that dK/dV's
// last workgroups leave idle (two launches would wait for dK/dV to drain).
// One LDS allocation, the larger of the two layouts.
template <int D, bool SOFTCAP, bool ALIBI>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dkdv_dq_kernel(BwdParams p, int n_dkdv) {
  static_assert(kDkdvThreads == kThreads, "one workgroup size");
  constexpr int kDkdvLds = D == 128 ? kDkdvLdsBytes : kW4LdsBytes;
  constexpr int kDqLds = 4 * kBN * D * 2;
  __shared__ __attribute__((aligned(1024))) char lds[kDkdvLds > kDqLds ? kDkdvLds : kDqLds];
  if ((int)blockIdx.x < n_dkdv) {
    if constexpr (D == 128)
      bwd_dkdv_body<D, SOFTCAP, ALIBI>(p, blockIdx.x, lds);
    else
      bwd_dkdv_w4_body<D, SOFTCAP, ALIBI>(p, blockIdx.x, lds);
  } else {
    bwd_dq_body<D, SOFTCAP, ALIBI>(p, blockIdx.x - n_dkdv, lds);
  }
}

}  // namespace

template <int D, bool SOFTCAP, bool ALIBI>
int launch_bwd_bf16(const BwdParams& p, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  const int64_t rows = (int64_t)p.B * p.H * p.nblk * BWD_RB;
  constexpr int RPB = kThreads / (D / 8);
  hipLaunchKernelGGL((bwd_prep_kernel<D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(kThreads),
                     0, s, p);
  int rc = (int)hipGetLastError();
  if (rc) return rc;
  // Key tiles of BWD_BK keys (head_dim 64) or kDkdvKeys keys (head_dim 128; the
  // workgroups past a sequence's keys exit at once).
  const int64_t ktiles = D == 128 ? (int64_t)p.num_k_tiles * (BWD_BK / kDkdvKeys) : p.num_k_tiles;
  const int64_t n_dkdv = ktiles * p.H * p.B;
  const int64_t n_dq = (int64_t)p.num_q_tiles * p.H * p.B;
  hipLaunchKernelGGL((bwd_dkdv_dq_kernel<D, SOFTCAP, ALIBI>), dim3((unsigned)(n_dkdv + n_dq)),
                     dim3(kThreads), 0, s, p, (int)n_dkdv);
  return (int)hipGetLastError();
}

// Row-term buffer of fa_bwd_noalloc (callers that cannot allocate device
// memory): a static device array, one copy per GPU the library runs on, held
// until the process ends. In host code `scratch` names a host-side stand-in;
// its device address on the current GPU comes from hipGetSymbolAddress, looked
// up once per device and kept.
static __device__ __align__(256) float scratch[NOALLOC_SCRATCH_FLOATS];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

int noalloc_scratch(float** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    g_scratch_ptr[dev] = (float*)ptr;
  }
  *out = g_scratch_ptr[dev];
  return 0;
}

#define FA_INST(D, SC, AL) template int launch_bwd_bf16<D, SC, AL>(const BwdParams&, void*);
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
