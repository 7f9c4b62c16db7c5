// bf16 tiled attention forward for gfx950 (MI355X).
//
// One workgroup of 4 wavefronts owns a 128-row query tile of one (batch, head)
// [and one key split when PAGED]. Each wavefront keeps its 32 query rows in
// registers and walks the key range its rows can see in 64-key tiles:
//   S^T = K Q^T     on v_mfma_f32_32x32x16_bf16 (K from LDS, Q from VGPRs)
//   score transform, mask, online softmax in VGPRs (row = lane pair l, l^32)
//   O^T += V^T P^T  on v_mfma_f32_32x32x16_bf16 (V read transposed from LDS
//                   with ds_read_b64_tr_b16, P from VGPRs)
// K and V tiles are double-buffered in LDS in their natural [key][d] layout:
// the next tile's global loads are issued before the current tile's math, and
// stored after it.
// (Tiled IO-aware forward with online softmax: "IO感知技术革命: FlashAttention如何
// 重塑大模型训练的经济学", sections on block tiling, online softmax and overlap of
// copies with compute; mask and score variants: flash-attn v2.0-v2.7 update
// article, v2.1-v2.6 entries; split + paged form: its v2.2 and v2.5 entries.)
#include <hip/hip_runtime.h>

#include "fa_device.h"

namespace fa {

namespace {

constexpr int kBM = BF16_BM;   // query rows per workgroup
constexpr int kBN = 64;        // keys per tile
constexpr int kThreads = 256;  // 4 wavefronts

// Wavefronts per SIMD the register budget is sized for: 2 lets one wavefront's
// softmax overlap another's MFMA work and keeps accumulators out of AGPRs.
#ifndef FA_PREFILL_WAVES
#define FA_PREFILL_WAVES 2
#endif

template <int D, bool SOFTCAP, bool ALIBI, bool PAGED>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(FA_PREFILL_WAVES, FA_PREFILL_WAVES))) void fwd_bf16_kernel(FwdParams p) {
  constexpr int KS = D / 16;             // MFMA k-steps of Q K^T
  constexpr int NDB = D / 32;            // 32-row blocks of O^T
  // LDS row strides (bf16) picked for conflict-free operand reads: K rows are
  // read 16 bytes per lane (32 lanes = 32 rows), V with transposed 8-byte reads
  // (16 lanes = 4 rows x 32 bytes, two 16-lane groups 16 d apart).
  constexpr int KSTR = D + 8;
  constexpr int VSTR = D + 32;
  constexpr int CPR = D / 8;             // 16-byte chunks per K/V row
  constexpr int KPT = kBN * CPR / kThreads;  // K/V rows each thread moves per tile (4 or 2)
  static_assert(KPT == 4 || KPT == 2, "tile split");

  __shared__ __attribute__((aligned(16))) uint16_t sK[2][kBN * KSTR];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][kBN * VSTR];

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, r = lane & 31, h2 = lane >> 5;
  const WorkItem wi = decode_work<PAGED>(p);
  const int b = wi.b, h = wi.h, s = wi.s;

  const int off = p.Nk - p.Nq;
  int slo = 0, shi = p.Nk;
  if constexpr (PAGED) split_range(p, s, slo, shi);

  const int q0 = wi.qt * kBM;
  const int q1 = min(p.Nq, q0 + kBM);
  const KeyBounds wg = key_bounds(q0, q1, off, slo, shi, p.window_left, p.window_right);
  if (wg.hi <= wg.lo) {
    write_empty_rows<PAGED>(p, b, h, s, q0, q1, D, tid, kThreads);
    return;
  }

  // This wavefront's rows and keys.
  const int wq0 = q0 + 32 * w;
  const int wq1 = min(p.Nq, wq0 + 32);
  const bool wave_live = wq0 < p.Nq;
  const KeyBounds wk = key_bounds(wq0, max(wq1, wq0 + 1), off, slo, shi, p.window_left,
                                  p.window_right);
  const int row = wq0 + r;
  const KeyBounds rk = key_bounds(row, row + 1, off, slo, shi, p.window_left, p.window_right);

  float slope_log2 = 0.0f;
  if constexpr (ALIBI) slope_log2 = p.alibi[h] * kLog2e;

  // Q fragment: row `row`, columns 16*ks + 8*h2 .. +7 (the B operand of S^T = K Q^T).
  bf16x8_t qf[KS];
  {
    const uint16_t* qp = (const uint16_t*)p.q + q_offset(p, b, min(row, p.Nq - 1), h, D) + 8 * h2;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4_t x = *(const u32x4_t*)(qp + 16 * ks);
      if (row >= p.Nq) x = u32x4_t{0, 0, 0, 0};
      qf[ks] = __builtin_bit_cast(bf16x8_t, x);
    }
  }

  // Tile movement: thread handles chunk `lc` of rows lg*KPT .. lg*KPT+KPT-1.
  const int lc = tid % CPR, lg = tid / CPR;
  u32x4_t kr[KPT], vr[KPT];
  auto load_tile = [&](int j0) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int key = j0 + lg * KPT + i;
      if (key < p.Nk) {
        const int64_t o = kv_offset<PAGED>(p, b, key, h, D) + 8 * lc;
        kr[i] = *(const u32x4_t*)((const uint16_t*)p.k + o);
        vr[i] = *(const u32x4_t*)((const uint16_t*)p.v + o);
      } else {
        kr[i] = u32x4_t{0, 0, 0, 0};
        vr[i] = u32x4_t{0, 0, 0, 0};
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      *(u32x4_t*)&sK[buf][(lg * KPT + i) * KSTR + 8 * lc] = kr[i];
      *(u32x4_t*)&sV[buf][(lg * KPT + i) * VSTR + 8 * lc] = vr[i];
    }
  };

  f32x16_t oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16_t{};
  // m_run: running max (log2 units). l_run: row sum of the bf16-rounded P that
  // feeds the PV product (normalises O). l_exact: row sum of the unrounded P
  // (gives the log-sum-exp).
  float m_run = kNegInf, l_run = 0.0f, l_exact = 0.0f;

  const int j_first = (wg.lo / kBN) * kBN;
  const int ntiles = (wg.hi - j_first + kBN - 1) / kBN;

  load_tile(j_first);
  store_tile(0);
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    const int j0 = j_first + it * kBN;
    const int buf = it & 1;
    const bool has_next = it + 1 < ntiles;
    if (has_next) load_tile(j0 + kBN);

    if (wave_live && j0 < wk.hi && j0 + kBN > wk.lo) {
      // ---- S^T = K Q^T for 64 keys (two 32-key blocks)
      f32x16_t sacc[2] = {f32x16_t{}, f32x16_t{}};
      const uint16_t* kb = &sK[buf][r * KSTR + 8 * h2];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const bf16x8_t a = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(kb + 32 * j * KSTR + 16 * ks));
          sacc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], sacc[j], 0, 0, 0);
        }
      }
      float t[2][16];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) t[j][v] = sacc[j][v];

      const bool full = j0 >= wk.flo && j0 + kBN <= wk.fhi;
      const float rel = (float)(row + off) - (float)(j0 + 4 * h2);
      transform_scores<2, SOFTCAP, ALIBI>(t, p, slope_log2, rel, !full, j0, rk.lo, rk.hi, h2);

      bool any_rescale;
      float base;
      const float alpha = online_max<2>(t, m_run, l_run, any_rescale, base, 0.0f);
      l_exact *= alpha;
      if (any_rescale) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
      }

      // ---- P (bf16, rounded to nearest even) and its row sum
      bf16x8_t pf[4];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        f32x8_t x;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          x[e] = fast_exp2(t[tt >> 1][(tt & 1) * 8 + e] - base);
          l_exact += x[e];
        }
        pf[tt] = __builtin_convertvector(x, bf16x8_t);
        l_run = sum_bf16x8(pf[tt], l_run);
      }

      // ---- O^T += V^T P^T: k-step tt covers keys 16*tt .. 16*tt+15. The A operand
      // (lane: d-row m = lane % 32, keys 16tt + 4*h2 + {0..3, 8..11}) comes from two
      // transposed reads: in each 16-lane group, lanes 4k..4k+3 address the four
      // 4-column chunks of key k, and lane i receives column i of those 4 keys.
      const int gl = lane & 15, sub = (lane >> 4) & 1;
      const uint16_t* vb = &sV[buf][(4 * h2 + (gl >> 2)) * VSTR + 16 * sub + 4 * (gl & 3)];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const uint16_t* vp = vb + 16 * tt * VSTR + 32 * db;
          const s16x4_t lo = ds_read_tr16(vp);
          const s16x4_t hi = ds_read_tr16(vp + 8 * VSTR);
          const s16x8_t x = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, x), pf[tt],
                                                             oacc[db], 0, 0, 0);
        }
      }
    }

    if (has_next) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = O / l, LSE = (m + log2 l) ln 2
  if (!wave_live) return;
  const float l_tot = l_run + other_half(l_run);
  const float l_ex = l_exact + other_half(l_exact);
  if (row >= p.Nq) return;
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  const float lse = l_ex > 0.0f ? (m_run + __log2f(l_ex)) * kLn2 : kNegInf;
  if constexpr (PAGED) {
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
    const int64_t ob = q_offset(p, b, row, h, D);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        store_out4(p, ob + 32 * db + 8 * g + 4 * h2, oacc[db][4 * g] * inv,
                   oacc[db][4 * g + 1] * inv, oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
    if (h2 == 0 && p.lse) p.lse[((int64_t)b * p.H + h) * p.Nq + row] = lse;
  }
}

}  // namespace

template <int D, bool SOFTCAP, bool ALIBI, bool PAGED>
int launch_fwd_bf16(const FwdParams& p, void* stream) {
  const int64_t groups = (int64_t)p.num_q_tiles * p.H * p.B * (PAGED ? p.num_splits : 1);
  hipLaunchKernelGGL((fwd_bf16_kernel<D, SOFTCAP, ALIBI, PAGED>), dim3((unsigned)groups),
                     dim3(kThreads), 0, (hipStream_t)stream, p);
  return (int)hipGetLastError();
}

#define FA_INST(D, SC, AL, PG) template int launch_fwd_bf16<D, SC, AL, PG>(const FwdParams&, void*);
#define FA_INST_D(D)                                                                        \
  FA_INST(D, false, false, false) FA_INST(D, false, true, false) FA_INST(D, true, false, false) \
  FA_INST(D, true, true, false) FA_INST(D, false, false, true) FA_INST(D, false, true, true)     \
  FA_INST(D, true, false, true) FA_INST(D, true, true, true)
FA_INST_D(64)
FA_INST_D(128)

}  // namespace fa
