// fp32 tiled attention forward for gfx950, on v_mfma_f32_32x32x2_f32.
//
// Same method and register layout as the bf16 kernel (S^T = K Q^T, online
// softmax per lane pair, O^T += V^T P^T), with fp32 operands throughout so that
// fp32 inputs keep fp32 products. One wavefront owns a 32-row query tile and
// walks 32-key tiles staged in LDS. Used for fp32 inputs, where problem sizes
// are small and accuracy, not throughput, is the point.
#include <hip/hip_runtime.h>

#include "fa_device.h"

namespace fa {

namespace {

constexpr int kBN = 32;
constexpr int kThreads = 64;

template <int D, bool SOFTCAP, bool ALIBI, bool PAGED>
__global__ __launch_bounds__(kThreads) void fwd_f32_kernel(FwdParams p) {
  constexpr int NDB = D / 32;
  // Row strides chosen so that the 64 lanes of each MFMA operand read hit 64 distinct banks.
  constexpr int KSTR = D + 2;  // lane (r, h2) reads K[r][2ks + h2]
  constexpr int VSTR = D + 8;  // lane (r, h2) reads V[key(h2)][32db + r], keys 4 apart
  __shared__ float sK[kBN * KSTR];
  __shared__ __attribute__((aligned(16))) float sV[kBN * VSTR];

  const int lane = threadIdx.x, r = lane & 31, h2 = lane >> 5;
  const WorkItem wi = decode_work<PAGED>(p);
  const int b = wi.b, h = wi.h, s = wi.s;
  const SeqInfo si = seq_info(p, b, h);
  const int nq = si.nq, nk = si.nk;
  if constexpr (PAGED) {
    // Append: one workgroup per (b, h) copies the new keys into their pages.
    if (p.k_new && s == 0 && wi.rank == 0) append_rows<float>(p, si, b, h, D, lane, kThreads);
  }
  const int qt = query_tile(wi, nq, F32_BM);
  if (qt < 0) return;  // a packed sequence shorter than the longest

  const int off = nk - nq;
  int slo = 0, shi = nk;
  if constexpr (PAGED) split_range(p, nk, s, slo, shi);

  const int q0 = qt * F32_BM;
  const int q1 = min(nq, q0 + F32_BM);
  const KeyBounds wk = key_bounds(q0, q1, off, slo, shi, p.window_left, p.window_right);
  if (wk.hi <= wk.lo) {
    write_empty_rows<PAGED>(p, si, b, h, s, q0, q1, D, lane, kThreads);
    return;
  }
  const int row = q0 + r;
  const KeyBounds rk = key_bounds(row, row + 1, off, slo, shi, p.window_left, p.window_right);

  float slope_log2 = 0.0f;
  if constexpr (ALIBI) slope_log2 = p.alibi[h] * kLog2e;
  const float c = exponent_scale<SOFTCAP, ALIBI>(p);

  float qf[D / 2];
  {
    const float* qp = (const float*)p.q + q_offset(p, si, min(row, nq - 1), h, D) + h2;
#pragma unroll
    for (int ks = 0; ks < D / 2; ++ks) qf[ks] = row < nq ? qp[2 * ks] : 0.0f;
  }

  f32x16_t oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16_t{};
  float m_run = kNegInf, l_run = 0.0f;

  const int j_first = (wk.lo / kBN) * kBN;
  for (int j0 = j_first; j0 < wk.hi; j0 += kBN) {
    __syncthreads();
    for (int idx = lane; idx < kBN * D / 4; idx += kThreads) {
      const int kk = idx / (D / 4), c = idx % (D / 4);
      const int key = j0 + kk;
      f32x4_t kx = {0.f, 0.f, 0.f, 0.f}, vx = {0.f, 0.f, 0.f, 0.f};
      if (key < nk) {
        // Appended keys (paged launches with k_new) come from k_new / v_new.
        const bool fresh = PAGED && key >= si.n_cached;
        const int64_t o = (fresh ? new_key_offset(p, si, b, key, h, D)
                                 : kv_offset<PAGED>(p, b, si, key, h, D)) + 4 * c;
        kx = *(const f32x4_t*)((const float*)(fresh ? p.k_new : p.k) + o);
        vx = *(const f32x4_t*)((const float*)(fresh ? p.v_new : p.v) + o);
      }
      float* kd = &sK[kk * KSTR + 4 * c];
      kd[0] = kx[0];
      kd[1] = kx[1];
      kd[2] = kx[2];
      kd[3] = kx[3];
      *(f32x4_t*)&sV[kk * VSTR + 4 * c] = vx;
    }
    __syncthreads();

    f32x16_t sacc = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < D / 2; ++ks)
      sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(sK[r * KSTR + 2 * ks + h2], qf[ks], sacc, 0, 0, 0);

    float t[1][16];
#pragma unroll
    for (int v = 0; v < 16; ++v) t[0][v] = sacc[v];
    const bool full = j0 >= wk.flo && j0 + kBN <= wk.fhi;
    const float rel = (float)(ALIBI ? alibi_anchor(row + off, rk) : row + off) - (float)(j0 + 4 * h2);
    transform_scores<1, SOFTCAP, ALIBI>(t, p, slope_log2, rel, !full, j0, rk.lo, rk.hi, h2);

    bool any_rescale;
    float mc;
    const float alpha =
        online_max<1>(t, c, m_run, l_run, any_rescale, mc, kLazyRescaleThreshold / c);
    if (any_rescale) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
    }
    float pr[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      pr[v] = fast_exp2(__builtin_fmaf(t[0][v], c, -mc));
      l_run += pr[v];
    }
    // k-step v pairs this lane's slot v (key acc_key(v, h2)) with V row of that key.
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float* vp = &sV[acc_key(v, h2) * VSTR + r];
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vp[32 * db], pr[v], oacc[db], 0, 0, 0);
    }
  }

  const float l_tot = half_sum(l_run);
  if (row >= nq) return;
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  float mref = m_run * c;  // the maximum in units of the unshifted ALiBi bias
  if constexpr (ALIBI) mref -= slope_log2 * (float)abs(row + off - alibi_anchor(row + off, rk));
  const float lse = l_tot > 0.0f ? (mref + __log2f(l_tot)) * kLn2 : kNegInf;
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

}  // namespace

template <int D, bool SOFTCAP, bool ALIBI, bool PAGED>
int launch_fwd_f32(const FwdParams& p, void* stream) {
  const int64_t groups = (int64_t)p.num_q_tiles * p.H * p.B * (PAGED ? p.num_splits : 1);
  hipLaunchKernelGGL((fwd_f32_kernel<D, SOFTCAP, ALIBI, PAGED>), dim3((unsigned)groups),
                     dim3(kThreads), 0, (hipStream_t)stream, p);
  return (int)hipGetLastError();
}

#define FA_INST(D, SC, AL, PG) template int launch_fwd_f32<D, SC, AL, PG>(const FwdParams&, void*);
#define FA_INST_D(D)                                                                        \
  FA_INST(D, false, false, false) FA_INST(D, false, true, false) FA_INST(D, true, false, false) \
  FA_INST(D, true, true, false) FA_INST(D, false, false, true) FA_INST(D, false, true, true)     \
  FA_INST(D, true, false, true) FA_INST(D, true, true, true)
FA_INST_D(64)
FA_INST_D(128)

}  // namespace fa
