// fp32 tiled attention forward for gfx950, on v_mfma_f32_32x32x2_f32.
//
// Same method and register layout as the bf16 kernel (S^T = K Q^T, online
// softmax per lane pair, O^T += V^T P^T), with fp32 operands throughout so that
// fp32 inputs keep fp32 products. A workgroup owns a 32-row query tile; its
// four wavefronts take every fourth 32-key tile of the tile's key range (each
// staging its own tiles in LDS), and their partial (max, sum, O) are merged by
// the log-sum-exp rule at the end. Used for fp32 inputs, where problem sizes
// are small and accuracy, not throughput, is the point: the four wavefronts
// spread a short problem over four SIMDs instead of one.
#include <hip/hip_runtime.h>

#include "fa_device.h"

namespace fa {

namespace {

constexpr int kBN = 32;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

// Orders the LDS writes of one wavefront before its following reads.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int D, bool SOFTCAP, bool ALIBI, bool PAGED>
__global__ __launch_bounds__(kThreads) void fwd_f32_kernel(FwdParams p) {
  constexpr int NDB = D / 32;
  // Row strides chosen so that the 64 lanes of each MFMA operand read hit 64 distinct banks.
  constexpr int KSTR = D + 2;  // lane (r, h2) reads K[r][2ks + h2]
  constexpr int VSTR = D + 8;  // lane (r, h2) reads V[key(h2)][32db + r], keys 4 apart
  constexpr int kStage = kBN * (KSTR + VSTR);      // floats of one wavefront's K and V tile
  constexpr int kMerge = NDB * 16 * 64 + 2 * 64;   // floats of one wavefront's partial output
  constexpr int kPerWave = kStage > kMerge ? kStage : kMerge;
  __shared__ __attribute__((aligned(16))) float smem[kWaves * kPerWave];

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, r = lane & 31, h2 = lane >> 5;
  float* sK = smem + w * kPerWave;
  float* sV = sK + kBN * KSTR;
  const WorkItem wi = decode_work<PAGED>(p);
  const int b = wi.b, h = wi.h, s = wi.s;
  const SeqInfo si = seq_info(p, b, h);
  const int nq = si.nq, nk = si.nk;
  if constexpr (PAGED) {
    // Append: one workgroup per (b, h) copies the new keys into their pages.
    if (p.k_new && s == 0 && wi.rank == 0) append_rows<float>(p, si, b, h, D, tid, kThreads);
  }
  const int qt = query_tile(p, wi, nq, F32_BM);
  if (qt < 0) return;  // a packed sequence shorter than the longest

  const int off = nk - nq;
  int slo = 0, shi = nk;
  if constexpr (PAGED) split_range(p, nk, s, slo, shi);

  const int q0 = qt * F32_BM;
  const int q1 = min(nq, q0 + F32_BM);
  const KeyBounds wk = key_bounds(q0, q1, off, slo, shi, p.window_left, p.window_right);
  if (wk.hi <= wk.lo) {
    write_empty_rows<PAGED>(p, si, b, h, s, q0, q1, D, tid, kThreads);
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
  for (int j0 = j_first + w * kBN; j0 < wk.hi; j0 += kWaves * kBN) {
    wave_lds_sync();  // the previous tile's reads came first
    // The tile's K and V, 16 bytes per lane per load: every load is issued
    // before any is stored (a rolled loop waited for each load in turn). Keys
    // past the end load the last key (in range) and are stored as zeros.
    constexpr int kLoadsPerLane = kBN * D / 4 / 64;
    f32x4_t kx[kLoadsPerLane], vx[kLoadsPerLane];
#pragma unroll
    for (int it = 0; it < kLoadsPerLane; ++it) {
      const int idx = lane + 64 * it;
      const int key = min(j0 + idx / (D / 4), nk - 1);
      // Appended keys (paged launches with k_new) come from k_new / v_new.
      const bool fresh = PAGED && key >= si.n_cached;
      const int64_t o = (fresh ? new_key_offset(p, si, b, key, h, D)
                               : kv_offset<PAGED>(p, b, si, key, h, D)) + 4 * (idx % (D / 4));
      kx[it] = *(const f32x4_t*)((const float*)(fresh ? p.k_new : p.k) + o);
      vx[it] = *(const f32x4_t*)((const float*)(fresh ? p.v_new : p.v) + o);
    }
#pragma unroll
    for (int it = 0; it < kLoadsPerLane; ++it) {
      const int idx = lane + 64 * it;
      const int kk = idx / (D / 4), c4 = idx % (D / 4);
      const bool in = j0 + kk < nk;
      float* kd = &sK[kk * KSTR + 4 * c4];
      kd[0] = in ? kx[it][0] : 0.0f;
      kd[1] = in ? kx[it][1] : 0.0f;
      kd[2] = in ? kx[it][2] : 0.0f;
      kd[3] = in ? kx[it][3] : 0.0f;
      *(f32x4_t*)&sV[kk * VSTR + 4 * c4] = in ? vx[it] : f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    wave_lds_sync();

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

  // Merge the wavefronts' partials: row max M = max_w m_w (log2 units), sum L =
  // sum_w l_w 2^(m_w - M), O = sum_w O_w 2^(m_w - M) / L. Each wavefront
  // publishes (m_w, l_w) per lane and its accumulators lane-contiguously.
  const float mw = m_run == kNegInf ? kNegInf : m_run * c;
  const float lw = half_sum(l_run);
  __syncthreads();  // every wavefront is done with its K/V stage
  {
    float* mine = smem + w * kPerWave;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) mine[(db * 16 + e) * 64 + lane] = oacc[db][e];
    mine[NDB * 16 * 64 + lane] = mw;
    mine[NDB * 16 * 64 + 64 + lane] = lw;
  }
  __syncthreads();
  float M = kNegInf;
#pragma unroll
  for (int u = 0; u < kWaves; ++u) M = fmaxf(M, smem[u * kPerWave + NDB * 16 * 64 + lane]);
  float wgt[kWaves];
  float L = 0.0f;
#pragma unroll
  for (int u = 0; u < kWaves; ++u) {
    const float mu = smem[u * kPerWave + NDB * 16 * 64 + lane];
    wgt[u] = M == kNegInf || mu == kNegInf ? 0.0f : fast_exp2(mu - M);
    L += smem[u * kPerWave + NDB * 16 * 64 + 64 + lane] * wgt[u];
  }
  if (row >= nq) return;
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
#pragma unroll
  for (int u = 0; u < kWaves; ++u) wgt[u] *= inv;
  float mref = M;  // the maximum in units of the unshifted ALiBi bias
  if constexpr (ALIBI) mref -= slope_log2 * (float)abs(row + off - alibi_anchor(row + off, rk));
  const float lse = L > 0.0f ? (mref + __log2f(L)) * kLn2 : kNegInf;
  // Wavefront w writes the 32-column blocks db = w, w + kWaves, ...
  for (int db = w; db < NDB; db += kWaves) {
    float ov[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float x = 0.0f;
#pragma unroll
      for (int u = 0; u < kWaves; ++u) x += smem[u * kPerWave + (db * 16 + e) * 64 + lane] * wgt[u];
      ov[e] = x;
    }
    if constexpr (PAGED) {
      const int64_t ro = (((int64_t)s * p.B + b) * p.H + h) * p.Nq + row;
      float* op = p.o_part + ro * D;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4_t x = {ov[4 * g], ov[4 * g + 1], ov[4 * g + 2], ov[4 * g + 3]};
        *(f32x4_t*)(op + 32 * db + 8 * g + 4 * h2) = x;
      }
    } else {
      const int64_t ob = q_offset(p, si, row, h, D);
#pragma unroll
      for (int g = 0; g < 4; ++g)
        store_out4(p, ob + 32 * db + 8 * g + 4 * h2, ov[4 * g], ov[4 * g + 1], ov[4 * g + 2],
                   ov[4 * g + 3]);
    }
  }
  if (w == 0 && h2 == 0) {
    if constexpr (PAGED)
      p.lse_part[(((int64_t)s * p.B + b) * p.H + h) * p.Nq + row] = lse;
    else if (p.lse)
      p.lse[si.lse0 + row] = lse;
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
