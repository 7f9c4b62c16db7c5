// Reduce step of split-KV: merge per-split normalised outputs by their
// log-sum-exps (flash-attn v2.0-v2.7 update article, v2.2 entry: a separate
// kernel merges the results of the blocks that each handled one key range).
//
//   L = m + log2(sum_s 2^(lse2_s - m)),  O = sum_s 2^(lse2_s - L) o_s
// computed in log2 units; rows with every split empty get O = 0, L = -inf.
// Rows are ordered head-fastest, so a workgroup writes neighbouring heads of
// the same token contiguously. Two forms:
//  - segment form (split counts up to D / 4, 16-byte aligned partials and
//    output): D / 4 lanes per row, each lane one 16-byte piece of the row, so
//    a wavefront merges 64 / (D / 4) rows at once. Lane q of a row's segment
//    loads split q's log-sum-exp; the partial vectors of the first splits are
//    loaded before those are reduced (they do not depend on them), and each
//    split's weight reaches the other lanes by a shuffle, so a row costs one
//    memory round trip when the split count is small.
//  - row form (any split count or alignment): one wavefront per row, 4-byte
//    pieces, the log-sum-exps read once per pass.
#include <hip/hip_runtime.h>

#include "fa_device.h"

namespace fa {

namespace {

constexpr int kRowsPerGroup = 4;

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  return x;
}

template <int D>
__global__ __launch_bounds__(64 * kRowsPerGroup) void combine_kernel(CombineParams p) {
  constexpr int PER_LANE = D / 64;
  const int lane = threadIdx.x & 63;
  const int64_t R = (int64_t)blockIdx.x * kRowsPerGroup + (threadIdx.x >> 6);
  const int64_t nrows = (int64_t)p.B * p.Nq * p.H;
  if (R >= nrows) return;
  const int h = (int)(R % p.H);
  const int64_t bi = R / p.H;
  const int i = (int)(bi % p.Nq);
  const int b = (int)(bi / p.Nq);

  const int64_t split_stride = (int64_t)p.B * p.H * p.Nq;
  const int64_t r0 = ((int64_t)b * p.H + h) * p.Nq + i;  // row index inside one split

  // Split log-sum-exps (log2 units) loaded by the lanes in parallel.
  float m = kNegInf;
  for (int s = lane; s < p.S; s += 64) m = fmaxf(m, p.lse_part[s * split_stride + r0] * kLog2e);
  m = wave_max(m);
  float tot = 0.0f;
  float acc[PER_LANE];
#pragma unroll
  for (int e = 0; e < PER_LANE; ++e) acc[e] = 0.0f;
  if (m != kNegInf) {
    for (int s = lane; s < p.S; s += 64) tot += fast_exp2(p.lse_part[s * split_stride + r0] * kLog2e - m);
    tot = wave_sum(tot);
    const float* op = p.o_part + r0 * D + lane;
#pragma unroll 8
    for (int s = 0; s < p.S; ++s) {
      const float wgt = fast_exp2(p.lse_part[s * split_stride + r0] * kLog2e - m);
#pragma unroll
      for (int e = 0; e < PER_LANE; ++e) acc[e] += wgt * op[s * split_stride * D + 64 * e];
    }
  }
  const float inv = tot > 0.0f ? 1.0f / tot : 0.0f;
  const int64_t ob = (((int64_t)b * p.Nq + i) * p.H + h) * D;
#pragma unroll
  for (int e = 0; e < PER_LANE; ++e) {
    const float x = acc[e] * inv;
    if (p.o_bf16)
      ((__bf16*)p.o)[ob + lane + 64 * e] = (__bf16)x;
    else
      ((float*)p.o)[ob + lane + 64 * e] = x;
  }
  if (lane == 0 && p.lse)
    p.lse[((int64_t)b * p.H + h) * p.Nq + i] = tot > 0.0f ? (m + __log2f(tot)) * kLn2 : kNegInf;
}


// Segment form (p.S <= D / 4; o_part 16-byte aligned, o 16-byte aligned for
// fp32 and 8-byte for bf16, checked by the launcher).
template <int D>
__global__ __launch_bounds__(256) void combine_seg_kernel(CombineParams p) {
  constexpr int LPR = D / 4;     // lanes per row: one 16-byte piece each
  constexpr int RPW = 64 / LPR;  // rows per wavefront
  constexpr int kChunk = 16;     // partial vectors loaded ahead of their use
  const int lane = threadIdx.x & 63;
  const int q = lane % LPR;
  const int seg = lane - q;
  const int64_t nrows = (int64_t)p.B * p.Nq * p.H;
  const int64_t R = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW + lane / LPR;
  const bool valid = R < nrows;  // lanes of a row past the end compute on row 0 and store nothing
  const int64_t Rv = valid ? R : 0;
  const int h = (int)(Rv % p.H);
  const int64_t bi = Rv / p.H;
  const int i = (int)(bi % p.Nq);
  const int b = (int)(bi / p.Nq);
  const int S = p.S;

  const int64_t split_stride = (int64_t)p.B * p.H * p.Nq;
  const int64_t r0 = ((int64_t)b * p.H + h) * p.Nq + i;
  // Loads are unconditional (indices clamped to the last split) so that none
  // waits for another; the surplus values are discarded.
  const float xl = p.lse_part[min(q, S - 1) * split_stride + r0];
  const f32x4_t* op = (const f32x4_t*)(p.o_part + r0 * D) + q;
  const int64_t vstride = split_stride * (D / 4);  // one split, in 16-byte pieces
  f32x4_t ov[kChunk];
#pragma unroll
  for (int c = 0; c < kChunk; ++c) ov[c] = op[min(c, S - 1) * vstride];
  const float x = q < S ? xl * kLog2e : kNegInf;

  float m = x;
#pragma unroll
  for (int k = LPR / 2; k >= 1; k >>= 1) m = fmaxf(m, __shfl_xor(m, k));
  const float e = m == kNegInf ? 0.0f : fast_exp2(x - m);
  float tot = e;
#pragma unroll
  for (int k = LPR / 2; k >= 1; k >>= 1) tot += __shfl_xor(tot, k);

  // (No branch on an all-empty row here: it would hold the loads above back
  // until the reduction is done. Such a row's output is set to 0 below.)
  f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
  auto accumulate = [&](int s0) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < kChunk; ++c) {
      if (s0 + c < S) {
        const float w = __shfl(e, seg + s0 + c);
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t] += w * ov[c][t];
      }
    }
  };
  accumulate(0);
  for (int s0 = kChunk; s0 < S; s0 += kChunk) {
#pragma unroll
    for (int c = 0; c < kChunk; ++c) ov[c] = op[min(s0 + c, S - 1) * vstride];
    accumulate(s0);
  }
  if (!valid) return;
  const float inv = tot > 0.0f ? 1.0f / tot : 0.0f;
  const int64_t ob = (((int64_t)b * p.Nq + i) * p.H + h) * D + 4 * q;
  f32x4_t y = {acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
  if (m == kNegInf) y = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  if (p.o_bf16) {
    typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
    const bf16x4_t yb = {(__bf16)y[0], (__bf16)y[1], (__bf16)y[2], (__bf16)y[3]};
    *(bf16x4_t*)((__bf16*)p.o + ob) = yb;
  } else {
    *(f32x4_t*)((float*)p.o + ob) = y;
  }
  if (q == 0 && p.lse)
    p.lse[((int64_t)b * p.H + h) * p.Nq + i] = tot > 0.0f ? (m + __log2f(tot)) * kLn2 : kNegInf;
}

}  // namespace

template <int D>
int launch_combine(const CombineParams& p, void* stream) {
  const int64_t nrows = (int64_t)p.B * p.Nq * p.H;
  const bool aligned = ((uintptr_t)p.o_part & 15) == 0 && ((uintptr_t)p.o & (p.o_bf16 ? 7 : 15)) == 0;
  if (p.S <= D / 4 && aligned) {
    constexpr int kRowsPerWg = 4 * (64 / (D / 4));
    const int64_t groups = (nrows + kRowsPerWg - 1) / kRowsPerWg;
    hipLaunchKernelGGL(combine_seg_kernel<D>, dim3((unsigned)groups), dim3(256), 0,
                       (hipStream_t)stream, p);
  } else {
    const int64_t groups = (nrows + kRowsPerGroup - 1) / kRowsPerGroup;
    hipLaunchKernelGGL(combine_kernel<D>, dim3((unsigned)groups), dim3(64 * kRowsPerGroup), 0,
                       (hipStream_t)stream, p);
  }
  return (int)hipGetLastError();
}

template int launch_combine<64>(const CombineParams&, void*);
template int launch_combine<128>(const CombineParams&, void*);

}  // namespace fa
