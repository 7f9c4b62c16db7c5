// Reduce step of split-KV: merge per-split normalised outputs by their
// log-sum-exps (flash-attn v2.0-v2.7 update article, v2.2 entry: a separate
// kernel merges the results of the blocks that each handled one key range).
//
// One wavefront per output row (b, h, i), rows ordered head-fastest so a
// workgroup writes neighbouring heads of the same token contiguously.
//   L = m + log2(sum_s 2^(lse2_s - m)),  O = sum_s 2^(lse2_s - L) o_s
// computed in log2 units; rows with every split empty get O = 0, L = -inf.
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

}  // namespace

template <int D>
int launch_combine(const CombineParams& p, void* stream) {
  const int64_t nrows = (int64_t)p.B * p.Nq * p.H;
  const int64_t groups = (nrows + kRowsPerGroup - 1) / kRowsPerGroup;
  hipLaunchKernelGGL(combine_kernel<D>, dim3((unsigned)groups), dim3(64 * kRowsPerGroup), 0,
                     (hipStream_t)stream, p);
  return (int)hipGetLastError();
}

template int launch_combine<64>(const CombineParams&, void*);
template int launch_combine<128>(const CombineParams&, void*);

}  // namespace fa
