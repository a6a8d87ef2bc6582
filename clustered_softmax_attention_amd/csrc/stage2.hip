// Stage 2 of MuSe: each query refines its cluster's summaries with its residual
// (gist.science summary of arXiv 2509.10406, Kernmechanismen 1 "Decompositie" and
// 2 "Fase 2"; pith.science review, "What carries the argument").
//
// Query n in cluster i, residual qt = q_n - qbar_i, table entry e (its block for
// causal calls, 0 otherwise):
//   l_j = log Z_ij + s qt . K_ij,   p = softmax_j(l),   L_n = logsumexp_j l_j,
//   o_n = sum_j p_j V_ij + s D_i qt.
// One thread per query; the residual is kept in registers for the logits and in
// LDS (lane-major) for the dipole product, whose table is stored key index first so
// that a row of D_i^T is contiguous.
#include "muse_kernels.hpp"

namespace muse {

constexpr int kS2Threads = 128;

template <typename T, int D>
__global__ void __launch_bounds__(kS2Threads) s2_refine_kernel(S2Args a) {
  __shared__ float s_q[D][kS2Threads];
  const int bh = blockIdx.y, tid = threadIdx.x;
  const long n = static_cast<long>(blockIdx.x) * kS2Threads + tid;
  const bool valid = n < a.N;
  const long nn = valid ? n : a.N - 1;
  const int b = a.causal ? static_cast<int>(nn / a.block) : 0;
  const size_t row = static_cast<size_t>(bh) * a.N + nn;
  const bool far_empty = a.causal && b == 0;
  if (far_empty) {
    if (valid) {
      a.l_far[row] = kNegInf;
      for (int d = 0; d < D; ++d) a.o_far[row * D + d] = 0.f;
    }
    return;
  }
  const int i = a.labels_q[row];
  const T* Q = static_cast<const T*>(a.q);
  const float* qb = a.qbar + (static_cast<size_t>(bh) * a.Cq + i) * D;
  float qt[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    qt[d] = Elem<T>::load(Q, row * D + d) - qb[d];
    s_q[d][tid] = qt[d];
  }
  const int e = a.causal ? b : 0;
  const size_t sidx = (static_cast<size_t>(bh) * a.nbS + e) * a.Cq + i;
  const float* lz = a.s_logz + sidx * a.Ck;
  const float* Kt = a.s_k + sidx * a.Ck * D;
  const float* Vt = a.s_v + sidx * a.Ck * D;

  float mx = kNegInf;
  for (int j = 0; j < a.Ck; ++j) {
    const float l0 = lz[j];
    if (l0 == kNegInf) continue;
    float dot = 0.f;
#pragma unroll
    for (int d = 0; d < D; ++d) dot = fmaf(qt[d], Kt[j * D + d], dot);
    mx = fmaxf(mx, l0 + a.scale * dot);
  }
  float acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) acc[d] = 0.f;
  float z = 0.f;
  for (int j = 0; j < a.Ck; ++j) {
    const float l0 = lz[j];
    if (l0 == kNegInf) continue;
    float dot = 0.f;
#pragma unroll
    for (int d = 0; d < D; ++d) dot = fmaf(qt[d], Kt[j * D + d], dot);
    const float p = __expf(l0 + a.scale * dot - mx);
    z += p;
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] = fmaf(p, Vt[j * D + d], acc[d]);
  }
  const float inv = 1.f / z;
#pragma unroll
  for (int d = 0; d < D; ++d) acc[d] *= inv;
  if (a.dipole) {
    const float* dipT = a.s_dipT + sidx * D * D;  // [dk][dv]
    for (int dk = 0; dk < D; ++dk) {
      const float x = a.scale * s_q[dk][tid];
#pragma unroll
      for (int dv = 0; dv < D; ++dv) acc[dv] = fmaf(dipT[dk * D + dv], x, acc[dv]);
    }
  }
  const float L = mx + __logf(z);
  if (!valid) return;
  if (a.causal) {
    a.l_far[row] = L;
#pragma unroll
    for (int d = 0; d < D; ++d) a.o_far[row * D + d] = acc[d];
  } else {
    if (a.lse_out) a.lse_out[row] = L;
    if (a.out_bf16) {
#pragma unroll
      for (int d = 0; d < D; ++d) static_cast<bf16*>(a.out)[row * D + d].bits = f32_to_bf16_bits(acc[d]);
    } else {
#pragma unroll
      for (int d = 0; d < D; ++d) static_cast<float*>(a.out)[row * D + d] = acc[d];
    }
  }
}

hipError_t launch_stage2(const S2Args& a, int dtype, hipStream_t s) {
  const dim3 g((a.N + kS2Threads - 1) / kS2Threads, a.BH);
  ProfScope ps_("s2_refine", s);
  if (dtype == 0) {
    if (a.D == 64) hipLaunchKernelGGL((s2_refine_kernel<float, 64>), g, dim3(kS2Threads), 0, s, a);
    else hipLaunchKernelGGL((s2_refine_kernel<float, 128>), g, dim3(kS2Threads), 0, s, a);
  } else {
    if (a.D == 64) hipLaunchKernelGGL((s2_refine_kernel<bf16, 64>), g, dim3(kS2Threads), 0, s, a);
    else hipLaunchKernelGGL((s2_refine_kernel<bf16, 128>), g, dim3(kS2Threads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace muse
