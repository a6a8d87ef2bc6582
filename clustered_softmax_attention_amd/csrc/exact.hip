// Exact softmax attention (gfx950): the comparator of the library and, with a block
// size, the exact attention on the diagonal blocks of causal MuSe (pith.science
// review of arXiv 2509.10406, caption of Figure 2), whose partial result is merged
// with the far-field approximation by log-sum-exp:
//   L = log(e^L_loc + e^L_far),  o = e^(L_loc - L) o_loc + e^(L_far - L) o_far.
//
// fp32 path: one thread per query, online softmax over chunks of 32 keys; all lanes
// of a wave visit the same key at the same time, so key and value rows are read
// once per wave.
#include "muse_kernels.hpp"

namespace muse {

constexpr int kExThreads = 128;
constexpr int kExChunk = 32;

__device__ __forceinline__ int wave_min_int(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = min(x, __shfl_xor(x, o, 64));
  return x;
}

__device__ __forceinline__ int wave_max_int(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = max(x, __shfl_xor(x, o, 64));
  return x;
}

template <typename T, int D>
__global__ void __launch_bounds__(kExThreads) exact_valu_kernel(ExactArgs a) {
  const int bh = blockIdx.y;
  const long n = static_cast<long>(blockIdx.x) * kExThreads + threadIdx.x;
  const bool valid = n < a.N;
  const long nn = valid ? n : a.N - 1;
  const size_t base = static_cast<size_t>(bh) * a.N;
  const T* Q = static_cast<const T*>(a.q) + base * D;
  const T* K = static_cast<const T*>(a.k) + base * D;
  const T* V = static_cast<const T*>(a.v) + base * D;
  float q[D];
#pragma unroll
  for (int d = 0; d < D; ++d) q[d] = a.scale * Elem<T>::load(Q, nn * D + d);
  const int kbeg = a.block > 0 ? static_cast<int>((nn / a.block) * a.block) : 0;
  const int kend = a.causal ? static_cast<int>(nn) + 1 : a.N;
  const int wbeg = wave_min_int(kbeg), wend = wave_max_int(kend);

  float m = kNegInf, l = 0.f;
  float acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) acc[d] = 0.f;
  for (int c0 = wbeg; c0 < wend; c0 += kExChunk) {
    float sc[kExChunk];
    float cmax = kNegInf;
#pragma unroll
    for (int u = 0; u < kExChunk; ++u) {
      const int key = c0 + u;
      float dot = 0.f;
      if (key < wend) {
#pragma unroll
        for (int d = 0; d < D; ++d) dot = fmaf(q[d], Elem<T>::load(K, static_cast<size_t>(key) * D + d), dot);
      }
      sc[u] = (key >= kbeg && key < kend) ? dot : kNegInf;
      cmax = fmaxf(cmax, sc[u]);
    }
    const float newm = fmaxf(m, cmax);
    const float alpha = (m == kNegInf) ? 0.f : __expf(m - newm);
    if (newm != kNegInf) {
      l *= alpha;
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] *= alpha;
      m = newm;
    }
#pragma unroll
    for (int u = 0; u < kExChunk; ++u) {
      const int key = c0 + u;
      if (key >= wend) break;
      const float p = (sc[u] == kNegInf) ? 0.f : __expf(sc[u] - m);
      l += p;
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] = fmaf(p, Elem<T>::load(V, static_cast<size_t>(key) * D + d), acc[d]);
    }
  }
  float L = m + __logf(l);
  const float inv = 1.f / l;
#pragma unroll
  for (int d = 0; d < D; ++d) acc[d] *= inv;
  if (!valid) return;
  const size_t row = base + n;
  if (a.l_far != nullptr) {
    const float lf = a.l_far[row];
    if (lf != kNegInf) {
      const float Lt = fmaxf(L, lf) + __logf(1.f + __expf(-fabsf(L - lf)));
      const float w0 = __expf(L - Lt), w1 = __expf(lf - Lt);
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] = w0 * acc[d] + w1 * a.o_far[row * D + d];
      L = Lt;
    }
  }
  if (a.lse_out) a.lse_out[row] = L;
  if (a.out_bf16) {
#pragma unroll
    for (int d = 0; d < D; ++d) static_cast<bf16*>(a.out)[row * D + d].bits = f32_to_bf16_bits(acc[d]);
  } else {
#pragma unroll
    for (int d = 0; d < D; ++d) static_cast<float*>(a.out)[row * D + d] = acc[d];
  }
}

hipError_t launch_exact(const ExactArgs& a, int dtype, hipStream_t s) {
  const dim3 g((a.N + kExThreads - 1) / kExThreads, a.BH);
  ProfScope ps_(a.block > 0 ? "local_block_exact" : "exact_valu", s);
  if (dtype == 0) {
    if (a.D == 64) hipLaunchKernelGGL((exact_valu_kernel<float, 64>), g, dim3(kExThreads), 0, s, a);
    else hipLaunchKernelGGL((exact_valu_kernel<float, 128>), g, dim3(kExThreads), 0, s, a);
  } else {
    if (a.D == 64) hipLaunchKernelGGL((exact_valu_kernel<bf16, 64>), g, dim3(kExThreads), 0, s, a);
    else hipLaunchKernelGGL((exact_valu_kernel<bf16, 128>), g, dim3(kExThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace muse
