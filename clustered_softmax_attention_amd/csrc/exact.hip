// Exact softmax attention (gfx950): the comparator of the library and, with a block
// size, the exact attention on the diagonal blocks of causal MuSe (pith.science
// review of arXiv 2509.10406, caption of Figure 2), whose partial result is merged
// with the far-field approximation by log-sum-exp:
//   L = log(e^L_loc + e^L_far),  o = e^(L_loc - L) o_loc + e^(L_far - L) o_far.
//
// bf16 path (flash_bf16): workgroup of 4 waves = 128 queries; key/value tiles of 64
// keys staged row-major in LDS (the next tile in registers meanwhile); per wave
// S^T = K Q^T on the matrix cores (32 keys x 32 queries per tile), online softmax along
// accumulator rows (one lane and its partner), O^T += V^T P^T with P rounded to bf16 and
// V^T read by the transpose read in the key order of the P accumulator. Workgroups are
// renumbered so that those of one head run on one XCD and share its L2.
// fp32 path: one thread per query, online softmax over chunks of 32 keys; all lanes
// of a wave visit the same key at the same time, so key and value rows are read
// once per wave.
#include "mfma.hpp"
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

template <int D>
__global__ void __launch_bounds__(256, 2) flash_bf16_kernel(ExactArgs a, int nqt) {
  constexpr int BQ = 128, BK = 64;
  constexpr int KST = D + 16;  // bf16 elements per K and V row in LDS (padded)
  constexpr int NKS = D / 16;
  constexpr int NMT = D / 32;
  constexpr int CH = D / 8;    // 16-byte chunks per row
  constexpr int NP = BK * CH / 256;  // 16-byte pieces per thread and tensor
  __shared__ __align__(16) uint16_t sK[BK * KST];
  __shared__ __align__(16) uint16_t sV[BK * KST];

  const int total = nqt * a.BH;
  // workgroup id -> (query tile, head) such that each XCD takes a contiguous range: the
  // query tiles of a head read the same keys and values
  const int id = xcd_contiguous(blockIdx.x, total);
  int qt = id % nqt;
  const int bh = id / nqt;
  if (a.causal) qt = nqt - 1 - qt;  // longest rows first
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, h = lane >> 5, c = lane & 31;
  const int N = a.N;
  const int q0 = qt * BQ;
  const int qi = q0 + wave * 32 + c;
  const bool qvalid = qi < N;
  const size_t base = static_cast<size_t>(bh) * N;
  const uint16_t* Q = static_cast<const uint16_t*>(a.q) + base * D;
  const uint16_t* K = static_cast<const uint16_t*>(a.k) + base * D;
  const uint16_t* V = static_cast<const uint16_t*>(a.v) + base * D;

  bf16x8_t qf[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    u16x8_t u = {0, 0, 0, 0, 0, 0, 0, 0};
    if (qvalid) u = *reinterpret_cast<const u16x8_t*>(Q + static_cast<size_t>(qi) * D + 16 * ks + 8 * h);
    qf[ks] = as_bf16x8(u);
  }
  const int qq = qvalid ? qi : N - 1;
  const int kbeg = a.block > 0 ? (qq / a.block) * a.block : 0;
  const int kend = a.causal ? qq + 1 : N;
  const int wkb_min = wave_min_int(kbeg), wkb_max = wave_max_int(kbeg);
  const int wke_min = wave_min_int(kend), wke_max = wave_max_int(kend);
  const int qlast = min(q0 + BQ, N) - 1;
  const int gkb = a.block > 0 ? (q0 / a.block) * a.block : 0;
  const int gke = a.causal ? qlast + 1 : N;
  const float sl2 = a.scale * 1.4426950408889634f;

  float m = -1e30f, l = 0.f;
  f32x16_t o[NMT];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) o[mt] = zero16();

  // the next tile's rows travel in registers while the current one is used
  u16x8_t pk[NP], pv[NP];
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      const int e = tid + 256 * q, r = e / CH, cc = e % CH, key = kt + r;
      pk[q] = u16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
      pv[q] = pk[q];
      if (key < N) {
        pk[q] = *reinterpret_cast<const u16x8_t*>(K + static_cast<size_t>(key) * D + cc * 8);
        pv[q] = *reinterpret_cast<const u16x8_t*>(V + static_cast<size_t>(key) * D + cc * 8);
      }
    }
  };
  if (gkb < gke) load_tile(gkb);
  for (int kt = gkb; kt < gke; kt += BK) {
    __syncthreads();  // the previous tile is consumed
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      const int e = tid + 256 * q, r = e / CH, cc = e % CH;
      *reinterpret_cast<u16x8_t*>(sK + r * KST + cc * 8) = pk[q];
      *reinterpret_cast<u16x8_t*>(sV + r * KST + cc * 8) = pv[q];
    }
    __syncthreads();
    if (kt + BK < gke) load_tile(kt + BK);
    if (kt >= wke_max || kt + BK <= wkb_min) continue;  // tile outside every row of this wave
    const bool full = kt >= wkb_max && kt + BK <= wke_min && kt + BK <= N;

    f32x16_t s[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      s[t] = zero16();
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const bf16x8_t af = as_bf16x8(*reinterpret_cast<const u16x8_t*>(sK + (32 * t + c) * KST + 16 * ks + 8 * h));
        s[t] = mfma32(af, qf[ks], s[t]);
      }
    }
    float mx = -1e30f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float x = s[t][v] * sl2;
        if (!full) {
          const int key = kt + 32 * t + 8 * (v >> 2) + 4 * h + (v & 3);
          if (key < kbeg || key >= kend) x = kNegInf;
        }
        s[t][v] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, xor32(mx));
    const float mn = fmaxf(m, mx);
    if (__ballot(mn > m) != 0ull) {  // rescale only when a row's running max grew (else alpha = 1)
      const float alpha = fast_exp2(m - mn);
      l *= alpha;
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[mt][v] *= alpha;
    }
    m = mn;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float p = fast_exp2(s[t][v] - mn);
        s[t][v] = p;
        l += p;
      }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int ss = 0; ss < 2; ++ss) {
        float pv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) pv[i] = s[t][8 * ss + i];
        const bf16x8_t bfr = pack_bf16x8(pv);
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt)
          o[mt] = mfma32(lds_operand_tr_acc(sV, KST, 32 * t + 16 * ss, 32 * mt, lane), bfr, o[mt]);
      }
  }
  const float lt = l + xor32(l);
  if (!qvalid) return;
  const float inv = 1.f / lt;
  float L = (m + __log2f(lt)) * 0.6931471805599453f;
  const size_t row = base + qi;
  float w0 = inv, w1 = 0.f;
  bool merge = false;
  if (a.l_far != nullptr) {
    const float lf = a.l_far[row];
    if (lf != kNegInf) {
      const float Lt = fmaxf(L, lf) + __logf(1.f + __expf(-fabsf(L - lf)));
      w0 = __expf(L - Lt) * inv;
      w1 = __expf(lf - Lt);
      L = Lt;
      merge = true;
    }
  }
  if (a.lse_out != nullptr && h == 0) a.lse_out[row] = L;
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = 32 * mt + 8 * g + 4 * h;
      float r4[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) r4[r] = o[mt][4 * g + r] * w0;
      if (merge) {
        const f32x4_t f = *reinterpret_cast<const f32x4_t*>(a.o_far + row * D + d0);
#pragma unroll
        for (int r = 0; r < 4; ++r) r4[r] += w1 * f[r];
      }
      if (a.out_bf16) {
        const u16x4_t u = {f32_to_bf16_bits(r4[0]), f32_to_bf16_bits(r4[1]), f32_to_bf16_bits(r4[2]),
                           f32_to_bf16_bits(r4[3])};
        *reinterpret_cast<u16x4_t*>(static_cast<uint16_t*>(a.out) + row * D + d0) = u;
      } else {
        const f32x4_t f = {r4[0], r4[1], r4[2], r4[3]};
        *reinterpret_cast<f32x4_t*>(static_cast<float*>(a.out) + row * D + d0) = f;
      }
    }
}

hipError_t launch_exact(const ExactArgs& a, int dtype, hipStream_t s) {
  const dim3 g((a.N + kExThreads - 1) / kExThreads, a.BH);
  if (dtype == 1) {
    const int nqt = (a.N + 127) / 128;
    ProfScope ps_(a.block > 0 ? "local_block_mfma" : "exact_mfma", s);
    if (a.D == 64) hipLaunchKernelGGL((flash_bf16_kernel<64>), dim3(nqt * a.BH), dim3(256), 0, s, a, nqt);
    else hipLaunchKernelGGL((flash_bf16_kernel<128>), dim3(nqt * a.BH), dim3(256), 0, s, a, nqt);
    return hipGetLastError();
  }
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
