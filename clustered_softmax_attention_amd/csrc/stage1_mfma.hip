// Matrix-core stage 1 for bf16 inputs (gfx950).
//
// The quantities are those of stage1.hip (pith.science review of arXiv 2509.10406,
// "What carries the argument"): for query centroid qbar_i and key m,
// a_im = s qbar_i . k_m; per (i, key cluster j, block b') the atom (max, sum exp, sum
// exp k, sum exp v); per (i, moment sub-block) the normalised sum w v k^T and its log
// mass. Here:
//   s1_scores      a_im for every centroid and key, [BH, Cq, N] fp32 (qbar split into
//                  bf16 hi + lo; keys are exact in bf16).
//   s1_atoms_mfma  one wave per (block, key cluster) bucket: per-centroid max of a over
//                  the bucket, then sum_m w_m k_m and sum_m w_m v_m as products
//                  K_seg^T W^T with the weights split into bf16 hi + lo.
//   s1_moments_f16 per (sub-block, centroid group): weights w = exp(a - max) from the
//                  scores (no running rescale), then sum_m w_m v_m k_m^T with fp16
//                  operands (the weights are applied to V^T with packed fp16 multiplies)
//                  and fp32 accumulation.
#include "mfma.hpp"
#include "muse_kernels.hpp"

namespace muse {

typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;

__device__ __forceinline__ f32x16_t mfma32_f16(const f16x8_t& a, const f16x8_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Workgroup = 256 keys (4 waves x 2 tiles of 32); dynamic LDS: qbar hi/lo [Cqp][D+8].
template <int D>
__global__ void __launch_bounds__(256) s1_scores_kernel(S1Args a) {
  extern __shared__ __align__(16) uint16_t sq[];
  constexpr int QST = D + 8;
  constexpr int NKS = D / 16;
  const int bh = blockIdx.y, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, h = lane >> 5, c = lane & 31;
  const int Cq = a.Cq, Cqp = (Cq + 31) & ~31, nt_n = Cqp / 32;
  uint16_t* qhi = sq;
  uint16_t* qlo = sq + Cqp * QST;
  for (int x = tid; x < Cqp * D; x += 256) {
    const int i = x / D, d = x % D;
    const float v = i < Cq ? a.qbar[(static_cast<size_t>(bh) * Cq + i) * D + d] : 0.f;
    const uint16_t hv = f32_to_bf16_bits(v);
    qhi[i * QST + d] = hv;
    qlo[i * QST + d] = f32_to_bf16_bits(v - bf16_to_f32(hv));
  }
  __syncthreads();
  const uint16_t* K = static_cast<const uint16_t*>(a.k) + static_cast<size_t>(bh) * a.N * D;
  float* S = a.scores + static_cast<size_t>(bh) * Cq * a.N;
  for (int tt = 0; tt < 2; ++tt) {
    const int kb = blockIdx.x * 256 + wave * 64 + tt * 32;
    if (kb >= a.N) break;
    const int key = kb + c;
    bf16x8_t ak[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      u16x8_t u = {0, 0, 0, 0, 0, 0, 0, 0};
      if (key < a.N) u = *reinterpret_cast<const u16x8_t*>(K + static_cast<size_t>(key) * D + 16 * ks + 8 * h);
      ak[ks] = as_bf16x8(u);
    }
    for (int nt = 0; nt < nt_n; ++nt) {
      f32x16_t acc = zero16();
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int o = (32 * nt + c) * QST + 16 * ks + 8 * h;
        acc = mfma32(ak[ks], as_bf16x8(*reinterpret_cast<const u16x8_t*>(qhi + o)), acc);
        acc = mfma32(ak[ks], as_bf16x8(*reinterpret_cast<const u16x8_t*>(qlo + o)), acc);
      }
      // lane (c, h): centroid 32 nt + c, keys kb + 8 g + 4 h + r
      const int i = 32 * nt + c;
      if (i >= Cq) continue;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int k0 = kb + 8 * g + 4 * h;
        if (k0 + 3 < a.N) {
          const f32x4_t f = {a.scale * acc[4 * g], a.scale * acc[4 * g + 1], a.scale * acc[4 * g + 2],
                             a.scale * acc[4 * g + 3]};
          *reinterpret_cast<f32x4_t*>(S + static_cast<size_t>(i) * a.N + k0) = f;
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (k0 + r < a.N) S[static_cast<size_t>(i) * a.N + k0 + r] = a.scale * acc[4 * g + r];
        }
      }
    }
  }
}

// One wave per (block b', key cluster j) bucket; 4 buckets per workgroup.
template <int D>
__global__ void __launch_bounds__(256) s1_atoms_mfma_kernel(S1Args a) {
  constexpr int NMT = D / 32;
  const int bh = blockIdx.y, wave = threadIdx.x >> 6, lane = threadIdx.x & 63, h = lane >> 5, c = lane & 31;
  const int Cq = a.Cq, Ck = a.Ck;
  const int u = blockIdx.x * 4 + wave;
  if (u >= a.nb * Ck) return;
  const int bp = u / Ck, j = u % Ck;
  const int32_t* offs = a.offs_k + static_cast<size_t>(bh) * (a.nb * Ck + 1);
  const int s0 = offs[u], n = offs[u + 1] - s0;
  const int32_t* perm = a.perm_k + static_cast<size_t>(bh) * a.N + s0;
  const uint16_t* K = static_cast<const uint16_t*>(a.k) + static_cast<size_t>(bh) * a.N * D;
  const uint16_t* V = static_cast<const uint16_t*>(a.v) + static_cast<size_t>(bh) * a.N * D;
  const size_t abase = (static_cast<size_t>(bh) * a.nb + bp) * Cq;
  for (int nt = 0; nt < (Cq + 31) / 32; ++nt) {
    const int i = 32 * nt + c;
    const bool iv = i < Cq;
    const float* Si = a.scores + (static_cast<size_t>(bh) * Cq + (iv ? i : 0)) * a.N;
    float mx = kNegInf;
    for (int k = h; k < n; k += 2) mx = fmaxf(mx, Si[perm[k]]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    f32x16_t ak[NMT], av[NMT];
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
      ak[mt] = zero16();
      av[mt] = zero16();
    }
    float z = 0.f;
    for (int k0 = 0; k0 < n; k0 += 16) {
      int key[8];
      float w[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int kk = k0 + 8 * h + e;
        key[e] = kk < n ? perm[kk] : -1;
        w[e] = (key[e] >= 0 && iv) ? __expf(Si[key[e]] - mx) : 0.f;
        z += w[e];
      }
      bf16x8_t whi, wlo;
      split_bf16x8(w, whi, wlo);
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) {
        const int d = 32 * mt + c;
        u16x8_t kv, vv;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          kv[e] = key[e] >= 0 ? K[static_cast<size_t>(key[e]) * D + d] : 0;
          vv[e] = key[e] >= 0 ? V[static_cast<size_t>(key[e]) * D + d] : 0;
        }
        ak[mt] = mfma32(as_bf16x8(kv), whi, ak[mt]);
        ak[mt] = mfma32(as_bf16x8(kv), wlo, ak[mt]);
        av[mt] = mfma32(as_bf16x8(vv), whi, av[mt]);
        av[mt] = mfma32(as_bf16x8(vv), wlo, av[mt]);
      }
    }
    z += __shfl_xor(z, 32, 64);
    if (!iv) continue;
    const size_t aidx = (abase + i) * Ck + j;
    if (h == 0) {
      a.at_m[aidx] = n > 0 ? mx : kNegInf;
      a.at_z[aidx] = z;
    }
    // lane (c, h): column = centroid i, rows d = 32 mt + 8 g + 4 h + r
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * mt + 8 * g + 4 * h;
        const f32x4_t fk = {ak[mt][4 * g], ak[mt][4 * g + 1], ak[mt][4 * g + 2], ak[mt][4 * g + 3]};
        const f32x4_t fv = {av[mt][4 * g], av[mt][4 * g + 1], av[mt][4 * g + 2], av[mt][4 * g + 3]};
        *reinterpret_cast<f32x4_t*>(a.at_k + aidx * D + d0) = fk;
        *reinterpret_cast<f32x4_t*>(a.at_v + aidx * D + d0) = fv;
      }
  }
}

// Sub-block moments with fp16 operands. D = 64: 8 centroids per workgroup, 2 per wave;
// D = 128: 2 centroids, each wave half of the 16 output tiles of one centroid.
// Static LDS: K^T, V^T [D][64+8] fp16 | weights [G][kMaxMbk] fp16 | max, sum [G].
constexpr int kMaxMbk = 1024;

template <int D>
__global__ void __launch_bounds__(256) s1_moments_f16_kernel(S1Args a) {
  constexpr int KC = 64;
  constexpr int TST = KC + 8;
  constexpr int G = D == 64 ? 8 : 2;
  constexpr int CPW = D == 64 ? 2 : 1;
  constexpr int NMT = D / 32;
  constexpr int NNT = 2;
  __shared__ __align__(16) _Float16 sKt[D * TST];
  __shared__ __align__(16) _Float16 sVt[D * TST];
  __shared__ __align__(16) _Float16 sw[G * kMaxMbk];
  __shared__ float smx[G], ssum[G];
  const int mb = blockIdx.x, ig = blockIdx.y, bh = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, h = lane >> 5, c = lane & 31;
  const int Cq = a.Cq, i0 = ig * G, ng = min(G, Cq - i0);
  const int key0 = mb * a.mbk, key1 = min(a.N, key0 + a.mbk), nkeys = key1 - key0;

  // weights: wave w takes centroids g = w, w + 4
  for (int g = wave; g < G; g += 4) {
    const float* Sg = a.scores + (static_cast<size_t>(bh) * Cq + i0 + (g < ng ? g : 0)) * a.N + key0;
    float mx = kNegInf;
    for (int k = lane; k < nkeys; k += 64) mx = fmaxf(mx, Sg[k]);
    mx = wave_max(mx);
    float sum = 0.f;
    for (int k = lane; k < kMaxMbk; k += 64) {
      const float w = (k < nkeys && g < ng) ? __expf(Sg[k < nkeys ? k : 0] - mx) : 0.f;
      sw[g * kMaxMbk + k] = static_cast<_Float16>(w);
      sum += w;
    }
    sum = wave_sum(sum);
    if (lane == 0) {
      smx[g] = mx;
      ssum[g] = sum;
    }
  }
  const int wc0 = D == 64 ? 2 * wave : wave / 2;
  const int nt0 = D == 64 ? 0 : 2 * (wave & 1);
  const uint16_t* K = static_cast<const uint16_t*>(a.k) + static_cast<size_t>(bh) * a.N * D;
  const uint16_t* V = static_cast<const uint16_t*>(a.v) + static_cast<size_t>(bh) * a.N * D;
  f32x16_t acc[CPW][NMT][NNT];
#pragma unroll
  for (int cc = 0; cc < CPW; ++cc)
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NNT; ++nt) acc[cc][mt][nt] = zero16();

  for (int c0 = 0; c0 < nkeys; c0 += KC) {
    const int nk = min(KC, nkeys - c0);
    __syncthreads();
    for (int x = tid; x < KC * (D / 8); x += 256) {
      const int r = x / (D / 8), cc8 = x % (D / 8);
      u16x8_t kv = {0, 0, 0, 0, 0, 0, 0, 0}, vv = {0, 0, 0, 0, 0, 0, 0, 0};
      if (r < nk) {
        kv = *reinterpret_cast<const u16x8_t*>(K + static_cast<size_t>(key0 + c0 + r) * D + cc8 * 8);
        vv = *reinterpret_cast<const u16x8_t*>(V + static_cast<size_t>(key0 + c0 + r) * D + cc8 * 8);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        sKt[(cc8 * 8 + e) * TST + r] = static_cast<_Float16>(bf16_to_f32(kv[e]));
        sVt[(cc8 * 8 + e) * TST + r] = static_cast<_Float16>(bf16_to_f32(vv[e]));
      }
    }
    __syncthreads();
    if (wc0 < ng) {
#pragma unroll
      for (int ks = 0; ks < KC / 16; ++ks) {
        const int kk = 16 * ks + 8 * h;
        f16x8_t bk[NNT];
#pragma unroll
        for (int nt = 0; nt < NNT; ++nt) bk[nt] = *reinterpret_cast<const f16x8_t*>(sKt + (32 * (nt0 + nt) + c) * TST + kk);
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) {
          const f16x8_t vr = *reinterpret_cast<const f16x8_t*>(sVt + (32 * mt + c) * TST + kk);
#pragma unroll
          for (int cc = 0; cc < CPW; ++cc) {
            const f16x8_t wr = *reinterpret_cast<const f16x8_t*>(sw + (wc0 + cc) * kMaxMbk + c0 + kk);
            const f16x8_t av = vr * wr;
#pragma unroll
            for (int nt = 0; nt < NNT; ++nt) acc[cc][mt][nt] = mfma32_f16(av, bk[nt], acc[cc][mt][nt]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int cc = 0; cc < CPW; ++cc) {
    const int g = wc0 + cc;
    if (g >= ng) continue;
    const int i = i0 + g;
    const size_t bidx = (static_cast<size_t>(bh) * a.nmb + mb) * Cq + i;
    const float sum = ssum[g];
    const float inv = sum > 0.f ? 1.f / sum : 0.f;
    if (lane == 0 && nt0 == 0) a.blk_lmass[bidx] = sum > 0.f ? smx[g] + __logf(sum) : kNegInf;
    float* out = a.blk_mom + bidx * D * D;
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NNT; ++nt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int dv = 32 * mt + 8 * (v >> 2) + 4 * h + (v & 3);
          out[static_cast<size_t>(dv) * D + 32 * (nt0 + nt) + c] = acc[cc][mt][nt][v] * inv;
        }
  }
}

template <int D>
static void launch_t(const S1Args& a, int which, hipStream_t s) {
  if (which == 0) {
    const size_t lds = static_cast<size_t>((a.Cq + 31) & ~31) * (D + 8) * 2 * sizeof(uint16_t);
    allow_lds((const void*)s1_scores_kernel<D>, lds);
    ProfScope ps_("s1_scores", s);
    hipLaunchKernelGGL((s1_scores_kernel<D>), dim3((a.N + 255) / 256, a.BH), dim3(256), lds, s, a);
  } else if (which == 1) {
    ProfScope ps_("s1_atoms_mfma", s);
    hipLaunchKernelGGL((s1_atoms_mfma_kernel<D>), dim3((a.nb * a.Ck + 3) / 4, a.BH), dim3(256), 0, s, a);
  } else {
    constexpr int G = D == 64 ? 8 : 2;
    ProfScope ps_("s1_moments_f16", s);
    hipLaunchKernelGGL((s1_moments_f16_kernel<D>), dim3(a.nmb, (a.Cq + G - 1) / G, a.BH), dim3(256), 0, s, a);
  }
}

// which: 0 scores, 1 atoms, 2 moments
void launch_stage1_mfma(const S1Args& a, int which, hipStream_t s) {
  if (a.D == 64) launch_t<64>(a, which, s);
  else launch_t<128>(a, which, s);
}

}  // namespace muse
