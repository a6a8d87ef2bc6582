// Exact softmax attention (gfx950): the comparator of the library and, with a block
// size, the exact attention on the diagonal blocks of causal MuSe (pith.science
// review of arXiv 2509.10406, caption of Figure 2), whose partial result is merged
// with the far-field approximation by log-sum-exp:
//   L = log(e^L_loc + e^L_far),  o = e^(L_loc - L) o_loc + e^(L_far - L) o_far.
//
// bf16 path (flash_bf16): workgroup of 4 waves = 128 queries; key/value tiles of 64
// keys staged row-major in LDS, two of each (the tiles after them in registers
// meanwhile), one barrier per tile; per wave S^T = K Q^T on the matrix cores (32 keys x
// 32 queries per tile), online softmax along accumulator rows (one lane and its
// partner), O^T += V^T P^T with P rounded to bf16 and V^T read by the transpose read in
// the key order of the P accumulator. The loop is software-pipelined: the products of
// the next tile's scores are issued between the exponentials of the current one, so
// the matrix cores and the vector ALU work at the same time within a wave. The running
// max is raised only when a row's products exceed it by 8 / (scale log2 e), which leaves
// the result unchanged (it is a stabiliser) and skips most rescaling passes. Workgroups
// are renumbered so that those of one head run on one XCD and share its L2.
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

// EXACT_P: the weights enter the product with V as bf16 hi + lo and the normaliser as
// their fp32 sum (output accurate to fp32 rounding; one more product per step), for the
// backward pass's recomputation of the forward.
// LSE32 (with EXACT_P false, when the log-sum-exp is an output): the log-sum-exp from a
// second, fp32 sum of the weights (one more add per weight), while the output keeps the
// sum of the bf16-rounded weights that enter its product with V.
template <int D, bool EXACT_P, bool LSE32>
__global__ void __launch_bounds__(256, 2) flash_bf16_kernel(ExactArgs a, int nqt) {
  constexpr int BQ = 128, BK = 64;
  constexpr int KST = D + 16;  // bf16 elements per K and V row in LDS (padded)
  constexpr int NKS = D / 16;
  constexpr int NMT = D / 32;
  constexpr int CH = D / 8;    // 16-byte chunks per row
  constexpr int NP = BK * CH / 256;  // 16-byte pieces per thread and tensor
  // two K and two V tiles: iteration j reads K of tile j + 1 and V of tile j while the
  // K of tile j + 2 and the V of tile j + 1 are stored into the other halves
  __shared__ __align__(16) uint16_t sK[2][BK * KST];
  __shared__ __align__(16) uint16_t sV[2][BK * KST];

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

  // queries past the end repeat the last one (their rows are not stored)
  const int qq = qvalid ? qi : N - 1;
  bf16x8_t qf[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks)
    qf[ks] = as_bf16x8(*reinterpret_cast<const u16x8_t*>(Q + static_cast<size_t>(qq) * D + 16 * ks + 8 * h));
  const int kbeg = a.block > 0 ? (qq / a.block) * a.block : 0;
  const int kend = a.causal ? qq + 1 : N;
  // wave-uniform bounds (scalar registers, so that the tile tests are scalar branches)
  const int wkb_min = __builtin_amdgcn_readfirstlane(wave_min_int(kbeg));
  const int wkb_max = __builtin_amdgcn_readfirstlane(wave_max_int(kbeg));
  const int wke_min = __builtin_amdgcn_readfirstlane(wave_min_int(kend));
  const int wke_max = __builtin_amdgcn_readfirstlane(wave_max_int(kend));
  const int qlast = min(q0 + BQ, N) - 1;
  const int gkb = a.block > 0 ? (q0 / a.block) * a.block : 0;
  const int gke = a.causal ? qlast + 1 : N;
  const int T = (gke - gkb + BK - 1) / BK;  // key tiles of this workgroup
  const float sl2 = a.scale * 1.4426950408889634f;
  const float thr = 8.f / sl2;

  // l: the row sum of the weights as they enter the product with V (the output's
  // normaliser); l32 (LSE32): their fp32 sum, for the log-sum-exp output (the bf16
  // rounding of a dominant weight would otherwise shift it by up to 2^-8)
  float m = -1e30f, l = 0.f, l32 = 0.f;
  f32x16_t o[NMT];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) o[mt] = zero16();

  u16x8_t rk[NP], rv[NP];
  auto load_rows = [&](const uint16_t* X, u16x8_t* r, int j) {
    const int kt = gkb + j * BK;
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      // rows past the end repeat the last row: their scores are masked and their weights
      // are zero, so they only need to be finite
      const int e = tid + 256 * q, row = e / CH, cc = e % CH, key = min(kt + row, N - 1);
      r[q] = *reinterpret_cast<const u16x8_t*>(X + static_cast<size_t>(key) * D + cc * 8);
    }
  };
  auto store_rows = [&](uint16_t* S, const u16x8_t* r) {
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      const int e = tid + 256 * q, row = e / CH, cc = e % CH;
      *reinterpret_cast<u16x8_t*>(S + row * KST + cc * 8) = r[q];
    }
  };
  auto scores = [&](const uint16_t* S, f32x16_t* s) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      s[t] = zero16();
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const bf16x8_t af = as_bf16x8(*reinterpret_cast<const u16x8_t*>(S + (32 * t + c) * KST + 16 * ks + 8 * h));
        s[t] = mfma32(af, qf[ks], s[t]);
      }
    }
  };
  auto needed = [&](int j) {
    const int kt = gkb + j * BK;
    return !(kt >= wke_max || kt + BK <= wkb_min);
  };

  // prologue (a workgroup has at least one key tile): K and V of tile 0 and K of tile 1
  // in LDS, the scores of tile 0, and K of tile 2 and V of tile 1 in registers
  load_rows(K, rk, 0);
  load_rows(V, rv, 0);
  store_rows(sK[0], rk);
  store_rows(sV[0], rv);
  load_rows(K, rk, min(1, T - 1));
  store_rows(sK[1], rk);
  __syncthreads();
  f32x16_t sA[2], sB[2];
  scores(sK[0], sA);
  load_rows(K, rk, min(2, T - 1));
  load_rows(V, rv, min(1, T - 1));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t ones = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};

  auto iteration = [&](int j, f32x16_t (&scur)[2], f32x16_t (&snxt)[2]) {
    __syncthreads();  // iteration j - 1 is done everywhere; its stores are visible
    const int kt = gkb + j * BK;
    if (needed(j)) {
      const bool full = kt >= wkb_max && kt + BK <= wke_min && kt + BK <= N;
      if (!full) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int key = kt + 32 * t + 8 * (v >> 2) + 4 * h + (v & 3);
            if (key < kbeg || key >= kend) scur[t][v] = kNegInf;
          }
      }
      // running max on the raw products q.k (the scale is folded into the exponent); it
      // is a stabiliser only, raised (with the accumulators rescaled) when a row's
      // products exceed it by more than 8 / sl2, so the weights stay below 2^8
      float mx = -1e30f;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int v = 0; v < 16; v += 2)
          mx = __builtin_elementwise_maximum(__builtin_elementwise_maximum(mx, scur[t][v]), scur[t][v + 1]);
      mx = __builtin_elementwise_maximum(mx, xor32(mx));
      if (__ballot(mx > m + thr) != 0ull) {
        const float mn = __builtin_elementwise_maximum(m, mx);
        const float alpha = fast_exp2((m - mn) * sl2);
        l *= alpha;
        if constexpr (LSE32) l32 *= alpha;
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
          for (int v = 0; v < 16; ++v) o[mt][v] *= alpha;
        m = mn;
      }
      const float nb = -m * sl2;
      // the next tile's scores on the matrix cores while this tile's weights are formed
      // (after the last tile they are computed from a stale half and not used): the
      // NKS k-steps of its two 32-key halves are spread over the four weight steps
      const uint16_t* sk = sK[(j + 1) & 1];
      snxt[0] = zero16();
      snxt[1] = zero16();
      // p = 2^(s sl2 - m sl2), rounded to bf16 for the product with V; the row sum is
      // taken of the same rounded weights (packed dot products with ones), so that
      // numerator and normaliser use identical values
      const uint16_t* sv = sV[j & 1];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int ss = 0; ss < 2; ++ss) {
#pragma unroll
          for (int u = 0; u < NKS / 4; ++u) {
            const int ks = (2 * t + ss) * (NKS / 4) + u;
#pragma unroll
            for (int tn = 0; tn < 2; ++tn) {
              const bf16x8_t af =
                  as_bf16x8(*reinterpret_cast<const u16x8_t*>(sk + (32 * tn + c) * KST + 16 * ks + 8 * h));
              snxt[tn] = mfma32(af, qf[ks], snxt[tn]);
            }
          }
          float pv[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) pv[i] = fast_exp2(fmaf(scur[t][8 * ss + i], sl2, nb));
          if constexpr (EXACT_P) {
            // the weights as bf16 hi + lo (fp32-accurate products with V) and their fp32 sum
            bf16x8_t ph, pl;
            split_bf16x8(pv, ph, pl);
#pragma unroll
            for (int i = 0; i < 8; ++i) l += pv[i];
#pragma unroll
            for (int mt = 0; mt < NMT; ++mt) {
              const bf16x8_t vt = lds_operand_tr_acc(sv, KST, 32 * t + 16 * ss, 32 * mt, lane);
              o[mt] = mfma32(vt, ph, o[mt]);
              o[mt] = mfma32(vt, pl, o[mt]);
            }
          } else {
            const bf16x8_t bfr = pack_bf16x8(pv);
            if constexpr (LSE32) l32 += ((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7]));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const bf16x2_t p2 = {bfr[2 * i], bfr[2 * i + 1]};
              l = __builtin_amdgcn_fdot2_f32_bf16(p2, ones, l, false);
            }
#pragma unroll
            for (int mt = 0; mt < NMT; ++mt)
              o[mt] = mfma32(lds_operand_tr_acc(sv, KST, 32 * t + 16 * ss, 32 * mt, lane), bfr, o[mt]);
          }
        }
    } else {
      scores(sK[(j + 1) & 1], snxt);
    }
    // stage K of tile j + 2 and V of tile j + 1 into the halves read in iteration j - 1;
    // unconditionally, past the last tile with repeated rows that are never read, so
    // that no branch separates a load from its wait
    store_rows(sK[j & 1], rk);
    store_rows(sV[(j + 1) & 1], rv);
    load_rows(K, rk, min(j + 3, T - 1));
    load_rows(V, rv, min(j + 2, T - 1));
  };
  for (int j = 0; j < T; j += 2) {
    iteration(j, sA, sB);
    if (j + 1 < T) iteration(j + 1, sB, sA);
  }
  const float lt = l + xor32(l);
  const float lt32 = LSE32 ? l32 + xor32(l32) : lt;
  if (!qvalid) return;
  const float inv = 1.f / lt;
  float L = (m * sl2 + __log2f(lt32)) * 0.6931471805599453f;
  const size_t row = base + qi;
  float w0 = inv, w1 = 0.f;
  bool merge = false;
  // the far-field row requested together with its log-sum-exp (a load under `merge`
  // would be issued and waited for one 16-byte piece at a time)
  f32x4_t ofar[NMT][4];
  if (a.l_far != nullptr) {
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        ofar[mt][g] = *reinterpret_cast<const f32x4_t*>(a.o_far + row * D + 32 * mt + 8 * g + 4 * h);
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
#pragma unroll
        for (int r = 0; r < 4; ++r) r4[r] += w1 * ofar[mt][g][r];
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
    const dim3 g(nqt * a.BH);
    if (a.exact_p) {
      if (a.D == 64) hipLaunchKernelGGL((flash_bf16_kernel<64, true, false>), g, dim3(256), 0, s, a, nqt);
      else hipLaunchKernelGGL((flash_bf16_kernel<128, true, false>), g, dim3(256), 0, s, a, nqt);
    } else if (a.lse_out != nullptr) {
      if (a.D == 64) hipLaunchKernelGGL((flash_bf16_kernel<64, false, true>), g, dim3(256), 0, s, a, nqt);
      else hipLaunchKernelGGL((flash_bf16_kernel<128, false, true>), g, dim3(256), 0, s, a, nqt);
    } else {
      if (a.D == 64) hipLaunchKernelGGL((flash_bf16_kernel<64, false, false>), g, dim3(256), 0, s, a, nqt);
      else hipLaunchKernelGGL((flash_bf16_kernel<128, false, false>), g, dim3(256), 0, s, a, nqt);
    }
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
