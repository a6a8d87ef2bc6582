// Stage 2 of MuSe: each query refines its cluster's summaries with its residual
// (gist.science summary of arXiv 2509.10406, Kernmechanismen 1 "Decompositie" and
// 2 "Fase 2"; pith.science review, "What carries the argument").
//
// Query n in cluster i, residual qt = q_n - qbar_i, table entry e (its block for
// causal calls, 0 otherwise):
//   l_j = log Z_ij + s qt . K_ij,   p = softmax_j(l),   L_n = logsumexp_j l_j,
//   o_n = sum_j p_j V_ij + s D_i qt.
// bf16 inputs (s2_mfma): queries are bucketed by (block, cluster) and cut into tiles
// of 32; one wave per tile computes on the matrix cores
//   l^T = K_i qt^T (Ck x 32), P = softmax over the Ck rows, O^T = V_i^T P^T + (s D_i) qt^T,
// with K_i, qt, V_i and P split into bf16 hi + lo parts (three products hi*hi, hi*lo,
// lo*hi; error ~2^-16 relative) and the dipole product in plain bf16 (a small term).
// fp32 inputs (s2_refine): one thread per query; the residual is kept in registers for
// the logits and in LDS (lane-major) for the dipole product, whose table is stored key
// index first so that a row of D_i^T is contiguous.
#include "mfma.hpp"
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
  const bool empty = !(z > 0.f);  // no far-field key at all
  const float inv = empty ? 0.f : 1.f / z;
#pragma unroll
  for (int d = 0; d < D; ++d) acc[d] *= inv;
  if (a.dipole && !empty) {
    const float* dip = a.s_dip + sidx * D * D;  // [dv][dk]
    for (int dk = 0; dk < D; ++dk) {
      const float x = a.scale * s_q[dk][tid];
#pragma unroll
      for (int dv = 0; dv < D; ++dv) acc[dv] = fmaf(dip[dv * D + dk], x, acc[dv]);
    }
  }
  const float L = empty ? kNegInf : mx + __logf(z);
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

// One workgroup per head: tiles of at most 32 consecutive queries inside one
// (block, cluster) bucket of the query permutation.
__global__ void s2_tiles_kernel(S2Args a) {
  const int bh = blockIdx.x;
  const int nbk = a.nb * a.Cq;
  const int32_t* offs = a.offs_q + static_cast<size_t>(bh) * (nbk + 1);
  int2* tiles = a.tiles + static_cast<size_t>(bh) * a.max_tiles;
  int* s_base = a.tile_base + static_cast<size_t>(bh) * (nbk + 1);
  // per-bucket tile counts, scanned by one thread (a few thousand buckets at most in practice)
  if (threadIdx.x == 0) {
    int run = 0;
    for (int u = 0; u < nbk; ++u) {
      s_base[u] = run;
      run += (offs[u + 1] - offs[u] + 31) / 32;
    }
    s_base[nbk] = run;
    a.ntiles[bh] = run;
  }
  __syncthreads();
  for (int u = threadIdx.x; u < nbk; u += blockDim.x) {
    const int n0 = offs[u], n1 = offs[u + 1];
    int t = s_base[u];
    for (int st = n0; st < n1; st += 32) tiles[t++] = make_int2(u, st);
  }
}

template <int D>
__global__ void __launch_bounds__(256) s2_mfma_kernel(S2Args a) {
  constexpr int NKS = D / 16;
  constexpr int NMT = D / 32;
  constexpr int MAXJT = kMaxClusters / 32;
  const int bh = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, h = lane >> 5, c = lane & 31;
  const int t = blockIdx.x * 4 + wave;
  if (t >= a.ntiles[bh]) return;  // whole wave leaves together
  const int2 tile = a.tiles[static_cast<size_t>(bh) * a.max_tiles + t];
  const int u = tile.x, st = tile.y;
  const int b = u / a.Cq, i = u % a.Cq;
  const int32_t* offs = a.offs_q + static_cast<size_t>(bh) * (a.nb * a.Cq + 1);
  const int n = min(32, offs[u + 1] - st);
  const bool valid = c < n;
  const int qn = a.perm_q[static_cast<size_t>(bh) * a.N + st + (valid ? c : 0)];
  const size_t row = static_cast<size_t>(bh) * a.N + qn;
  if (a.causal && b == 0) {  // the first block has no far field
    if (valid) {
      if (h == 0) a.l_far[row] = kNegInf;
      for (int d = h * (D / 2); d < (h + 1) * (D / 2); d += 4) {
        const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
        *reinterpret_cast<f32x4_t*>(a.o_far + row * D + d) = z;
      }
    }
    return;
  }
  const int e = a.causal ? b : 0;
  const size_t sidx = (static_cast<size_t>(bh) * a.nbS + e) * a.Cq + i;
  const int Ck = a.Ck;
  const int njt = (Ck + 31) / 32;

  // residual query fragments (B operand: column = query c, k = d)
  const uint16_t* Q = static_cast<const uint16_t*>(a.q);
  const float* qb = a.qbar + (static_cast<size_t>(bh) * a.Cq + i) * D;
  bf16x8_t qhi[NKS], qlo[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    const int d0 = 16 * ks + 8 * h;
    const u16x8_t u8 = *reinterpret_cast<const u16x8_t*>(Q + row * D + d0);
    float x[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) x[r] = valid ? bf16_to_f32(u8[r]) - qb[d0 + r] : 0.f;
    split_bf16x8(x, qhi[ks], qlo[ks]);
  }

  // logits^T, in log2 units
  const float* lz = a.s_logz + sidx * Ck;
  const uint16_t* khi = a.t_khi + sidx * Ck * D;
  const uint16_t* klo = a.t_klo + sidx * Ck * D;
  const float sl2 = a.scale * 1.4426950408889634f;
  f32x16_t lg[MAXJT];
  float mx = -1e30f;
#pragma unroll
  for (int jt = 0; jt < MAXJT; ++jt) {
    if (jt >= njt) break;
    f32x16_t acc = zero16();
    const int j = 32 * jt + c;
    const bool jok = j < Ck;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      u16x8_t ah = {0, 0, 0, 0, 0, 0, 0, 0}, al = {0, 0, 0, 0, 0, 0, 0, 0};
      if (jok) {
        ah = *reinterpret_cast<const u16x8_t*>(khi + static_cast<size_t>(j) * D + 16 * ks + 8 * h);
        al = *reinterpret_cast<const u16x8_t*>(klo + static_cast<size_t>(j) * D + 16 * ks + 8 * h);
      }
      acc = mfma32(as_bf16x8(ah), qhi[ks], acc);
      acc = mfma32(as_bf16x8(ah), qlo[ks], acc);
      acc = mfma32(as_bf16x8(al), qhi[ks], acc);
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int jj = 32 * jt + 8 * (v >> 2) + 4 * h + (v & 3);
      const float l0 = jj < Ck ? lz[jj] : kNegInf;
      const float x = (l0 == kNegInf) ? kNegInf : l0 * 1.4426950408889634f + sl2 * acc[v];
      acc[v] = x;
      mx = fmaxf(mx, x);
    }
    lg[jt] = acc;
  }
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  float z = 0.f;
#pragma unroll
  for (int jt = 0; jt < MAXJT; ++jt) {
    if (jt >= njt) break;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float p = fast_exp2(lg[jt][v] - mx);
      lg[jt][v] = p;
      z += p;
    }
  }
  z += __shfl_xor(z, 32, 64);
  const float invz = z > 0.f ? 1.f / z : 0.f;  // z == 0: no far-field key at all

  // O^T = V^T P^T (split), then / z, then + (s D_i) qt^T
  const uint16_t* vthi = a.t_vthi + sidx * Ck * D;
  const uint16_t* vtlo = a.t_vtlo + sidx * Ck * D;
  f32x16_t o[NMT];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) o[mt] = zero16();
#pragma unroll
  for (int jt = 0; jt < MAXJT; ++jt) {
    if (jt >= njt) break;
#pragma unroll
    for (int ss = 0; ss < 2; ++ss) {
      float pv[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) pv[r] = lg[jt][8 * ss + r];
      bf16x8_t phi, plo;
      split_bf16x8(pv, phi, plo);
      const int j0 = 32 * jt + 16 * ss + 4 * h;
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) {
        const size_t rofs = static_cast<size_t>(32 * mt + c) * Ck;
        u16x8_t vh = {0, 0, 0, 0, 0, 0, 0, 0}, vl = {0, 0, 0, 0, 0, 0, 0, 0};
        if ((Ck & 3) == 0) {  // 8-byte aligned groups of 4 (j0 is a multiple of 4)
          if (j0 < Ck) {
            const u16x4_t h4 = *reinterpret_cast<const u16x4_t*>(vthi + rofs + j0);
            const u16x4_t l4 = *reinterpret_cast<const u16x4_t*>(vtlo + rofs + j0);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              vh[r] = h4[r];
              vl[r] = l4[r];
            }
          }
          if (j0 + 8 < Ck) {
            const u16x4_t h4 = *reinterpret_cast<const u16x4_t*>(vthi + rofs + j0 + 8);
            const u16x4_t l4 = *reinterpret_cast<const u16x4_t*>(vtlo + rofs + j0 + 8);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              vh[4 + r] = h4[r];
              vl[4 + r] = l4[r];
            }
          }
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if (j0 + r < Ck) {
              vh[r] = vthi[rofs + j0 + r];
              vl[r] = vtlo[rofs + j0 + r];
            }
            if (j0 + 8 + r < Ck) {
              vh[4 + r] = vthi[rofs + j0 + 8 + r];
              vl[4 + r] = vtlo[rofs + j0 + 8 + r];
            }
          }
        }
        o[mt] = mfma32(as_bf16x8(vh), phi, o[mt]);
        o[mt] = mfma32(as_bf16x8(vh), plo, o[mt]);
        o[mt] = mfma32(as_bf16x8(vl), phi, o[mt]);
      }
    }
  }
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[mt][v] *= invz;
  if (a.dipole) {
    const uint16_t* dip = a.t_dip + sidx * D * D;
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const u16x8_t ad = *reinterpret_cast<const u16x8_t*>(dip + static_cast<size_t>(32 * mt + c) * D + 16 * ks + 8 * h);
        o[mt] = mfma32(as_bf16x8(ad), qhi[ks], o[mt]);
      }
  }
  // lanes (c, h) hold rows d = 32 mt + 8 g + 4 h + r of query c
  if (!valid) return;
  const float L = z > 0.f ? (mx + __log2f(z)) * 0.6931471805599453f : kNegInf;
  if (a.causal) {
    if (h == 0) a.l_far[row] = L;
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4_t f = {o[mt][4 * g], o[mt][4 * g + 1], o[mt][4 * g + 2], o[mt][4 * g + 3]};
        *reinterpret_cast<f32x4_t*>(a.o_far + row * D + 32 * mt + 8 * g + 4 * h) = f;
      }
  } else {
    if (a.lse_out != nullptr && h == 0) a.lse_out[row] = L;
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * mt + 8 * g + 4 * h;
        if (a.out_bf16) {
          const u16x4_t u4 = {f32_to_bf16_bits(o[mt][4 * g]), f32_to_bf16_bits(o[mt][4 * g + 1]),
                              f32_to_bf16_bits(o[mt][4 * g + 2]), f32_to_bf16_bits(o[mt][4 * g + 3])};
          *reinterpret_cast<u16x4_t*>(static_cast<uint16_t*>(a.out) + row * D + d0) = u4;
        } else {
          const f32x4_t f = {o[mt][4 * g], o[mt][4 * g + 1], o[mt][4 * g + 2], o[mt][4 * g + 3]};
          *reinterpret_cast<f32x4_t*>(static_cast<float*>(a.out) + row * D + d0) = f;
        }
      }
  }
}

hipError_t launch_stage2(const S2Args& a, int dtype, hipStream_t s) {
  if (dtype == 1) {
    {
      ProfScope ps_("s2_tiles", s);
      hipLaunchKernelGGL(s2_tiles_kernel, dim3(a.BH), dim3(256), 0, s, a);
    }
    ProfScope ps_("s2_mfma", s);
    const dim3 gm((a.max_tiles + 3) / 4, a.BH);
    if (a.D == 64) hipLaunchKernelGGL((s2_mfma_kernel<64>), gm, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((s2_mfma_kernel<128>), gm, dim3(256), 0, s, a);
    return hipGetLastError();
  }
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
