// Backward pass of the MuSe forward (gfx950), acausal and causal (prefix form).
//
// The reviews note that the method's backward pass uses the same approximations as its
// forward and that its error was never measured (pith.science review, "Reading between
// the lines"). Differentiated here: the forward output o(q, k, v) with the K-means labels
// held fixed (the clustering is piecewise constant in q and k). With s the softmax scale,
// for query n of query cluster i (qt_n = q_n - qbar_i, qbar_i the member mean) and key m
// of key cluster j:
//   stage 2  o_n = sum_j p_nj V_ij + s D_i qt_n,   p_n = softmax_j (log Z_ij + s qt_n . K_ij)
//   stage 1  a_im = s qbar_i . k_m,  w_im = exp(a_im - log Z_ij),  log Z_ij = lse_{m in j} a_im,
//            K_ij = sum w k,  V_ij = sum w v,  P_ij = softmax_j log Z_ij,
//            D_i = sum_j P_ij C_ij  with  C_ij = sum w v k^T - V_ij K_ij^T  (tilted)  or
//            C_ij = Cov_j (untilted: the plain covariance of cluster j)
// (pith.science review, "What carries the argument" and "Assumptions & free parameters";
// gist.science summary, Kernmechanismen 2). The gradients, in reverse:
//   bw_refine    per query cluster i: dL/dlog Z_i., dL/dK_i., dL/dV_i., dL/dD_i (G_Dip_i),
//                the residual part of dq and its sum (the stage-2 part of dL/dqbar_i).
//   bw_prep_i    per i: P_i., log sum_j Z_ij, G_Dip_i in bf16 hi + lo (both layouts), and
//                dK'_ij = dL/dK_ij - P_ij G_Dip_i^T V_ij, dV'_ij = dL/dV_ij - P_ij G_Dip_i K_ij
//                (the tilted dipole's C_ij depends on K_ij and V_ij), V_ij^T G_Dip_i K_ij.
//   bw_prep_j    (untilted) per j: dL/dP_ij = <G_Dip_i, Cov_j>, sum_i P_ij G_Dip_i, means.
//   bw_scores    a_im at every key position (bucket order).
//   bw_keys_a    (tilted) per 128 keys, on the matrix cores: Q_im = v_m^T G_Dip_i k_m, and
//                the dipole's direct terms  dk_m = sum_i p_im G_Dip_i^T v_m,
//                dv_m = sum_i p_im G_Dip_i k_m  (p_im = w_im P_ij = exp(a_im) / sum_j Z_ij).
//   bw_dlogz     per i: dL/dP_ij = sum_{m in j} w_im Q_im - V_ij^T G_Dip_i K_ij (tilted),
//                dL/dlog Z_ij through P, and sum_{m in j} w_im dL/dw_im in closed form.
//   bw_keys_b    per 64 keys: dL/dw_im, da_im = w_im (dL/dw_im - sum_j + dL/dlog Z_ij), the
//                rest of dk_m and dv_m, and per tile s sum_m w dL/dw k_m for dL/dqbar.
//   bw_centroid  per i: dL/dqbar_i, spread over the members (qbar is their mean).
// Causal calls (block b's far field summarises the keys of blocks < b and is merged with
// exact attention inside the block by log-sum-exp; gist.science summary, Kernmechanismen
// 3; pith.science review, caption of Figure 2) add:
//   bw_merge     the merge's backward: the far field's and the in-block part's shares of
//                dL/do and dL/d(log normaliser).
//   (per entry)  bw_refine, bw_prep_i for every (block, query cluster) against table entry
//                b; bw_entry: dL/dlog Z - S through the dipole's aggregated form.
//   bw_suffix    the suffix sums over the later entries that a key's gradient needs.
//   bw_keys_a/b  against the suffix tables of the key's block.
//   bw_local_*   the exact in-block attention's backward.
// All arithmetic in fp32 (bf16 inputs are exact in it); the matrix-core products split
// G_Dip (and fp32 keys and values) into bf16 hi + lo. Every sum runs in a fixed order.
#include "mfma.hpp"
#include "muse_kernels.hpp"

namespace muse {

constexpr int kBwQT = 16;   // queries per tile of the stage-2 backward
constexpr int kBwGST = kBwD + 8;  // LDS row stride (bf16) of the staged G_Dip tiles

// dL/dlog Z, dL/dK, dL/dV, dL/dD of one query cluster and the residual part of dq.
// LDS: K_i. and V_i. rows and D_i (fp32, rows padded to 68 floats: 16-byte reads by 16
// lanes hit distinct banks), the tile's residuals and upstream gradients, and the tile's
// weights p and dl = dL/dlogit; every product reads its operands 4 at a time.
// Causal calls: one workgroup per (block b, query cluster i) bucket, against table entry
// b, with the far field's share of the upstream gradient (fp32) and of dL/dlog-normaliser.
template <typename T, typename TG>
__global__ void __launch_bounds__(256) bw_refine_kernel(BwArgs a) {
  constexpr int D = kBwD, DP = D + 4, CP = kMaxClusters + 4, QT = kBwQT;
  __shared__ __align__(16) float sK[kMaxClusters * DP];
  __shared__ __align__(16) float sV[kMaxClusters * DP];
  __shared__ __align__(16) float sDip[D * DP];
  __shared__ __align__(16) float sQt[QT * DP];
  __shared__ __align__(16) float sG[QT * DP];
  __shared__ __align__(16) float sL[QT * CP];
  __shared__ __align__(16) float sDl[QT * CP];
  __shared__ float sLz[kMaxClusters];
  __shared__ float sQbar[D];
  __shared__ int sRow[QT];
  __shared__ float sDL[QT];    // dL/d(log normaliser) of the tile's queries (causal far field)
  __shared__ __align__(16) float sRed[QT][D];
  const int e = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int Cq = a.Cq, Ck = a.Ck, N = a.N, Ck4 = (Ck + 3) & ~3;
  const int nbS = a.causal ? a.nb : 1;
  const int i = e % Cq;
  const float s = a.scale;
  const bool dip = a.dipole != 0;
  const size_t ti = static_cast<size_t>(bh) * nbS * Cq + e;  // table entry e / Cq, cluster i
  // tables; rows Ck .. Ck4 - 1 of K and columns Ck .. Ck4 - 1 of dl stay zero
  for (int e = tid; e < Ck4 * D; e += 256) {
    const int j = e / D, d = e % D;
    sK[j * DP + d] = j < Ck ? a.tk[ti * Ck * D + e] : 0.f;
    sV[j * DP + d] = j < Ck ? a.tv[ti * Ck * D + e] : 0.f;
  }
  for (int e = tid; e < D * D; e += 256) sDip[(e / D) * DP + e % D] = dip ? a.dip[ti * D * D + e] : 0.f;
  for (int e = tid; e < QT * CP; e += 256) sDl[e] = 0.f;
  for (int j = tid; j < Ck; j += 256) sLz[j] = a.logz[ti * Ck + j];
  if (tid < D) sQbar[tid] = a.qbar[(static_cast<size_t>(bh) * Cq + i) * D + tid];
  const int32_t* offq = a.offs_q + static_cast<size_t>(bh) * (nbS * Cq + 1);
  const int o0 = offq[e], o1 = offq[e + 1];
  const int32_t* perm = a.perm_q + static_cast<size_t>(bh) * N;
  const T* Q = static_cast<const T*>(a.q) + static_cast<size_t>(bh) * N * D;
  const TG* G = static_cast<const TG*>(a.causal ? static_cast<const void*>(a.o_far) : a.dout) + static_cast<size_t>(bh) * N * D;
  const float* dLn = a.causal ? a.l_far + static_cast<size_t>(bh) * N : nullptr;
  float* dq = a.dq + static_cast<size_t>(bh) * N * D;
  // summary-gradient accumulators: dL/dK, dL/dV of cluster aj, dims ad0 .. ad0 + 31
  const int aj = tid >> 1, ad0 = (tid & 1) * 32;
  f32x4_t gk[8], gv[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) gk[r] = gv[r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // dL/dD_i: row pv (value index), columns pd0 .. pd0 + 15
  const int pv = tid >> 2, pd0 = (tid & 3) * 16;
  f32x4_t gdp[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) gdp[r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float glz = 0.f;                                  // dL/dlog Z_ij for j = tid
  const int eq = tid >> 4, ed0 = (tid & 15) * 4;    // dq: query eq of the tile, dims ed0 .. ed0 + 3
  f32x4_t qbs = {0.f, 0.f, 0.f, 0.f};               // - sum of this thread's dq values
  // this thread's elements of a query tile: rows wave + 4 r (r < 4), dimension lane; the
  // next tile's rows travel in registers while the current tile is processed
  constexpr int RPT = QT * D / 256;
  int pn[RPT];
  float pq[RPT], pg[RPT], pdl[RPT];
  auto fetch = [&](int t0) {
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      const int qq = wave + 4 * r;
      pn[r] = t0 + qq < o1 ? perm[t0 + qq] : -1;
    }
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      pq[r] = pn[r] >= 0 ? Elem<T>::load(Q, static_cast<size_t>(pn[r]) * D + lane) : 0.f;
      pg[r] = pn[r] >= 0 ? Elem<TG>::load(G, static_cast<size_t>(pn[r]) * D + lane) : 0.f;
      pdl[r] = (dLn != nullptr && pn[r] >= 0) ? dLn[pn[r]] : 0.f;
    }
  };
  if (o0 < o1) fetch(o0);
  __syncthreads();
  for (int t0 = o0; t0 < o1; t0 += QT) {
    const int nq = min(QT, o1 - t0);
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      const int qq = wave + 4 * r;
      sQt[qq * DP + lane] = pn[r] >= 0 ? pq[r] - sQbar[lane] : 0.f;
      sG[qq * DP + lane] = pg[r];
      if (lane == 0) {
        sRow[qq] = pn[r];
        sDL[qq] = pdl[r];
      }
    }
    __syncthreads();
    if (t0 + QT < o1) fetch(t0 + QT);
    {
      // logits and dp_nj = g_n . V_ij: cluster j, queries q0 .. q0 + 7
      const int j = tid & 127, q0 = (tid >> 7) * 8;
      if (j < Ck) {
        float l[8], dp[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) l[r] = dp[r] = 0.f;
        for (int d = 0; d < D; d += 4) {
          const f32x4_t k4 = *reinterpret_cast<const f32x4_t*>(&sK[j * DP + d]);
          const f32x4_t v4 = *reinterpret_cast<const f32x4_t*>(&sV[j * DP + d]);
#pragma unroll
          for (int r = 0; r < 8; ++r) {
            const f32x4_t q4 = *reinterpret_cast<const f32x4_t*>(&sQt[(q0 + r) * DP + d]);
            const f32x4_t g4 = *reinterpret_cast<const f32x4_t*>(&sG[(q0 + r) * DP + d]);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              l[r] = fmaf(q4[c], k4[c], l[r]);
              dp[r] = fmaf(g4[c], v4[c], dp[r]);
            }
          }
        }
        const float lz = sLz[j];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          sL[(q0 + r) * CP + j] = lz == kNegInf ? kNegInf : lz + s * l[r];
          sDl[(q0 + r) * CP + j] = dp[r];
        }
      }
    }
    __syncthreads();
    // softmax over the key clusters and dl = p (dp - sum_j p dp): a wave per row
    for (int qq = wave; qq < QT; qq += 4) {
      float lv[2], dv2[2], mx = kNegInf;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int j = lane + 64 * t;
        lv[t] = j < Ck ? sL[qq * CP + j] : kNegInf;
        dv2[t] = j < Ck ? sDl[qq * CP + j] : 0.f;
        mx = fmaxf(mx, lv[t]);
      }
      mx = wave_max(mx);
      float e2[2], z = 0.f;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        e2[t] = lv[t] == kNegInf ? 0.f : __expf(lv[t] - mx);
        z += e2[t];
      }
      z = wave_sum(z);
      const float inv = (z > 0.f && qq < nq) ? 1.f / z : 0.f;
      float rs = 0.f;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        e2[t] *= inv;
        rs = fmaf(e2[t], dv2[t], rs);
      }
      rs = wave_sum(rs) - sDL[qq];  // the log normaliser's gradient adds p dL/dL_far
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int j = lane + 64 * t;
        if (j < Ck) {
          sL[qq * CP + j] = e2[t];
          sDl[qq * CP + j] = e2[t] * (dv2[t] - rs);
        }
      }
    }
    __syncthreads();
    if (aj < Ck) {
      for (int qq = 0; qq < nq; ++qq) {
        const float p = sL[qq * CP + aj], dl = sDl[qq * CP + aj];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const f32x4_t g4 = *reinterpret_cast<const f32x4_t*>(&sG[qq * DP + ad0 + 4 * r]);
          const f32x4_t q4 = *reinterpret_cast<const f32x4_t*>(&sQt[qq * DP + ad0 + 4 * r]);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            gv[r][c] = fmaf(p, g4[c], gv[r][c]);
            gk[r][c] = fmaf(dl, q4[c], gk[r][c]);
          }
        }
      }
    }
    if (tid < Ck)
      for (int qq = 0; qq < nq; ++qq) glz += sDl[qq * CP + tid];
    if (dip) {
      for (int qq = 0; qq < nq; ++qq) {
        const float g = sG[qq * DP + pv];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const f32x4_t q4 = *reinterpret_cast<const f32x4_t*>(&sQt[qq * DP + pd0 + 4 * r]);
#pragma unroll
          for (int c = 0; c < 4; ++c) gdp[r][c] = fmaf(g, q4[c], gdp[r][c]);
        }
      }
    }
    {
      // dq_n = s sum_j dl_nj K_ij + s D_i^T g_n: query eq, dims ed0 .. ed0 + 3
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
      for (int j = 0; j < Ck4; j += 4) {
        const f32x4_t dl4 = *reinterpret_cast<const f32x4_t*>(&sDl[eq * CP + j]);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const f32x4_t k4 = *reinterpret_cast<const f32x4_t*>(&sK[(j + t) * DP + ed0]);
#pragma unroll
          for (int c = 0; c < 4; ++c) acc[c] = fmaf(dl4[t], k4[c], acc[c]);
        }
      }
      if (dip) {
        for (int vv = 0; vv < D; vv += 4) {
          const f32x4_t g4 = *reinterpret_cast<const f32x4_t*>(&sG[eq * DP + vv]);
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const f32x4_t d4 = *reinterpret_cast<const f32x4_t*>(&sDip[(vv + t) * DP + ed0]);
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[c] = fmaf(g4[t], d4[c], acc[c]);
          }
        }
      }
      if (eq < nq) {
        const f32x4_t x = {s * acc[0], s * acc[1], s * acc[2], s * acc[3]};
        *reinterpret_cast<f32x4_t*>(dq + static_cast<size_t>(sRow[eq]) * D + ed0) = x;
#pragma unroll
        for (int c = 0; c < 4; ++c) qbs[c] -= x[c];
      }
    }
    __syncthreads();  // the tile buffers are rewritten next
  }
  if (aj < Ck) {
    const size_t o = (ti * Ck + aj) * D + ad0;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      *reinterpret_cast<f32x4_t*>(a.g_k + o + 4 * r) = f32x4_t{s * gk[r][0], s * gk[r][1], s * gk[r][2], s * gk[r][3]};
      *reinterpret_cast<f32x4_t*>(a.g_v + o + 4 * r) = gv[r];
    }
  }
  if (tid < Ck) a.g_logz[ti * Ck + tid] = glz;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const f32x4_t x = dip ? f32x4_t{s * gdp[r][0], s * gdp[r][1], s * gdp[r][2], s * gdp[r][3]}
                          : f32x4_t{0.f, 0.f, 0.f, 0.f};
    *reinterpret_cast<f32x4_t*>(a.g_dip + ti * D * D + static_cast<size_t>(pv) * D + pd0 + 4 * r) = x;
  }
  *reinterpret_cast<f32x4_t*>(&sRed[eq][ed0]) = qbs;
  __syncthreads();
  if (tid < D) {
    float x = 0.f;
    for (int q = 0; q < QT; ++q) x += sRed[q][tid];
    a.dqbar2[ti * D + tid] = x;
  }
}

// The stage-2 backward on the matrix cores (bf16 inputs): one workgroup per bucket as
// above, 32 queries per tile. The fp32 operands (K_i., V_i., D_i, the residuals qt, an
// fp32 upstream gradient, p and dl) enter as bf16 hi + lo (three products where both
// sides are fp32, so every product is fp32-accurate up to about 2^-16). Per tile:
//   wave w (key clusters 32 w .. 32 w + 31): L^T = K qt^T and dP^T = V g^T, then the
//     softmax over all clusters (cross-wave max and sums through LDS), p and
//     dl = p (dp - sum_j p dp + dL) stored transposed (cluster rows) as bf16 hi, lo;
//     dL/dV^T += g^T P and dL/dK^T += qt^T dl for its clusters (accumulators over the
//     bucket), and dL/dlog Z partials;
//   waves 0, 1 (dimensions 32 w ..): dq^T = K^T dl^T + D_i^T g^T;
//   waves 2, 3: dL/dD_i += g^T qt (two 32 x 32 tiles each).
// Operands that run along the LDS rows are read by the transpose read.
constexpr int kRfQT = 32, kRfST = kBwD + 8, kRfPT = kRfQT + 8;

__host__ __device__ constexpr size_t bw_refine_mfma_lds(int Ck) {
  const size_t ckp = 32 * static_cast<size_t>((Ck + 31) / 32);
  return sizeof(uint16_t) * (4 * ckp * kRfST + 2 * kBwD * kRfST + 4 * kRfQT * kRfST + 4 * ckp * kRfPT) +
         sizeof(float) * (3 * 4 * kRfQT + ckp + kBwD + kRfQT) + sizeof(int) * kRfQT;
}

template <typename TG>
__global__ void __launch_bounds__(256) bw_refine_mfma_kernel(BwArgs a) {
  constexpr int D = kBwD, ST = kRfST, PT = kRfPT, QT = kRfQT, NKS = D / 16;
  constexpr bool GF = sizeof(TG) == 4;  // fp32 upstream gradient: hi + lo
  extern __shared__ __align__(16) unsigned char lds_raw[];
  const int e = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x, lane = tid & 63, h = lane >> 5, c = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int Cq = a.Cq, Ck = a.Ck, N = a.N, njt = (Ck + 31) / 32, Ckp = 32 * njt;
  const int nbS = a.causal ? a.nb : 1;
  const int i = e % Cq;
  const float s = a.scale;
  const bool dip = a.dipole != 0;
  const size_t ti = static_cast<size_t>(bh) * nbS * Cq + e;
  uint16_t* sKh = reinterpret_cast<uint16_t*>(lds_raw);
  uint16_t* sKl = sKh + Ckp * ST;
  uint16_t* sVh = sKl + Ckp * ST;
  uint16_t* sVl = sVh + Ckp * ST;
  uint16_t* sDh = sVl + Ckp * ST;   // D_i rows v
  uint16_t* sDl = sDh + D * ST;
  uint16_t* sQh = sDl + D * ST;     // tile residual rows
  uint16_t* sQl = sQh + QT * ST;
  uint16_t* sGh = sQl + QT * ST;    // tile upstream-gradient rows
  uint16_t* sGl = sGh + QT * ST;
  uint16_t* sPh = sGl + QT * ST;    // P^T: cluster rows, query columns
  uint16_t* sPl = sPh + Ckp * PT;
  uint16_t* sLh = sPl + Ckp * PT;   // dl^T
  uint16_t* sLl = sLh + Ckp * PT;
  float* sRed = reinterpret_cast<float*>(sLl + Ckp * PT);  // [3][4][QT]: max, sum, sum e dp
  float* sLz = sRed + 3 * 4 * QT;
  float* sQbar = sLz + Ckp;
  float* sDL = sQbar + D;
  int* sRow = reinterpret_cast<int*>(sDL + QT);
  auto split_store = [&](uint16_t* hi, uint16_t* lo, int o, float x) {
    const uint16_t xh = f32_to_bf16_bits(x);
    hi[o] = xh;
    lo[o] = f32_to_bf16_bits(x - bf16_to_f32(xh));
  };
  // the bucket's tables (rows Ck .. Ckp - 1 zero, their log Z -inf), four values per
  // thread and step: 16-byte loads, hi and lo written 8 bytes at a time
  auto split4 = [&](uint16_t* hi, uint16_t* lo, int o, const f32x4_t& x) {
    u16x4_t h4, l4;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      h4[u] = f32_to_bf16_bits(x[u]);
      l4[u] = f32_to_bf16_bits(x[u] - bf16_to_f32(h4[u]));
    }
    *reinterpret_cast<u16x4_t*>(hi + o) = h4;
    *reinterpret_cast<u16x4_t*>(lo + o) = l4;
  };
  for (int x = tid; x < Ckp * D / 4; x += 256) {
    const int j = x / (D / 4), d = 4 * (x % (D / 4));
    const f32x4_t z4 = {0.f, 0.f, 0.f, 0.f};
    const f32x4_t kv = j < Ck ? *reinterpret_cast<const f32x4_t*>(a.tk + (ti * Ck + j) * D + d) : z4;
    const f32x4_t vv = j < Ck ? *reinterpret_cast<const f32x4_t*>(a.tv + (ti * Ck + j) * D + d) : z4;
    split4(sKh, sKl, j * ST + d, kv);
    split4(sVh, sVl, j * ST + d, vv);
  }
  for (int x = tid; x < D * D / 4; x += 256) {
    const int r = x / (D / 4), d = 4 * (x % (D / 4));
    const f32x4_t z4 = {0.f, 0.f, 0.f, 0.f};
    split4(sDh, sDl, r * ST + d, dip ? *reinterpret_cast<const f32x4_t*>(a.dip + ti * D * D + r * D + d) : z4);
  }
  for (int j = tid; j < Ckp; j += 256) sLz[j] = j < Ck ? a.logz[ti * Ck + j] : kNegInf;
  if (tid < D) sQbar[tid] = a.qbar[(static_cast<size_t>(bh) * Cq + i) * D + tid];
  const int32_t* offq = a.offs_q + static_cast<size_t>(bh) * (nbS * Cq + 1);
  const int o0 = offq[e], o1 = offq[e + 1];
  const int32_t* perm = a.perm_q + static_cast<size_t>(bh) * N;
  const uint16_t* Q = static_cast<const uint16_t*>(a.q) + static_cast<size_t>(bh) * N * D;
  const TG* G = static_cast<const TG*>(a.causal ? static_cast<const void*>(a.o_far) : a.dout) + static_cast<size_t>(bh) * N * D;
  const float* dLn = a.causal ? a.l_far + static_cast<size_t>(bh) * N : nullptr;
  float* dq = a.dq + static_cast<size_t>(bh) * N * D;
  const bool ownj = 32 * wave < Ck;  // this wave's clusters exist
  f32x16_t gvt[2], gkt[2], dqa, gdp[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) gvt[q] = gkt[q] = gdp[q] = zero16();
  float glz[16], qbs[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) glz[v] = qbs[v] = 0.f;
  __syncthreads();
  for (int t0 = o0; t0 < o1; t0 += QT) {
    // stage the tile: thread -> query row tid / 8, dimensions 8 (tid % 8) .. + 7
    {
      const int r = tid >> 3, d0 = (tid & 7) * 8;
      const int n = t0 + r < o1 ? perm[t0 + r] : -1;
      float qv[8], gv[8];
      if (n >= 0) {
        const u16x8_t q8 = *reinterpret_cast<const u16x8_t*>(Q + static_cast<size_t>(n) * D + d0);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          qv[u] = bf16_to_f32(q8[u]) - sQbar[d0 + u];
          gv[u] = Elem<TG>::load(G, static_cast<size_t>(n) * D + d0 + u);
        }
      } else {
#pragma unroll
        for (int u = 0; u < 8; ++u) qv[u] = gv[u] = 0.f;
      }
      bf16x8_t qh, ql, gh, gl;
      split_bf16x8(qv, qh, ql);
      split_bf16x8(gv, gh, gl);
      *reinterpret_cast<bf16x8_t*>(&sQh[r * ST + d0]) = qh;
      *reinterpret_cast<bf16x8_t*>(&sQl[r * ST + d0]) = ql;
      *reinterpret_cast<bf16x8_t*>(&sGh[r * ST + d0]) = gh;
      *reinterpret_cast<bf16x8_t*>(&sGl[r * ST + d0]) = gl;
      if ((tid & 7) == 0) {
        sRow[r] = n;
        sDL[r] = (dLn != nullptr && n >= 0) ? dLn[n] : 0.f;
      }
    }
    __syncthreads();
    // logits and dp for this wave's clusters (rows 32 w + 8 (v / 4) + 4 h + v % 4, query c)
    f32x16_t lt = zero16(), dpt = zero16();
    if (ownj) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int ok = (32 * wave + c) * ST + 16 * ks + 8 * h, oq = c * ST + 16 * ks + 8 * h;
        const bf16x8_t kh = *reinterpret_cast<const bf16x8_t*>(&sKh[ok]), kl = *reinterpret_cast<const bf16x8_t*>(&sKl[ok]);
        const bf16x8_t vh = *reinterpret_cast<const bf16x8_t*>(&sVh[ok]), vl = *reinterpret_cast<const bf16x8_t*>(&sVl[ok]);
        const bf16x8_t qh = *reinterpret_cast<const bf16x8_t*>(&sQh[oq]), ql = *reinterpret_cast<const bf16x8_t*>(&sQl[oq]);
        const bf16x8_t gh = *reinterpret_cast<const bf16x8_t*>(&sGh[oq]);
        lt = mfma32(kh, qh, lt);
        lt = mfma32(kh, ql, lt);
        lt = mfma32(kl, qh, lt);
        dpt = mfma32(vh, gh, dpt);
        dpt = mfma32(vl, gh, dpt);
        if (GF) dpt = mfma32(vh, *reinterpret_cast<const bf16x8_t*>(&sGl[oq]), dpt);
      }
    }
    float lg[16], mx = kNegInf;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float lz = ownj ? sLz[32 * wave + 8 * (v >> 2) + 4 * h + (v & 3)] : kNegInf;
      lg[v] = lz == kNegInf ? kNegInf : lz + s * lt[v];
      mx = fmaxf(mx, lg[v]);
    }
    mx = fmaxf(mx, xor32(mx));
    if (h == 0) sRed[wave * QT + c] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(sRed[c], sRed[QT + c]), fmaxf(sRed[2 * QT + c], sRed[3 * QT + c]));
    float ev[16], z = 0.f, zd = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      ev[v] = lg[v] == kNegInf ? 0.f : __expf(lg[v] - mx);
      z += ev[v];
      zd = fmaf(ev[v], dpt[v], zd);
    }
    z += xor32(z);
    zd += xor32(zd);
    if (h == 0) {
      sRed[4 * QT + wave * QT + c] = z;
      sRed[8 * QT + wave * QT + c] = zd;
    }
    __syncthreads();
    const float zt = (sRed[4 * QT + c] + sRed[5 * QT + c]) + (sRed[6 * QT + c] + sRed[7 * QT + c]);
    const float zdt = (sRed[8 * QT + c] + sRed[9 * QT + c]) + (sRed[10 * QT + c] + sRed[11 * QT + c]);
    const bool qok = sRow[c] >= 0;
    const float inv = (zt > 0.f && qok) ? 1.f / zt : 0.f;
    const float rs = zdt * inv - sDL[c];  // sum_j p dp - dL/dL_far
    if (ownj) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float p = ev[v] * inv;
        const float dl = p * (dpt[v] - rs);
        glz[v] += dl;
        const int o = (32 * wave + 8 * (v >> 2) + 4 * h + (v & 3)) * PT + c;
        split_store(sPh, sPl, o, p);
        split_store(sLh, sLl, o, dl);
      }
    }
    __syncthreads();
    if (ownj) {
      // dL/dV^T += g^T P, dL/dK^T += qt^T dl (dimension rows, this wave's cluster columns)
#pragma unroll
      for (int ks = 0; ks < QT / 16; ++ks) {
        const int ob = (32 * wave + c) * PT + 16 * ks + 8 * h;
        const bf16x8_t ph = *reinterpret_cast<const bf16x8_t*>(&sPh[ob]), pl = *reinterpret_cast<const bf16x8_t*>(&sPl[ob]);
        const bf16x8_t lh = *reinterpret_cast<const bf16x8_t*>(&sLh[ob]), ll = *reinterpret_cast<const bf16x8_t*>(&sLl[ob]);
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
          const bf16x8_t gth = lds_operand_tr(sGh, ST, 16 * ks, 32 * dt, lane);
          const bf16x8_t qth = lds_operand_tr(sQh, ST, 16 * ks, 32 * dt, lane);
          const bf16x8_t qtl = lds_operand_tr(sQl, ST, 16 * ks, 32 * dt, lane);
          gvt[dt] = mfma32(gth, ph, gvt[dt]);
          gvt[dt] = mfma32(gth, pl, gvt[dt]);
          if (GF) gvt[dt] = mfma32(lds_operand_tr(sGl, ST, 16 * ks, 32 * dt, lane), ph, gvt[dt]);
          gkt[dt] = mfma32(qth, lh, gkt[dt]);
          gkt[dt] = mfma32(qth, ll, gkt[dt]);
          gkt[dt] = mfma32(qtl, lh, gkt[dt]);
        }
      }
    }
    if (wave < 2) {
      // dq^T = K^T dl^T + D^T g^T for dimensions 32 wave .. + 31, query columns
      dqa = zero16();
      for (int js = 0; js < Ckp / 16; ++js) {
        const bf16x8_t kth = lds_operand_tr(sKh, ST, 16 * js, 32 * wave, lane);
        const bf16x8_t ktl = lds_operand_tr(sKl, ST, 16 * js, 32 * wave, lane);
        const bf16x8_t lth = lds_operand_tr(sLh, PT, 16 * js, 0, lane);
        const bf16x8_t ltl = lds_operand_tr(sLl, PT, 16 * js, 0, lane);
        dqa = mfma32(kth, lth, dqa);
        dqa = mfma32(kth, ltl, dqa);
        dqa = mfma32(ktl, lth, dqa);
      }
      if (dip) {
#pragma unroll
        for (int vs = 0; vs < NKS; ++vs) {
          const bf16x8_t dth = lds_operand_tr(sDh, ST, 16 * vs, 32 * wave, lane);
          const bf16x8_t dtl = lds_operand_tr(sDl, ST, 16 * vs, 32 * wave, lane);
          const int og = c * ST + 16 * vs + 8 * h;
          const bf16x8_t gh = *reinterpret_cast<const bf16x8_t*>(&sGh[og]);
          dqa = mfma32(dth, gh, dqa);
          dqa = mfma32(dtl, gh, dqa);
          if (GF) dqa = mfma32(dth, *reinterpret_cast<const bf16x8_t*>(&sGl[og]), dqa);
        }
      }
      const int n = sRow[c];
      if (n >= 0) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d0 = 32 * wave + 8 * g4 + 4 * h;
          const f32x4_t x = {s * dqa[4 * g4], s * dqa[4 * g4 + 1], s * dqa[4 * g4 + 2], s * dqa[4 * g4 + 3]};
          *reinterpret_cast<f32x4_t*>(dq + static_cast<size_t>(n) * D + d0) = x;
#pragma unroll
          for (int u = 0; u < 4; ++u) qbs[4 * g4 + u] -= x[u];
        }
      }
    } else if (dip) {
      // dL/dD_i (rows v, columns d) += g^T qt: tiles (vt, dt) = (wave - 2, 0 and 1)
      const int vt = wave - 2;
#pragma unroll
      for (int ks = 0; ks < QT / 16; ++ks) {
        const bf16x8_t gth = lds_operand_tr(sGh, ST, 16 * ks, 32 * vt, lane);
        const bf16x8_t gtl = GF ? lds_operand_tr(sGl, ST, 16 * ks, 32 * vt, lane) : gth;
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
          const bf16x8_t qh = lds_operand_tr(sQh, ST, 16 * ks, 32 * dt, lane);
          const bf16x8_t ql = lds_operand_tr(sQl, ST, 16 * ks, 32 * dt, lane);
          gdp[dt] = mfma32(gth, qh, gdp[dt]);
          gdp[dt] = mfma32(gth, ql, gdp[dt]);
          if (GF) gdp[dt] = mfma32(gtl, qh, gdp[dt]);
        }
      }
    }
    __syncthreads();  // the tile buffers are rewritten next
  }
  // summary gradients of this wave's clusters: lane column j = 32 wave + c, rows d
  const int j = 32 * wave + c;
  if (ownj && j < Ck) {
    const size_t o = (ti * Ck + j) * D;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * dt + 8 * g4 + 4 * h;
        *reinterpret_cast<f32x4_t*>(a.g_v + o + d0) =
            f32x4_t{gvt[dt][4 * g4], gvt[dt][4 * g4 + 1], gvt[dt][4 * g4 + 2], gvt[dt][4 * g4 + 3]};
        *reinterpret_cast<f32x4_t*>(a.g_k + o + d0) =
            f32x4_t{s * gkt[dt][4 * g4], s * gkt[dt][4 * g4 + 1], s * gkt[dt][4 * g4 + 2], s * gkt[dt][4 * g4 + 3]};
      }
  }
  if (wave >= 2) {
    const int vt = wave - 2;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        // element v: row v_idx = 32 vt + 8 (v / 4) + 4 h + v % 4, column d = 32 dt + c
        const int vi = 32 * vt + 8 * (v >> 2) + 4 * h + (v & 3);
        a.g_dip[ti * D * D + static_cast<size_t>(vi) * D + 32 * dt + c] = dip ? s * gdp[dt][v] : 0.f;
      }
  }
  // dL/dlog Z (sum over the queries: lanes c) and the stage-2 part of dL/dqbar (waves 0, 1:
  // sum over the query columns), through LDS in a fixed order
  float* red = reinterpret_cast<float*>(sPh);  // free now: [Ckp][33] then [D][33]
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int r = 32 * wave + 8 * (v >> 2) + 4 * h + (v & 3);
    if (ownj) red[r * 33 + c] = glz[v];
  }
  float* red2 = red + Ckp * 33;
  if (wave < 2)
#pragma unroll
    for (int v = 0; v < 16; ++v) red2[(32 * wave + 8 * (v >> 2) + 4 * h + (v & 3)) * 33 + c] = qbs[v];
  __syncthreads();
  if (tid < Ck) {
    float x = 0.f;
    for (int q = 0; q < 32; ++q) x += red[tid * 33 + q];
    a.g_logz[ti * Ck + tid] = x;
  }
  if (tid < D) {
    float x = 0.f;
    for (int q = 0; q < 32; ++q) x += red2[tid * 33 + q];
    a.dqbar2[ti * D + tid] = x;
  }
}

// Per query cluster i: P_i., log sum_j Z_ij, the bf16 hi/lo copies of G_Dip_i (tilted,
// acausal), and for every key cluster j: dK'_ij, dV'_ij and V_ij^T G_Dip_i K_ij. Two
// clusters at a time (threads 0-127: j, 128-255: j + 1; of each half, 64 threads per
// output dimension). Causal calls: one workgroup per (table entry, query cluster); an
// entry whose row has no keys (entry 0) gets P = 0 and log sum = -inf.
__global__ void __launch_bounds__(256) bw_prep_i_kernel(BwArgs a) {
  constexpr int D = kBwD, DP = D + 1;
  __shared__ float sGd[D * DP];
  __shared__ float sP[kMaxClusters];
  __shared__ float sKr[2][D], sVr[2][D], sY[2][D];
  const int bh = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int Cq = a.Cq, Ck = a.Ck;
  const size_t ti = static_cast<size_t>(bh) * (a.causal ? a.nb : 1) * Cq + blockIdx.x;
  const bool tilted = a.dipole == 1;
  if (wave == 0) {
    float l[2], mx = kNegInf;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int j = lane + 64 * t;
      l[t] = j < Ck ? a.logz[ti * Ck + j] : kNegInf;
      mx = fmaxf(mx, l[t]);
    }
    mx = wave_max(mx);
    float e2[2], z = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      e2[t] = l[t] == kNegInf ? 0.f : __expf(l[t] - mx);
      z += e2[t];
    }
    z = wave_sum(z);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int j = lane + 64 * t;
      if (j < Ck) {
        const float pj = z > 0.f ? e2[t] / z : 0.f;
        sP[j] = pj;
        a.P[ti * Ck + j] = pj;
      }
    }
    if (lane == 0) a.lz[ti] = z > 0.f ? mx + __logf(z) : kNegInf;
  }
  if (tilted)
    for (int e = tid; e < D * D; e += 256) sGd[(e / D) * DP + e % D] = a.g_dip[ti * D * D + e];
  __syncthreads();
  if (tilted && !a.causal) {
    uint16_t* gd = a.gd + ti * 4 * D * D;
    for (int e = tid; e < D * D; e += 256) {
      const int r = e / D, c = e % D;
      const float x = sGd[r * DP + c];   // G_Dip[v = r][d = c]
      const float y = sGd[c * DP + r];   // transpose: row d = r, column v = c
      const uint16_t xh = f32_to_bf16_bits(x), yh = f32_to_bf16_bits(y);
      gd[e] = xh;
      gd[D * D + e] = f32_to_bf16_bits(x - bf16_to_f32(xh));
      gd[2 * D * D + e] = yh;
      gd[3 * D * D + e] = f32_to_bf16_bits(y - bf16_to_f32(yh));
    }
  }
  const int half = tid >> 7, t = tid & 127;
  for (int j0 = 0; j0 < Ck; j0 += 2) {
    const int j = j0 + half;
    const bool ok = j < Ck;
    const size_t tj = (ti * Ck + (ok ? j : 0)) * D;
    __syncthreads();  // the previous pair's rows are consumed
    if (t < D) {
      sKr[half][t] = ok ? a.tk[tj + t] : 0.f;
      sVr[half][t] = ok ? a.tv[tj + t] : 0.f;
    }
    __syncthreads();
    if (ok) {
      const float pj = sP[j];
      if (t < D) {  // dK'[d] = dL/dK[d] - P sum_v G_Dip[v][d] V[v]
        float x = 0.f;
        if (tilted)
          for (int vv = 0; vv < D; ++vv) x = fmaf(sGd[vv * DP + t], sVr[half][vv], x);
        a.dKp[tj + t] = a.g_k[tj + t] - pj * x;
      } else {      // y[v] = sum_d G_Dip[v][d] K[d];  dV'[v] = dL/dV[v] - P y[v]
        const int vv = t - D;
        float y = 0.f;
        if (tilted)
          for (int d = 0; d < D; ++d) y = fmaf(sGd[vv * DP + d], sKr[half][d], y);
        a.dVp[tj + vv] = a.g_v[tj + vv] - pj * y;
        sY[half][vv] = y;
      }
    }
    __syncthreads();
    if (tilted && ok && t < D) {  // one whole wave (0 or 2) per half
      const float z = wave_sum(sVr[half][t] * sY[half][t]);
      if (t == 0) a.vgk[ti * Ck + j] = z;
    }
  }
}

// Untilted dipole, per key cluster j: dL/dP_ij = <G_Dip_i, Cov_j> for every i, the matrix
// sum_i P_ij G_Dip_i and the cluster's key and value means.
template <typename T>
__global__ void __launch_bounds__(256) bw_prep_j_kernel(BwArgs a) {
  constexpr int D = kBwD, EPT = D * D / 256;
  __shared__ float sRed[4];
  const int j = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int Cq = a.Cq, Ck = a.Ck, N = a.N;
  const size_t tj = static_cast<size_t>(bh) * Ck + j;
  float cv[EPT], dc[EPT];
#pragma unroll
  for (int r = 0; r < EPT; ++r) {
    cv[r] = a.cov[tj * D * D + tid + 256 * r];
    dc[r] = 0.f;
  }
  for (int i = 0; i < Cq; ++i) {
    const size_t ti = static_cast<size_t>(bh) * Cq + i;
    const float p = a.P[ti * Ck + j];
    float part = 0.f;
#pragma unroll
    for (int r = 0; r < EPT; ++r) {
      const float g = a.g_dip[ti * D * D + tid + 256 * r];
      dc[r] = fmaf(p, g, dc[r]);
      part = fmaf(g, cv[r], part);
    }
    part = wave_sum(part);
    __syncthreads();  // the previous value was read
    if (lane == 0) sRed[wave] = part;
    __syncthreads();
    if (tid == 0) a.dP[ti * Ck + j] = (sRed[0] + sRed[1]) + (sRed[2] + sRed[3]);
  }
#pragma unroll
  for (int r = 0; r < EPT; ++r) a.dcov[tj * D * D + tid + 256 * r] = dc[r];
  const int32_t* offk = a.offs_k + static_cast<size_t>(bh) * (Ck + 1);
  const int m0 = offk[j];
  const int m1 = a.klen != nullptr ? m0 + a.klen[tj] : offk[j + 1];  // the kept prefix under a cap
  if (tid < 2 * D) {
    const T* X = static_cast<const T*>(tid < D ? a.k : a.v) + static_cast<size_t>(bh) * N * D;
    const int d = tid % D;
    const int32_t* perm = a.perm_k + static_cast<size_t>(bh) * N;
    float sum = 0.f;
    for (int pp = m0; pp < m1; ++pp) sum += Elem<T>::load(X, static_cast<size_t>(perm[pp]) * D + d);
    const float mean = m1 > m0 ? sum / static_cast<float>(m1 - m0) : 0.f;
    (tid < D ? a.kmean : a.vmean)[tj * D + d] = mean;
  }
}

// Causal calls: backward of the log-sum-exp merge of the exact in-block part (o_loc,
// L_loc) and the far field (o_far, L_far):  o = e^(L_far - L) o_far + e^(L_loc - L) o_loc
// with L = log(e^L_far + e^L_loc). With g = dL/do and the weights af, al:
//   dL/do_far = af g,  dL/dL_far = af g . (o_far - o),  dL/do_loc = al g,
// and for the in-block backward delta = dL/do_loc . o_loc - dL/dL_loc = al g . o.
// One wave per query row; the far-field arrays and o_loc are overwritten in place.
template <typename T>
__global__ void __launch_bounds__(256) bw_merge_kernel(BwArgs a) {
  constexpr int D = kBwD;
  const size_t row = static_cast<size_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= static_cast<size_t>(a.BH) * a.N) return;
  const float lf = a.l_far[row], ll = a.l_loc[row];
  float af = 0.f, al = 1.f;
  if (lf != kNegInf) {
    const float L = fmaxf(lf, ll) + __logf(1.f + __expf(-fabsf(lf - ll)));
    af = __expf(lf - L);
    al = __expf(ll - L);
  }
  const float g = Elem<T>::load(static_cast<const T*>(a.dout), row * D + lane);
  const float of = a.o_far[row * D + lane], ol = a.o_loc[row * D + lane];
  const float o = af * of + al * ol;
  const float go = wave_sum(g * o), gf = wave_sum(g * of);
  a.o_far[row * D + lane] = af * g;
  a.o_loc[row * D + lane] = al * g;
  if (lane == 0) {
    a.l_far[row] = af * (gf - go);
    a.delta_loc[row] = al * go;
  }
}

// Causal calls, per (table entry b, query cluster i): with the dipole differentiated
// through D_i = E_i - sum_j P_ij V_ij K_ij^T, E_i = sum_m p_im v_m k_m^T (p_im = w_im
// P_ij = exp(a_im - lz_i)), which equals the per-cluster form sum_j P_ij C_ij, the total
//   dL/dlog Z_ij - S_ij = G_logZ_ij - P_ij (V_ij^T G K_ij + <G, D_i>) - (dK'.K + dV'.V)
// (S_ij = sum_{m in j} w dL/dw over the K and V paths; the E path's per-key term is
// p_im v_m^T G k_m). Written to dlogz.
__global__ void __launch_bounds__(256) bw_entry_kernel(BwArgs a) {
  constexpr int D = kBwD;
  __shared__ float sRed[4];
  const int bh = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int Cq = a.Cq, Ck = a.Ck;
  const size_t ti = static_cast<size_t>(bh) * a.nb * Cq + blockIdx.x;
  const bool tilted = a.dipole == 1;
  float ge = 0.f;
  if (tilted) {
    float x = 0.f;
    for (int e = tid; e < D * D; e += 256) x = fmaf(a.g_dip[ti * D * D + e], a.dip[ti * D * D + e], x);
    x = wave_sum(x);
    if (lane == 0) sRed[wave] = x;
    __syncthreads();
    ge = (sRed[0] + sRed[1]) + (sRed[2] + sRed[3]);
  }
  for (int j = wave; j < Ck; j += 4) {
    const size_t tj = (ti * Ck + j) * D;
    float x = 0.f;
    if (a.logz[ti * Ck + j] != kNegInf) {
      x = a.g_logz[ti * Ck + j] - wave_sum(fmaf(a.dKp[tj + lane], a.tk[tj + lane], a.dVp[tj + lane] * a.tv[tj + lane]));
      if (tilted) x -= a.P[ti * Ck + j] * (a.vgk[ti * Ck + j] + ge);
    }
    if (lane == 0) a.dlogz[ti * Ck + j] = x;
  }
}

// Causal calls: a key m of block b' enters table entries b' + 1 .. nb - 1, with weights
// w^b_im = exp(a_im - log Z^b_ij) = w^{b'+1}_im exp(log Z^{b'+1}_ij - log Z^b_ij) and
// p^b_im = p^{b'+1}_im exp(lz^{b'+1}_i - lz^b_i); both factors are at most 1 (the sums
// only grow with b). So its gradient needs, per (b', i, j), the suffix sums
//   sdk = sum_{b > b'} exp(log Z^{b'+1} - log Z^b) dK'^b  (and sdv, st of dL/dlog Z - S)
// and per (b', i) sh = sum_{b > b'} exp(lz^{b'+1} - lz^b) G_Dip^b, each by one backward
// recurrence X^{b'} = Y^{b'+1} + r X^{b'+1} over the blocks (zero at b' = nb - 1).
// Part one: 64 threads (one per dimension) per (i, j) pair, four pairs per workgroup.
__global__ void __launch_bounds__(256) bw_suffix_kernel(BwArgs a) {
  constexpr int D = kBwD;
  const int bh = blockIdx.y, tid = threadIdx.x, d = tid & 63;
  const int Cq = a.Cq, Ck = a.Ck, nb = a.nb;
  const int ij = blockIdx.x * 4 + (tid >> 6);
  if (ij >= Cq * Ck) return;
  const size_t CC = static_cast<size_t>(Cq) * Ck;
  const size_t e0 = static_cast<size_t>(bh) * nb * CC + ij;  // (entry 0, i, j)
  float xk = 0.f, xv = 0.f, xt = 0.f;
  a.sdk[(e0 + (nb - 1) * CC) * D + d] = 0.f;
  a.sdv[(e0 + (nb - 1) * CC) * D + d] = 0.f;
  if (d == 0) a.st[e0 + (nb - 1) * CC] = 0.f;
  for (int bp = nb - 2; bp >= 0; --bp) {
    const size_t e1 = e0 + (bp + 1) * CC;
    const float l1 = a.logz[e1];
    const float l2 = bp + 2 < nb ? a.logz[e1 + CC] : kNegInf;
    const float r = (l1 == kNegInf || l2 == kNegInf) ? 0.f : __expf(l1 - l2);
    xk = fmaf(r, xk, a.dKp[e1 * D + d]);
    xv = fmaf(r, xv, a.dVp[e1 * D + d]);
    xt = fmaf(r, xt, a.dlogz[e1]);
    a.sdk[(e0 + bp * CC) * D + d] = xk;
    a.sdv[(e0 + bp * CC) * D + d] = xv;
    if (d == 0) a.st[e0 + bp * CC] = xt;
  }
}

// Part two (tilted): per (i, head), sh for every b', written as the bf16 hi + lo copies the
// per-key matrix-core pass reads (rows v, then the transpose with rows d).
__global__ void __launch_bounds__(256) bw_suffix_dip_kernel(BwArgs a) {
  constexpr int D = kBwD, DP = D + 1, EPT = D * D / 256;
  __shared__ float sX[D * DP];
  const int i = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int Cq = a.Cq, nb = a.nb;
  float x[EPT];
#pragma unroll
  for (int r = 0; r < EPT; ++r) x[r] = 0.f;
  for (int bp = nb - 1; bp >= 0; --bp) {
    if (bp + 1 < nb) {
      const size_t e1 = (static_cast<size_t>(bh) * nb + bp + 1) * Cq + i;
      const float l1 = a.lz[e1];
      const float l2 = bp + 2 < nb ? a.lz[e1 + Cq] : kNegInf;
      const float r = (l1 == kNegInf || l2 == kNegInf) ? 0.f : __expf(l1 - l2);
#pragma unroll
      for (int q = 0; q < EPT; ++q) x[q] = fmaf(r, x[q], a.g_dip[e1 * D * D + tid + 256 * q]);
    }
    __syncthreads();  // the previous entry's transpose reads are done
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
      const int e = tid + 256 * q;
      sX[(e / D) * DP + e % D] = x[q];
    }
    __syncthreads();
    uint16_t* gd = a.gd + ((static_cast<size_t>(bh) * nb + bp) * Cq + i) * 4 * D * D;
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
      const int e = tid + 256 * q, r = e / D, c = e % D;
      const float y = sX[c * DP + r];  // transpose: row d = r, column v = c
      const uint16_t xh = f32_to_bf16_bits(x[q]), yh = f32_to_bf16_bits(y);
      gd[e] = xh;
      gd[D * D + e] = f32_to_bf16_bits(x[q] - bf16_to_f32(xh));
      gd[2 * D * D + e] = yh;
      gd[3 * D * D + e] = f32_to_bf16_bits(y - bf16_to_f32(yh));
    }
  }
}

// a_im = s qbar_i . k_m at every key position (bucket order): four threads per key
// (16 dimensions each, summed over the quad).
template <typename T>
__global__ void __launch_bounds__(256) bw_scores_kernel(BwArgs a) {
  constexpr int D = kBwD, KT = kBwKeyTile, DQ = D / 4;
  __shared__ float sQb[kMaxClusters * D];
  const int bh = blockIdx.y, tid = threadIdx.x, kk = tid >> 2, d0 = (tid & 3) * DQ;
  const int N = a.N, Cq = a.Cq;
  for (int e0 = tid; e0 < Cq * D; e0 += 256 * 8) {  // eight loads in flight per thread
    float qv[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) qv[q] = a.qbar[static_cast<size_t>(bh) * Cq * D + min(e0 + 256 * q, Cq * D - 1)];
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (e0 + 256 * q < Cq * D) sQb[e0 + 256 * q] = qv[q];
  }
  const int pos = blockIdx.x * KT + kk;
  const bool valid = pos < N;
  const int key = valid ? a.perm_k[static_cast<size_t>(bh) * N + pos] : 0;
  const T* K = static_cast<const T*>(a.k) + static_cast<size_t>(bh) * N * D;
  float kf[DQ];
#pragma unroll
  for (int e = 0; e < DQ; ++e) kf[e] = Elem<T>::load(K, static_cast<size_t>(key) * D + d0 + e);  // key 0 if invalid
#pragma unroll
  for (int e = 0; e < DQ; ++e) kf[e] = valid ? kf[e] : 0.f;
  __syncthreads();
  float* A = a.A + static_cast<size_t>(bh) * Cq * N;
  for (int i = 0; i < Cq; ++i) {
    float x = 0.f;
#pragma unroll
    for (int e = 0; e < DQ; ++e) x = fmaf(sQb[i * D + d0 + e], kf[e], x);
    x += dpp_f32<0xB1>(x);  // lane ^ 1
    x += dpp_f32<0x4E>(x);  // lane ^ 2
    if (valid && (tid & 3) == 0) A[static_cast<size_t>(i) * N + pos] = a.scale * x;
  }
}

// Tilted dipole, 128 keys per workgroup (a wave per 32 consecutive key positions), query
// clusters in order with G_Dip_i (bf16 hi + lo, both layouts) staged in LDS, double
// buffered: on the matrix cores u^T = G_Dip_i K^T (rows v, column = key) and
// t^T = G_Dip_i^T V^T (rows d); then Q_im = v_m . u_m, and the accumulators
// dv_m += p_im u_m, dk_m += p_im t_m, written as the dipole terms of dk and dv.
// Causal calls: the workgroups tile each key block separately (positions in bucket order
// are grouped by block), and a key of block b' takes the suffix sum sh of block b' in
// place of G_Dip_i and p^{b'+1}_im as its weight; keys of the last block enter no table.
// NW waves per workgroup (32 keys each): 8 when the key blocks are multiples of 256 keys,
// so that every staged G tile serves 256 keys.
template <typename T, int NW>
__global__ void __launch_bounds__(64 * NW) bw_keys_a_kernel(BwArgs a) {
  constexpr int D = kBwD, GST = kBwGST, NKS = D / 16, NMT = D / 32, NT = 64 * NW, KPW = 32 * NW;
  constexpr int NPF = 4 * D * D / 8 / NT;  // 16-byte pieces of the four tiles per thread
  constexpr bool F32 = sizeof(T) == 4;
  __shared__ __align__(16) uint16_t sGd[2][4 * D * GST];
  const int bh = blockIdx.y, tid = threadIdx.x, lane = tid & 63, h = lane >> 5, c = lane & 31;
  const int wave = tid >> 6;
  const int N = a.N, Cq = a.Cq, Ck = a.Ck;
  const int blk = a.causal ? a.block : N, tpb = (blk + KPW - 1) / KPW;
  const int bp = blockIdx.x / tpb;           // key block (0 when acausal)
  const int pend = min(N, (bp + 1) * blk);
  const int pos = bp * blk + (blockIdx.x % tpb) * KPW + wave * 32 + c;
  const bool valid = pos < pend;
  const bool last = a.causal && bp == a.nb - 1;  // uniform: no table entry after this block
  const int nbW = a.causal ? a.nb : 1;
  const size_t ew = static_cast<size_t>(bh) * nbW + (a.causal ? bp + 1 : 0);  // weights' entry
  const size_t eg = static_cast<size_t>(bh) * nbW + (a.causal ? bp : 0);      // G tiles' entry
  const int key = valid ? a.perm_k[static_cast<size_t>(bh) * N + pos] : 0;
  const int j = valid ? min(max(a.labels_k[static_cast<size_t>(bh) * N + key], 0), Ck - 1) : 0;
  // a key left out by the cluster size cap is in no summary: weights zero
  const bool kept = valid && (a.kdrop == nullptr || a.kdrop[static_cast<size_t>(bh) * N + key] == 0);
  const T* K = static_cast<const T*>(a.k) + static_cast<size_t>(bh) * N * D;
  const T* V = static_cast<const T*>(a.v) + static_cast<size_t>(bh) * N * D;
  // B operands: key c, dimensions 16 ks + 8 h .. + 7 (bf16 hi, and lo for fp32 inputs)
  // (the row of key `key`, 0 for an invalid lane, is loaded unconditionally and zeroed
  // after: loads under the lane's validity are issued and waited for one at a time)
  bf16x8_t kh[NKS], kl[NKS], vh[NKS], vl[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    float x[8], y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const size_t o = static_cast<size_t>(key) * D + 16 * ks + 8 * h + e;
      x[e] = Elem<T>::load(K, o);
      y[e] = Elem<T>::load(V, o);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x[e] = valid ? x[e] : 0.f;
      y[e] = valid ? y[e] : 0.f;
    }
    split_bf16x8(x, kh[ks], kl[ks]);
    split_bf16x8(y, vh[ks], vl[ks]);
  }
  // v_m at the accumulator rows 32 mt + 8 g + 4 h + r
  float vq[NMT * 16];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
    for (int v = 0; v < 16; ++v)
      vq[16 * mt + v] = Elem<T>::load(V, static_cast<size_t>(key) * D + 32 * mt + 8 * (v >> 2) + 4 * h + (v & 3));
#pragma unroll
  for (int v = 0; v < NMT * 16; ++v) vq[v] = valid ? vq[v] : 0.f;
  u16x8_t pf[NPF];
  auto fetch = [&](int i) {
    const uint16_t* src = a.gd + (eg * Cq + i) * 4 * D * D;
#pragma unroll
    for (int q = 0; q < NPF; ++q) pf[q] = *reinterpret_cast<const u16x8_t*>(src + 8 * (tid + NT * q));
  };
  auto stage = [&](int buf) {
#pragma unroll
    for (int q = 0; q < NPF; ++q) {
      const int e = 8 * (tid + NT * q), arr = e / (D * D), rem = e % (D * D);
      *reinterpret_cast<u16x8_t*>(&sGd[buf][arr * D * GST + (rem / D) * GST + rem % D]) = pf[q];
    }
  };
  f32x16_t adk[NMT], adv[NMT];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) adk[mt] = adv[mt] = zero16();
  const int nci = last ? 0 : Cq;  // query clusters visited
  if (nci > 0) {
    fetch(0);
    stage(0);
  }
  __syncthreads();
  const float* Arow = a.A + static_cast<size_t>(bh) * Cq * N;
  // this key's score and the entry's log masses for cluster i, requested one cluster ahead
  auto fetch_s = [&](int i, float& av, float& lzij, float& lzi) {
    const size_t ti = ew * Cq + i;
    av = Arow[static_cast<size_t>(i) * N + min(pos, N - 1)];  // unconditional (zeroed below)
    av = valid ? av : 0.f;
    lzij = a.logz[ti * Ck + j];
    lzi = a.lz[ti];
  };
  float cav = 0.f, clzij = kNegInf, clzi = kNegInf, nav = 0.f, nlzij = kNegInf, nlzi = kNegInf;
  if (nci > 0) fetch_s(0, cav, clzij, clzi);
  for (int i = 0; i < nci; ++i) {
    const int buf = i & 1;
    if (i + 1 < Cq) fetch(i + 1);  // the next tiles travel during this cluster's products
    if (i + 1 < nci) fetch_s(i + 1, nav, nlzij, nlzi);
    const float av = cav, lzij = clzij, lzi = clzi;
    const float w = (kept && lzij != kNegInf) ? __expf(av - lzij) : 0.f;
    const float p = (kept && lzi != kNegInf) ? __expf(av - lzi) : 0.f;
    const uint16_t* g = sGd[buf];
    // u^T = G K^T, then t^T = G^T V^T, each folded into its accumulator before the next
    // (one 32-row tile pair of registers live at a time)
    float qp = 0.f;
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
      f32x16_t u = zero16();
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int o = (32 * mt + c) * GST + 16 * ks + 8 * h;
        const bf16x8_t gh = as_bf16x8(*reinterpret_cast<const u16x8_t*>(g + o));
        const bf16x8_t gl = as_bf16x8(*reinterpret_cast<const u16x8_t*>(g + D * GST + o));
        u = mfma32(gh, kh[ks], u);
        u = mfma32(gl, kh[ks], u);
        if (F32) u = mfma32(gh, kl[ks], u);
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        qp = fmaf(vq[16 * mt + v], u[v], qp);
        adv[mt][v] = fmaf(p, u[v], adv[mt][v]);
      }
    }
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
      f32x16_t t = zero16();
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int o = (32 * mt + c) * GST + 16 * ks + 8 * h;
        const bf16x8_t th = as_bf16x8(*reinterpret_cast<const u16x8_t*>(g + 2 * D * GST + o));
        const bf16x8_t tl = as_bf16x8(*reinterpret_cast<const u16x8_t*>(g + 3 * D * GST + o));
        t = mfma32(th, vh[ks], t);
        t = mfma32(tl, vh[ks], t);
        if (F32) t = mfma32(th, vl[ks], t);
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) adk[mt][v] = fmaf(p, t[v], adk[mt][v]);
    }
    const float qv = qp + xor32(qp);
    if (valid && h == 0) {
      const size_t o = (static_cast<size_t>(bh) * Cq + i) * N + pos;
      a.Q[o] = qv;
      if (!a.causal) a.WQ[o] = w * qv;
    }
    if (i + 1 < Cq) stage(buf ^ 1);
    cav = nav;
    clzij = nlzij;
    clzi = nlzi;
    __syncthreads();
  }
  if (last && valid && h == 0)
    for (int i = 0; i < Cq; ++i) a.Q[(static_cast<size_t>(bh) * Cq + i) * N + pos] = 0.f;
  if (valid) {
    float* dk = a.dk + (static_cast<size_t>(bh) * N + key) * D;
    float* dv = a.dv + (static_cast<size_t>(bh) * N + key) * D;
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * mt + 8 * g4 + 4 * h;
        *reinterpret_cast<f32x4_t*>(dk + d0) = f32x4_t{adk[mt][4 * g4], adk[mt][4 * g4 + 1], adk[mt][4 * g4 + 2], adk[mt][4 * g4 + 3]};
        *reinterpret_cast<f32x4_t*>(dv + d0) = f32x4_t{adv[mt][4 * g4], adv[mt][4 * g4 + 1], adv[mt][4 * g4 + 2], adv[mt][4 * g4 + 3]};
      }
  }
}

// Per query cluster i: dL/dP_ij (tilted: sum over the bucket of w Q, a wave per cluster in
// a fixed reduction order, minus V^T G_Dip K; untilted: from bw_prep_j), then
//   dL/dlog Z_ij = G_logZ_ij + P_ij (dL/dP_ij - sum_j' P_ij' dL/dP_ij'),
//   S_ij = sum_{m in j} w_im dL/dw_im = dK'.K + dV'.V (+ P (dL/dP + V^T G_Dip K), tilted),
// and the part  s sum_j (dL/dlog Z_ij - S_ij) K_ij  of dL/dqbar_i (sum_m w_im k_m = K_ij).
__global__ void __launch_bounds__(256) bw_dlogz_kernel(BwArgs a) {
  constexpr int D = kBwD;
  __shared__ float sdP[kMaxClusters], sdl[kMaxClusters], sS[kMaxClusters];
  const int i = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int Cq = a.Cq, Ck = a.Ck, N = a.N;
  const size_t ti = static_cast<size_t>(bh) * Cq + i;
  const bool tilted = a.dipole == 1;
  const int32_t* offk = a.offs_k + static_cast<size_t>(bh) * (Ck + 1);
  for (int j = wave; j < Ck; j += 4) {
    float x = 0.f;
    if (tilted) {
      const int m0 = offk[j], m1 = offk[j + 1];
      const float* wq = a.WQ + ti * N;
      for (int pp = m0 + lane; pp < m1; pp += 64) x += wq[pp];
      x = wave_sum(x) - a.vgk[ti * Ck + j];
    } else if (a.dipole == 2) {
      x = a.dP[ti * Ck + j];
    }
    if (lane == 0) sdP[j] = x;
  }
  __syncthreads();
  if (wave == 0) {
    float pd = 0.f;
    for (int j = lane; j < Ck; j += 64) pd = fmaf(a.P[ti * Ck + j], sdP[j], pd);
    pd = wave_sum(pd);
    for (int j = lane; j < Ck; j += 64) {
      const float x = a.g_logz[ti * Ck + j] + (a.logz[ti * Ck + j] == kNegInf ? 0.f : a.P[ti * Ck + j] * (sdP[j] - pd));
      sdl[j] = x;
      a.dlogz[ti * Ck + j] = x;
    }
  }
  for (int j = wave; j < Ck; j += 4) {
    const size_t tj = (ti * Ck + j) * D;
    float x = 0.f;
    if (a.logz[ti * Ck + j] != kNegInf) {
      x = wave_sum(fmaf(a.dKp[tj + lane], a.tk[tj + lane], a.dVp[tj + lane] * a.tv[tj + lane]));
      if (tilted) x += a.P[ti * Ck + j] * (sdP[j] + a.vgk[ti * Ck + j]);
    }
    if (lane == 0) {
      sS[j] = x;
      a.sij[ti * Ck + j] = x;
    }
  }
  __syncthreads();
  if (tid < D) {
    float acc = 0.f;
    for (int j = 0; j < Ck; ++j)
      if (a.logz[ti * Ck + j] != kNegInf) acc = fmaf(sdl[j] - sS[j], a.tk[(ti * Ck + j) * D + tid], acc);
    a.dqbar1[ti * D + tid] = a.scale * acc;
  }
}

// 64 keys per workgroup (four threads per key, 16 dimensions each): over the query
// clusters in order, dL/dw_im = dK'_ij . k_m + dV'_ij . v_m (+ P_ij Q_im, tilted),
// da_im = w_im (dL/dw_im - S_ij + dL/dlog Z_ij), and
//   dk_m += sum_i (w_im dK'_ij + s da_im qbar_i),  dv_m += sum_i w_im dV'_ij
// on top of the tilted dipole's terms (bw_keys_a) or, untilted, plus the covariance terms
// (sum_i P_ij G_Dip_i)^T (v_m - mean v) / n_j and (sum_i P_ij G_Dip_i)(k_m - mean k) / n_j.
// Then the tile's s sum_m w_im dL/dw_im k_m for every i (one partial per tile).
// Dynamic LDS (floats): qbar [Cq][D] | w dL/dw [Cq][KT + 1] | key rows [KT][D + 1] |
// value rows [KT][D + 1] (untilted only).
__host__ __device__ constexpr size_t bw_keys_b_lds(int Cq, int dipole) {
  return sizeof(float) * (static_cast<size_t>(Cq) * kBwD + static_cast<size_t>(Cq) * (kBwKeyTile + 1) +
                          (dipole == 2 ? 2 : 1) * static_cast<size_t>(kBwKeyTile) * (kBwD + 1));
}

// Causal calls (a tile lies in one key block b', the block being a multiple of the tile):
// with the suffix sums of block b' and the weights of entry b' + 1,
//   da_im = w (sdk . k_m + sdv . v_m + st) + p v_m^T sh k_m,
//   dk_m += sum_i (w sdk + s da_im qbar_i),  dv_m += sum_i w sdv,
// and the tile partial is s sum_m da_im k_m (all of dL/dqbar's stage-1 part).
template <typename T>
__global__ void __launch_bounds__(256) bw_keys_b_kernel(BwArgs a) {
  constexpr int D = kBwD, KT = kBwKeyTile, DQ = D / 4, RP = D + 1;
  extern __shared__ __align__(16) float dyn[];
  const int bh = blockIdx.y, tid = threadIdx.x, kk = tid >> 2, d0 = (tid & 3) * DQ;
  const int N = a.N, Cq = a.Cq, Ck = a.Ck;
  const int bp = a.causal ? (blockIdx.x * KT) / a.block : 0;  // key block of the tile
  const bool last = a.causal && bp == a.nb - 1;               // enters no table entry
  const size_t ew = static_cast<size_t>(bh) * (a.causal ? a.nb : 1) + (a.causal ? bp + 1 : 0);
  const size_t es = static_cast<size_t>(bh) * (a.causal ? a.nb : 1) + bp;  // suffix entry (causal)
  float* sQb = dyn;
  float* sWd = sQb + Cq * D;
  float* sKr = sWd + Cq * (KT + 1);
  float* sVr = sKr + KT * RP;  // untilted only
  const float s = a.scale;
  for (int e0 = tid; e0 < Cq * D; e0 += 256 * 8) {  // eight loads in flight per thread
    float qv[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) qv[q] = a.qbar[static_cast<size_t>(bh) * Cq * D + min(e0 + 256 * q, Cq * D - 1)];
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (e0 + 256 * q < Cq * D) sQb[e0 + 256 * q] = qv[q];
  }
  const int pos = blockIdx.x * KT + kk;
  const bool valid = pos < N;
  const int key = valid ? a.perm_k[static_cast<size_t>(bh) * N + pos] : 0;
  const int j = valid ? min(max(a.labels_k[static_cast<size_t>(bh) * N + key], 0), Ck - 1) : 0;
  // a key left out by the cluster size cap is in no summary: weights zero
  const bool kept = valid && (a.kdrop == nullptr || a.kdrop[static_cast<size_t>(bh) * N + key] == 0);
  const T* K = static_cast<const T*>(a.k) + static_cast<size_t>(bh) * N * D;
  const T* V = static_cast<const T*>(a.v) + static_cast<size_t>(bh) * N * D;
  float kf[DQ], vf[DQ], dk[DQ], dv[DQ];
  float* dkr = a.dk + (static_cast<size_t>(bh) * N + key) * D + d0;
  float* dvr = a.dv + (static_cast<size_t>(bh) * N + key) * D + d0;
  // the rows of key `key` (0 for an invalid lane) loaded unconditionally and zeroed after:
  // loads under the lane's validity are issued and waited for one at a time
#pragma unroll
  for (int e = 0; e < DQ; ++e) {
    kf[e] = Elem<T>::load(K, static_cast<size_t>(key) * D + d0 + e);
    vf[e] = Elem<T>::load(V, static_cast<size_t>(key) * D + d0 + e);
    dk[e] = dkr[e];
    dv[e] = dvr[e];
  }
#pragma unroll
  for (int e = 0; e < DQ; ++e) {
    kf[e] = valid ? kf[e] : 0.f;
    vf[e] = valid ? vf[e] : 0.f;
    sKr[kk * RP + d0 + e] = kf[e];
    if (a.dipole == 2) sVr[kk * RP + d0 + e] = vf[e];
    dk[e] = (a.dipole == 1 && valid) ? dk[e] : 0.f;
    dv[e] = (a.dipole == 1 && valid) ? dv[e] : 0.f;
  }
  __syncthreads();
  // the table rows of query cluster i + 1 are requested while cluster i is used (they do
  // not depend on the computation): one memory round trip per cluster is hidden
  struct Rows {
    float lzij, kpv[DQ], vpv[DQ], x0, x1, x2, x3;
  };
  auto fetch = [&](int i, Rows& r) {
    const size_t ti = ew * Cq + i;
    const size_t tij = ti * Ck + j;
    const size_t sij_ = (es * Cq + i) * Ck + j;  // suffix tables (causal)
    r.lzij = a.logz[tij];
    const float* kp = a.causal ? a.sdk + sij_ * D + d0 : a.dKp + tij * D + d0;
    const float* vp = a.causal ? a.sdv + sij_ * D + d0 : a.dVp + tij * D + d0;
#pragma unroll
    for (int e = 0; e < DQ; e += 4) {
      const f32x4_t k4 = *reinterpret_cast<const f32x4_t*>(kp + e);
      const f32x4_t v4 = *reinterpret_cast<const f32x4_t*>(vp + e);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        r.kpv[e + q] = k4[q];
        r.vpv[e + q] = v4[q];
      }
    }
    const float qi = a.dipole == 1 ? a.Q[(static_cast<size_t>(bh) * Cq + i) * N + pos] : 0.f;
    if (a.causal) {
      r.x0 = a.lz[ti];
      r.x1 = qi;
      r.x2 = a.st[sij_];
      r.x3 = 0.f;
    } else {
      r.x0 = a.dipole == 1 ? a.P[tij] : 0.f;
      r.x1 = qi;
      r.x2 = a.sij[tij];
      r.x3 = a.dlogz[tij];
    }
  };
  Rows cur, nxt;
  const int nci = last ? 0 : Cq;
  if (nci > 0) fetch(0, cur);
  for (int i = 0; i < nci; ++i) {
    if (i + 1 < nci) fetch(i + 1, nxt);
    float x = 0.f;
#pragma unroll
    for (int e = 0; e < DQ; ++e) x = fmaf(sQb[i * D + d0 + e], kf[e], x);
    x += dpp_f32<0xB1>(x);
    x += dpp_f32<0x4E>(x);
    const float av = s * x;
    const float lzij = cur.lzij;
    const float w = (kept && lzij != kNegInf) ? __expf(av - lzij) : 0.f;
    const float* kpv = cur.kpv;
    const float* vpv = cur.vpv;
    float y = 0.f;
#pragma unroll
    for (int e = 0; e < DQ; ++e) y = fmaf(kpv[e], kf[e], fmaf(vpv[e], vf[e], y));
    y += dpp_f32<0xB1>(y);
    y += dpp_f32<0x4E>(y);
    float da;
    if (a.causal) {
      const float lzi = cur.x0;
      const float p = (a.dipole == 1 && kept && lzi != kNegInf) ? __expf(av - lzi) : 0.f;
      da = fmaf(w, y + cur.x2, p * cur.x1);
    } else {
      if (a.dipole == 1 && kept) y += cur.x0 * cur.x1;
      da = w * (y - cur.x2 + cur.x3);
    }
#pragma unroll
    for (int e = 0; e < DQ; ++e) {
      dk[e] = fmaf(w, kpv[e], fmaf(s * da, sQb[i * D + d0 + e], dk[e]));
      dv[e] = fmaf(w, vpv[e], dv[e]);
    }
    if ((tid & 3) == 0) sWd[i * (KT + 1) + kk] = a.causal ? da : w * y;
    cur = nxt;
  }
  if (last)
    for (int e = tid; e < Cq * (KT + 1); e += 256) sWd[e] = 0.f;
  if (a.dipole == 2 && kept) {
    // covariance terms with the cluster's dL/dCov = sum_i P_ij G_Dip_i (over its kept keys)
    const size_t tj = static_cast<size_t>(bh) * Ck + j;
    const float* dc = a.dcov + tj * D * D;
    const float* km = a.kmean + tj * D;
    const float* vm = a.vmean + tj * D;
    const int32_t* offk = a.offs_k + static_cast<size_t>(bh) * (Ck + 1);
    const int nj = a.klen != nullptr ? a.klen[tj] : offk[j + 1] - offk[j];
    const float inv_n = 1.f / static_cast<float>(max(1, nj));
    for (int d = 0; d < D; ++d) {
      const float kc = sKr[kk * RP + d] - km[d];  // k_m - mean k, dimension d
      const float vc = sVr[kk * RP + d] - vm[d];  // v_m - mean v, dimension (value) d
#pragma unroll
      for (int e = 0; e < DQ; ++e) {
        dv[e] = fmaf(dc[static_cast<size_t>(d0 + e) * D + d] * inv_n, kc, dv[e]);  // row v = d0 + e
        dk[e] = fmaf(dc[static_cast<size_t>(d) * D + d0 + e] * inv_n, vc, dk[e]);  // row v = d, col d0 + e
      }
    }
  }
  if (valid) {
#pragma unroll
    for (int e = 0; e < DQ; ++e) {
      dkr[e] = dk[e];
      dvr[e] = dv[e];
    }
  }
  __syncthreads();
  // s sum over the tile's keys of w dL/dw k, for every (i, d)
  float* part = a.dqbar_part + (static_cast<size_t>(bh) * a.ntb + blockIdx.x) * Cq * D;
  for (int e = tid; e < Cq * D; e += 256) {
    const int i = e / D, d = e % D;
    float acc = 0.f;
    for (int q = 0; q < KT; ++q) acc = fmaf(sWd[i * (KT + 1) + q], sKr[q * RP + d], acc);
    part[e] = s * acc;
  }
}

// dL/dqbar_i = stage-2 part + s sum_j (dL/dlog Z_ij - S_ij) K_ij + the key tiles' partials
// (in tile order), then dq_n += dL/dqbar_i / n_i for every member n of cluster i.
__global__ void __launch_bounds__(256) bw_centroid_kernel(BwArgs a) {
  constexpr int D = kBwD;
  __shared__ float sRed[4][D];
  __shared__ float sTot[D];
  const int i = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x, d = tid & 63, g = tid >> 6;
  const int Cq = a.Cq, N = a.N;
  const size_t ti = static_cast<size_t>(bh) * Cq + i;
  // this thread's tiles g, g + 4, ... in order, eight loads in flight at a time
  float acc = 0.f;
  const float* src = a.dqbar_part + (static_cast<size_t>(bh) * a.ntb * Cq + i) * D + d;
  const size_t stride = static_cast<size_t>(Cq) * D;
  for (int t0 = g; t0 < a.ntb; t0 += 32) {
    float x[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) x[r] = t0 + 4 * r < a.ntb ? src[(t0 + 4 * r) * stride] : 0.f;
#pragma unroll
    for (int r = 0; r < 8; ++r) acc += x[r];
  }
  sRed[g][d] = acc;
  __syncthreads();
  // causal calls: the stage-2 parts of every table entry (in entry order); the stage-1
  // part is all in the key tiles' partials
  const int nbS = a.causal ? a.nb : 1;
  const int32_t* offq = a.offs_q + static_cast<size_t>(bh) * (nbS * Cq + 1);
  if (tid < D) {
    float x = a.causal ? 0.f : a.dqbar1[ti * D + tid];
    for (int b = 0; b < nbS; ++b) x += a.dqbar2[((static_cast<size_t>(bh) * nbS + b) * Cq + i) * D + tid];
    sTot[tid] = x + ((sRed[0][tid] + sRed[1][tid]) + (sRed[2][tid] + sRed[3][tid]));
  }
  __syncthreads();
  int n_i = 0;
  for (int b = 0; b < nbS; ++b) n_i += offq[b * Cq + i + 1] - offq[b * Cq + i];
  if (n_i == 0) return;
  const float inv = 1.f / static_cast<float>(n_i);
  const int32_t* perm = a.perm_q + static_cast<size_t>(bh) * N;
  float* dq = a.dq + static_cast<size_t>(bh) * N * D;
  for (int b = 0; b < nbS; ++b) {
    const int o0 = offq[b * Cq + i], o1 = offq[b * Cq + i + 1];
    // four rows per pass (a wave per row), four passes' loads in flight
    for (int r0 = 0; r0 < o1 - o0; r0 += 16) {
      float* row[4];
      float x[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = r0 + 4 * q + g;
        row[q] = r < o1 - o0 ? dq + static_cast<size_t>(perm[o0 + r]) * D + d : nullptr;
        x[q] = row[q] != nullptr ? *row[q] : 0.f;
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (row[q] != nullptr) *row[q] = x[q] + sTot[d] * inv;
    }
  }
}

// Causal calls: backward of the exact attention inside each block (queries n and keys
// m <= n of one block), P_nm = exp(s q_n . k_m - L_loc_n), with g_n = dL/do_loc:
//   dV_m = sum_n P_nm g_n,  dS_nm = P_nm (g_n . v_m - delta_n),
//   dK_m = s sum_n dS_nm q_n,  dQ_n = s sum_m dS_nm k_m,
// delta_n = g_n . o_loc_n - dL/dL_loc_n. fp32 arithmetic on 64 x 64 tiles staged in LDS
// (rows padded to 68 floats), each thread holding a 4 x 4 block of every product; the
// results are added to the far-field gradients already in dk, dv (bw_local_kv: one
// workgroup per key tile, over the query tiles of its block from the diagonal on) and
// dq (bw_local_q: one per query tile, over the key tiles up to the diagonal).
constexpr int kLocT = 64, kLocRS = kLocT + 4;

template <typename T>
__device__ __forceinline__ void loc_stage_rows(float* dst, const T* src, int row0, int tid) {
  constexpr int D = kBwD;
#pragma unroll
  for (int q = 0; q < kLocT * D / 256; ++q) {
    const int e = tid + 256 * q, r = e / D, d = e % D;
    dst[r * kLocRS + d] = Elem<T>::load(src, static_cast<size_t>(row0 + r) * D + d);
  }
}

// S = Q K^T and dP = G V^T for queries 4 ty + r and keys 4 tx + c of the staged tiles,
// then P and dS with the causal mask (key position <= query position).
__device__ __forceinline__ void loc_scores(const float* sQ, const float* sG, const float* sK, const float* sV,
                                           const float* sL, const float* sDel, int ty, int tx, int n0, int m0,
                                           float scale, float (&P)[4][4], float (&dS)[4][4]) {
  constexpr int D = kBwD;
  float sc[4][4], dp[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) sc[r][c] = dp[r][c] = 0.f;
  for (int d = 0; d < D; d += 4) {
    f32x4_t q4[4], g4[4], k4[4], v4[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      q4[r] = *reinterpret_cast<const f32x4_t*>(&sQ[(4 * ty + r) * kLocRS + d]);
      g4[r] = *reinterpret_cast<const f32x4_t*>(&sG[(4 * ty + r) * kLocRS + d]);
      k4[r] = *reinterpret_cast<const f32x4_t*>(&sK[(4 * tx + r) * kLocRS + d]);
      v4[r] = *reinterpret_cast<const f32x4_t*>(&sV[(4 * tx + r) * kLocRS + d]);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          sc[r][c] = fmaf(q4[r][u], k4[c][u], sc[r][c]);
          dp[r][c] = fmaf(g4[r][u], v4[c][u], dp[r][c]);
        }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int n = 4 * ty + r;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int m = 4 * tx + c;
      const float p = (m0 + m <= n0 + n) ? __expf(scale * sc[r][c] - sL[n]) : 0.f;
      P[r][c] = p;
      dS[r][c] = p * (dp[r][c] - sDel[n]);
    }
  }
}

template <typename T>
__global__ void __launch_bounds__(256) bw_local_kv_kernel(BwArgs a) {
  constexpr int D = kBwD, TT = kLocT, RS = kLocRS;
  __shared__ __align__(16) float sK[TT * RS], sV[TT * RS], sQ[TT * RS], sG[TT * RS], sP[TT * RS], sS[TT * RS];
  __shared__ float sL[TT], sDel[TT];
  const int bh = blockIdx.y, tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const int N = a.N, m0 = blockIdx.x * TT, bend = (m0 / a.block + 1) * a.block;
  const size_t base = static_cast<size_t>(bh) * N;
  const T* Q = static_cast<const T*>(a.q) + base * D;
  const T* K = static_cast<const T*>(a.k) + base * D;
  const T* V = static_cast<const T*>(a.v) + base * D;
  const float* G = a.o_loc + base * D;  // dL/do_loc
  loc_stage_rows<T>(sK, K, m0, tid);
  loc_stage_rows<T>(sV, V, m0, tid);
  float accV[4][4], accK[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) accV[r][c] = accK[r][c] = 0.f;
  for (int n0 = m0; n0 < bend; n0 += TT) {
    __syncthreads();  // the previous query tile is consumed
    loc_stage_rows<T>(sQ, Q, n0, tid);
    loc_stage_rows<float>(sG, G, n0, tid);
    if (tid < TT) {
      sL[tid] = a.l_loc[base + n0 + tid];
      sDel[tid] = a.delta_loc[base + n0 + tid];
    }
    __syncthreads();
    float P[4][4], dS[4][4];
    loc_scores(sQ, sG, sK, sV, sL, sDel, ty, tx, n0, m0, a.scale, P, dS);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      *reinterpret_cast<f32x4_t*>(&sP[(4 * ty + r) * RS + 4 * tx]) = f32x4_t{P[r][0], P[r][1], P[r][2], P[r][3]};
      *reinterpret_cast<f32x4_t*>(&sS[(4 * ty + r) * RS + 4 * tx]) = f32x4_t{dS[r][0], dS[r][1], dS[r][2], dS[r][3]};
    }
    __syncthreads();
    // keys 4 ty + r, dimensions 4 tx + c
    for (int n = 0; n < TT; ++n) {
      const f32x4_t p4 = *reinterpret_cast<const f32x4_t*>(&sP[n * RS + 4 * ty]);
      const f32x4_t s4 = *reinterpret_cast<const f32x4_t*>(&sS[n * RS + 4 * ty]);
      const f32x4_t g4 = *reinterpret_cast<const f32x4_t*>(&sG[n * RS + 4 * tx]);
      const f32x4_t q4 = *reinterpret_cast<const f32x4_t*>(&sQ[n * RS + 4 * tx]);
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          accV[r][c] = fmaf(p4[r], g4[c], accV[r][c]);
          accK[r][c] = fmaf(s4[r], q4[c], accK[r][c]);
        }
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const size_t o = (base + m0 + 4 * ty + r) * D + 4 * tx;
    f32x4_t dk4 = *reinterpret_cast<const f32x4_t*>(a.dk + o);
    f32x4_t dv4 = *reinterpret_cast<const f32x4_t*>(a.dv + o);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      dk4[c] = fmaf(a.scale, accK[r][c], dk4[c]);
      dv4[c] += accV[r][c];
    }
    *reinterpret_cast<f32x4_t*>(a.dk + o) = dk4;
    *reinterpret_cast<f32x4_t*>(a.dv + o) = dv4;
  }
}

template <typename T>
__global__ void __launch_bounds__(256) bw_local_q_kernel(BwArgs a) {
  constexpr int D = kBwD, TT = kLocT, RS = kLocRS;
  __shared__ __align__(16) float sK[TT * RS], sV[TT * RS], sQ[TT * RS], sG[TT * RS], sSt[TT * RS];
  __shared__ float sL[TT], sDel[TT];
  const int bh = blockIdx.y, tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const int N = a.N, n0 = blockIdx.x * TT, bbeg = (n0 / a.block) * a.block;
  const size_t base = static_cast<size_t>(bh) * N;
  const T* Q = static_cast<const T*>(a.q) + base * D;
  const T* K = static_cast<const T*>(a.k) + base * D;
  const T* V = static_cast<const T*>(a.v) + base * D;
  const float* G = a.o_loc + base * D;
  loc_stage_rows<T>(sQ, Q, n0, tid);
  loc_stage_rows<float>(sG, G, n0, tid);
  if (tid < TT) {
    sL[tid] = a.l_loc[base + n0 + tid];
    sDel[tid] = a.delta_loc[base + n0 + tid];
  }
  float acc[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[r][c] = 0.f;
  for (int m0 = bbeg; m0 <= n0; m0 += TT) {
    __syncthreads();  // the previous key tile is consumed
    loc_stage_rows<T>(sK, K, m0, tid);
    loc_stage_rows<T>(sV, V, m0, tid);
    __syncthreads();
    float P[4][4], dS[4][4];
    loc_scores(sQ, sG, sK, sV, sL, sDel, ty, tx, n0, m0, a.scale, P, dS);
    // dS transposed: row = key, column = query
#pragma unroll
    for (int c = 0; c < 4; ++c)
      *reinterpret_cast<f32x4_t*>(&sSt[(4 * tx + c) * RS + 4 * ty]) = f32x4_t{dS[0][c], dS[1][c], dS[2][c], dS[3][c]};
    __syncthreads();
    // queries 4 ty + r, dimensions 4 tx + c
    for (int m = 0; m < TT; ++m) {
      const f32x4_t s4 = *reinterpret_cast<const f32x4_t*>(&sSt[m * RS + 4 * ty]);
      const f32x4_t k4 = *reinterpret_cast<const f32x4_t*>(&sK[m * RS + 4 * tx]);
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[r][c] = fmaf(s4[r], k4[c], acc[r][c]);
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const size_t o = (base + n0 + 4 * ty + r) * D + 4 * tx;
    f32x4_t dq4 = *reinterpret_cast<const f32x4_t*>(a.dq + o);
#pragma unroll
    for (int c = 0; c < 4; ++c) dq4[c] = fmaf(a.scale, acc[r][c], dq4[c]);
    *reinterpret_cast<f32x4_t*>(a.dq + o) = dq4;
  }
}

// The same on the matrix cores (bf16 inputs): 32 x 32 x 16 bf16 products with fp32
// accumulation; the fp32 operands (dL/do_loc, P, dS) enter as bf16 hi + lo, so every
// product is fp32-accurate (hi hi + hi lo + lo hi where both operands are fp32). A
// workgroup of two waves takes 64 positions, a wave 32 of them.
// bw_local_kv_mfma: a wave's 32 keys m (K and V rows in registers) over the query tiles of
// the block from the diagonal on (Q rows, dL/do_loc as hi and lo, L_loc, delta staged in
// LDS). Per 32-query chunk: S = Q K^T and dP = G V^T with queries as rows (a lane holds
// its key's column), P and dS elementwise, then dV^T += G^T P and dK^T += Q^T dS with the
// accumulators as B operands and G^T, Q^T read by the LDS transpose read.
constexpr int kLocST = kBwD + 8;  // bf16 row stride of the staged tiles (16-byte aligned rows)

// NWK waves per workgroup (32 keys each; 4 when the block is a multiple of 128 keys), so
// that every staged query tile serves 32 NWK keys.
template <int NWK>
__global__ void __launch_bounds__(64 * NWK) bw_local_kv_mfma_kernel(BwArgs a) {
  constexpr int D = kBwD, ST = kLocST, NKS = D / 16, NMT = D / 32, TT = 64, NT = 64 * NWK;
  __shared__ __align__(16) uint16_t sQ[TT * ST], sGh[TT * ST], sGl[TT * ST];
  __shared__ float sL[TT], sDel[TT];
  const int bh = blockIdx.y, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, h = lane >> 5, c = lane & 31;
  const int N = a.N, m0 = blockIdx.x * 32 * NWK, bend = (m0 / a.block + 1) * a.block;
  const int mk = m0 + 32 * wave + c;  // this lane's key
  const size_t base = static_cast<size_t>(bh) * N;
  const uint16_t* Q = static_cast<const uint16_t*>(a.q) + base * D;
  const uint16_t* K = static_cast<const uint16_t*>(a.k) + base * D;
  const uint16_t* V = static_cast<const uint16_t*>(a.v) + base * D;
  const float* G = a.o_loc + base * D;  // dL/do_loc
  const float sl2 = a.scale * 1.4426950408889634f;
  bf16x8_t kb[NKS], vb[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    kb[ks] = as_bf16x8(*reinterpret_cast<const u16x8_t*>(K + static_cast<size_t>(mk) * D + 16 * ks + 8 * h));
    vb[ks] = as_bf16x8(*reinterpret_cast<const u16x8_t*>(V + static_cast<size_t>(mk) * D + 16 * ks + 8 * h));
  }
  f32x16_t dvt[NMT], dkt[NMT];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) dvt[mt] = dkt[mt] = zero16();
  for (int n0 = m0; n0 < bend; n0 += TT) {
    __syncthreads();  // the previous query tile is consumed
    // Q rows (bf16) and G rows (fp32 -> hi, lo): 16-byte pieces, 8 bf16 / 4 floats each
#pragma unroll
    for (int q = 0; q < TT * D / 8 / NT; ++q) {
      const int e = tid + NT * q, r = e / (D / 8), cc = e % (D / 8);
      *reinterpret_cast<u16x8_t*>(&sQ[r * ST + 8 * cc]) =
          *reinterpret_cast<const u16x8_t*>(Q + static_cast<size_t>(n0 + r) * D + 8 * cc);
    }
#pragma unroll
    for (int q = 0; q < TT * D / 4 / NT; ++q) {
      const int e = tid + NT * q, r = e / (D / 4), cc = e % (D / 4);
      const f32x4_t g4 = *reinterpret_cast<const f32x4_t*>(G + static_cast<size_t>(n0 + r) * D + 4 * cc);
      u16x4_t hi, lo;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        hi[u] = f32_to_bf16_bits(g4[u]);
        lo[u] = f32_to_bf16_bits(g4[u] - bf16_to_f32(hi[u]));
      }
      *reinterpret_cast<u16x4_t*>(&sGh[r * ST + 4 * cc]) = hi;
      *reinterpret_cast<u16x4_t*>(&sGl[r * ST + 4 * cc]) = lo;
    }
    if (tid < TT) {
      sL[tid] = a.l_loc[base + n0 + tid];
      sDel[tid] = a.delta_loc[base + n0 + tid];
    }
    __syncthreads();
#pragma unroll
    for (int qc = 0; qc < 2; ++qc) {
      if (n0 + 32 * qc + 31 < m0 + 32 * wave) continue;  // every query of the chunk precedes the wave's keys
      f32x16_t sc = zero16(), dp = zero16();
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int o = (32 * qc + c) * ST + 16 * ks + 8 * h;
        sc = mfma32(as_bf16x8(*reinterpret_cast<const u16x8_t*>(&sQ[o])), kb[ks], sc);
        dp = mfma32(as_bf16x8(*reinterpret_cast<const u16x8_t*>(&sGh[o])), vb[ks], dp);
        dp = mfma32(as_bf16x8(*reinterpret_cast<const u16x8_t*>(&sGl[o])), vb[ks], dp);
      }
      // P and dS: element v is query row 8 (v / 4) + 4 h + v % 4 of the chunk, key mk
      float pv[16], dsv[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = 32 * qc + 8 * (v >> 2) + 4 * h + (v & 3);
        const float p = (mk <= n0 + r) ? fast_exp2(fmaf(sc[v], sl2, -sL[r] * 1.4426950408889634f)) : 0.f;
        pv[v] = p;
        dsv[v] = p * (dp[v] - sDel[r]);
      }
#pragma unroll
      for (int ss = 0; ss < 2; ++ss) {
        bf16x8_t ph, pl, dh, dl;
        split_bf16x8(pv + 8 * ss, ph, pl);
        split_bf16x8(dsv + 8 * ss, dh, dl);
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) {
          const bf16x8_t gth = lds_operand_tr_acc(sGh, ST, 32 * qc + 16 * ss, 32 * mt, lane);
          const bf16x8_t gtl = lds_operand_tr_acc(sGl, ST, 32 * qc + 16 * ss, 32 * mt, lane);
          const bf16x8_t qt = lds_operand_tr_acc(sQ, ST, 32 * qc + 16 * ss, 32 * mt, lane);
          dvt[mt] = mfma32(gth, ph, dvt[mt]);
          dvt[mt] = mfma32(gth, pl, dvt[mt]);
          dvt[mt] = mfma32(gtl, ph, dvt[mt]);
          dkt[mt] = mfma32(qt, dh, dkt[mt]);
          dkt[mt] = mfma32(qt, dl, dkt[mt]);
        }
      }
    }
  }
  // dV^T and dK^T: this lane's key mk, dimensions 32 mt + 8 g + 4 h + 0..3
  float* dkr = a.dk + (base + mk) * D;
  float* dvr = a.dv + (base + mk) * D;
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = 32 * mt + 8 * g + 4 * h;
      f32x4_t k4 = *reinterpret_cast<const f32x4_t*>(dkr + d0);
      f32x4_t v4 = *reinterpret_cast<const f32x4_t*>(dvr + d0);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        k4[u] = fmaf(a.scale, dkt[mt][4 * g + u], k4[u]);
        v4[u] += dvt[mt][4 * g + u];
      }
      *reinterpret_cast<f32x4_t*>(dkr + d0) = k4;
      *reinterpret_cast<f32x4_t*>(dvr + d0) = v4;
    }
}

// bw_local_q_mfma: a wave's 32 queries n (Q rows and dL/do_loc as hi and lo in registers,
// L_loc and delta of the lane's query) over the key tiles of the block up to the diagonal
// (K and V rows staged in LDS). Per 32-key chunk: S^T = K Q^T and dP^T = V G^T with keys
// as rows (a lane holds its query's column), P^T and dS^T elementwise, then
// dQ^T += K^T dS^T with dS^T as the B operand and K^T read by the LDS transpose read.
__global__ void __launch_bounds__(128) bw_local_q_mfma_kernel(BwArgs a) {
  constexpr int D = kBwD, ST = kLocST, NKS = D / 16, NMT = D / 32, TT = 64;
  __shared__ __align__(16) uint16_t sK[TT * ST], sV[TT * ST];
  const int bh = blockIdx.y, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, h = lane >> 5, c = lane & 31;
  const int N = a.N, n0 = blockIdx.x * TT, bbeg = (n0 / a.block) * a.block;
  const int nq = n0 + 32 * wave + c;  // this lane's query
  const size_t base = static_cast<size_t>(bh) * N;
  const uint16_t* Q = static_cast<const uint16_t*>(a.q) + base * D;
  const uint16_t* K = static_cast<const uint16_t*>(a.k) + base * D;
  const uint16_t* V = static_cast<const uint16_t*>(a.v) + base * D;
  const float* G = a.o_loc + base * D;
  const float sl2 = a.scale * 1.4426950408889634f;
  bf16x8_t qb[NKS], gh[NKS], gl[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    qb[ks] = as_bf16x8(*reinterpret_cast<const u16x8_t*>(Q + static_cast<size_t>(nq) * D + 16 * ks + 8 * h));
    float g8[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) g8[u] = G[static_cast<size_t>(nq) * D + 16 * ks + 8 * h + u];
    split_bf16x8(g8, gh[ks], gl[ks]);
  }
  const float lq = a.l_loc[base + nq] * 1.4426950408889634f, dq_del = a.delta_loc[base + nq];
  f32x16_t acc[NMT];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) acc[mt] = zero16();
  for (int m0 = bbeg; m0 <= n0; m0 += TT) {
    __syncthreads();  // the previous key tile is consumed
#pragma unroll
    for (int q = 0; q < TT * D / 8 / 128; ++q) {
      const int e = tid + 128 * q, r = e / (D / 8), cc = e % (D / 8);
      *reinterpret_cast<u16x8_t*>(&sK[r * ST + 8 * cc]) =
          *reinterpret_cast<const u16x8_t*>(K + static_cast<size_t>(m0 + r) * D + 8 * cc);
      *reinterpret_cast<u16x8_t*>(&sV[r * ST + 8 * cc]) =
          *reinterpret_cast<const u16x8_t*>(V + static_cast<size_t>(m0 + r) * D + 8 * cc);
    }
    __syncthreads();
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      if (m0 + 32 * kc > n0 + 32 * wave + 31) continue;  // every key of the chunk follows the wave's queries
      f32x16_t st = zero16(), dpt = zero16();
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int o = (32 * kc + c) * ST + 16 * ks + 8 * h;
        const bf16x8_t kr = as_bf16x8(*reinterpret_cast<const u16x8_t*>(&sK[o]));
        const bf16x8_t vr = as_bf16x8(*reinterpret_cast<const u16x8_t*>(&sV[o]));
        st = mfma32(kr, qb[ks], st);
        dpt = mfma32(vr, gh[ks], dpt);
        dpt = mfma32(vr, gl[ks], dpt);
      }
      // P^T and dS^T: element v is key row 8 (v / 4) + 4 h + v % 4 of the chunk, query nq
      float dsv[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int mkey = m0 + 32 * kc + 8 * (v >> 2) + 4 * h + (v & 3);
        const float p = (mkey <= nq) ? fast_exp2(fmaf(st[v], sl2, -lq)) : 0.f;
        dsv[v] = p * (dpt[v] - dq_del);
      }
#pragma unroll
      for (int ss = 0; ss < 2; ++ss) {
        bf16x8_t dh, dl;
        split_bf16x8(dsv + 8 * ss, dh, dl);
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) {
          const bf16x8_t kt = lds_operand_tr_acc(sK, ST, 32 * kc + 16 * ss, 32 * mt, lane);
          acc[mt] = mfma32(kt, dh, acc[mt]);
          acc[mt] = mfma32(kt, dl, acc[mt]);
        }
      }
    }
  }
  float* dqr = a.dq + (base + nq) * D;
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = 32 * mt + 8 * g + 4 * h;
      f32x4_t q4 = *reinterpret_cast<const f32x4_t*>(dqr + d0);
#pragma unroll
      for (int u = 0; u < 4; ++u) q4[u] = fmaf(a.scale, acc[mt][4 * g + u], q4[u]);
      *reinterpret_cast<f32x4_t*>(dqr + d0) = q4;
    }
}

template <typename T>
static void launch_backward_t(const BwArgs& a, hipStream_t s) {
  const int nbS = a.causal ? a.nb : 1;
  const dim3 gi(a.Cq, a.BH), ge(nbS * a.Cq, a.BH), gk((a.N + kBwKeyTile - 1) / kBwKeyTile, a.BH);
  if (a.causal) {
    ProfScope ps_("bw_merge", s);
    hipLaunchKernelGGL((bw_merge_kernel<T>), dim3((a.BH * a.N + 3) / 4), dim3(256), 0, s, a);
  }
  if (sizeof(T) == 2) {
    const size_t lds = bw_refine_mfma_lds(a.Ck);
    ProfScope ps_("bw_refine_mfma", s);
    if (a.causal) {
      allow_lds((const void*)bw_refine_mfma_kernel<float>, lds);
      hipLaunchKernelGGL(bw_refine_mfma_kernel<float>, ge, dim3(256), lds, s, a);
    } else {
      allow_lds((const void*)bw_refine_mfma_kernel<bf16>, lds);
      hipLaunchKernelGGL(bw_refine_mfma_kernel<bf16>, ge, dim3(256), lds, s, a);
    }
  } else {
    ProfScope ps_("bw_refine", s);
    if (a.causal) hipLaunchKernelGGL((bw_refine_kernel<T, float>), ge, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((bw_refine_kernel<T, T>), ge, dim3(256), 0, s, a);
  }
  {
    ProfScope ps_("bw_prep_i", s);
    hipLaunchKernelGGL(bw_prep_i_kernel, ge, dim3(256), 0, s, a);
  }
  if (a.causal) {
    {
      ProfScope ps_("bw_entry", s);
      hipLaunchKernelGGL(bw_entry_kernel, ge, dim3(256), 0, s, a);
    }
    {
      ProfScope ps_("bw_suffix", s);
      hipLaunchKernelGGL(bw_suffix_kernel, dim3((a.Cq * a.Ck + 3) / 4, a.BH), dim3(256), 0, s, a);
    }
    if (a.dipole == 1) {
      ProfScope ps_("bw_suffix_dip", s);
      hipLaunchKernelGGL(bw_suffix_dip_kernel, gi, dim3(256), 0, s, a);
    }
  }
  if (a.dipole == 2) {
    ProfScope ps_("bw_prep_j", s);
    hipLaunchKernelGGL((bw_prep_j_kernel<T>), dim3(a.Ck, a.BH), dim3(256), 0, s, a);
  }
  if (a.dipole == 1) {
    {
      ProfScope ps_("bw_scores", s);
      hipLaunchKernelGGL((bw_scores_kernel<T>), gk, dim3(256), 0, s, a);
    }
    const int blk = a.causal ? a.block : a.N;
    ProfScope ps_("bw_keys_a", s);
    if (sizeof(T) == 2 && blk % 256 == 0)  // (fp32 inputs: their hi/lo operands need the registers of 4 waves)
      hipLaunchKernelGGL((bw_keys_a_kernel<T, 8>), dim3(nbS * (blk / 256), a.BH), dim3(512), 0, s, a);
    else
      hipLaunchKernelGGL((bw_keys_a_kernel<T, 4>), dim3(nbS * ((blk + 127) / 128), a.BH), dim3(256), 0, s, a);
  }
  if (!a.causal) {
    ProfScope ps_("bw_dlogz", s);
    hipLaunchKernelGGL(bw_dlogz_kernel, gi, dim3(256), 0, s, a);
  }
  {
    const size_t lds = bw_keys_b_lds(a.Cq, a.dipole);
    allow_lds((const void*)bw_keys_b_kernel<T>, lds);
    ProfScope ps_("bw_keys_b", s);
    hipLaunchKernelGGL((bw_keys_b_kernel<T>), gk, dim3(256), lds, s, a);
  }
  {
    ProfScope ps_("bw_centroid", s);
    hipLaunchKernelGGL(bw_centroid_kernel, gi, dim3(256), 0, s, a);
  }
  if (a.causal) {
    const dim3 gl(a.N / kLocT, a.BH);
    constexpr bool MF = sizeof(T) == 2;
    {
      ProfScope ps_(MF ? "bw_local_kv_mfma" : "bw_local_kv", s);
      if (MF && a.block % 128 == 0)
        hipLaunchKernelGGL(bw_local_kv_mfma_kernel<4>, dim3(a.N / 128, a.BH), dim3(256), 0, s, a);
      else if (MF)
        hipLaunchKernelGGL(bw_local_kv_mfma_kernel<2>, gl, dim3(128), 0, s, a);
      else hipLaunchKernelGGL((bw_local_kv_kernel<T>), gl, dim3(256), 0, s, a);
    }
    ProfScope ps_(MF ? "bw_local_q_mfma" : "bw_local_q", s);
    if (MF) hipLaunchKernelGGL(bw_local_q_mfma_kernel, gl, dim3(128), 0, s, a);
    else hipLaunchKernelGGL((bw_local_q_kernel<T>), gl, dim3(256), 0, s, a);
  }
}

hipError_t launch_backward(const BwArgs& a, int dtype, hipStream_t s) {
  if (dtype == 0) launch_backward_t<float>(a, s);
  else launch_backward_t<bf16>(a, s);
  return hipGetLastError();
}

}  // namespace muse
