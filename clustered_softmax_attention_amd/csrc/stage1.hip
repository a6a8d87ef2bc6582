// Stage 1 of MuSe: coarse query centroids attend to fine key clusters (gfx950).
//
// For query centroid qbar_i and the keys m of key cluster j (pith.science review of
// arXiv 2509.10406, "What carries the argument"; gist.science summary,
// Kernmechanismen 2, "Exponential Tilting"), with a_m = s qbar_i . k_m:
//   log Z_ij = logsumexp_m a_m,   K_ij = sum_m w_m k_m,   V_ij = sum_m w_m v_m,
//   w_m = exp(a_m) / Z_ij,  and the aggregated dipole
//   D_i = sum_j P_ij C_ij = E_i[v k^T] - sum_j P_ij V_ij K_ij^T,
// where P_ij = Z_ij / sum_j' Z_ij' and E_i is the expectation under the softmax of
// a_m over all keys (the two forms are equal because P_ij w_m = exp(a_m) / Z_i).
//
// Keys are processed per spatial block b' ("atoms" (i, j, b')): acausal calls have
// a single block. Causal calls accumulate the atoms of all preceding blocks
// (gist.science summary, Kernmechanismen 3) by a log-sum-exp fold over blocks.
//
// Kernels (all sums in a fixed order; no floating-point atomics):
//   s1_atoms      one workgroup per (j, b', head): online log-sum-exp over the
//                 bucket's keys for every centroid i.
//   s1_moments    one workgroup per (i, b', head): block-normalised sum w v k^T.
//   s1_prefix     fold of atoms over blocks -> log Z, K, V tables.
//   s1_mom_prefix fold of block moments over blocks -> E_i[v k^T] per table entry.
//                 Causal entry e covers blocks [0, e), or with the hierarchical
//                 decomposition the square's key blocks [e - lowbit(e), e) (pith.science
//                 review, Figure 2 caption: MuSe on the squares below the diagonal).
//   s1_dip_final  D_i = E_i[v k^T] - sum_j P_ij V_ij K_ij^T (value index first).
//   s1_cluster_cov, s1_untilted_dip  the untilted dipole (acausal): per key cluster
//                 covariance Cov_j, then D_i = sum_j P_ij Cov_j.
// The bf16 kernels (matrix cores) are in stage1_mfma.hip; this file launches them, the
// atoms on a second stream beside the scores and moments.
#include <mutex>

#include "mfma.hpp"
#include "muse_kernels.hpp"

namespace muse {

// keys staged in LDS per step (fewer for D = 128 to keep LDS under budget)
template <int D>
struct S1Keys {
  static constexpr int value = D == 64 ? 64 : 32;
};

// LDS: qb [Cq][D] | kc [64][D] | vc [64][D] | sa [Cq][64] | sm, sz, salpha [Cq]
template <typename T, int D>
__global__ void __launch_bounds__(256) s1_atoms_kernel(S1Args a) {
  constexpr int kS1Keys = S1Keys<D>::value;
  extern __shared__ __align__(16) float sh[];
  const int j = blockIdx.x, bp = blockIdx.y, bh = blockIdx.z;
  const int Cq = a.Cq, Ck = a.Ck, tid = threadIdx.x;
  float* qb = sh;
  float* kc = qb + Cq * D;
  float* vc = kc + kS1Keys * D;
  float* sa = vc + kS1Keys * D;
  float* sm = sa + Cq * kS1Keys;
  float* sz = sm + Cq;
  float* salpha = sz + Cq;

  const int32_t* offs = a.offs_k + static_cast<size_t>(bh) * (a.nb * Ck + 1);
  // the bucket's positions, or with a cluster size cap its kept prefix
  const int seg0 = offs[bp * Ck + j];
  const int seg1 = a.klen ? seg0 + a.klen[static_cast<size_t>(bh) * a.nb * Ck + bp * Ck + j] : offs[bp * Ck + j + 1];
  const int32_t* perm = a.perm_k + static_cast<size_t>(bh) * a.N;
  const T* K = static_cast<const T*>(a.k) + static_cast<size_t>(bh) * a.N * D;
  const T* V = static_cast<const T*>(a.v) + static_cast<size_t>(bh) * a.N * D;

  for (int e = tid; e < Cq * D; e += 256) qb[e] = a.qbar[static_cast<size_t>(bh) * Cq * D + e];
  for (int i = tid; i < Cq; i += 256) {
    sm[i] = kNegInf;
    sz[i] = 0.f;
  }
  constexpr int kMaxPairs = kMaxClusters * D / 256;
  const int npairs = (Cq * D + 255) / 256;
  float accK[kMaxPairs], accV[kMaxPairs];
#pragma unroll
  for (int r = 0; r < kMaxPairs; ++r) accK[r] = accV[r] = 0.f;

  for (int c0 = seg0; c0 < seg1; c0 += kS1Keys) {
    const int nk = min(kS1Keys, seg1 - c0);
    __syncthreads();
    for (int e = tid; e < nk * D; e += 256) {
      const int m = e / D, d = e % D;
      const size_t row = static_cast<size_t>(perm[c0 + m]) * D;
      kc[e] = Elem<T>::load(K, row + d);
      vc[e] = Elem<T>::load(V, row + d);
    }
    __syncthreads();
    for (int e = tid; e < Cq * kS1Keys; e += 256) {
      const int i = e / kS1Keys, m = e % kS1Keys;
      float dot = 0.f;
      if (m < nk) {
#pragma unroll 16
        for (int d = 0; d < D; ++d) dot = fmaf(qb[i * D + d], kc[m * D + d], dot);
      }
      sa[e] = m < nk ? a.scale * dot : kNegInf;
    }
    __syncthreads();
    for (int i = tid; i < Cq; i += 256) {
      float cmax = kNegInf;
      for (int m = 0; m < nk; ++m) cmax = fmaxf(cmax, sa[i * kS1Keys + m]);
      const float newm = fmaxf(sm[i], cmax);
      const float alpha = (sm[i] == kNegInf) ? 0.f : __expf(sm[i] - newm);
      float zc = 0.f;
      for (int m = 0; m < kS1Keys; ++m) {
        const float e = (m < nk) ? __expf(sa[i * kS1Keys + m] - newm) : 0.f;
        sa[i * kS1Keys + m] = e;
        zc += e;
      }
      sz[i] = sz[i] * alpha + zc;
      sm[i] = newm;
      salpha[i] = alpha;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kMaxPairs; ++r) {
      if (r >= npairs) break;
      const int p = tid + 256 * r;
      if (p >= Cq * D) break;
      const int i = p / D, d = p % D;
      float sk = 0.f, sv = 0.f;
      for (int m = 0; m < nk; ++m) {
        const float w = sa[i * kS1Keys + m];
        sk = fmaf(w, kc[m * D + d], sk);
        sv = fmaf(w, vc[m * D + d], sv);
      }
      accK[r] = accK[r] * salpha[i] + sk;
      accV[r] = accV[r] * salpha[i] + sv;
    }
  }
  __syncthreads();
  const size_t abase = (static_cast<size_t>(bh) * a.nb + bp) * Cq;  // [.., i, j]
  for (int i = tid; i < Cq; i += 256) {
    a.at_m[(abase + i) * Ck + j] = sm[i];
    a.at_z[(abase + i) * Ck + j] = sz[i];
  }
#pragma unroll
  for (int r = 0; r < kMaxPairs; ++r) {
    if (r >= npairs) break;
    const int p = tid + 256 * r;
    if (p >= Cq * D) break;
    const int i = p / D, d = p % D;
    a.at_k[((abase + i) * Ck + j) * D + d] = accK[r];
    a.at_v[((abase + i) * Ck + j) * D + d] = accV[r];
  }
}

// Block log-mass R_ib' = logsumexp_j (m_ij + log z_ij) and block-normalised moments
// sum_m exp(a_m - R) v_m k_m^T over the keys of block b'.
// Thread layout: 16x16 grid of threads, each owning a (D/16)x(D/16) tile of (dv, dk).
template <typename T, int D>
__global__ void __launch_bounds__(256) s1_moments_kernel(S1Args a) {
  constexpr int TD = D / 16;
  constexpr int kS1Keys = S1Keys<D>::value;
  extern __shared__ __align__(16) float sh[];
  const int i = blockIdx.x, bp = blockIdx.y, bh = blockIdx.z;
  const int Cq = a.Cq, Ck = a.Ck, tid = threadIdx.x;
  float* qb = sh;                  // [D]
  float* kc = qb + D;              // [64][D]
  float* vc = kc + kS1Keys * D;    // [64][D]
  float* w = vc + kS1Keys * D;     // [64]
  float* red = w + kS1Keys;        // [1]

  for (int d = tid; d < D; d += 256) qb[d] = a.qbar[(static_cast<size_t>(bh) * Cq + i) * D + d];
  const size_t abase = ((static_cast<size_t>(bh) * a.nb + bp) * Cq + i) * Ck;
  if (tid < 64) {
    float mx = kNegInf;
    for (int j = tid; j < Ck; j += 64) {
      const float z = a.at_z[abase + j];
      if (z > 0.f) mx = fmaxf(mx, a.at_m[abase + j] + __logf(z));
    }
    mx = wave_max(mx);
    float s = 0.f;
    for (int j = tid; j < Ck; j += 64) {
      const float z = a.at_z[abase + j];
      if (z > 0.f) s += __expf(a.at_m[abase + j] + __logf(z) - mx);
    }
    s = wave_sum(s);
    if (tid == 0) red[0] = (mx == kNegInf) ? kNegInf : mx + __logf(s);
  }
  __syncthreads();
  const float R = red[0];
  if (tid == 0) a.blk_lmass[(static_cast<size_t>(bh) * a.nmb + bp) * Cq + i] = R;

  const int tr = tid / 16, tc = tid % 16;  // rows dv = tr*TD.., cols dk = tc*TD..
  float acc[TD][TD];
#pragma unroll
  for (int x = 0; x < TD; ++x)
#pragma unroll
    for (int y = 0; y < TD; ++y) acc[x][y] = 0.f;

  const int key0 = a.causal ? bp * a.block : 0;
  const int key1 = a.causal ? key0 + a.block : a.N;
  const T* K = static_cast<const T*>(a.k) + static_cast<size_t>(bh) * a.N * D;
  const T* V = static_cast<const T*>(a.v) + static_cast<size_t>(bh) * a.N * D;
  if (R != kNegInf) {
    for (int c0 = key0; c0 < key1; c0 += kS1Keys) {
      const int nk = min(kS1Keys, key1 - c0);
      __syncthreads();
      for (int e = tid; e < nk * D; e += 256) {
        kc[e] = Elem<T>::load(K, static_cast<size_t>(c0) * D + e);
        vc[e] = Elem<T>::load(V, static_cast<size_t>(c0) * D + e);
      }
      __syncthreads();
      if (tid < kS1Keys) {
        float dot = 0.f;
        if (tid < nk) {
#pragma unroll 16
          for (int d = 0; d < D; ++d) dot = fmaf(qb[d], kc[tid * D + d], dot);
        }
        // keys left out by a cluster size cap weigh nothing
        const bool in = tid < nk && (a.kdrop == nullptr || a.kdrop[static_cast<size_t>(bh) * a.N + c0 + tid] == 0);
        w[tid] = in ? __expf(a.scale * dot - R) : 0.f;
      }
      __syncthreads();
      for (int m = 0; m < nk; ++m) {
        const float wm = w[m];
        float vr[TD], kr[TD];
#pragma unroll
        for (int x = 0; x < TD; ++x) vr[x] = wm * vc[m * D + tr * TD + x];
#pragma unroll
        for (int y = 0; y < TD; ++y) kr[y] = kc[m * D + tc * TD + y];
#pragma unroll
        for (int x = 0; x < TD; ++x)
#pragma unroll
          for (int y = 0; y < TD; ++y) acc[x][y] = fmaf(vr[x], kr[y], acc[x][y]);
      }
    }
  }
  float* out = a.blk_mom + ((static_cast<size_t>(bh) * a.nmb + bp) * Cq + i) * D * D;
#pragma unroll
  for (int x = 0; x < TD; ++x)
#pragma unroll
    for (int y = 0; y < TD; ++y) out[(tr * TD + x) * D + tc * TD + y] = acc[x][y];
}

// Acausal tables of the general path (a single key block, whose atoms are whole): per
// (query centroid i, head), for every key cluster j, log Z_ij = m + log z and the tilted
// means K_ij = (sum w k) / z, V_ij = (sum w v) / z (zero for an empty cluster).
__global__ void __launch_bounds__(256) s1_tables_acausal_kernel(S1Args a) {
  const int i = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int D = a.D, Cq = a.Cq, Ck = a.Ck;
  const size_t base = (static_cast<size_t>(bh) * Cq + i) * Ck;
  for (int j = tid; j < Ck; j += 256) {
    const float z = a.at_z[base + j];
    a.s_logz[base + j] = z > 0.f ? a.at_m[base + j] + __logf(z) : kNegInf;
  }
  for (int e = tid; e < Ck * D; e += 256) {
    const float z = a.at_z[base + e / D];
    const float inv = z > 0.f ? 1.f / z : 0.f;
    a.s_k[base * D + e] = a.at_k[base * D + e] * inv;
    a.s_v[base * D + e] = a.at_v[base * D + e] * inv;
  }
}

constexpr int kHierLevels = 12;  // binary-counter depth of the hierarchical folds (nb < 2^11)

// Fold atoms over blocks: one workgroup per (j, i, head), 2*D threads (K then V dims).
// HIER: causal entries of the hierarchical squares (an instance of its own, so that the
// batched prefix fold does not change its register allocation).
template <bool HIER>
__global__ void s1_prefix_kernel(S1Args a) {
  const int j = blockIdx.x, i = blockIdx.y, bh = blockIdx.z;
  const int D = a.D, Cq = a.Cq, Ck = a.Ck;
  const int t = threadIdx.x;
  const bool isK = t < D;
  const int d = isK ? t : t - D;
  float rm = kNegInf, rz = 0.f, racc = 0.f;
  auto emit = [&](int b) {
    const size_t sidx = ((static_cast<size_t>(bh) * a.nbS + b) * Cq + i) * Ck + j;
    const bool any = rz > 0.f;
    if (t == 0) a.s_logz[sidx] = any ? rm + __logf(rz) : kNegInf;
    float* dst = isK ? a.s_k : a.s_v;
    dst[sidx * D + d] = any ? racc / rz : 0.f;
  };
  // blocks [b0, b1) folded in order, their atoms requested eight at a time; with
  // prefix_emit, entry b is written before block b joins (entry b: blocks < b)
  auto fold = [&](int b0, int b1, bool prefix_emit) {
    for (int c0 = b0; c0 < b1; c0 += 8) {
      float m8[8], z8[8], x8[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        m8[q] = kNegInf;
        z8[q] = 0.f;
        x8[q] = 0.f;
        if (c0 + q < b1) {
          const size_t aidx = ((static_cast<size_t>(bh) * a.nb + c0 + q) * Cq + i) * Ck + j;
          m8[q] = a.at_m[aidx];
          z8[q] = a.at_z[aidx];
          x8[q] = (isK ? a.at_k : a.at_v)[aidx * D + d];
        }
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if (c0 + q >= b1) break;
        if (prefix_emit) emit(c0 + q);
        if (z8[q] > 0.f) {
          const float nm = fmaxf(rm, m8[q]);
          const float f0 = (rz > 0.f) ? __expf(rm - nm) : 0.f;
          const float f1 = __expf(m8[q] - nm);
          rz = rz * f0 + z8[q] * f1;
          racc = racc * f0 + x8[q] * f1;
          rm = nm;
        }
      }
    }
  };
  if (HIER && a.nb < (1 << (kHierLevels - 1))) {
    // entry e: the square's key blocks [e - lowbit(e), e), by a binary counter over the
    // blocks: block b is pushed as a node and merged with the ctz(b + 1) nodes on top of
    // the stack (each the fold of the blocks just before it), which leaves exactly entry
    // b + 1's square on top. Left (earlier) operands first; entry 0 stays empty.
    float sm[kHierLevels], sz[kHierLevels], sa[kHierLevels];
    int top = 0;
    emit(0);
    for (int c0 = 0; c0 < a.nb; c0 += 8) {
      float m8[8], z8[8], x8[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        m8[q] = kNegInf;
        z8[q] = 0.f;
        x8[q] = 0.f;
        if (c0 + q < a.nb) {
          const size_t aidx = ((static_cast<size_t>(bh) * a.nb + c0 + q) * Cq + i) * Ck + j;
          m8[q] = a.at_m[aidx];
          z8[q] = a.at_z[aidx];
          x8[q] = (isK ? a.at_k : a.at_v)[aidx * D + d];
        }
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int b = c0 + q;
        if (b >= a.nb) break;
        const bool has = z8[q] > 0.f;
        float cm = has ? m8[q] : kNegInf, cz = has ? z8[q] : 0.f, ca = has ? x8[q] : 0.f;
        for (int t = __builtin_ctz(b + 1); t > 0; --t) {
          --top;
          const float lm = sm[top], lz = sz[top], la = sa[top];
          const float nm = fmaxf(lm, cm);
          const float f0 = lz > 0.f ? __expf(lm - nm) : 0.f;
          const float f1 = cz > 0.f ? __expf(cm - nm) : 0.f;
          cz = lz * f0 + cz * f1;
          ca = la * f0 + ca * f1;
          cm = nm;
        }
        sm[top] = cm;
        sz[top] = cz;
        sa[top] = ca;
        ++top;
        if (b + 1 < a.nb) {
          rm = cm;
          rz = cz;
          racc = ca;
          emit(b + 1);
        }
      }
    }
    return;
  }
  if (HIER) {
    // very many blocks: entry e folded directly from its square's blocks, one at a time
    for (int e = 0; e < a.nb; ++e) {
      rm = kNegInf;
      rz = 0.f;
      racc = 0.f;
      for (int b = e - (e & -e); b < e; ++b) {
        const size_t aidx = ((static_cast<size_t>(bh) * a.nb + b) * Cq + i) * Ck + j;
        const float m = a.at_m[aidx], z = a.at_z[aidx];
        if (z > 0.f) {
          const float x = (isK ? a.at_k : a.at_v)[aidx * D + d];
          const float nm = fmaxf(rm, m);
          const float f0 = (rz > 0.f) ? __expf(rm - nm) : 0.f;
          const float f1 = __expf(m - nm);
          rz = rz * f0 + z * f1;
          racc = racc * f0 + x * f1;
          rm = nm;
        }
      }
      emit(e);
    }
    return;
  }
  fold(0, a.nb, a.causal != 0);
  if (!a.causal) emit(0);
}

// Fold sub-block moments: thread per (dv, dk) element; every table entry is normalised
// by its mass. Causal entry b holds the sub-blocks of blocks < b (HIER: of its square).
template <bool HIER>
__global__ void s1_mom_prefix_kernel(S1Args a) {
  const int D = a.D, Cq = a.Cq;
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  const int i = blockIdx.y, bh = blockIdx.z;
  if (e >= D * D) return;
  const int per_block = a.causal ? a.block / a.mbk : a.nmb;
  float rR = kNegInf, racc = 0.f;
  auto emit = [&](int b) {
    const size_t sbase = ((static_cast<size_t>(bh) * a.nbS + b) * Cq + i) * D * D;
    a.s_dip[sbase + e] = (rR == kNegInf) ? 0.f : racc;  // [dv][dk]
  };
  // sub-blocks [m0, m1) folded in order, requested eight at a time; with prefix_emit,
  // entry b is written before the first sub-block of block b joins
  auto fold = [&](int m0, int m1, bool prefix_emit) {
    for (int c0 = m0; c0 < m1; c0 += 8) {
      float R8[8], x8[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        R8[q] = kNegInf;
        x8[q] = 0.f;
        if (c0 + q < m1) {
          const size_t bidx = (static_cast<size_t>(bh) * a.nmb + c0 + q) * Cq + i;
          R8[q] = a.blk_lmass[bidx];
          x8[q] = a.blk_mom[bidx * D * D + e];
        }
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int mb = c0 + q;
        if (mb >= m1) break;
        if (prefix_emit && mb % per_block == 0) emit(mb / per_block);
        const float R = R8[q];
        if (R != kNegInf) {
          const float nR = (rR == kNegInf) ? R : fmaxf(rR, R) + __logf(1.f + __expf(-fabsf(rR - R)));
          const float f0 = (rR == kNegInf) ? 0.f : __expf(rR - nR);
          const float f1 = __expf(R - nR);
          racc = racc * f0 + x8[q] * f1;
          rR = nR;
        }
      }
    }
  };
  if (HIER && a.nb < (1 << (kHierLevels - 1))) {
    // entry b: the sub-blocks of the square's key blocks [b - lowbit(b), b), by a binary
    // counter over the blocks as in s1_prefix (a block's node is the fold of its
    // sub-blocks; left operands first; entry 0 stays empty)
    float sR[kHierLevels], sA[kHierLevels];
    int top = 0;
    emit(0);
    float cR = kNegInf, cA = 0.f;  // the block being built
    for (int c0 = 0; c0 < a.nmb; c0 += 8) {
      float R8[8], x8[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        R8[q] = kNegInf;
        x8[q] = 0.f;
        if (c0 + q < a.nmb) {
          const size_t bidx = (static_cast<size_t>(bh) * a.nmb + c0 + q) * Cq + i;
          R8[q] = a.blk_lmass[bidx];
          x8[q] = a.blk_mom[bidx * D * D + e];
        }
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int mb = c0 + q;
        if (mb >= a.nmb) break;
        const float R = R8[q];
        if (R != kNegInf) {
          const float nR = (cR == kNegInf) ? R : fmaxf(cR, R) + __logf(1.f + __expf(-fabsf(cR - R)));
          const float f0 = (cR == kNegInf) ? 0.f : __expf(cR - nR);
          const float f1 = __expf(R - nR);
          cA = cA * f0 + x8[q] * f1;
          cR = nR;
        }
        if ((mb + 1) % per_block != 0) continue;
        const int b = mb / per_block;
        for (int t = __builtin_ctz(b + 1); t > 0; --t) {
          --top;
          const float lR = sR[top], lA = sA[top];
          const float nR = lR == kNegInf ? cR : (cR == kNegInf ? lR : fmaxf(lR, cR) + __logf(1.f + __expf(-fabsf(lR - cR))));
          const float f0 = lR == kNegInf ? 0.f : __expf(lR - nR);
          const float f1 = cR == kNegInf ? 0.f : __expf(cR - nR);
          cA = lA * f0 + cA * f1;
          cR = nR;
        }
        sR[top] = cR;
        sA[top] = cA;
        ++top;
        if (b + 1 < a.nb) {
          rR = cR;
          racc = cA;
          emit(b + 1);
        }
        cR = kNegInf;
        cA = 0.f;
      }
    }
    return;
  }
  if (HIER) {
    // very many blocks: entry b folded directly from its square's sub-blocks
    for (int b = 0; b < a.nb; ++b) {
      rR = kNegInf;
      racc = 0.f;
      for (int mb = (b - (b & -b)) * per_block; mb < b * per_block; ++mb) {
        const size_t bidx = (static_cast<size_t>(bh) * a.nmb + mb) * Cq + i;
        const float R = a.blk_lmass[bidx];
        if (R != kNegInf) {
          const float x = a.blk_mom[bidx * D * D + e];
          const float nR = (rR == kNegInf) ? R : fmaxf(rR, R) + __logf(1.f + __expf(-fabsf(rR - R)));
          const float f0 = (rR == kNegInf) ? 0.f : __expf(rR - nR);
          const float f1 = __expf(R - nR);
          racc = racc * f0 + x * f1;
          rR = nR;
        }
      }
      emit(b);
    }
    return;
  }
  fold(0, a.nmb, a.causal != 0);
  if (!a.causal) emit(0);
}

// D_i = E_i[v k^T] - sum_j P_ij V_ij K_ij^T for one table entry; one workgroup per
// (i, b, head); thread tiles as in s1_moments. fp32 tables; the bf16 path uses
// s1_dip_final_mfma (stage1_mfma.hip), which also packs the tables.
template <int D>
__global__ void __launch_bounds__(256) s1_dip_final_kernel(S1Args a) {
  constexpr int TD = D / 16;
  extern __shared__ __align__(16) float sh[];
  const int i = blockIdx.x, b = blockIdx.y, bh = blockIdx.z;
  const int Cq = a.Cq, Ck = a.Ck, tid = threadIdx.x;
  if (a.causal && b == 0) return;  // block 0 has no far field
  const size_t sidx = ((static_cast<size_t>(bh) * a.nbS + b) * Cq + i);
  float* P = sh;                    // [Ck]
  float* kc = P + kMaxClusters;     // [32][D]
  float* vc = kc + 32 * D;          // [32][D]
  float* red = vc + 32 * D;
  if (tid < 64) {
    float mx = kNegInf;
    for (int j = tid; j < Ck; j += 64) mx = fmaxf(mx, a.s_logz[sidx * Ck + j]);
    mx = wave_max(mx);
    float s = 0.f;
    for (int j = tid; j < Ck; j += 64) {
      const float l = a.s_logz[sidx * Ck + j];
      const float p = (l == kNegInf) ? 0.f : __expf(l - mx);
      P[j] = p;
      s += p;
    }
    s = wave_sum(s);
    if (tid == 0) red[0] = s;
  }
  __syncthreads();
  const float inv = red[0] > 0.f ? 1.f / red[0] : 0.f;
  const int tr = tid / 16, tc = tid % 16;
  float acc[TD][TD];
#pragma unroll
  for (int x = 0; x < TD; ++x)
#pragma unroll
    for (int y = 0; y < TD; ++y) acc[x][y] = 0.f;
  for (int j0 = 0; j0 < Ck; j0 += 32) {
    const int nj = min(32, Ck - j0);
    __syncthreads();
    for (int e = 4 * tid; e < nj * D; e += 4 * 256) {
      const size_t g = (sidx * Ck + j0) * D + e;
      const f32x4_t k4 = *reinterpret_cast<const f32x4_t*>(a.s_k + g);
      const f32x4_t v4 = *reinterpret_cast<const f32x4_t*>(a.s_v + g);
      *reinterpret_cast<f32x4_t*>(kc + e) = k4;
      *reinterpret_cast<f32x4_t*>(vc + e) = v4;
    }
    __syncthreads();
    for (int jj = 0; jj < nj; ++jj) {
      const float p = P[j0 + jj] * inv;
      float vr[TD], kr[TD];
#pragma unroll
      for (int x = 0; x < TD; ++x) vr[x] = p * vc[jj * D + tr * TD + x];
#pragma unroll
      for (int y = 0; y < TD; ++y) kr[y] = kc[jj * D + tc * TD + y];
#pragma unroll
      for (int x = 0; x < TD; ++x)
#pragma unroll
        for (int y = 0; y < TD; ++y) acc[x][y] = fmaf(vr[x], kr[y], acc[x][y]);
    }
  }
  float* dip = a.s_dip + sidx * D * D;
#pragma unroll
  for (int x = 0; x < TD; ++x)
#pragma unroll
    for (int y = 0; y < TD; ++y) {
      const size_t o = static_cast<size_t>(tr * TD + x) * D + (tc * TD + y);  // [dv][dk]
      dip[o] = dip[o] - acc[x][y];
    }
}

// bf16 hi/lo copies of one table entry (i, e) for the matrix-core stage 2: K_ij and
// V_ij row-major, and s * D_i (value index first).
__global__ void __launch_bounds__(256) s1_pack_kernel(S1Args a) {
  const int i = blockIdx.x, e = blockIdx.y, bh = blockIdx.z;
  const int D = a.D, Ck = a.Ck, tid = threadIdx.x;
  const size_t sidx = (static_cast<size_t>(bh) * a.nbS + e) * a.Cq + i;
  const float* K = a.s_k + sidx * Ck * D;
  const float* V = a.s_v + sidx * Ck * D;
  for (int x = 4 * tid; x < Ck * D; x += 4 * 256) {
    const f32x4_t k4 = *reinterpret_cast<const f32x4_t*>(K + x);
    const f32x4_t v4 = *reinterpret_cast<const f32x4_t*>(V + x);
    u16x4_t kh, kl, vh, vl;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      kh[q] = f32_to_bf16_bits(k4[q]);
      kl[q] = f32_to_bf16_bits(k4[q] - bf16_to_f32(kh[q]));
      vh[q] = f32_to_bf16_bits(v4[q]);
      vl[q] = f32_to_bf16_bits(v4[q] - bf16_to_f32(vh[q]));
    }
    *reinterpret_cast<u16x4_t*>(a.t_khi + sidx * Ck * D + x) = kh;
    *reinterpret_cast<u16x4_t*>(a.t_klo + sidx * Ck * D + x) = kl;
    *reinterpret_cast<u16x4_t*>(a.t_vhi + sidx * Ck * D + x) = vh;
    *reinterpret_cast<u16x4_t*>(a.t_vlo + sidx * Ck * D + x) = vl;
  }
  if (a.dipole) {
    const float* dip = a.s_dip + sidx * D * D;  // [dv][dk]
    for (int x = tid; x < D * D; x += 256) a.t_dip[sidx * D * D + x] = f32_to_bf16_bits(a.scale * dip[x]);
  }
}

// Untilted dipole, acausal (the paper's partially specialised dipole: the tilted C_ij
// replaced by the plain within-cluster covariance of key cluster j; gist.science
// Kernmechanismen 2 and the pith.science referee's note on the covariance of Algorithm 3):
//   Cov_j = (1/n_j) sum_{m in S_j} (v_m - vbar_j)(k_m - kbar_j)^T   (value index first),
// one workgroup per (cluster j, head), two passes over the cluster's keys (means, then
// centred products; every sum in key order). Keys are staged KC at a time in LDS as
// fp32 (four threads per row, each with one permutation entry and 16-byte loads); a
// cluster of at most KC keys is staged once for both passes. Thread (tr, tc) holds
// rows TD tr .. TD tr + TD - 1 and columns TD tc .. TD tc + TD - 1 (TD = D / 16).
template <typename T>
__device__ __forceinline__ void load8_f32(const T* p, float* out);
template <>
__device__ __forceinline__ void load8_f32<bf16>(const bf16* p, float* out) {
  const u16x8_t u = *reinterpret_cast<const u16x8_t*>(p);
#pragma unroll
  for (int e = 0; e < 8; ++e) out[e] = bf16_to_f32(u[e]);
}
template <>
__device__ __forceinline__ void load8_f32<float>(const float* p, float* out) {
  const f32x4_t a = *reinterpret_cast<const f32x4_t*>(p), b = *reinterpret_cast<const f32x4_t*>(p + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    out[e] = a[e];
    out[4 + e] = b[e];
  }
}

// KC keys staged per step: 64, or 2048 / D for the short buckets of causal calls (a
// smaller LDS footprint, so that more workgroups share a CU).
template <typename T, int D, int KC>
__global__ void __launch_bounds__(256) s1_cluster_cov_kernel(S1Args a) {
  constexpr int TD = D / 16, EPT = D * KC / 256, SST = D + 4;  // EPT: staged elements per thread
  static_assert(EPT % 8 == 0, "whole 8-element loads per thread");
  __shared__ __align__(16) float sk[KC * SST];
  __shared__ __align__(16) float sv[KC * SST];
  __shared__ float smk[D], smv[D];
  // acausal: bucket j = key cluster j; causal: bucket u = b * Ck + j (key block b)
  const int j = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x, tr = tid / 16, tc = tid % 16;
  const int32_t* offs = a.offs_k + static_cast<size_t>(bh) * (a.nb * a.Ck + 1);
  // the bucket's members, or with a cluster size cap its kept prefix
  const int m0 = offs[j], m1 = a.klen ? m0 + a.klen[static_cast<size_t>(bh) * a.nb * a.Ck + j] : offs[j + 1];
  const int n = m1 - m0;
  const int32_t* perm = a.perm_k + static_cast<size_t>(bh) * a.N;
  const T* K = static_cast<const T*>(a.k) + static_cast<size_t>(bh) * a.N * D;
  const T* V = static_cast<const T*>(a.v) + static_cast<size_t>(bh) * a.N * D;
  const int sr = tid / (D / EPT), sc = (tid % (D / EPT)) * EPT;  // staged row and first column of this thread
  auto stage = [&](int c0) {  // keys c0 .. c0 + KC - 1 of the cluster (zeros past its end)
    float kf[EPT], vf[EPT];
    const int m = c0 + sr;
    if (m < m1) {
      const size_t row = static_cast<size_t>(perm[m]) * D + sc;
#pragma unroll
      for (int q = 0; q < EPT / 8; ++q) {
        load8_f32<T>(K + row + 8 * q, kf + 8 * q);
        load8_f32<T>(V + row + 8 * q, vf + 8 * q);
      }
    } else {
#pragma unroll
      for (int e = 0; e < EPT; ++e) kf[e] = vf[e] = 0.f;
    }
#pragma unroll
    for (int q = 0; q < EPT / 4; ++q) {
      *reinterpret_cast<f32x4_t*>(sk + sr * SST + sc + 4 * q) = f32x4_t{kf[4 * q], kf[4 * q + 1], kf[4 * q + 2], kf[4 * q + 3]};
      *reinterpret_cast<f32x4_t*>(sv + sr * SST + sc + 4 * q) = f32x4_t{vf[4 * q], vf[4 * q + 1], vf[4 * q + 2], vf[4 * q + 3]};
    }
  };
  const bool once = n <= KC;  // the staged chunk serves both passes
  // pass 1: means (thread d < D sums k, D <= thread < 2D sums v)
  float sum = 0.f;
  for (int c0 = m0; c0 < m1; c0 += KC) {
    __syncthreads();
    stage(c0);
    __syncthreads();
    const int nk = min(KC, m1 - c0);
    if (tid < 2 * D) {
      const float* col = tid < D ? sk + tid : sv + (tid - D);
#pragma unroll 8
      for (int r = 0; r < nk; ++r) sum += col[r * SST];
    }
  }
  if (tid < D) smk[tid] = n > 0 ? sum / static_cast<float>(n) : 0.f;
  else if (tid < 2 * D) smv[tid - D] = n > 0 ? sum / static_cast<float>(n) : 0.f;
  __syncthreads();
  if (a.causal) {
    const size_t u = static_cast<size_t>(bh) * a.nb * a.Ck + j;
    if (tid < D) a.ub_mk[u * D + tid] = smk[tid];
    else if (tid < 2 * D) a.ub_mv[u * D + tid - D] = smv[tid - D];
    if (tid == 0) a.ub_n[u] = static_cast<float>(n);
  }
  float mk[TD], mv[TD];
#pragma unroll
  for (int x = 0; x < TD; ++x) {
    mv[x] = smv[TD * tr + x];
    mk[x] = smk[TD * tc + x];
  }
  // pass 2: centred products
  float acc[TD][TD];
#pragma unroll
  for (int x = 0; x < TD; ++x)
#pragma unroll
    for (int y = 0; y < TD; ++y) acc[x][y] = 0.f;
  for (int c0 = m0; c0 < m1; c0 += KC) {
    if (!once) {
      __syncthreads();
      stage(c0);
      __syncthreads();
    }
    const int nk = min(KC, m1 - c0);
#pragma unroll 4
    for (int r = 0; r < nk; ++r) {
      float vr[TD], kr[TD];
#pragma unroll
      for (int x = 0; x < TD; ++x) {
        vr[x] = sv[r * SST + TD * tr + x] - mv[x];
        kr[x] = sk[r * SST + TD * tc + x] - mk[x];
      }
#pragma unroll
      for (int x = 0; x < TD; ++x)
#pragma unroll
        for (int y = 0; y < TD; ++y) acc[x][y] = fmaf(vr[x], kr[y], acc[x][y]);
    }
  }
  // acausal: the covariance (1/n); causal: the bucket's centred sum, combined over blocks later
  const float inv = a.causal ? 1.f : (n > 0 ? 1.f / static_cast<float>(n) : 0.f);
  float* cov = a.causal ? a.ub_c + (static_cast<size_t>(bh) * a.nb * a.Ck + j) * D * D
                        : a.cov_k + (static_cast<size_t>(bh) * a.Ck + j) * D * D;
#pragma unroll
  for (int x = 0; x < TD; ++x)
#pragma unroll
    for (int y = 0; y < TD; y += 4) {
      const f32x4_t f = {acc[x][y] * inv, acc[x][y + 1] * inv, acc[x][y + 2] * inv, acc[x][y + 3] * inv};
      *reinterpret_cast<f32x4_t*>(cov + static_cast<size_t>(TD * tr + x) * D + TD * tc + y) = f;
    }
}

// Untilted dipole, acausal: D_i = sum_j P_ij Cov_j with P_ij = softmax_j(log Z_ij) from the
// finalised log Z table, for all query clusters of a head: one workgroup per (256
// elements of D x D, head), a thread per element, query clusters in groups of 32 (their
// P rows in LDS, zero past Ck), the covariances of eight clusters requested at a time,
// sums over j in cluster order. Writes s * D_i in bf16 (matrix-core stage 2) or D_i in
// fp32.
template <int D>
__global__ void __launch_bounds__(256) s1_untilted_dip_kernel(S1Args a) {
  constexpr int IG = 32, JB = 8;
  __shared__ float sP[IG][kMaxClusters];
  const int bh = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int e = blockIdx.x * 256 + tid;  // < D * D (the grid covers it exactly)
  const int Cq = a.Cq, Ck = a.Ck, Ckr = (Ck + JB - 1) / JB * JB;
  const float* cov = a.cov_k + static_cast<size_t>(bh) * Ck * D * D + e;
  for (int i0 = 0; i0 < Cq; i0 += IG) {
    const int ni = min(IG, Cq - i0);
    __syncthreads();  // the previous group's rows are consumed
    for (int ii = wave; ii < IG; ii += 4) {  // a wave per query cluster: softmax over j
      float l[kMaxClusters / 64];
      float mx = kNegInf;
      const float* lz = a.s_logz + (static_cast<size_t>(bh) * a.nbS * Cq + i0 + ii) * Ck;
#pragma unroll
      for (int q = 0; q < kMaxClusters / 64; ++q) {
        const int jj = lane + 64 * q;
        l[q] = ii < ni && jj < Ck ? lz[jj] : kNegInf;
        mx = fmaxf(mx, l[q]);
      }
      mx = wave_max(mx);
      float sum = 0.f;
#pragma unroll
      for (int q = 0; q < kMaxClusters / 64; ++q) {
        l[q] = l[q] == kNegInf ? 0.f : __expf(l[q] - mx);
        sum += l[q];
      }
      sum = wave_sum(sum);
      const float inv = sum > 0.f ? 1.f / sum : 0.f;
#pragma unroll
      for (int q = 0; q < kMaxClusters / 64; ++q) sP[ii][lane + 64 * q] = l[q] * inv;
    }
    __syncthreads();
    float acc[IG];
#pragma unroll
    for (int ii = 0; ii < IG; ++ii) acc[ii] = 0.f;
    for (int j0 = 0; j0 < Ckr; j0 += JB) {
      float cv[JB];
#pragma unroll
      for (int q = 0; q < JB; ++q) cv[q] = j0 + q < Ck ? cov[static_cast<size_t>(j0 + q) * D * D] : 0.f;
#pragma unroll
      for (int q = 0; q < JB; ++q)
#pragma unroll
        for (int ii = 0; ii < IG; ++ii) acc[ii] = fmaf(sP[ii][j0 + q], cv[q], acc[ii]);
    }
    for (int ii = 0; ii < ni; ++ii) {
      const size_t sidx = static_cast<size_t>(bh) * a.nbS * Cq + i0 + ii;  // entry 0
      if (a.t_dip != nullptr) a.t_dip[sidx * D * D + e] = f32_to_bf16_bits(a.scale * acc[ii]);
      else a.s_dip[sidx * D * D + e] = acc[ii];
    }
  }
}

// Untilted dipole, causal: per (head, key cluster j) the count and means of the cluster's
// keys in the blocks before b, for every entry b (entry 0: none), folded block by block in
// block order: n' = n + n_b, mean' = mean + (mean_b - mean) n_b / n'. Thread d holds
// dimension d of the key and the value mean.
template <int D>
__global__ void __launch_bounds__(D) s1_untilted_prefix_kernel(S1Args a) {
  const int j = blockIdx.x, bh = blockIdx.y, d = threadIdx.x, Ck = a.Ck;
  float n = 0.f, mk = 0.f, mv = 0.f;
  for (int b = 0; b < a.nb; ++b) {
    const size_t e = (static_cast<size_t>(bh) * a.nb + b) * Ck + j;  // entry b and bucket (b, j)
    a.up_mk[e * D + d] = mk;
    a.up_mv[e * D + d] = mv;
    if (d == 0) a.up_n[e] = n;
    const float nb_ = a.ub_n[e];
    if (nb_ > 0.f) {
      const float n1 = n + nb_, f = nb_ / n1;
      mk += (a.ub_mk[e * D + d] - mk) * f;
      mv += (a.ub_mv[e * D + d] - mv) * f;
      n = n1;
    }
  }
}

// Untilted dipole, causal: D_i^{<b} = sum_j P_ij^{<b} Cov_j^{<b} for every entry b >= 1,
// with Cov_j^{<b} the plain covariance of key cluster j over the keys of the blocks
// before b and P_ij^{<b} = softmax_j log Z_ij^{<b} from the entry's tables. One workgroup
// per (64 consecutive elements of D x D, head) walks the blocks in order and keeps, for
// each of its elements, the running centred sum C_j of every cluster, spread over four
// threads (clusters q, q + 4, ... of thread q). Adding block b - 1 to it is the pairwise
// combination of centred sums,
//   C_j += C_(b-1,j) + n n_b / (n + n_b) (mv_b - mv)[dv] (mk_b - mk)[dk],
// with the prefix (n, mk, mv) of entry b - 1 and the bucket's own (n_b, mk_b, mv_b); then
// D_i = sum_j (P_ij / n_j) C_j for 32 query clusters at a time (the weights in LDS),
// summed over the four threads of an element. Entry 0 (no earlier keys) is zero. Writes
// s * D_i in bf16 (matrix-core stage 2) or D_i in fp32.
template <int D>
__global__ void __launch_bounds__(256) s1_untilted_causal_kernel(S1Args a) {
  constexpr int EL = 64, IG = 32, JR = kMaxClusters / 4;
  __shared__ float sA[kMaxClusters * EL];
  __shared__ float sW[IG * kMaxClusters];
  __shared__ float sF[kMaxClusters];
  __shared__ float sN[kMaxClusters];
  const int bh = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int el = tid >> 2, q = tid & 3;
  const int e0 = blockIdx.x * EL;            // first element; the grid covers D * D exactly
  const int e = e0 + el;
  const int dv = e0 / D;                     // one value row per workgroup (EL <= D)
  const int Cq = a.Cq, Ck = a.Ck;
  const size_t hb = static_cast<size_t>(bh) * a.nb;
  float C[JR];
#pragma unroll
  for (int r = 0; r < JR; ++r) C[r] = 0.f;
  auto store = [&](int b, int i, float val) {
    const size_t sidx = (hb + b) * Cq + i;
    if (a.t_dip != nullptr) a.t_dip[sidx * D * D + e] = f32_to_bf16_bits(a.scale * val);
    else a.s_dip[sidx * D * D + e] = val;
  };
  if (q == 0)
    for (int i = 0; i < Cq; ++i) store(0, i, 0.f);
  for (int b = 1; b < a.nb; ++b) {
    const size_t u = (hb + b - 1) * Ck;      // buckets (b - 1, j) and prefix entry b - 1
    __syncthreads();                         // the previous block's LDS is consumed
    for (int jj = tid; jj < Ck; jj += 256) {
      const float n0 = a.up_n[u + jj], n1 = a.ub_n[u + jj];
      const float f = (n0 > 0.f && n1 > 0.f) ? n0 * n1 / (n0 + n1) : 0.f;
      sF[jj] = f * (a.ub_mv[(u + jj) * D + dv] - a.up_mv[(u + jj) * D + dv]);
      sN[jj] = n0 + n1;
    }
    __syncthreads();
    for (int x = tid; x < Ck * EL; x += 256) {
      const int jj = x / EL, ex = x % EL, dk = (e0 + ex) % D;
      const float dkv = a.ub_mk[(u + jj) * D + dk] - a.up_mk[(u + jj) * D + dk];
      sA[x] = a.ub_c[(u + jj) * D * D + e0 + ex] + sF[jj] * dkv;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < JR; ++r) {
      const int jj = q + 4 * r;
      if (jj < Ck) C[r] += sA[jj * EL + el];
    }
    for (int i0 = 0; i0 < Cq; i0 += IG) {
      const int ni = min(IG, Cq - i0);
      __syncthreads();                       // sW of the previous group is consumed
      for (int ii = wave; ii < IG; ii += 4) {  // a wave per query cluster: softmax over j
        float l[kMaxClusters / 64];
        float mx = kNegInf;
        const float* lz = a.s_logz + ((hb + b) * Cq + i0 + ii) * Ck;
#pragma unroll
        for (int t = 0; t < kMaxClusters / 64; ++t) {
          const int jj = lane + 64 * t;
          l[t] = ii < ni && jj < Ck ? lz[jj] : kNegInf;
          mx = fmaxf(mx, l[t]);
        }
        mx = wave_max(mx);
        float sum = 0.f;
#pragma unroll
        for (int t = 0; t < kMaxClusters / 64; ++t) {
          l[t] = l[t] == kNegInf ? 0.f : __expf(l[t] - mx);
          sum += l[t];
        }
        sum = wave_sum(sum);
        const float inv = sum > 0.f ? 1.f / sum : 0.f;
#pragma unroll
        for (int t = 0; t < kMaxClusters / 64; ++t) {
          const int jj = lane + 64 * t;
          const float nj = jj < Ck ? sN[jj] : 0.f;
          sW[ii * kMaxClusters + jj] = nj > 0.f ? l[t] * inv / nj : 0.f;
        }
      }
      __syncthreads();
      float acc[IG];
#pragma unroll
      for (int ii = 0; ii < IG; ++ii) acc[ii] = 0.f;
#pragma unroll
      for (int r = 0; r < JR; ++r) {
        const int jj = q + 4 * r;
        if (jj >= Ck) break;
#pragma unroll
        for (int ii = 0; ii < IG; ++ii) acc[ii] = fmaf(sW[ii * kMaxClusters + jj], C[r], acc[ii]);
      }
      // sum over the four threads of the element (lanes 4 el .. 4 el + 3, a DPP quad)
#pragma unroll
      for (int ii = 0; ii < IG; ++ii) {
        float v = acc[ii];
        v += dpp_f32<0xB1>(v);  // l ^ 1
        v += dpp_f32<0x4E>(v);  // l ^ 2
        acc[ii] = v;
      }
#pragma unroll
      for (int ii = 0; ii < IG; ii += 4)
        if (i0 + ii + q < Cq) store(b, i0 + ii + q, acc[ii + q]);
    }
  }
}

template <typename T, int D>
static void launch_untilted(const S1Args& a, int part, hipStream_t s) {
  if (part == 0) {
    {
      ProfScope ps_("s1_cluster_cov", s);
      if (a.causal)
        hipLaunchKernelGGL((s1_cluster_cov_kernel<T, D, 2048 / D>), dim3(a.nb * a.Ck, a.BH), dim3(256), 0, s, a);
      else
        hipLaunchKernelGGL((s1_cluster_cov_kernel<T, D, 64>), dim3(a.nb * a.Ck, a.BH), dim3(256), 0, s, a);
    }
    if (a.causal) {
      ProfScope ps_("s1_untilted_prefix", s);
      hipLaunchKernelGGL(s1_untilted_prefix_kernel<D>, dim3(a.Ck, a.BH), dim3(D), 0, s, a);
    }
  } else if (a.causal) {
    ProfScope ps_("s1_untilted_causal", s);
    hipLaunchKernelGGL(s1_untilted_causal_kernel<D>, dim3(D * D / 64, a.BH), dim3(256), 0, s, a);
  } else {
    ProfScope ps_("s1_untilted_dip", s);
    hipLaunchKernelGGL((s1_untilted_dip_kernel<D>), dim3((D * D + 255) / 256, a.BH), dim3(256), 0, s, a);
  }
}

// A second stream per device (default priority, created on first use and kept until the
// process ends) on which the atoms run beside the scores and the block moments: the
// atoms read only the clustering, the moments read the scores, and the tables need both.
static hipStream_t side_stream() {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static hipStream_t streams[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (streams[dev] == nullptr) {
    hipStream_t st = nullptr;
    if (hipStreamCreateWithFlags(&st, hipStreamNonBlocking) != hipSuccess) return nullptr;
    streams[dev] = st;
  }
  return streams[dev];
}

template <typename T, int D>
static void launch_stage1_t(const S1Args& a, hipStream_t s) {
  constexpr int kS1Keys = S1Keys<D>::value;
  const bool mf = sizeof(T) == 2;  // bf16 inputs: matrix-core kernels
  if (mf && a.retr == nullptr && !a.hier && !a.tables_f32) {
    // acausal: one table entry per (head, i), finalised in a single pass; causal without
    // retrieval: one scan over the blocks writes every entry (the hierarchical squares
    // take the general path below: per entry folds of the merged atoms and moments). The atoms (with their
    // merge) go to the side stream, forked from and joined back into the caller's stream
    // by events; without a side stream or events everything runs on the caller's stream.
    hipStream_t side = a.one_stream ? nullptr : side_stream();
    hipEvent_t fork = nullptr, join = nullptr;
    bool two = side != nullptr && hipEventCreateWithFlags(&fork, hipEventDisableTiming) == hipSuccess &&
               hipEventCreateWithFlags(&join, hipEventDisableTiming) == hipSuccess &&
               hipEventRecord(fork, s) == hipSuccess && hipStreamWaitEvent(side, fork, 0) == hipSuccess;
    launch_stage1_mfma(a, 1, two ? side : s);
    if (two && hipEventRecord(join, side) != hipSuccess) {
      (void)hipStreamSynchronize(side);  // the join cannot be enqueued: wait on the host
      two = false;
    }
    const bool untilted = a.dipole == 2;
    if (untilted) {
      launch_untilted<T, D>(a, 0, s);  // per key cluster covariance (needs no scores)
    } else {
      launch_stage1_mfma(a, 0, s);
      if (a.dipole) launch_stage1_mfma(a, 2, s);
    }
    if (two && hipStreamWaitEvent(s, join, 0) != hipSuccess) (void)hipStreamSynchronize(side);
    if (fork != nullptr) (void)hipEventDestroy(fork);
    if (join != nullptr) (void)hipEventDestroy(join);
    if (untilted) {
      S1Args af = a;
      af.dipole = 0;  // the tables without the tilted dipole
      launch_stage1_mfma(af, a.causal ? 4 : 3, s);
      launch_untilted<T, D>(a, 1, s);
    } else {
      launch_stage1_mfma(a, a.causal ? 4 : 3, s);
    }
    return;
  }
  if (mf) {
    launch_stage1_mfma(a, 0, s);
    launch_stage1_mfma(a, 1, s);
  } else {
    const size_t lds_atoms = sizeof(float) * (static_cast<size_t>(a.Cq) * D + 2 * kS1Keys * D +
                                              static_cast<size_t>(a.Cq) * kS1Keys + 3 * a.Cq);
    allow_lds((const void*)s1_atoms_kernel<T, D>, lds_atoms);
    ProfScope ps_("s1_atoms", s);
    hipLaunchKernelGGL((s1_atoms_kernel<T, D>), dim3(a.Ck, a.nb, a.BH), dim3(256), lds_atoms, s, a);
  }
  if (!a.causal) {
    ProfScope ps_("s1_tables", s);
    hipLaunchKernelGGL(s1_tables_acausal_kernel, dim3(a.Cq, a.BH), dim3(256), 0, s, a);
  } else {
    ProfScope ps_("s1_prefix", s);
    if (a.hier) hipLaunchKernelGGL(s1_prefix_kernel<true>, dim3(a.Ck, a.Cq, a.BH), dim3(2 * D), 0, s, a);
    else hipLaunchKernelGGL(s1_prefix_kernel<false>, dim3(a.Ck, a.Cq, a.BH), dim3(2 * D), 0, s, a);
  }
  if (a.dipole == 2) {  // untilted (no retrieval, no hierarchy): per key cluster covariances
    launch_untilted<T, D>(a, 0, s);
    launch_untilted<T, D>(a, 1, s);
    if (a.t_khi != nullptr) {
      ProfScope ps_("s1_pack", s);
      hipLaunchKernelGGL(s1_pack_kernel, dim3(a.Cq, a.nbS, a.BH), dim3(256), 0, s, a);
    }
    return;
  }
  if (a.dipole) {
    if (mf) {
      launch_stage1_mfma(a, 2, s);
    } else {
      const size_t lds_mom = sizeof(float) * (D + 2 * kS1Keys * D + kS1Keys + 4);
      allow_lds((const void*)s1_moments_kernel<T, D>, lds_mom);
      ProfScope ps_("s1_moments", s);
      hipLaunchKernelGGL((s1_moments_kernel<T, D>), dim3(a.Cq, a.nb, a.BH), dim3(256), lds_mom, s, a);
    }
    {
      ProfScope ps_("s1_mom_prefix", s);
      if (a.causal && a.hier)
        hipLaunchKernelGGL(s1_mom_prefix_kernel<true>, dim3((D * D + 255) / 256, a.Cq, a.BH), dim3(256), 0, s, a);
      else
        hipLaunchKernelGGL(s1_mom_prefix_kernel<false>, dim3((D * D + 255) / 256, a.Cq, a.BH), dim3(256), 0, s, a);
    }
  }
  if (a.retr != nullptr) launch_retrieval(*a.retr, 0, sizeof(T) == 2 ? 1 : 0, s);
  if (a.dipole) {
    if (a.t_khi != nullptr) {
      launch_stage1_mfma(a, 5, s);  // matrix cores, with the packing of the bf16 tables
    } else {
      const size_t lds_fin = sizeof(float) * (kMaxClusters + 64 * D + 4);
      allow_lds((const void*)s1_dip_final_kernel<D>, lds_fin);
      ProfScope ps_("s1_dip_final", s);
      hipLaunchKernelGGL((s1_dip_final_kernel<D>), dim3(a.Cq, a.nbS, a.BH), dim3(256), lds_fin, s, a);
    }
  }
  if (a.t_khi != nullptr && !a.dipole) {  // with the dipole, the finalise packs the tables
    ProfScope ps_("s1_pack", s);
    hipLaunchKernelGGL(s1_pack_kernel, dim3(a.Cq, a.nbS, a.BH), dim3(256), 0, s, a);
  }
}

hipError_t launch_stage1_pack(const S1Args& a, hipStream_t s) {
  ProfScope ps_("s1_pack", s);
  hipLaunchKernelGGL(s1_pack_kernel, dim3(a.Cq, a.nbS, a.BH), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_stage1(const S1Args& a, int dtype, hipStream_t s) {
  if (dtype == 0) {
    if (a.D == 64) launch_stage1_t<float, 64>(a, s);
    else launch_stage1_t<float, 128>(a, s);
  } else {
    if (a.D == 64) launch_stage1_t<bf16, 64>(a, s);
    else launch_stage1_t<bf16, 128>(a, s);
  }
  return hipGetLastError();
}

}  // namespace muse
