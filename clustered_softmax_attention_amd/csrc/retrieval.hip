// Retrieval for causal MuSe (gist.science summary of arXiv 2509.10406, Kernmechanismen 4):
// for each query cluster i and block b >= 1,
//   1. the k1 key clusters j with the largest tilted-summary score log Z^{<b}_ij (the log
//      mass of cluster j's earlier keys seen from qbar_i),
//   2. inside each, the k2 earlier blocks b' with the largest atom log mass
//      m_ij(b') + log z_ij(b'),
// and the keys of the chosen (cluster, block) atoms are attended exactly; the summaries
// cover the remaining earlier keys only. Descending order with ties to the lower index;
// empty candidates are never chosen.
//
//   retr_select  one wave per (i, b): the selection, stored as k1 rows of
//                (j, b'_1 .. b'_k2), -1 padded.
//   retr_tables  one workgroup per (i, b): table entry (b, i) becomes the far field
//                without the retrieved atoms: chosen clusters are re-merged from their
//                unselected atoms (no subtraction of log-sum-exps), and the second
//                moment becomes (M - sum_R w v k^T) / (1 - sum_R w) with w relative to the
//                prefix mass.
//   retr_exact   one workgroup per (i, b): exact softmax over the retrieved keys for the
//                bucket's queries, merged by log-sum-exp into the far-field partial result.
//   retr_exact_mfma  (bf16 inputs) the same on the matrix cores, one workgroup per
//                chunk of up to 128 queries of one bucket (the stage-2 chunks).
//   retr_moment_mfma (bf16 inputs) the second-moment part of retr_tables on the matrix
//                cores, run before it (it needs the prefix log mass of the unmodified
//                entry).
#include "mfma.hpp"
#include "muse_kernels.hpp"

namespace muse {

// wave-wide argmax with ties to the lower index; every lane gets the winner
__device__ __forceinline__ void wave_argmax(float& v, int& idx) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(v, o, 64);
    const int oi = __shfl_xor(idx, o, 64);
    if (ov > v || (ov == v && oi < idx)) {
      v = ov;
      idx = oi;
    }
  }
}

// One wave per (i, b): the k1 clusters first (LDS only), then per chosen cluster its
// block scores, loaded once for all k2 picks (each lane's rows requested together,
// unconditionally at a clamped block index), a chosen entry marked by a score of -inf.
// Dynamic LDS: nb floats (the block scores of one cluster).
__global__ void __launch_bounds__(64) retr_select_kernel(RetrArgs a) {
  extern __shared__ float s_bs[];
  __shared__ float s_sj[kMaxClusters];
  __shared__ int s_out[kMaxRetrRow];  // the selection row, written out at the end
  const int i = blockIdx.x, b = blockIdx.y, bh = blockIdx.z;
  const int lane = threadIdx.x;
  const int Ck = a.Ck, k1 = a.k1, k2 = a.k2, row = k1 * (1 + k2);
  int32_t* out = a.sel + ((static_cast<size_t>(bh) * a.nb + b) * a.Cq + i) * row;
  if (b == 0) {
    for (int x = lane; x < row; x += 64) out[x] = -1;
    return;
  }
  const size_t sidx = (static_cast<size_t>(bh) * a.nb + b) * a.Cq + i;
  {
    float l[kMaxClusters / 64];
#pragma unroll
    for (int q = 0; q < kMaxClusters / 64; ++q) l[q] = a.s_logz[sidx * Ck + min(lane + 64 * q, Ck - 1)];
#pragma unroll
    for (int q = 0; q < kMaxClusters / 64; ++q)
      if (lane + 64 * q < Ck) s_sj[lane + 64 * q] = l[q];
  }
  __syncthreads();
  // clusters: highest prefix log mass first, ties to the lower index; -inf ends the list
  for (int t = 0; t < k1; ++t) {
    float v = kNegInf;
    int idx = 1 << 30;
    for (int j = lane; j < Ck; j += 64)
      if (s_sj[j] != kNegInf && (s_sj[j] > v || (s_sj[j] == v && j < idx))) {
        v = s_sj[j];
        idx = j;
      }
    wave_argmax(v, idx);
    const int j = v == kNegInf ? -1 : idx;
    if (lane == 0) {
      if (j >= 0) s_sj[j] = kNegInf;
      s_out[t * (1 + k2)] = j;
    }
    __syncthreads();
  }
  // blocks of each chosen cluster: highest atom log mass among blocks < b, ties to the
  // earlier block; empty atoms never chosen
  for (int t = 0; t < k1; ++t) {
    const int j = s_out[t * (1 + k2)];
    int* o = s_out + t * (1 + k2);
    if (j < 0) {
      for (int x = lane; x < k2; x += 64) o[1 + x] = -1;
      continue;
    }
    for (int bb0 = 0; bb0 < b; bb0 += 64) {
      const int bb = bb0 + lane;
      const size_t aidx = ((static_cast<size_t>(bh) * a.nb + min(bb, b - 1)) * a.Cq + i) * Ck + j;
      const float z = a.at_z[aidx], m = a.at_m[aidx];
      if (bb < b) s_bs[bb] = z > 0.f ? m + __logf(z) : kNegInf;
    }
    __syncthreads();
    for (int u = 0; u < k2; ++u) {
      float bv = kNegInf;
      int bi = 1 << 30;
      for (int bb = lane; bb < b; bb += 64) {
        const float sv = s_bs[bb];
        if (sv != kNegInf && (sv > bv || (sv == bv && bb < bi))) {
          bv = sv;
          bi = bb;
        }
      }
      wave_argmax(bv, bi);
      if (lane == 0) {
        o[1 + u] = bv == kNegInf ? -1 : bi;
        if (bv != kNegInf) s_bs[bi] = kNegInf;
      }
      __syncthreads();
    }
  }
  __syncthreads();
  for (int x = lane; x < row; x += 64) {
    out[x] = s_out[x];
    if (a.trace != nullptr) a.trace[((static_cast<size_t>(bh) * a.nb + b) * a.Cq + i) * row + x] = s_out[x];
  }
}

__device__ __forceinline__ bool atom_selected(const int32_t* selrow, int k2, int bb) {
  for (int u = 0; u < k2; ++u)
    if (selrow[1 + u] == bb) return true;
  return false;
}

// The retrieved atoms of (b, i) as ranges of the key permutation, in selection order
// (cluster t, then its blocks): range w = t k2 + u starts at start[w] and holds the
// concatenated positions [cum[w], cum[w + 1]); unchosen or empty atoms are empty ranges.
// Called by one whole wave (a pair per lane, then a wave prefix sum); returns the number
// of ranges, k1 k2.
__device__ int retr_ranges(const int32_t* selrow, const int32_t* offk, int Ck, int k1, int k2, int* start,
                           int* cum) {
  const int lane = lane_id(), np = k1 * k2;
  int run = 0;
  for (int w0 = 0; w0 < np; w0 += 64) {
    const int w = w0 + lane;
    int p0 = 0, len = 0;
    if (w < np) {
      const int t = w / k2, u = w % k2;
      const int j = selrow[t * (1 + k2)], bb = selrow[t * (1 + k2) + 1 + u];
      if (j >= 0 && bb >= 0) {
        p0 = offk[bb * Ck + j];
        len = offk[bb * Ck + j + 1] - p0;
      }
    }
    int incl = len;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    if (w < np) {
      start[w] = p0;
      cum[w] = run + incl - len;
    }
    run += __shfl(incl, 63, 64);
  }
  if (lane == 0) cum[np] = run;
  return np;
}

// keys staged per step (LDS stays under 64 KiB)
template <int D>
struct RetrChunk {
  static constexpr int value = D == 64 ? 64 : 32;
};

// 256 threads; LDS: key/value chunk [KCH][D] fp32, weights, reductions.
template <typename T, int D>
__global__ void __launch_bounds__(256) retr_tables_kernel(RetrArgs a) {
  constexpr int TD = D / 16;
  constexpr int KCH = RetrChunk<D>::value;
  __shared__ float s_k[KCH * D];
  __shared__ float s_v[KCH * D];
  __shared__ float s_w[64];
  __shared__ float s_q[D];
  __shared__ float s_red[2];
  __shared__ int s_sel[kMaxRetrRow];
  __shared__ int s_start[kMaxRetrRow];    // retrieved atoms as ranges of the key permutation
  __shared__ int s_cum[kMaxRetrRow + 1];  // exclusive prefix of the range lengths
  __shared__ int s_row[KCH];              // key rows of the staged chunk
  __shared__ int s_nr;
  const int i = blockIdx.x, b = blockIdx.y, bh = blockIdx.z;
  const int tid = threadIdx.x;
  if (b == 0) return;
  const int Ck = a.Ck, k1 = a.k1, k2 = a.k2, row = k1 * (1 + k2);
  const int32_t* sel = a.sel + ((static_cast<size_t>(bh) * a.nb + b) * a.Cq + i) * row;
  static_assert(kMaxRetrRow <= 256 && D <= 256, "one element per thread");
  {
    // both requested before either is stored (a load under the thread's bound would wait
    // for itself)
    const int32_t sv = sel[min(tid, row - 1)];
    const float qv = a.qbar[(static_cast<size_t>(bh) * a.Cq + i) * D + min(tid, D - 1)];
    if (tid < row) s_sel[tid] = sv;
    if (tid < D) s_q[tid] = qv;
  }
  const size_t sidx = (static_cast<size_t>(bh) * a.nb + b) * a.Cq + i;
  // prefix log mass (before any entry is rewritten), for the fp32 second moment
  const bool mom32 = a.dipole && sizeof(T) == 4;
  if (mom32 && tid < 64) {
    float mx = kNegInf;
    for (int j = tid; j < Ck; j += 64) mx = fmaxf(mx, a.s_logz[sidx * Ck + j]);
    mx = wave_max(mx);
    float sm = 0.f;
    for (int j = tid; j < Ck; j += 64) {
      const float l = a.s_logz[sidx * Ck + j];
      if (l != kNegInf) sm += __expf(l - mx);
    }
    sm = wave_sum(sm);
    if (tid == 0) s_red[0] = mx == kNegInf ? kNegInf : mx + __logf(sm);
  }
  __syncthreads();
  const float Rpre = mom32 ? s_red[0] : kNegInf;

  // 1. remainder summaries of the chosen clusters (re-merged from unselected atoms): the
  // k1 x 2D (cluster, feature) folds spread over all threads
  for (int w = tid; w < k1 * 2 * D; w += 256) {
    const int t = w / (2 * D), x = w % (2 * D);
    const int* sr = s_sel + t * (1 + k2);
    const int j = sr[0];
    if (j < 0) continue;
    {
      const bool isK = x < D;
      const int d = isK ? x : x - D;
      float rm = kNegInf, rz = 0.f, racc = 0.f;
      // eight blocks' atoms requested at a time, folded in block order
      for (int bb0 = 0; bb0 < b; bb0 += 8) {
        float m8[8], z8[8], x8[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int bb = bb0 + q;
          m8[q] = kNegInf;
          z8[q] = 0.f;
          x8[q] = 0.f;
          if (bb < b && !atom_selected(sr, k2, bb)) {
            const size_t aidx = ((static_cast<size_t>(bh) * a.nb + bb) * a.Cq + i) * Ck + j;
            m8[q] = a.at_m[aidx];
            z8[q] = a.at_z[aidx];
            x8[q] = (isK ? a.at_k : a.at_v)[aidx * D + d];
          }
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          if (!(z8[q] > 0.f)) continue;
          const float nm = fmaxf(rm, m8[q]);
          const float f0 = rz > 0.f ? __expf(rm - nm) : 0.f;
          const float f1 = __expf(m8[q] - nm);
          rz = rz * f0 + z8[q] * f1;
          racc = racc * f0 + x8[q] * f1;
          rm = nm;
        }
      }
      const bool any = rz > 0.f;
      if (x == 0) a.s_logz[sidx * Ck + j] = any ? rm + __logf(rz) : kNegInf;
      (isK ? a.s_k : a.s_v)[(sidx * Ck + j) * D + d] = any ? racc / rz : 0.f;
    }
  }
  // bf16 inputs: the second moment was handled by retr_moment_mfma
  if (!mom32 || Rpre == kNegInf) return;

  // 2. second moment without the retrieved keys
  const int tr = tid / 16, tc = tid % 16;
  float acc[TD][TD];
#pragma unroll
  for (int x = 0; x < TD; ++x)
#pragma unroll
    for (int y = 0; y < TD; ++y) acc[x][y] = 0.f;
  float wsum = 0.f;  // meaningful in thread 0
  const T* K = static_cast<const T*>(a.k) + static_cast<size_t>(bh) * a.N * D;
  const T* V = static_cast<const T*>(a.v) + static_cast<size_t>(bh) * a.N * D;
  const int32_t* perm = a.perm_k + static_cast<size_t>(bh) * a.N;
  const int32_t* offs = a.offs_k + static_cast<size_t>(bh) * (a.nb * Ck + 1);
  if (tid < 64) {
    const int n = retr_ranges(s_sel, offs, Ck, k1, k2, s_start, s_cum);
    if (tid == 0) s_nr = n;
  }
  __syncthreads();
  const int nr = s_nr, nR = s_cum[nr];
  // the retrieved keys in chunks of KCH of their concatenation (several atoms per chunk)
  for (int c0 = 0; c0 < nR; c0 += KCH) {
    const int nk = min(KCH, nR - c0);
    __syncthreads();  // previous chunk consumed
    if (tid < nk) {
      const int pos = c0 + tid;
      int lo = 0, hi = nr - 1;  // last range with s_cum <= pos
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_cum[mid] <= pos) lo = mid;
        else hi = mid - 1;
      }
      s_row[tid] = perm[s_start[lo] + pos - s_cum[lo]];
    }
    __syncthreads();
    for (int x = tid; x < nk * D; x += 256) {
      const int r = x / D, d = x % D;
      const size_t rowi = static_cast<size_t>(s_row[r]) * D + d;
      s_k[x] = Elem<T>::load(K, rowi);
      s_v[x] = Elem<T>::load(V, rowi);
    }
    __syncthreads();
    if (tid < 64) {
      float w = 0.f;
      if (tid < nk) {
        float dot = 0.f;
        for (int d = 0; d < D; ++d) dot = fmaf(s_q[d], s_k[tid * D + d], dot);
        w = __expf(a.scale * dot - Rpre);
      }
      s_w[tid] = w;
      const float ws = wave_sum(w);
      if (tid == 0) wsum += ws;
    }
    __syncthreads();
    for (int m = 0; m < nk; ++m) {
      const float wm = s_w[m];
#pragma unroll
      for (int x = 0; x < TD; ++x)
#pragma unroll
        for (int y = 0; y < TD; ++y) acc[x][y] = fmaf(wm * s_v[m * D + tr * TD + x], s_k[m * D + tc * TD + y], acc[x][y]);
    }
  }
  if (tid == 0) s_red[1] = wsum;
  __syncthreads();
  const float rest = 1.f - s_red[1];
  const float inv = rest > 1e-30f ? 1.f / rest : 0.f;
  float* dip = a.s_dip + sidx * D * D;  // [dv][dk], holds the prefix E[v k^T]
#pragma unroll
  for (int x = 0; x < TD; ++x)
#pragma unroll
    for (int y = 0; y < TD; ++y) {
      const size_t o = static_cast<size_t>(tr * TD + x) * D + (tc * TD + y);
      dip[o] = (dip[o] - acc[x][y]) * inv;
    }
}

// Exact softmax over the retrieved keys for the queries of bucket (b, i), merged into
// the far-field partial result (o_far, l_far). One thread per query, keys staged in LDS.
template <typename T, int D>
__global__ void __launch_bounds__(256) retr_exact_kernel(RetrArgs a) {
  constexpr int KCH = RetrChunk<D>::value;
  __shared__ float s_k[KCH * D];
  __shared__ float s_v[KCH * D];
  __shared__ int s_sel[kMaxRetrRow];
  const int i = blockIdx.x, b = blockIdx.y, bh = blockIdx.z;
  const int tid = threadIdx.x;
  if (b == 0) return;
  const int Ck = a.Ck, k1 = a.k1, k2 = a.k2, row = k1 * (1 + k2);
  const int32_t* sel = a.sel + ((static_cast<size_t>(bh) * a.nb + b) * a.Cq + i) * row;
  for (int x = tid; x < row; x += 256) s_sel[x] = sel[x];
  const int32_t* offq = a.offs_q + static_cast<size_t>(bh) * (a.nb * a.Cq + 1);
  const int q0 = offq[b * a.Cq + i], q1 = offq[b * a.Cq + i + 1];
  const T* Q = static_cast<const T*>(a.q) + static_cast<size_t>(bh) * a.N * D;
  const T* K = static_cast<const T*>(a.k) + static_cast<size_t>(bh) * a.N * D;
  const T* V = static_cast<const T*>(a.v) + static_cast<size_t>(bh) * a.N * D;
  const int32_t* permq = a.perm_q + static_cast<size_t>(bh) * a.N;
  const int32_t* permk = a.perm_k + static_cast<size_t>(bh) * a.N;
  const int32_t* offk = a.offs_k + static_cast<size_t>(bh) * (a.nb * Ck + 1);
  __syncthreads();
  for (int qb = q0; qb < q1; qb += 256) {
    const int qp = qb + tid;
    const bool valid = qp < q1;
    const int qn = valid ? permq[qp] : 0;
    float q[D];
#pragma unroll
    for (int d = 0; d < D; ++d) q[d] = a.scale * Elem<T>::load(Q, static_cast<size_t>(qn) * D + d);
    float m = kNegInf, l = 0.f;
    float acc[D];
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] = 0.f;
    for (int t = 0; t < k1; ++t) {
      const int j = s_sel[t * (1 + k2)];
      if (j < 0) continue;
      for (int u = 0; u < k2; ++u) {
        const int bb = s_sel[t * (1 + k2) + 1 + u];
        if (bb < 0) continue;
        const int p0 = offk[bb * Ck + j], p1 = offk[bb * Ck + j + 1];
        for (int c0 = p0; c0 < p1; c0 += KCH) {
          const int nk = min(KCH, p1 - c0);
          __syncthreads();
          for (int x = tid; x < nk * D; x += 256) {
            const int r = x / D, d = x % D;
            const size_t rowi = static_cast<size_t>(permk[c0 + r]) * D + d;
            s_k[x] = Elem<T>::load(K, rowi);
            s_v[x] = Elem<T>::load(V, rowi);
          }
          __syncthreads();
          for (int r = 0; r < nk; ++r) {
            float dot = 0.f;
#pragma unroll
            for (int d = 0; d < D; ++d) dot = fmaf(q[d], s_k[r * D + d], dot);
            if (dot > m) {
              const float f = m == kNegInf ? 0.f : __expf(m - dot);
              l *= f;
#pragma unroll
              for (int d = 0; d < D; ++d) acc[d] *= f;
              m = dot;
            }
            const float p = __expf(dot - m);
            l += p;
#pragma unroll
            for (int d = 0; d < D; ++d) acc[d] = fmaf(p, s_v[r * D + d], acc[d]);
          }
        }
      }
    }
    if (!valid || l == 0.f) continue;
    const size_t rowq = static_cast<size_t>(bh) * a.N + qn;
    const float LR = m + __logf(l);
    const float lf = a.l_far[rowq];
    const float Lt = lf == kNegInf ? LR : fmaxf(LR, lf) + __logf(1.f + __expf(-fabsf(LR - lf)));
    const float w0 = __expf(LR - Lt) / l;
    const float w1 = lf == kNegInf ? 0.f : __expf(lf - Lt);
#pragma unroll
    for (int d = 0; d < D; ++d) a.o_far[rowq * D + d] = w0 * acc[d] + w1 * a.o_far[rowq * D + d];
    a.l_far[rowq] = Lt;
  }
}

// Position pos of the concatenated retrieved ranges -> key row (head-local index).
__device__ __forceinline__ int retr_key_row(const int* s_start, const int* s_cum, int nr, const int32_t* permk,
                                            int pos) {
  int lo = 0, hi = nr - 1;  // last range with s_cum <= pos
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_cum[mid] <= pos) lo = mid;
    else hi = mid - 1;
  }
  return permk[s_start[lo] + pos - s_cum[lo]];
}

// Matrix-core exact part for bf16 inputs. One workgroup of 4 waves per stage-2 chunk (up
// to 128 queries of bucket (b, i)). With more than 64 queries, wave w takes queries
// 32 w .. + 31 and all keys; with at most 64 (the usual case), wave w takes queries
// 32 (w & 1) .. + 31 and, of every 64 staged keys, keys 32 (w >> 1) .. + 31, so that all
// four waves work. The retrieved keys are the concatenation of the
// chosen atoms' ranges of the key permutation; 64 at a time are gathered (16-byte row
// pieces) into one of two LDS buffers while the other is in use, one barrier per step.
// On the matrix cores
//   l^T = K q^T (32 keys x 32 queries; bf16 operands are exact, fp32 accumulation),
//   online softmax over the keys, O^T += V^T P^T (P split into bf16 hi + lo),
// and at the end the two key halves of each query group (when split) are merged by
// log-sum-exp and the result merged into the far field of the query.
template <int D>
struct RetrExactCfg {
  static constexpr int JC = 64, KST = D + 8, NKS = D / 16, NMT = D / 32;
  static constexpr int NK = JC * D / 8 / 256;  // 16-byte row pieces per thread and tensor
  static constexpr size_t lds_bytes = 2 * 2 * JC * KST * sizeof(uint16_t);
};

// D = 64: four workgroups per compute unit (128 registers, three of them spilled); the
// kernel waits on its gathers, so the extra workgroup in flight pays (6 % at 16k tokens
// against three workgroups without spills).
template <int D>
__global__ void __launch_bounds__(256, D == 64 ? 4 : 2) retr_exact_mfma_kernel(RetrArgs a) {
  using Cfg = RetrExactCfg<D>;
  constexpr int NKS = Cfg::NKS, NMT = Cfg::NMT, JC = Cfg::JC, KST = Cfg::KST, NK = Cfg::NK;
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t* sK = reinterpret_cast<uint16_t*>(smem);  // [2][JC * KST]
  uint16_t* sV = sK + 2 * JC * KST;                   // [2][JC * KST]
  __shared__ int s_start[kMaxRetrRow];    // first permutation position of each range
  __shared__ int s_cum[kMaxRetrRow + 1];  // exclusive prefix of the range lengths
  __shared__ int s_nr;
  const int bh = blockIdx.y, tix = blockIdx.x, tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, h = lane >> 5, c = lane & 31;
  if (tix >= a.ntiles[bh]) return;  // whole workgroup leaves together
  const int2 tile = a.tiles[static_cast<size_t>(bh) * a.max_tiles + tix];
  const int u = tile.x, b = u / a.Cq, i = u % a.Cq;
  if (b == 0) return;  // the first block retrieves nothing
  const int32_t* offq = a.offs_q + static_cast<size_t>(bh) * (a.nb * a.Cq + 1);
  const int qend = min(offq[u + 1], tile.y + kS2Chunk);  // this chunk's queries end here
  const bool split = qend - tile.y <= 64;                // uniform
  const int g = split ? wave & 1 : wave, kp = split ? wave >> 1 : 0;
  const int Ck = a.Ck, k1 = a.k1, k2 = a.k2, row = k1 * (1 + k2);
  if (wave == 0) {
    const int32_t* sel = a.sel + ((static_cast<size_t>(bh) * a.nb + b) * a.Cq + i) * row;
    const int32_t* offk = a.offs_k + static_cast<size_t>(bh) * (a.nb * Ck + 1);
    const int n = retr_ranges(sel, offk, Ck, k1, k2, s_start, s_cum);
    if (lane == 0) s_nr = n;
  }
  const int st = tile.y + 32 * g;
  const int nw = max(0, min(32, qend - st));  // queries of this wave
  const bool valid = c < nw;
  const int qn = a.perm_q[static_cast<size_t>(bh) * a.N + min(st + c, a.N - 1)];
  const size_t rowq = static_cast<size_t>(bh) * a.N + qn;
  // query fragments (B operand: column = query c, k = d); exact in bf16
  const uint16_t* Q = static_cast<const uint16_t*>(a.q);
  bf16x8_t qf[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) qf[ks] = as_bf16x8(*reinterpret_cast<const u16x8_t*>(Q + rowq * D + 16 * ks + 8 * h));
  __syncthreads();
  const int nr = s_nr, nR = s_cum[nr];
  if (nR == 0) return;  // nothing retrieved (uniform: read from LDS by every thread)
  const uint16_t* K = static_cast<const uint16_t*>(a.k) + static_cast<size_t>(bh) * a.N * D;
  const uint16_t* V = static_cast<const uint16_t*>(a.v) + static_cast<size_t>(bh) * a.N * D;
  const int32_t* permk = a.perm_k + static_cast<size_t>(bh) * a.N;
  // the gather runs two steps ahead in two stages: the key rows of step ch + 2 (loads of
  // the permutation) and the K, V rows of step ch + 1 are requested together, so that no
  // load waits on another inside a step
  int prow[NK];
  u16x8_t pk[NK], pv[NK];
  auto resolve = [&](int ch) {
#pragma unroll
    for (int q = 0; q < NK; ++q) {
      const int pos = ch * JC + (tid + 256 * q) / (D / 8);
      prow[q] = pos < nR ? retr_key_row(s_start, s_cum, nr, permk, pos) : -1;
    }
  };
  auto fetch = [&]() {
#pragma unroll
    for (int q = 0; q < NK; ++q) {
      const int d8 = ((tid + 256 * q) % (D / 8)) * 8;
      pk[q] = u16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
      pv[q] = pk[q];
      if (prow[q] >= 0) {
        const size_t kr = static_cast<size_t>(prow[q]) * D + d8;
        pk[q] = *reinterpret_cast<const u16x8_t*>(K + kr);
        pv[q] = *reinterpret_cast<const u16x8_t*>(V + kr);
      }
    }
  };
  auto store_chunk = [&](int buf) {
#pragma unroll
    for (int q = 0; q < NK; ++q) {
      const int x = tid + 256 * q, r = x / (D / 8), d8 = (x % (D / 8)) * 8;
      *reinterpret_cast<u16x8_t*>(sK + buf * JC * KST + r * KST + d8) = pk[q];
      *reinterpret_cast<u16x8_t*>(sV + buf * JC * KST + r * KST + d8) = pv[q];
    }
  };
  const int nch = (nR + JC - 1) / JC;
  resolve(0);
  fetch();
  store_chunk(0);
  if (nch > 1) resolve(1);
  __syncthreads();
  const float sl2 = a.scale * 1.4426950408889634f;
  float mx = kNegInf, z = 0.f;  // running max (log2 units) and sum of this lane pair's query
  f32x16_t o[NMT];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) o[mt] = zero16();
  for (int ch = 0; ch < nch; ++ch) {
    if (ch + 1 < nch) {  // in flight during this step
      fetch();
      if (ch + 2 < nch) resolve(ch + 2);
    }
    for (int sub = kp; sub < 2; sub += split ? 2 : 1) {
      const int k0 = ch * JC + 32 * sub;  // first of these 32 keys
      if (nw == 0 || k0 >= nR) break;
      const uint16_t* kt = sK + (ch & 1) * JC * KST + 32 * sub * KST;
      const uint16_t* vt = sV + (ch & 1) * JC * KST + 32 * sub * KST;
      // logits^T of the 32 keys (rows = keys, column = query), log2 units
      f32x16_t lg = zero16();
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        lg = mfma32(as_bf16x8(*reinterpret_cast<const u16x8_t*>(kt + c * KST + 16 * ks + 8 * h)), qf[ks], lg);
      float cm = kNegInf;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = k0 + 8 * (v >> 2) + 4 * h + (v & 3);
        const float x = key < nR ? sl2 * lg[v] : kNegInf;
        lg[v] = x;
        cm = fmaxf(cm, x);
      }
      cm = fmaxf(cm, xor32(cm));
      const float mn = fmaxf(mx, cm);  // finite: key k0 < nR is among the 32
      const float alpha = mx == kNegInf ? 0.f : fast_exp2(mx - mn);
      const bool grow = mn > mx && mx != kNegInf;
      mx = mn;
      float zs = 0.f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float p = fast_exp2(lg[v] - mn);
        lg[v] = p;
        zs += p;
      }
      z = z * alpha + zs + xor32(zs);
      if (__ballot(grow) != 0ull) {
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
          for (int v = 0; v < 16; ++v) o[mt][v] *= alpha;
      }
      // O^T += V^T P^T: k-slots of step ss are rows 16 ss + 4 h + 0..3 and 16 ss + 8 + 4 h + 0..3
#pragma unroll
      for (int ss = 0; ss < 2; ++ss) {
        float pv8[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) pv8[r] = lg[8 * ss + r];
        bf16x8_t phi, plo;
        split_bf16x8(pv8, phi, plo);
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) {
          const bf16x8_t hv = lds_operand_tr_acc(vt, KST, 16 * ss, 32 * mt, lane);
          o[mt] = mfma32(hv, phi, o[mt]);
          o[mt] = mfma32(hv, plo, o[mt]);
        }
      }
    }
    if (ch + 1 < nch) store_chunk((ch + 1) & 1);  // the buffer of step ch - 1, free since its barrier
    __syncthreads();
  }
  // split workgroups: merge the key halves of each query group, waves kp = 1 hand (max,
  // sum, O) over in LDS
  // (lane-major, so that the partner lane reads the same index)
  float* xo = reinterpret_cast<float*>(smem);  // [2][NMT][16][64]
  float* xm = xo + 2 * NMT * 16 * 64;         // [2][64]
  float* xz = xm + 2 * 64;                    // [2][64]
  if (split && kp == 1) {
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
      for (int v = 0; v < 16; ++v) xo[((g * NMT + mt) * 16 + v) * 64 + lane] = o[mt][v];
    xm[g * 64 + lane] = mx;
    xz[g * 64 + lane] = z;
  }
  __syncthreads();
  if (kp == 1 || !valid) return;
  if (split) {
    const float m1 = xm[g * 64 + lane], z1 = xz[g * 64 + lane];
    const float M = fmaxf(mx, m1);  // finite: this wave saw key 0
    const float f0 = fast_exp2(mx - M), f1 = m1 == kNegInf ? 0.f : fast_exp2(m1 - M);
    z = z * f0 + z1 * f1;
    mx = M;
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
      for (int v = 0; v < 16; ++v) o[mt][v] = o[mt][v] * f0 + xo[((g * NMT + mt) * 16 + v) * 64 + lane] * f1;
  }
  // merge with the far field of the query: L = log(e^LR + e^Lf), o = e^(LR-L) o_R + e^(Lf-L) o_f
  const float LR = (mx + __log2f(z)) * 0.6931471805599453f;
  const float lf = a.l_far[rowq];
  const float Lt = lf == kNegInf ? LR : fmaxf(LR, lf) + log1pf(__expf(-fabsf(LR - lf)));
  const float w0 = __expf(LR - Lt) / z, w1 = lf == kNegInf ? 0.f : __expf(lf - Lt);
  // lanes (c, h) hold rows d = 32 mt + 8 gg + 4 h + r of query c
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) {
      float* dst = a.o_far + rowq * D + 32 * mt + 8 * gg + 4 * h;
      const f32x4_t f = *reinterpret_cast<const f32x4_t*>(dst);
      f32x4_t r;
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = w0 * o[mt][4 * gg + e] + w1 * f[e];
      *reinterpret_cast<f32x4_t*>(dst) = r;
    }
  if (h == 0) a.l_far[rowq] = Lt;
}

// Second moment without the retrieved keys for bf16 inputs, one workgroup of 4 waves per
// (i, b): E_i[v k^T] of the entry becomes (E - sum_R w v k^T) / (1 - sum_R w), with
// w_m = exp(s qbar_i . k_m - R) relative to the prefix log mass R. The retrieved keys are
// gathered 64 at a time into one of two LDS buffers (K and V rows, exact in bf16) while
// the other is in use, one barrier per step; each key's weight comes from the D / 8
// threads that load its row (fp32 partial dots, summed across those lanes) and is staged
// beside the rows; sum_R (w v) k^T on the matrix cores with w v split into bf16 hi + lo.
template <int D>
struct RetrMomCfg {
  static constexpr int JC = 64, ST = D + 8, NDT = D / 32, TPW = NDT * NDT / 4, NP = JC * D / 8 / 256, TPR = D / 8;
  static constexpr size_t lds_bytes = 2 * 2 * JC * ST * sizeof(uint16_t) + 2 * JC * sizeof(float);
};

template <int D>
__global__ void __launch_bounds__(256) retr_moment_mfma_kernel(RetrArgs a) {
  using Cfg = RetrMomCfg<D>;
  constexpr int JC = Cfg::JC, ST = Cfg::ST, NDT = Cfg::NDT, TPW = Cfg::TPW, NP = Cfg::NP, TPR = Cfg::TPR;
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t* sK = reinterpret_cast<uint16_t*>(smem);       // [2][JC * ST]
  uint16_t* sV = sK + 2 * JC * ST;                         // [2][JC * ST]
  float* sW = reinterpret_cast<float*>(sV + 2 * JC * ST);  // [2][JC]
  __shared__ float s_red[1 + 4];
  __shared__ int s_start[kMaxRetrRow];
  __shared__ int s_cum[kMaxRetrRow + 1];
  __shared__ int s_nr;
  const int i = blockIdx.x, b = blockIdx.y, bh = blockIdx.z;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int h = lane >> 5;
  if (b == 0) return;
  const int Ck = a.Ck, k1 = a.k1, k2 = a.k2, row = k1 * (1 + k2);
  const size_t sidx = (static_cast<size_t>(bh) * a.nb + b) * a.Cq + i;
  if (wave == 0) {
    // prefix log mass of the entry
    float mx = kNegInf;
    for (int j = lane; j < Ck; j += 64) mx = fmaxf(mx, a.s_logz[sidx * Ck + j]);
    mx = wave_max(mx);
    float sm = 0.f;
    for (int j = lane; j < Ck; j += 64) {
      const float l = a.s_logz[sidx * Ck + j];
      if (l != kNegInf) sm += __expf(l - mx);
    }
    sm = wave_sum(sm);
    if (lane == 0) s_red[0] = mx == kNegInf ? kNegInf : mx + __logf(sm);
  } else if (wave == 1) {
    const int32_t* sel = a.sel + sidx * row;
    const int32_t* offk = a.offs_k + static_cast<size_t>(bh) * (a.nb * Ck + 1);
    const int n = retr_ranges(sel, offk, Ck, k1, k2, s_start, s_cum);
    if (lane == 0) s_nr = n;
  }
  // this thread's 8 features of s qbar_i (every row piece it loads starts at feature d8)
  const int d8 = (tid % TPR) * 8;
  float qs[8];
  {
    const float* qb = a.qbar + (static_cast<size_t>(bh) * a.Cq + i) * D + d8;
#pragma unroll
    for (int e = 0; e < 8; ++e) qs[e] = a.scale * qb[e];
  }
  __syncthreads();
  const float Rpre = s_red[0];
  const int nr = s_nr, nR = s_cum[nr];
  if (Rpre == kNegInf || nR == 0) return;  // uniform (LDS values)
  const uint16_t* K = static_cast<const uint16_t*>(a.k) + static_cast<size_t>(bh) * a.N * D;
  const uint16_t* V = static_cast<const uint16_t*>(a.v) + static_cast<size_t>(bh) * a.N * D;
  const int32_t* permk = a.perm_k + static_cast<size_t>(bh) * a.N;
  // the gather runs two steps ahead in two stages (key rows of step ch + 2, K and V rows
  // of step ch + 1, requested together)
  int prow[NP];
  u16x8_t pk[NP], pv[NP];
  auto resolve = [&](int ch) {
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      const int pos = ch * JC + (tid + 256 * q) / TPR;
      prow[q] = pos < nR ? retr_key_row(s_start, s_cum, nr, permk, pos) : -1;
    }
  };
  auto fetch = [&]() {
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      pk[q] = u16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
      pv[q] = pk[q];
      if (prow[q] >= 0) {
        const size_t kr = static_cast<size_t>(prow[q]) * D + d8;
        pk[q] = *reinterpret_cast<const u16x8_t*>(K + kr);
        pv[q] = *reinterpret_cast<const u16x8_t*>(V + kr);
      }
    }
  };
  float wsum = 0.f;  // lanes with tid % TPR == 0: their rows' weights
  auto store_chunk = [&](int ch) {
    const int buf = ch & 1;
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      const int r = (tid + 256 * q) / TPR;
      *reinterpret_cast<u16x8_t*>(sK + buf * JC * ST + r * ST + d8) = pk[q];
      *reinterpret_cast<u16x8_t*>(sV + buf * JC * ST + r * ST + d8) = pv[q];
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) dot = fmaf(qs[e], bf16_to_f32(pk[q][e]), dot);
#pragma unroll
      for (int o = 1; o < TPR; o <<= 1) dot += __shfl_xor(dot, o, 64);
      if (tid % TPR == 0) {
        const float w = ch * JC + r < nR ? __expf(dot - Rpre) : 0.f;
        sW[buf * JC + r] = w;
        wsum += w;
      }
    }
  };
  f32x16_t acc[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) acc[t] = zero16();
  const int nch = (nR + JC - 1) / JC;
  resolve(0);
  fetch();
  store_chunk(0);
  if (nch > 1) resolve(1);
  __syncthreads();
  for (int ch = 0; ch < nch; ++ch) {
    if (ch + 1 < nch) {  // in flight during this step
      fetch();
      if (ch + 2 < nch) resolve(ch + 2);
    }
    const int buf = ch & 1;
    const uint16_t* kt = sK + buf * JC * ST;
    const uint16_t* vt = sV + buf * JC * ST;
    const int nks = min(JC, nR - ch * JC + 15) / 16;  // 16-key steps holding retrieved keys
    for (int ks = 0; ks < nks; ++ks) {
      float pw[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) pw[q] = sW[buf * JC + 16 * ks + 8 * h + q];
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const int ot = wave * TPW + t, dvt = ot / NDT, dkt = ot % NDT;
        const u16x8_t vb = __builtin_bit_cast(u16x8_t, lds_operand_tr(vt, ST, 16 * ks, 32 * dvt, lane));
        float av[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) av[q] = bf16_to_f32(vb[q]) * pw[q];
        bf16x8_t ah, al;
        split_bf16x8(av, ah, al);
        const bf16x8_t kb = lds_operand_tr(kt, ST, 16 * ks, 32 * dkt, lane);
        acc[t] = mfma32(ah, kb, acc[t]);
        acc[t] = mfma32(al, kb, acc[t]);
      }
    }
    if (ch + 1 < nch) store_chunk(ch + 1);  // the buffer of step ch - 1, free since its barrier
    __syncthreads();
  }
  {
    const float ws = wave_sum(wsum);
    if (lane == 0) s_red[1 + wave] = ws;
  }
  __syncthreads();
  const float rest = 1.f - ((s_red[1] + s_red[2]) + (s_red[3] + s_red[4]));
  const float inv = rest > 1e-30f ? 1.f / rest : 0.f;
  float* dip = a.s_dip + sidx * D * D;  // [dv][dk], holds the prefix E[v k^T]
  // lanes (c, h) hold rows dv = 32 dvt + 8 (v / 4) + 4 h + v % 4 of column dk = 32 dkt + c
  const int c = lane & 31;
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int ot = wave * TPW + t, dvt = ot / NDT, dkt = ot % NDT;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const size_t o = static_cast<size_t>(32 * dvt + 8 * (v >> 2) + 4 * h + (v & 3)) * D + 32 * dkt + c;
      dip[o] = (dip[o] - acc[t][v]) * inv;
    }
  }
}

hipError_t launch_retrieval(const RetrArgs& a, int phase, int dtype, hipStream_t s) {
  const dim3 g(a.Cq, a.nb, a.BH);
  if (phase == 0) {
    {
      ProfScope ps_("retr_select", s);
      hipLaunchKernelGGL(retr_select_kernel, g, dim3(64), sizeof(float) * a.nb, s, a);
    }
    if (dtype == 1 && a.dipole) {
      ProfScope ps_("retr_moment_mfma", s);
      if (a.D == 64) {
        allow_lds((const void*)retr_moment_mfma_kernel<64>, RetrMomCfg<64>::lds_bytes);
        hipLaunchKernelGGL((retr_moment_mfma_kernel<64>), g, dim3(256), RetrMomCfg<64>::lds_bytes, s, a);
      } else {
        allow_lds((const void*)retr_moment_mfma_kernel<128>, RetrMomCfg<128>::lds_bytes);
        hipLaunchKernelGGL((retr_moment_mfma_kernel<128>), g, dim3(256), RetrMomCfg<128>::lds_bytes, s, a);
      }
    }
    ProfScope ps_("retr_tables", s);
    if (dtype == 0) {
      if (a.D == 64) hipLaunchKernelGGL((retr_tables_kernel<float, 64>), g, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((retr_tables_kernel<float, 128>), g, dim3(256), 0, s, a);
    } else {
      if (a.D == 64) hipLaunchKernelGGL((retr_tables_kernel<bf16, 64>), g, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((retr_tables_kernel<bf16, 128>), g, dim3(256), 0, s, a);
    }
  } else {
    ProfScope ps_("retr_exact", s);
    if (dtype == 1 && a.tiles != nullptr) {
      const dim3 gm(a.max_tiles, a.BH);
      if (a.D == 64) {
        allow_lds((const void*)retr_exact_mfma_kernel<64>, RetrExactCfg<64>::lds_bytes);
        hipLaunchKernelGGL((retr_exact_mfma_kernel<64>), gm, dim3(256), RetrExactCfg<64>::lds_bytes, s, a);
      } else {
        allow_lds((const void*)retr_exact_mfma_kernel<128>, RetrExactCfg<128>::lds_bytes);
        hipLaunchKernelGGL((retr_exact_mfma_kernel<128>), gm, dim3(256), RetrExactCfg<128>::lds_bytes, s, a);
      }
    } else if (dtype == 0) {
      if (a.D == 64) hipLaunchKernelGGL((retr_exact_kernel<float, 64>), g, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((retr_exact_kernel<float, 128>), g, dim3(256), 0, s, a);
    } else {
      if (a.D == 64) hipLaunchKernelGGL((retr_exact_kernel<bf16, 64>), g, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((retr_exact_kernel<bf16, 128>), g, dim3(256), 0, s, a);
    }
  }
  return hipGetLastError();
}

}  // namespace muse
