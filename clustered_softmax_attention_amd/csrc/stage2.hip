// Stage 2 of MuSe: each query refines its cluster's summaries with its residual
// (gist.science summary of arXiv 2509.10406, Kernmechanismen 1 "Decompositie" and
// 2 "Fase 2"; pith.science review, "What carries the argument").
//
// Query n in cluster i, residual qt = q_n - qbar_i, table entry e (its block for
// causal calls, 0 otherwise):
//   l_j = log Z_ij + s qt . K_ij,   p = softmax_j(l),   L_n = logsumexp_j l_j,
//   o_n = sum_j p_j V_ij + s D_i qt.
// bf16 inputs (s2_mfma): queries are bucketed by (block, cluster) and cut into chunks
// of up to 128 (a workgroup; 32 per wave); on the matrix cores
//   l^T = K_i qt^T (Ck x 32), P = softmax over the Ck rows, O^T = V_i^T P^T + (s D_i) qt^T,
// with K_i, qt, V_i and P split into bf16 hi + lo parts (three products hi*hi, hi*lo,
// lo*hi; error ~2^-16 relative) and the dipole product in plain bf16 (a small term).
// fp32 inputs (s2_refine): one wave per query; the logits with the lanes over key
// clusters (the residual broadcast from LDS), the weighted values with the lanes over
// dimensions, and the dipole row by row (lanes over the key dimension, a wave sum each).
// With the hierarchical decomposition (pith.science review, Figure 2 caption) a query of
// block b sees the entries e = b, b & (b - 1), ... > 0, one per square below the
// diagonal; their (o, L) are merged by log-sum-exp, L = log(e^L1 + e^L2),
// o = e^(L1 - L) o1 + e^(L2 - L) o2.
#include "mfma.hpp"
#include "muse_kernels.hpp"

namespace muse {

template <typename T, int D>
__global__ void __launch_bounds__(256) s2_refine_kernel(S2Args a) {
  constexpr int NP = D / 64;  // dimensions per lane
  __shared__ float s_qt[4][D];
  __shared__ float s_p[4][kMaxClusters];
  const int bh = blockIdx.y, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const long n = static_cast<long>(blockIdx.x) * 4 + wave;
  if (n >= a.N) return;  // the whole wave
  const int b = a.causal ? static_cast<int>(n / a.block) : 0;
  const size_t row = static_cast<size_t>(bh) * a.N + n;
  if (a.causal && b == 0) {  // no earlier block: empty far field
    if (lane == 0) a.l_far[row] = kNegInf;
#pragma unroll
    for (int q = 0; q < NP; ++q) a.o_far[row * D + lane + 64 * q] = 0.f;
    return;
  }
  const int i = a.labels_q[row];
  const T* Q = static_cast<const T*>(a.q);
  const float* qb = a.qbar + (static_cast<size_t>(bh) * a.Cq + i) * D;
  float qt[NP];
#pragma unroll
  for (int q = 0; q < NP; ++q) {
    const int d = lane + 64 * q;
    qt[q] = Elem<T>::load(Q, row * D + d) - qb[d];
    s_qt[wave][d] = qt[q];
  }
  const int Ck = a.Ck;
  int e = a.causal ? b : 0;
  for (bool first = true;; first = false) {
    const size_t sidx = (static_cast<size_t>(bh) * a.nbS + e) * a.Cq + i;
    const float* lz = a.s_logz + sidx * Ck;
    const float* Kt = a.s_k + sidx * Ck * D;
    const float* Vt = a.s_v + sidx * Ck * D;
    // logits: lanes over key clusters (row j of K_i read 16 bytes at a time)
    float l[2], mx = kNegInf;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int j = lane + 64 * t;
      l[t] = kNegInf;
      if (j < Ck && lz[j] != kNegInf) {
        float dot = 0.f;
        for (int d = 0; d < D; d += 4) {
          const f32x4_t k4 = *reinterpret_cast<const f32x4_t*>(Kt + static_cast<size_t>(j) * D + d);
          const f32x4_t q4 = *reinterpret_cast<const f32x4_t*>(&s_qt[wave][d]);
          dot = fmaf(q4[0], k4[0], fmaf(q4[1], k4[1], fmaf(q4[2], k4[2], fmaf(q4[3], k4[3], dot))));
        }
        l[t] = lz[j] + a.scale * dot;
      }
      mx = fmaxf(mx, l[t]);
    }
    mx = wave_max(mx);
    float z = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int j = lane + 64 * t;
      const float p = l[t] == kNegInf ? 0.f : __expf(l[t] - mx);
      z += p;
      if (j < Ck) s_p[wave][j] = p;
    }
    z = wave_sum(z);
    const bool empty = !(z > 0.f);  // no far-field key at all
    const float inv = empty ? 0.f : 1.f / z;
    // o = sum_j p_j V_ij: lanes over dimensions, clusters in order
    float acc[NP];
#pragma unroll
    for (int q = 0; q < NP; ++q) acc[q] = 0.f;
    for (int j = 0; j < Ck; ++j) {
      const float p = s_p[wave][j];
#pragma unroll
      for (int q = 0; q < NP; ++q) acc[q] = fmaf(p, Vt[static_cast<size_t>(j) * D + lane + 64 * q], acc[q]);
    }
#pragma unroll
    for (int q = 0; q < NP; ++q) acc[q] *= inv;
    if (a.dipole && !empty) {
      // s D_i qt: rows dv of D_i read whole (lanes over dk), one wave sum per row
      const float* dip = a.s_dip + sidx * D * D;  // [dv][dk]
      for (int dv = 0; dv < D; ++dv) {
        float part = 0.f;
#pragma unroll
        for (int q = 0; q < NP; ++q) part = fmaf(dip[static_cast<size_t>(dv) * D + lane + 64 * q], qt[q], part);
        part = wave_sum(part);
        if ((dv & 63) == lane) acc[dv >> 6] = fmaf(a.scale, part, acc[dv >> 6]);
      }
    }
    const float L = empty ? kNegInf : mx + __logf(z);
    if (a.causal && !first) {
      // a further square: merge into the far field written so far (this row)
      const float L0 = a.l_far[row];
      const float Ln = L0 == kNegInf ? L : (L == kNegInf ? L0 : fmaxf(L0, L) + log1pf(__expf(-fabsf(L0 - L))));
      const float w0 = L0 == kNegInf ? 0.f : __expf(L0 - Ln), w1 = L == kNegInf ? 0.f : __expf(L - Ln);
#pragma unroll
      for (int q = 0; q < NP; ++q) {
        float* o = a.o_far + row * D + lane + 64 * q;
        *o = w0 * *o + w1 * acc[q];
      }
      if (lane == 0) a.l_far[row] = Ln;
    } else if (a.causal) {
      if (lane == 0) a.l_far[row] = L;
#pragma unroll
      for (int q = 0; q < NP; ++q) a.o_far[row * D + lane + 64 * q] = acc[q];
    } else {
      if (a.lse_out && lane == 0) a.lse_out[row] = L;
#pragma unroll
      for (int q = 0; q < NP; ++q) {
        const size_t o = row * D + lane + 64 * q;
        if (a.out_bf16) static_cast<bf16*>(a.out)[o].bits = f32_to_bf16_bits(acc[q]);
        else static_cast<float*>(a.out)[o] = acc[q];
      }
    }
    e = a.hier ? (e & (e - 1)) : 0;
    if (e == 0) break;
  }
}

// Matrix-core stage 2: one workgroup of 4 waves per chunk of up to 128 queries of one
// bucket (wave w: queries 32 w .. 32 w + 31 of the chunk). The bucket's tables stream
// through LDS in chunks of 32 key clusters (cooperative 16-byte loads, the next chunk in
// registers while the current one is used), with an online softmax across chunks.
// LDS: K hi/lo, V hi/lo [32][D+16] row-major | log Z [32] | s D_i [D][D+8] (bf16); the
// V^T operand of O^T = V^T P^T comes from the row-major V rows by the transpose read in
// the key order of the P accumulator.
template <int D>
struct S2Cfg {
  static constexpr int JC = 32;
  static constexpr int KST = D + 16;
  static constexpr int DST = D + 8;
  static constexpr int NK = JC * D / 8 / 256;   // 16-byte K (and V) pieces per thread and part (hi, lo)
  static constexpr int ND = D * D / 8 / 256;    // 16-byte dipole pieces per thread
};

// HIER: one further square of the hierarchy per launch: entry e = b with its lowest set
// bit cleared `level` times (blocks with fewer squares leave at once), merged by
// log-sum-exp into the far field the earlier launches wrote (o_far, l_far); the first
// square of every block is the single entry of the HIER = false instance.
template <int D, bool HIER>
__global__ void __launch_bounds__(256, D == 64 ? 3 : 2) s2_mfma_kernel(S2Args a) {
  using Cfg = S2Cfg<D>;
  constexpr int NKS = D / 16, NMT = D / 32, JC = Cfg::JC, KST = Cfg::KST, DST = Cfg::DST;
  constexpr int NK = Cfg::NK, ND = Cfg::ND;
  __shared__ __align__(16) uint16_t sKh[JC * KST];
  __shared__ __align__(16) uint16_t sKl[JC * KST];
  __shared__ __align__(16) uint16_t sVh[JC * KST];
  __shared__ __align__(16) uint16_t sVl[JC * KST];
  __shared__ __align__(16) uint16_t sDip[D * DST];
  __shared__ float slz[JC];
  // acausal: the chunks of one query cluster (consecutive in the chunk order) read the
  // same tables, so each XCD takes a contiguous range of (head, chunk); causal tables
  // are per (block, cluster), read by about one chunk each, and stay round-robin
  const int lin0 = blockIdx.x + gridDim.x * blockIdx.y;
  const int lin = a.nbS == 1 ? xcd_contiguous(lin0, gridDim.x * gridDim.y) : lin0;
  const int bh = lin / gridDim.x, tix = lin % gridDim.x, tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, h = lane >> 5, c = lane & 31;
  if (tix >= a.ntiles[bh]) return;  // whole workgroup leaves together
  const int2 tile = a.tiles[static_cast<size_t>(bh) * a.max_tiles + tix];
  const int u = tile.x, b = u / a.Cq, i = u % a.Cq;
  const int32_t* offs = a.offs_q + static_cast<size_t>(bh) * (a.nb * a.Cq + 1);
  const int st = tile.y + 32 * wave;
  // the permutation entry is requested beside the bucket end, not after it (past the
  // bucket it is a neighbour's entry, which no lane uses): one dependent round trip fewer
  const int qn = a.perm_q[static_cast<size_t>(bh) * a.N + min(st + c, a.N - 1)];
  const int nw = max(0, min(32, offs[u + 1] - st));  // queries of this wave
  const bool valid = c < nw;
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
  // the table entry: e = b (acausal: 0), or the level-th square of the block's chain
  int e = a.causal ? b : 0;
  if (HIER) {
    for (int t = 0; t < a.level; ++t) e &= e - 1;
    if (e == 0) return;  // fewer squares: the whole workgroup leaves together
  }
  const int Ck = a.Ck, njc = (Ck + JC - 1) / JC;
  const uint16_t *khi, *klo, *vhi, *vlo, *dip;
  const float* lz;
  auto set_entry = [&](int ee) {
    const size_t sidx = (static_cast<size_t>(bh) * a.nbS + ee) * a.Cq + i;
    khi = a.t_khi + sidx * Ck * D;
    klo = a.t_klo + sidx * Ck * D;
    vhi = a.t_vhi + sidx * Ck * D;
    vlo = a.t_vlo + sidx * Ck * D;
    dip = a.t_dip + sidx * D * D;
    lz = a.s_logz + sidx * Ck;
  };
  set_entry(e);

  // chunk jc of the tables into registers
  u16x8_t pkh[NK], pkl[NK], pvh[NK], pvl[NK];
  float plz = kNegInf;
  auto load_chunk = [&](int jc) {
    const int j0 = jc * JC;
#pragma unroll
    for (int q = 0; q < NK; ++q) {
      const int x = tid + 256 * q, jj = x / (D / 8), d8 = (x % (D / 8)) * 8;
      pkh[q] = u16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
      pkl[q] = pkh[q];
      pvh[q] = pkh[q];
      pvl[q] = pkh[q];
      if (j0 + jj < Ck) {
        const size_t o = static_cast<size_t>(j0 + jj) * D + d8;
        pkh[q] = *reinterpret_cast<const u16x8_t*>(khi + o);
        pkl[q] = *reinterpret_cast<const u16x8_t*>(klo + o);
        pvh[q] = *reinterpret_cast<const u16x8_t*>(vhi + o);
        pvl[q] = *reinterpret_cast<const u16x8_t*>(vlo + o);
      }
    }
    plz = (tid < JC && j0 + tid < Ck) ? lz[j0 + tid] : kNegInf;
  };
  u16x8_t pd[ND];
  auto load_dip = [&]() {
    if (a.dipole) {
#pragma unroll
      for (int q = 0; q < ND; ++q) {
        const int x = tid + 256 * q, r = x / (D / 8), c8 = (x % (D / 8)) * 8;
        pd[q] = *reinterpret_cast<const u16x8_t*>(dip + static_cast<size_t>(r) * D + c8);
      }
    }
  };
  auto store_dip = [&]() {
    if (a.dipole) {
#pragma unroll
      for (int q = 0; q < ND; ++q) {
        const int x = tid + 256 * q, r = x / (D / 8), c8 = (x % (D / 8)) * 8;
        *reinterpret_cast<u16x8_t*>(sDip + r * DST + c8) = pd[q];
      }
    }
  };
  load_chunk(0);
  load_dip();

  // residual query fragments (B operand: column = query c, k = d); the rows are requested
  // before any of the loads above is waited for
  const uint16_t* Q = static_cast<const uint16_t*>(a.q);
  const float* qb = a.qbar + (static_cast<size_t>(bh) * a.Cq + i) * D;
  u16x8_t qr[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) qr[ks] = *reinterpret_cast<const u16x8_t*>(Q + row * D + 16 * ks + 8 * h);
  store_dip();
  // (the centroid's elements are loaded unconditionally, as whole vectors: a load under
  // the lane's validity would be issued and waited for one element at a time)
  bf16x8_t qhi[NKS], qlo[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    const int d0 = 16 * ks + 8 * h;
    const f32x4_t c0 = *reinterpret_cast<const f32x4_t*>(qb + d0);
    const f32x4_t c1 = *reinterpret_cast<const f32x4_t*>(qb + d0 + 4);
    const float cb[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
    float x[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) x[r] = valid ? bf16_to_f32(qr[ks][r]) - cb[r] : 0.f;
    split_bf16x8(x, qhi[ks], qlo[ks]);
  }

  const float sl2 = a.scale * 1.4426950408889634f;
  {
    float mx = kNegInf, z = 0.f;  // running max (log2 units) and sum of this lane pair's query
    f32x16_t o[NMT];
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) o[mt] = zero16();
    for (int jc = 0; jc < njc; ++jc) {
      __syncthreads();  // previous chunk consumed
#pragma unroll
      for (int q = 0; q < NK; ++q) {
        const int x = tid + 256 * q, jj = x / (D / 8), d8 = (x % (D / 8)) * 8;
        *reinterpret_cast<u16x8_t*>(sKh + jj * KST + d8) = pkh[q];
        *reinterpret_cast<u16x8_t*>(sKl + jj * KST + d8) = pkl[q];
        *reinterpret_cast<u16x8_t*>(sVh + jj * KST + d8) = pvh[q];
        *reinterpret_cast<u16x8_t*>(sVl + jj * KST + d8) = pvl[q];
      }
      if (tid < JC) slz[tid] = plz;
      __syncthreads();
      if (jc + 1 < njc) load_chunk(jc + 1);
      if (nw == 0) continue;
      // logits^T of the chunk (rows j, column = query), log2 units
      f32x16_t lg = zero16();
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const bf16x8_t ah = as_bf16x8(*reinterpret_cast<const u16x8_t*>(sKh + c * KST + 16 * ks + 8 * h));
        const bf16x8_t al = as_bf16x8(*reinterpret_cast<const u16x8_t*>(sKl + c * KST + 16 * ks + 8 * h));
        lg = mfma32(ah, qhi[ks], lg);
        lg = mfma32(ah, qlo[ks], lg);
        lg = mfma32(al, qhi[ks], lg);
      }
      float cm = kNegInf;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4_t l4 = *reinterpret_cast<const f32x4_t*>(slz + 8 * g + 4 * h);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float l0 = l4[r];
          const float x = l0 == kNegInf ? kNegInf : l0 * 1.4426950408889634f + sl2 * lg[4 * g + r];
          lg[4 * g + r] = x;
          cm = fmaxf(cm, x);
        }
      }
      cm = fmaxf(cm, xor32(cm));
      const float mn = fmaxf(mx, cm);
      if (mn == kNegInf) continue;  // no key cluster yet: nothing to add (same for the lane pair)
      const float alpha = mx == kNegInf ? 0.f : fast_exp2(mx - mn);
      // the sums need rescaling only when a lane's running max grew and it had summed before
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
      // O^T += V^T P^T (split): k-slots of step ss are rows 16 ss + 4 h + 0..3 and 16 ss + 8 + 4 h + 0..3
#pragma unroll
      for (int ss = 0; ss < 2; ++ss) {
        float pv[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) pv[r] = lg[8 * ss + r];
        bf16x8_t phi, plo;
        split_bf16x8(pv, phi, plo);
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) {
          const bf16x8_t hv = lds_operand_tr_acc(sVh, KST, 16 * ss, 32 * mt, lane);
          const bf16x8_t lv = lds_operand_tr_acc(sVl, KST, 16 * ss, 32 * mt, lane);
          o[mt] = mfma32(hv, phi, o[mt]);
          o[mt] = mfma32(hv, plo, o[mt]);
          o[mt] = mfma32(lv, phi, o[mt]);
        }
      }
    }
    if (nw > 0) {
      const float invz = z > 0.f ? 1.f / z : 0.f;  // z == 0: no far-field key at all
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[mt][v] *= invz;
      if (a.dipole) {
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) {
            const u16x8_t ad = *reinterpret_cast<const u16x8_t*>(sDip + (32 * mt + c) * DST + 16 * ks + 8 * h);
            o[mt] = mfma32(as_bf16x8(ad), qhi[ks], o[mt]);
          }
      }
      float L = z > 0.f ? (mx + __log2f(z)) * 0.6931471805599453f : kNegInf;
      // lanes (c, h) hold rows d = 32 mt + 8 g + 4 h + r of query c
      if (valid && HIER) {
        // log-sum-exp merge of this square into the far field of the earlier launches
        const float L0 = a.l_far[row];
        const float Ln = L0 == kNegInf ? L : (L == kNegInf ? L0 : fmaxf(L0, L) + log1pf(__expf(-fabsf(L0 - L))));
        const float w0 = L0 == kNegInf ? 0.f : __expf(L0 - Ln), w1 = L == kNegInf ? 0.f : __expf(L - Ln);
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x4_t f = *reinterpret_cast<const f32x4_t*>(a.o_far + row * D + 32 * mt + 8 * g + 4 * h);
#pragma unroll
            for (int r = 0; r < 4; ++r) o[mt][4 * g + r] = w0 * f[r] + w1 * o[mt][4 * g + r];
          }
        L = Ln;
      }
      if (valid && a.causal) {
        if (h == 0) a.l_far[row] = L;
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x4_t f = {o[mt][4 * g], o[mt][4 * g + 1], o[mt][4 * g + 2], o[mt][4 * g + 3]};
            *reinterpret_cast<f32x4_t*>(a.o_far + row * D + 32 * mt + 8 * g + 4 * h) = f;
          }
      } else if (valid) {
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
  }
}

hipError_t launch_stage2(const S2Args& a, int dtype, hipStream_t s) {
  if (dtype == 1) {
    ProfScope ps_("s2_mfma", s);
    const dim3 gm(a.max_tiles, a.BH);
    if (a.D == 64) {
      hipLaunchKernelGGL((s2_mfma_kernel<64, false>), gm, dim3(256), 0, s, a);
    } else {
      hipLaunchKernelGGL((s2_mfma_kernel<128, false>), gm, dim3(256), 0, s, a);
    }
    if (a.causal && a.hier) {
      // the further squares of the hierarchy, one chain level per launch (at most the bit
      // length of nb - 1 squares per block)
      int levels = 0;
      for (int x = a.nb - 1; x > 0; x >>= 1) ++levels;
      S2Args al = a;
      for (int lv = 1; lv < levels; ++lv) {
        al.level = lv;
        if (a.D == 64) hipLaunchKernelGGL((s2_mfma_kernel<64, true>), gm, dim3(256), 0, s, al);
        else hipLaunchKernelGGL((s2_mfma_kernel<128, true>), gm, dim3(256), 0, s, al);
      }
    }
    return hipGetLastError();
  }
  const dim3 g((a.N + 3) / 4, a.BH);  // a wave per query
  ProfScope ps_("s2_refine", s);
  if (dtype == 0) {
    if (a.D == 64) hipLaunchKernelGGL((s2_refine_kernel<float, 64>), g, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((s2_refine_kernel<float, 128>), g, dim3(256), 0, s, a);
  } else {
    if (a.D == 64) hipLaunchKernelGGL((s2_refine_kernel<bf16, 64>), g, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((s2_refine_kernel<bf16, 128>), g, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace muse
