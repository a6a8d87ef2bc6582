// Matrix-core stage 1 for bf16 inputs (gfx950).
//
// The quantities are those of stage1.hip (pith.science review of arXiv 2509.10406,
// "What carries the argument"): for query centroid qbar_i and key m,
// a_im = s qbar_i . k_m; per (i, key cluster j, block b') the atom (max, sum exp, sum
// exp k, sum exp v); per (i, moment sub-block) the normalised sum w v k^T and its log
// mass. Here:
// Keys are visited in bucketed order (the key permutation sorted by block, then key
// cluster), so that a bucket, a block and a moment sub-block are contiguous ranges of
// positions:
//   s1_scores      a_i(pos) = s qbar_i . k_perm[pos] for every centroid and position,
//                  [BH, Cq, N] fp32 (qbar split into bf16 hi + lo; keys are exact).
//   s1_atoms_mfma  one wave per work item (a run of at most kAtomSeg positions of one
//                  (block, key cluster) bucket; s1_atoms_merge folds the items of a
//                  bucket): the item's scores
//                  recomputed on the matrix cores in steps of 32 keys (keys as rows, so
//                  the max is lane-local, online across steps), and sum w k, sum w v as
//                  K^T W, V^T W with the weight accumulator as B operand and the key and
//                  value rows read from a row-major LDS tile by the transpose read.
//   s1_moments_f16 per (key range, centroid group): weights w = exp(a - max) from the
//                  scores (no running rescale), then sum_m w_m v_m k_m^T with fp16
//                  operands (the weights are applied to the value fragments with packed
//                  fp16 multiplies) and fp32 accumulation.
//   s1_finalize_acausal, s1_causal_scan  the tables of stage 2 (acausal: one entry;
//                  causal: every block's prefix), below.
//   s1_dip_final_mfma  the dipole and bf16 tables of one entry on the general path
//                  (retrieval, hierarchy), from the folded atoms and moments.
#include "mfma.hpp"
#include "muse_kernels.hpp"

#include <algorithm>

namespace muse {

typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;

__device__ __forceinline__ f32x16_t mfma32_f16(const f16x8_t& a, const f16x8_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// sc * qbar of the head split into bf16 hi + lo rows of stride QST, padded with zero rows
// to Cqp; every thread's elements are requested before any is stored (eight at a time,
// clamped indices), so that the staging costs one memory round trip, not one per element.
template <int D, int NT>
__device__ __forceinline__ void stage_qbar_split(const float* qb, int Cq, int Cqp, float sc, uint16_t* qhi,
                                                 uint16_t* qlo, int QST, int tid) {
  const int n = Cqp * D, nv = Cq * D;
  for (int x0 = tid; x0 < n; x0 += 8 * NT) {
    float v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = qb[min(x0 + NT * q, nv - 1)];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int x = x0 + NT * q;
      if (x < n) {
        const int i = x / D, d = x % D;
        const float y = i < Cq ? sc * v[q] : 0.f;
        const uint16_t hv = f32_to_bf16_bits(y);
        qhi[i * QST + d] = hv;
        qlo[i * QST + d] = f32_to_bf16_bits(y - bf16_to_f32(hv));
      }
    }
  }
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
  const uint16_t* K = static_cast<const uint16_t*>(a.k) + static_cast<size_t>(bh) * a.N * D;
  const int32_t* perm = a.perm_k + static_cast<size_t>(bh) * a.N;
  float* S = a.scores + static_cast<size_t>(bh) * Cq * a.N;
  // the key rows of this wave's two 32-position tiles are requested before the centroids
  // are staged (permutation entries of both tiles, then their rows), one round trip each
  int keys[2];
  bf16x8_t ak2[2][NKS];
  // (unconditional loads with clamped positions, so that they issue back to back; the
  // rows past the end are masked below)
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) keys[tt] = perm[min(static_cast<int>(blockIdx.x) * 256 + wave * 64 + tt * 32 + c, a.N - 1)];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      ak2[tt][ks] = as_bf16x8(*reinterpret_cast<const u16x8_t*>(K + static_cast<size_t>(keys[tt]) * D + 16 * ks + 8 * h));
  stage_qbar_split<D, 256>(a.qbar + static_cast<size_t>(bh) * Cq * D, Cq, Cqp, 1.f, qhi, qlo, QST, tid);
  __syncthreads();
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int kb = blockIdx.x * 256 + wave * 64 + tt * 32;  // first position of the tile
    if (kb >= a.N) break;
    const int pos = kb + c;
    const int key = keys[tt];
    // bit p of dmask: position kb + p is left out by a cluster size cap (score -inf)
    const bool drop = a.kdrop != nullptr && pos < a.N && a.kdrop[static_cast<size_t>(bh) * a.N + key] != 0;
    const uint32_t dmask = static_cast<uint32_t>(__ballot(drop));
    const bf16x8_t* ak = ak2[tt];
    for (int nt = 0; nt < nt_n; ++nt) {
      f32x16_t acc = zero16();
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int o = (32 * nt + c) * QST + 16 * ks + 8 * h;
        acc = mfma32(ak[ks], as_bf16x8(*reinterpret_cast<const u16x8_t*>(qhi + o)), acc);
        acc = mfma32(ak[ks], as_bf16x8(*reinterpret_cast<const u16x8_t*>(qlo + o)), acc);
      }
      // lane (c, h): centroid 32 nt + c, positions kb + 8 g + 4 h + r; the max over the
      // tile's 32 positions goes to tmax (position ranges of the moments are whole tiles)
      const int i = 32 * nt + c;
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          acc[4 * g + r] *= a.scale;
          if ((dmask >> (8 * g + 4 * h + r)) & 1u) acc[4 * g + r] = kNegInf;
        }
      float tm = kNegInf;
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (kb + 8 * g + 4 * h + r < a.N) tm = fmaxf(tm, acc[4 * g + r]);
      tm = fmaxf(tm, xor32(tm));
      if (i >= Cq) continue;
      if (h == 0) a.tmax[(static_cast<size_t>(bh) * Cq + i) * ((a.N + 31) / 32) + kb / 32] = tm;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int k0 = kb + 8 * g + 4 * h;
        if (k0 + 3 < a.N) {
          const f32x4_t f = {acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]};
          *reinterpret_cast<f32x4_t*>(S + static_cast<size_t>(i) * a.N + k0) = f;
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (k0 + r < a.N) S[static_cast<size_t>(i) * a.N + k0 + r] = acc[4 * g + r];
        }
      }
    }
  }
}

constexpr int kAtomChunk = 32;  // positions per step
constexpr int kMergeGrid = 64;  // merge workgroups per head (each loops over the multi-item buckets)
constexpr int kFinQB = 4;       // work items of a bucket folded per batch by the acausal finalise

// Atoms over work items (a run of at most kAtomSeg positions of one (block, key cluster)
// bucket), for every query centroid in tiles of 32. A wave takes `ipw` consecutive items
// (chosen by the launcher from the item count: one for a few hundred items per head,
// more when there are thousands of small buckets) as one pipeline: while a step of 32 keys is on the
// matrix cores, the rows of the next step (of this item or the next) are in flight, and
// the permutation entries of the item after next are gathered (lane l holds position l
// of its item; the row loads take them by lane shuffle). The workgroup first stages
// s qbar (split into bf16 hi + lo) in LDS for its four waves. Per step, rows gathered into
// a wave-private row-major LDS tile give on the matrix cores
//   S = K_step (s qbar)^T   (32 keys x 32 centroids; keys exact),
// so that lane (c, h) holds 16 keys of centroid c and the max over the item is
// lane-local plus the partner lane l^32 (online across steps, sums rescaled when it
// grows). The weights w = exp(S - max), split into hi + lo, are directly the B operand
// of  sum w k = K^T W  and  sum w v = V^T W,  whose A operands come from the same LDS
// tile through the transpose read in the accumulator's key order. A bucket of one item
// writes its atom; the items of a larger bucket write partial atoms that are folded
// later (s1_atoms_merge, or the acausal finalise).
template <int D>
__global__ void __launch_bounds__(256, D == 64 ? 3 : 1) s1_atoms_mfma_kernel(S1Args a, int ipw) {
  constexpr int NKS = D / 16, NMT = D / 32, KC = kAtomChunk, ST = D + 8, QST = D + 8;
  constexpr int NP = KC * (D / 8) / 64;  // 16-byte row pieces per lane and tensor
  static_assert(kAtomSeg <= 64, "one permutation entry per lane");
  __shared__ __align__(16) uint16_t sK[4][KC * ST];
  __shared__ __align__(16) uint16_t sV[4][KC * ST];
  extern __shared__ __align__(16) uint16_t sq[];  // s qbar hi, lo [Cqp][QST]
  const int bh = blockIdx.y, tid = threadIdx.x, lane = tid & 63, h = lane >> 5, c = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int Cq = a.Cq, Ck = a.Ck, nbC = a.nb * Ck, Cqp = (Cq + 31) & ~31;
  const int max_items = atom_max_items(nbC, a.N);
  const int g0 = (blockIdx.x * 4 + wave) * ipw;  // first item of this wave
  const int4* items = a.items_k + static_cast<size_t>(bh) * max_items;
  const int32_t* perm = a.perm_k + static_cast<size_t>(bh) * a.N;
  auto header = [&](int r) { return r < ipw && g0 + r < max_items ? items[g0 + r] : make_int4(0, -1, -1, 0); };
  auto gather = [&](const int4& hd) { return lane < hd.y ? perm[hd.x + lane] : 0; };
  int4 hd = header(0), hd_nx = header(1);
  int pl = gather(hd), pl_nx = gather(hd_nx);
  uint16_t* qhi = sq;
  uint16_t* qlo = sq + Cqp * QST;
  stage_qbar_split<D, 256>(a.qbar + static_cast<size_t>(bh) * Cq * D, Cq, Cqp, a.scale, qhi, qlo, QST, tid);
  __syncthreads();
  if (hd.y < 0) return;  // no item (padding); no workgroup barrier below
  const uint16_t* K = static_cast<const uint16_t*>(a.k) + static_cast<size_t>(bh) * a.N * D;
  const uint16_t* V = static_cast<const uint16_t*>(a.v) + static_cast<size_t>(bh) * a.N * D;
  uint16_t* kt = sK[wave];
  uint16_t* vt = sV[wave];
  auto wave_sync = [] {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  u16x8_t pk[NP], pv[NP];
  // rows p0 .. p0 + 31 of an item whose permutation entries are in pls
  auto load_rows = [&](int pls, int n, int p0) {
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      const int x = lane + 64 * q, r = x / (D / 8), c8 = (x % (D / 8)) * 8;
      const int key = __shfl(pls, p0 + r, 64);
      pk[q] = u16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
      pv[q] = pk[q];
      if (p0 + r < n) {
        const size_t row = static_cast<size_t>(key) * D + c8;
        pk[q] = *reinterpret_cast<const u16x8_t*>(K + row);
        pv[q] = *reinterpret_cast<const u16x8_t*>(V + row);
      }
    }
  };
  for (int nt = 0; nt < Cqp / 32; ++nt) {
    const int i = 32 * nt + c;
    if (nt > 0) {  // the pipeline restarts for each tile of 32 centroids
      hd = header(0);
      hd_nx = header(1);
      pl = gather(hd);
      pl_nx = gather(hd_nx);
    }
    if (hd.y > 0) load_rows(pl, hd.y, 0);
    for (int r = 0; r < ipw; ++r) {
      if (hd.y < 0) break;  // padding items end the list
      const int n = hd.y, u = hd.w, bp = u / Ck, j = u % Ck;
      f32x16_t ak[NMT], av[NMT];
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) {
        ak[mt] = zero16();
        av[mt] = zero16();
      }
      float mx = kNegInf, z = 0.f;
      for (int p0 = 0; p0 < n; p0 += KC) {
        wave_sync();  // the previous step's tiles are consumed
#pragma unroll
        for (int q = 0; q < NP; ++q) {
          const int x = lane + 64 * q, rr = x / (D / 8), c8 = (x % (D / 8)) * 8;
          *reinterpret_cast<u16x8_t*>(kt + rr * ST + c8) = pk[q];
          *reinterpret_cast<u16x8_t*>(vt + rr * ST + c8) = pv[q];
        }
        wave_sync();
        // the next step's rows in flight: this item's, or the next item's first
        if (p0 + KC < n) load_rows(pl, n, p0 + KC);
        else if (hd_nx.y > 0) load_rows(pl_nx, hd_nx.y, 0);
        f32x16_t sc = zero16();
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const bf16x8_t ka = as_bf16x8(*reinterpret_cast<const u16x8_t*>(kt + c * ST + 16 * ks + 8 * h));
          const int qo = (32 * nt + c) * QST + 16 * ks + 8 * h;
          sc = mfma32(ka, as_bf16x8(*reinterpret_cast<const u16x8_t*>(qhi + qo)), sc);
          sc = mfma32(ka, as_bf16x8(*reinterpret_cast<const u16x8_t*>(qlo + qo)), sc);
        }
        // rows of sc: keys p0 + 8 (v/4) + 4 h + v%4
        float cm = kNegInf;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = p0 + 8 * (v >> 2) + 4 * h + (v & 3);
          if (key >= n) sc[v] = kNegInf;
          cm = fmaxf(cm, sc[v]);
        }
        cm = fmaxf(cm, xor32(cm));
        if (cm > mx) {  // the same for the lane pair
          const float f = mx == kNegInf ? 0.f : __expf(mx - cm);
          z *= f;
#pragma unroll
          for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              ak[mt][v] *= f;
              av[mt][v] *= f;
            }
          mx = cm;
        }
        float w[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          w[v] = __expf(sc[v] - mx);
          z += w[v];
        }
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          bf16x8_t whi, wlo;
          split_bf16x8(w + 8 * s, whi, wlo);
#pragma unroll
          for (int mt = 0; mt < NMT; ++mt) {
            const bf16x8_t kf = lds_operand_tr_acc(kt, ST, 16 * s, 32 * mt, lane);
            const bf16x8_t vf = lds_operand_tr_acc(vt, ST, 16 * s, 32 * mt, lane);
            ak[mt] = mfma32(kf, whi, ak[mt]);
            ak[mt] = mfma32(kf, wlo, ak[mt]);
            av[mt] = mfma32(vf, whi, av[mt]);
            av[mt] = mfma32(vf, wlo, av[mt]);
          }
        }
      }
      // an empty item issued no rows for the next one
      if (n == 0 && hd_nx.y > 0) load_rows(pl_nx, hd_nx.y, 0);
      z += xor32(z);
      if (i < Cq) {
        // the bucket's atom, or the item's partial when the bucket has several items
        const bool part = hd.z >= 0;
        const size_t aidx = part ? (static_cast<size_t>(bh) * atom_max_partials(a.N) + hd.z) * Cq + i
                                 : ((static_cast<size_t>(bh) * a.nb + bp) * Cq + i) * Ck + j;
        float* out_k = part ? a.pt_k : a.at_k;
        float* out_v = part ? a.pt_v : a.at_v;
        if (h == 0) {
          (part ? a.pt_m : a.at_m)[aidx] = n > 0 ? mx : kNegInf;
          (part ? a.pt_z : a.at_z)[aidx] = z;
        }
        // lane (c, h): column = centroid i, rows d = 32 mt + 8 g + 4 h + r
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int d0 = 32 * mt + 8 * g4 + 4 * h;
            const f32x4_t fk = {ak[mt][4 * g4], ak[mt][4 * g4 + 1], ak[mt][4 * g4 + 2], ak[mt][4 * g4 + 3]};
            const f32x4_t fv = {av[mt][4 * g4], av[mt][4 * g4 + 1], av[mt][4 * g4 + 2], av[mt][4 * g4 + 3]};
            *reinterpret_cast<f32x4_t*>(out_k + aidx * D + d0) = fk;
            *reinterpret_cast<f32x4_t*>(out_v + aidx * D + d0) = fv;
          }
      }
      // advance: the next item becomes current, the one after it is gathered
      hd = hd_nx;
      pl = pl_nx;
      hd_nx = header(r + 2);
      pl_nx = gather(hd_nx);
    }
  }
}

// Buckets of several work items: the items' partial atoms folded in item order with the
// log-sum-exp rule (running max M, sums rescaled by exp(m - M)) into the bucket's atom.
// kMergeGrid workgroups of NT threads per head walk the list of such buckets (NT = 512
// when the Cq D / 2 pairs fit, else 1024); threads over the (centroid, float4 of the K
// and V sums) pairs, four items per batch with all of a batch's loads in flight (one
// batch for buckets of up to 4 kAtomSeg keys).
template <int D, int NT>
__global__ void __launch_bounds__(NT) s1_atoms_merge_kernel(S1Args a) {
  constexpr int F4 = D / 2;  // float4s of one centroid's K and V sums
  constexpr int QB = 4;
  const int bh = blockIdx.y, tid = threadIdx.x;
  const int Cq = a.Cq, Ck = a.Ck;
  const int4* multi = a.multi_k + static_cast<size_t>(bh) * (1 + atom_max_multi(a.N));
  const float* __restrict__ pm = a.pt_m;
  const float* __restrict__ pz = a.pt_z;
  // the list head and this workgroup's first entry travel together (the entry is in
  // bounds whatever the count: gridDim.x <= atom_max_multi)
  const int count = multi[0].x;
  int4 e4 = multi[1 + blockIdx.x];
  for (int mb = blockIdx.x; mb < count; mb += gridDim.x) {
    if (mb != static_cast<int>(blockIdx.x)) e4 = multi[1 + mb];
    const int u = e4.x, ni = e4.z, bp = u / Ck, j = u % Ck;
    const size_t pb = static_cast<size_t>(bh) * atom_max_partials(a.N) + e4.y;
    const size_t abase = (static_cast<size_t>(bh) * a.nb + bp) * Cq;
    for (int e = tid; e < Cq * F4; e += NT) {
      const int i = e / F4, f = e % F4;
      const bool isv = f >= D / 4;
      const int d4 = 4 * (isv ? f - D / 4 : f);
      const float* __restrict__ src = isv ? a.pt_v : a.pt_k;
      float M = kNegInf, z = 0.f;
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
      for (int q0 = 0; q0 < ni; q0 += QB) {
        float m[QB], zz[QB];
        f32x4_t x[QB];
#pragma unroll
        for (int q = 0; q < QB; ++q) {
          m[q] = kNegInf;
          zz[q] = 0.f;
          x[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          if (q0 + q < ni) {
            const size_t pi = (pb + q0 + q) * Cq + i;
            m[q] = pm[pi];
            zz[q] = pz[pi];
            x[q] = *reinterpret_cast<const f32x4_t*>(src + pi * D + d4);
          }
        }
        float bm = M;
#pragma unroll
        for (int q = 0; q < QB; ++q) bm = fmaxf(bm, m[q]);
        const float rs = M == kNegInf ? 0.f : __expf(M - bm);
        z *= rs;
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c] *= rs;
#pragma unroll
        for (int q = 0; q < QB; ++q) {
          const float w = m[q] == kNegInf ? 0.f : __expf(m[q] - bm);
          z = fmaf(w, zz[q], z);
#pragma unroll
          for (int c = 0; c < 4; ++c) acc[c] = fmaf(w, x[q][c], acc[c]);
        }
        M = bm;
      }
      const size_t ai = (abase + i) * Ck + j;
      if (f == 0) {
        a.at_m[ai] = M;
        a.at_z[ai] = z;
      }
      *reinterpret_cast<f32x4_t*>((isv ? a.at_v : a.at_k) + ai * D + d4) = acc;
    }
  }
}

// Block moments with fp16 operands over a contiguous range of positions of the bucketed
// order (a causal block, or a slice of an acausal sequence; at most kMaxMomKeys
// positions, whose permutation entries are staged in LDS): one workgroup of 8 waves
// per (range, group of G centroids, head). Weights w = exp(a - max over the range) come
// from the scores; every chunk of K and V rows (128 keys at D = 64, 64 at D = 128) is
// gathered once, converted to
// fp16 (exact for bf16 values in fp16 range) and stored row-major in LDS, where the
// transpose read hands both MFMA operands over with the key index along k:
//   sum_m w_m v_m k_m^T = (V^T diag(w)) K,  A = v fragment * w (packed fp16), B = k fragment.
// D = 64: 16 centroids per workgroup, 2 per wave, all 4 output tiles of each;
// D = 128: 4 centroids, wave w takes centroid w/2, value tiles 2(w%2)..2(w%2)+1, all
// 4 key tiles. Output [dv][dk], normalised by the range's weight sum.
template <int D>
struct MomCfg {
  static constexpr int G = moments_group(D);   // centroids per workgroup
  static constexpr int CW = D == 64 ? 2 : 1;   // centroids per wave
  static constexpr int NDV = 2;                // value tiles per wave
  static constexpr int NDK = D / 32;           // key tiles per wave
  static constexpr int KC = D == 64 ? 128 : 64;  // keys per chunk (two chunks are in LDS)
  static constexpr int ST = D + 16;            // LDS row stride (fp16 elements)
  static constexpr int NPRE = KC * (D / 8) / 512;  // 16-byte row pieces per thread and tensor
  static constexpr int NWQ = (G * KC + 511) / 512;   // chunk weights per thread
};

// LDS holds two chunks (rows and weights): chunk c is used from one buffer while chunk
// c + 1 is written to the other and chunk c + 2 travels in registers; one barrier per chunk.
template <int D>
__global__ void __launch_bounds__(512) s1_moments_f16_kernel(S1Args a) {
  using Cfg = MomCfg<D>;
  constexpr int G = Cfg::G, CW = Cfg::CW, NDV = Cfg::NDV, NDK = Cfg::NDK, KC = Cfg::KC, ST = Cfg::ST;
  constexpr int NPRE = Cfg::NPRE, NWQ = Cfg::NWQ;
  __shared__ __align__(16) uint16_t sK[2][KC * ST];
  __shared__ __align__(16) uint16_t sV[2][KC * ST];
  __shared__ __align__(16) _Float16 sw[2][G * KC];
  __shared__ int s_perm[kMaxMomKeys];
  __shared__ float smx[G], ssum[G], spart[G * KC / 64];
  const int mb = blockIdx.x, ig = blockIdx.y, bh = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, h = lane >> 5;
  const int Cq = a.Cq, i0 = ig * G, ng = min(G, Cq - i0);
  const int key0 = mb * a.mbk, key1 = min(a.N, key0 + a.mbk), nkeys = key1 - key0;
  const float* S = a.scores + (static_cast<size_t>(bh) * Cq + i0) * a.N + key0;
  const int32_t* perm = a.perm_k + static_cast<size_t>(bh) * a.N + key0;
  // the range's permutation entries, eight per thread requested at a time (clamped)
  for (int k0 = tid; k0 < nkeys; k0 += 512 * 8) {
    int pv8[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) pv8[q] = perm[min(k0 + 512 * q, nkeys - 1)];
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (k0 + 512 * q < nkeys) s_perm[k0 + 512 * q] = pv8[q];
  }

  // max of the scores over the range, per centroid, from the maxima of its 32-position
  // tiles (the range starts on a tile): 32 lanes (a half-wave) per centroid
  const int ntl = (a.N + 31) / 32, t0 = key0 / 32, t1 = (key1 + 31) / 32;
  for (int g0 = 2 * wave; g0 < G; g0 += 16) {
    const int g = g0 + h;
    float mx = kNegInf;
    if (g < ng) {
      const float* Tg = a.tmax + (static_cast<size_t>(bh) * Cq + i0 + g) * ntl;
      for (int tb = t0; tb < t1; tb += 32 * 8) {
        float x[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int tt = tb + (lane & 31) + 32 * q;
          x[q] = tt < t1 ? Tg[tt] : kNegInf;
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) mx = fmaxf(mx, x[q]);
      }
    }
    mx = half_wave_max(mx);
    if ((lane & 31) == 0 && g < G) smx[g] = mx;
  }
  const uint16_t* K = static_cast<const uint16_t*>(a.k) + static_cast<size_t>(bh) * a.N * D;
  const uint16_t* V = static_cast<const uint16_t*>(a.v) + static_cast<size_t>(bh) * a.N * D;
  u16x8_t pk[NPRE], pv[NPRE];
  float ps[NWQ];
  auto load_chunk = [&](int c0) {
#pragma unroll
    for (int q = 0; q < NPRE; ++q) {
      const int x = tid + 512 * q;
      const int r = x / (D / 8), c8 = x % (D / 8);
      pk[q] = u16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
      pv[q] = u16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
      if (c0 + r < nkeys) {
        const size_t row = static_cast<size_t>(s_perm[c0 + r]) * D + c8 * 8;
        pk[q] = *reinterpret_cast<const u16x8_t*>(K + row);
        pv[q] = *reinterpret_cast<const u16x8_t*>(V + row);
      }
    }
#pragma unroll
    for (int q = 0; q < NWQ; ++q) {
      const int x = tid + 512 * q;
      const int g = x / KC, k = x % KC;
      ps[q] = kNegInf;
      if (x < G * KC && g < ng && c0 + k < nkeys) ps[q] = S[static_cast<size_t>(g) * a.N + c0 + k];
    }
  };
  // bf16 -> fp16 of eight values (exact in fp16's normal range)
  auto to_f16 = [](const u16x8_t& u) {
    f16x8_t o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = static_cast<_Float16>(bf16_to_f32(u[e]));
    return __builtin_bit_cast(u16x8_t, o);
  };
  float wsum[NWQ];
#pragma unroll
  for (int q = 0; q < NWQ; ++q) wsum[q] = 0.f;
  // registers -> LDS buffer bf
  auto stage = [&](int bf) {
#pragma unroll
    for (int q = 0; q < NPRE; ++q) {
      const int x = tid + 512 * q;
      const int r = x / (D / 8), c8 = x % (D / 8);
      *reinterpret_cast<u16x8_t*>(&sK[bf][r * ST + c8 * 8]) = to_f16(pk[q]);
      *reinterpret_cast<u16x8_t*>(&sV[bf][r * ST + c8 * 8]) = to_f16(pv[q]);
    }
#pragma unroll
    for (int q = 0; q < NWQ; ++q) {
      const int x = tid + 512 * q;
      if (x >= G * KC) break;
      const int g = x / KC;
      const _Float16 wh = static_cast<_Float16>(ps[q] == kNegInf ? 0.f : __expf(ps[q] - smx[g]));
      sw[bf][x] = wh;
      wsum[q] += static_cast<float>(wh);
    }
  };
  __syncthreads();  // s_perm, smx
  const int nch = (nkeys + KC - 1) / KC;
  if (nch > 0) {
    load_chunk(0);
    stage(0);
  }
  if (nch > 1) load_chunk(KC);
  __syncthreads();

  f32x16_t acc[CW][NDV][NDK];
#pragma unroll
  for (int cc = 0; cc < CW; ++cc)
#pragma unroll
    for (int dv = 0; dv < NDV; ++dv)
#pragma unroll
      for (int dk = 0; dk < NDK; ++dk) acc[cc][dv][dk] = zero16();
  const int gw = D == 64 ? CW * wave : wave / 2;         // first centroid (in the group) of this wave
  const int dv0 = D == 64 ? 0 : NDV * (wave & 1);        // first value tile of this wave

  for (int ch = 0; ch < nch; ++ch) {
    const int bf = ch & 1;
    if (gw < ng) {
#pragma unroll
      for (int ks = 0; ks < KC / 16; ++ks) {
        f16x8_t wr[CW];
#pragma unroll
        for (int cc = 0; cc < CW; ++cc) wr[cc] = *reinterpret_cast<const f16x8_t*>(&sw[bf][(gw + cc) * KC + 16 * ks + 8 * h]);
        f16x8_t bk[NDK];
#pragma unroll
        for (int dk = 0; dk < NDK; ++dk)
          bk[dk] = __builtin_bit_cast(f16x8_t, lds_operand_tr(sK[bf], ST, 16 * ks, 32 * dk, lane));
#pragma unroll
        for (int dv = 0; dv < NDV; ++dv) {
          const f16x8_t vr = __builtin_bit_cast(f16x8_t, lds_operand_tr(sV[bf], ST, 16 * ks, 32 * (dv0 + dv), lane));
#pragma unroll
          for (int cc = 0; cc < CW; ++cc) {
            const f16x8_t av = vr * wr[cc];
#pragma unroll
            for (int dk = 0; dk < NDK; ++dk) acc[cc][dv][dk] = mfma32_f16(av, bk[dk], acc[cc][dv][dk]);
          }
        }
      }
    }
    if (ch + 1 < nch) stage(bf ^ 1);                 // chunk ch + 1 into the other buffer
    if (ch + 2 < nch) load_chunk((ch + 2) * KC);     // chunk ch + 2 in flight
    __syncthreads();
  }
  // weight sums: per wave (64 consecutive weights of one centroid), then per centroid
  // in wave order
#pragma unroll
  for (int q = 0; q < NWQ; ++q) {
    const int x = tid + 512 * q;
    if (x >= G * KC) break;  // uniform per wave
    const float sp = wave_sum(wsum[q]);
    if (lane == 0) spart[x / 64] = sp;
  }
  __syncthreads();
  if (tid < G) {
    float sum = 0.f;
    for (int p = 0; p < KC / 64; ++p) sum += spart[tid * (KC / 64) + p];
    ssum[tid] = sum;
  }
  __syncthreads();
  const int c = lane & 31;
#pragma unroll
  for (int cc = 0; cc < CW; ++cc) {
    const int g = gw + cc;
    if (g >= ng) continue;
    const int i = i0 + g;
    const size_t bidx = (static_cast<size_t>(bh) * a.nmb + mb) * Cq + i;
    const float sum = ssum[g];
    const float inv = sum > 0.f ? 1.f / sum : 0.f;
    if (lane == 0 && dv0 == 0) a.blk_lmass[bidx] = sum > 0.f ? smx[g] + __logf(sum) : kNegInf;
    float* out = a.blk_mom + bidx * D * D;
#pragma unroll
    for (int dv = 0; dv < NDV; ++dv)
#pragma unroll
      for (int dk = 0; dk < NDK; ++dk)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = 32 * (dv0 + dv) + 8 * (v >> 2) + 4 * h + (v & 3);
          out[static_cast<size_t>(row) * D + 32 * dk + c] = acc[cc][dv][dk][v] * inv;
        }
  }
}

// Acausal tables for the matrix-core stage 2 in one pass: one workgroup (4 waves) per
// (query centroid i, head). From the atoms of the single key block and the moment
// slices it writes log Z_ij, the bf16 hi/lo tables of K_ij and V_ij (row-major), and
// s * D_i with
//   D_i = E_i[v k^T] - sum_j P_ij V_ij K_ij^T,
// E_i[v k^T] the mass-weighted mean of the slice moments, preset (negated) in the
// accumulator layout, and sum_j P_ij V_ij K_ij^T on the matrix cores with both operands
// split into bf16 hi + lo (hi.hi + hi.lo + lo.hi) and read through the transpose read
// from row-major LDS tiles of 64 key clusters. A cluster whose bucket was cut into
// several work items has its atom folded here from the items' partial atoms (log-sum-exp
// in item order). Every load that depends on nothing (the atom sums of all clusters, the
// slices' log masses and the first slices' moments) is issued at the start.
template <int D>
__global__ void __launch_bounds__(256, 2) s1_finalize_acausal_kernel(S1Args a) {
  constexpr int JC = 64;
  constexpr int ST = D + 16;
  constexpr int NDT = D / 32;
  constexpr int TPW = NDT * NDT / 4;  // dipole output tiles per wave
  constexpr int NCH = kMaxClusters / JC;  // cluster chunks
  constexpr int NF = JC * D / 4 / 256;    // float4 of a chunk's K (and V) sums per thread
  constexpr int MB = D == 64 ? 4 : 1;     // moment slices loaded per batch
  // the four chunk tiles, one buffer: after the last chunk it stages s * D_i
  __shared__ __align__(16) uint16_t sT[4 * JC * ST];
  uint16_t* const sKh = sT;
  uint16_t* const sKl = sT + JC * ST;
  uint16_t* const sVh = sT + 2 * JC * ST;
  uint16_t* const sVl = sT + 3 * JC * ST;
  constexpr int DST = D + 8;  // row stride of the staged dipole
  static_assert(D * DST <= 4 * JC * ST, "the staged dipole fits in the chunk tiles");
  __shared__ __align__(16) float sP[kMaxClusters];
  __shared__ float sM[kMaxClusters], sInv[kMaxClusters];
  __shared__ float sW[kMaxClusters][kFinQB];  // item weights exp(m_q - M) of the first kFinQB items
  __shared__ int2 sMeta[kMaxClusters];
  __shared__ float red[8];
  const int i = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, h = lane >> 5, c = lane & 31;
  const int Cq = a.Cq, Ck = a.Ck;
  const size_t sidx = static_cast<size_t>(bh) * Cq + i;  // one table entry per (head, i)
  const size_t aidx0 = sidx * Ck;                         // atoms of the single block
  const size_t pb = static_cast<size_t>(bh) * atom_max_partials(a.N);

  // ---- loads that depend on nothing
  int2 mt = make_int2(-1, 1);
  float m0 = kNegInf, z0 = 0.f;
  if (tid < Ck) {
    mt = a.bmeta_k[static_cast<size_t>(bh) * Ck + tid];  // (first partial slot or -1, items)
    m0 = a.at_m[aidx0 + tid];
    z0 = a.at_z[aidx0 + tid];
  }
  // atom sums of every cluster (stale for clusters of several items, which are replaced);
  // at D = 128 they are loaded chunk by chunk (registers)
  constexpr int PCH = D == 64 ? NCH : 0;
  auto load_atoms = [&](int cc, f32x4_t* k4, f32x4_t* v4) {
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int e = tid + 256 * f;
      const int j = min(cc * JC + e / (D / 4), Ck - 1), d4 = (e % (D / 4)) * 4;
      k4[f] = *reinterpret_cast<const f32x4_t*>(a.at_k + (aidx0 + j) * D + d4);
      v4[f] = *reinterpret_cast<const f32x4_t*>(a.at_v + (aidx0 + j) * D + d4);
    }
  };
  f32x4_t ak4[PCH > 0 ? PCH : 1][NF], av4[PCH > 0 ? PCH : 1][NF];
#pragma unroll
  for (int cc = 0; cc < PCH; ++cc)
    if (cc * JC < Ck) load_atoms(cc, ak4[cc], av4[cc]);
  // log masses of the first MB slices and their moments in the accumulator layout
  float R0[MB], mv0[MB][TPW][16];
  if (a.dipole) {
#pragma unroll
    for (int u = 0; u < MB; ++u) {
      const int mb = min(u, a.nmb - 1);
      const size_t bidx = (static_cast<size_t>(bh) * a.nmb + mb) * Cq + i;
      R0[u] = u < a.nmb ? a.blk_lmass[bidx] : kNegInf;
      const float* M = a.blk_mom + bidx * D * D;
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const int ot = wave * TPW + t, dvt = ot / NDT, dkt = ot % NDT;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = 32 * dvt + 8 * (v >> 2) + 4 * h + (v & 3);
          mv0[u][t][v] = M[static_cast<size_t>(row) * D + 32 * dkt + c];
        }
      }
    }
  }

  // ---- log Z_ij and P_ij = softmax_j log Z_ij; a cluster of several items folds the
  // items' (max, sum) kFinQB items' loads at a time
  float lz = kNegInf;
  if (tid < Ck) {
    float m = m0, z = z0;
    if (mt.x >= 0) {
      m = kNegInf;
      z = 0.f;
      for (int q0 = 0; q0 < mt.y; q0 += kFinQB) {
        float mq[kFinQB], zq[kFinQB];
#pragma unroll
        for (int q = 0; q < kFinQB; ++q) {
          const size_t pi = (pb + mt.x + min(q0 + q, mt.y - 1)) * Cq + i;
          mq[q] = a.pt_m[pi];
          zq[q] = a.pt_z[pi];
          if (q0 + q >= mt.y) mq[q] = kNegInf;
        }
        float bm = m;
#pragma unroll
        for (int q = 0; q < kFinQB; ++q) bm = fmaxf(bm, mq[q]);
        z *= m == kNegInf ? 0.f : __expf(m - bm);
#pragma unroll
        for (int q = 0; q < kFinQB; ++q) z = fmaf(mq[q] == kNegInf ? 0.f : __expf(mq[q] - bm), zq[q], z);
        m = bm;
      }
      // weights of the first items relative to the final max (the rest are recomputed)
#pragma unroll
      for (int q = 0; q < kFinQB; ++q) {
        const float mq = q < mt.y ? a.pt_m[(pb + mt.x + q) * Cq + i] : kNegInf;
        sW[tid][q] = mq == kNegInf ? 0.f : __expf(mq - m);
      }
    }
    sMeta[tid] = mt;
    sM[tid] = m;
    sInv[tid] = z > 0.f ? 1.f / z : 0.f;
    lz = z > 0.f ? m + __logf(z) : kNegInf;
    a.s_logz[sidx * Ck + tid] = lz;
  }
  float mx = wave_max(lz);
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float p = (tid < Ck && lz != kNegInf) ? __expf(lz - mx) : 0.f;
  const float ps = wave_sum(p);
  __syncthreads();
  if (lane == 0) red[wave] = ps;
  __syncthreads();
  const float psum = (red[0] + red[1]) + (red[2] + red[3]);
  if (tid < kMaxClusters) sP[tid] = psum > 0.f ? p / psum : 0.f;

  // ---- -E_i[v k^T] in the accumulator layout: rows dv = 32 dvt + 8 (v/4) + 4 h + v%4,
  // col dk = 32 dkt + c; the slice moments weighted by their normalised masses, folded in
  // slice order
  f32x16_t acc[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) acc[t] = zero16();
  if (a.dipole) {
    float Rm = kNegInf;
#pragma unroll
    for (int u = 0; u < MB; ++u) Rm = fmaxf(Rm, R0[u]);
    for (int mb = MB; mb < a.nmb; ++mb) Rm = fmaxf(Rm, a.blk_lmass[(static_cast<size_t>(bh) * a.nmb + mb) * Cq + i]);
    float ws = 0.f;
#pragma unroll
    for (int u = 0; u < MB; ++u) ws += R0[u] == kNegInf ? 0.f : __expf(R0[u] - Rm);
    for (int mb = MB; mb < a.nmb; ++mb) {
      const float R = a.blk_lmass[(static_cast<size_t>(bh) * a.nmb + mb) * Cq + i];
      ws += R == kNegInf ? 0.f : __expf(R - Rm);
    }
    const float winv = ws > 0.f ? 1.f / ws : 0.f;
#pragma unroll
    for (int u = 0; u < MB; ++u) {
      const float w = R0[u] == kNegInf ? 0.f : __expf(R0[u] - Rm) * winv;
      if (w == 0.f) continue;
#pragma unroll
      for (int t = 0; t < TPW; ++t)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[t][v] = fmaf(-w, mv0[u][t][v], acc[t][v]);
    }
    for (int mb0 = MB; mb0 < a.nmb; mb0 += MB) {
      float mv[MB][TPW][16], w[MB];
#pragma unroll
      for (int u = 0; u < MB; ++u) {
        const int mb = min(mb0 + u, a.nmb - 1);
        const size_t bidx = (static_cast<size_t>(bh) * a.nmb + mb) * Cq + i;
        const float R = mb0 + u < a.nmb ? a.blk_lmass[bidx] : kNegInf;
        w[u] = R == kNegInf ? 0.f : __expf(R - Rm) * winv;
        const float* M = a.blk_mom + bidx * D * D;
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
          const int ot = wave * TPW + t, dvt = ot / NDT, dkt = ot % NDT;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int row = 32 * dvt + 8 * (v >> 2) + 4 * h + (v & 3);
            mv[u][t][v] = M[static_cast<size_t>(row) * D + 32 * dkt + c];
          }
        }
      }
#pragma unroll
      for (int u = 0; u < MB; ++u) {
        if (w[u] == 0.f) continue;
#pragma unroll
        for (int t = 0; t < TPW; ++t)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[t][v] = fmaf(-w[u], mv[u][t][v], acc[t][v]);
      }
    }
  }

  // ---- per chunk of 64 clusters: normalised K_ij, V_ij (global tables, LDS hi/lo
  // tiles), then sum_j P_ij V_ij K_ij^T over the chunk
#pragma unroll
  for (int cc = 0; cc < NCH; ++cc) {
    const int j0 = cc * JC;
    if (j0 >= Ck) break;
    __syncthreads();  // sP, sMeta complete / previous chunk consumed
    f32x4_t ck4[NF], cv4[NF];
    if (cc < PCH) {
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        ck4[f] = ak4[cc < PCH ? cc : 0][f];
        cv4[f] = av4[cc < PCH ? cc : 0][f];
      }
    } else {
      load_atoms(cc, ck4, cv4);
    }
    float kk[NF][4], vv[NF][4];
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int e = tid + 256 * f;
      const int jj = e / (D / 4), d4 = (e % (D / 4)) * 4, j = j0 + jj;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        kk[f][q] = 0.f;
        vv[f][q] = 0.f;
      }
      if (j < Ck) {
        const int2 mj = sMeta[j];
        const float inv = sInv[j];
        if (mj.x < 0) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            kk[f][q] = ck4[f][q] * inv;
            vv[f][q] = cv4[f][q] * inv;
          }
        } else {
          for (int q0 = 0; q0 < mj.y; q0 += kFinQB) {
            f32x4_t k4[kFinQB], v4[kFinQB];
            float w[kFinQB];
#pragma unroll
            for (int q = 0; q < kFinQB; ++q) {
              const size_t pi = (pb + mj.x + min(q0 + q, mj.y - 1)) * Cq + i;
              k4[q] = *reinterpret_cast<const f32x4_t*>(a.pt_k + pi * D + d4);
              v4[q] = *reinterpret_cast<const f32x4_t*>(a.pt_v + pi * D + d4);
              if (q0 == 0) {
                w[q] = sW[j][q];
              } else {
                const float mq = a.pt_m[pi];
                w[q] = (q0 + q < mj.y && mq != kNegInf) ? __expf(mq - sM[j]) : 0.f;
              }
            }
#pragma unroll
            for (int q = 0; q < kFinQB; ++q) {
              const float wq = w[q] * inv;
#pragma unroll
              for (int c4 = 0; c4 < 4; ++c4) {
                kk[f][c4] = fmaf(wq, k4[q][c4], kk[f][c4]);
                vv[f][c4] = fmaf(wq, v4[q][c4], vv[f][c4]);
              }
            }
          }
        }
      }
    }
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int e = tid + 256 * f;
      const int jj = e / (D / 4), d4 = (e % (D / 4)) * 4, j = j0 + jj;
      u16x4_t kh, kl, vh, vl;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        kh[q] = f32_to_bf16_bits(kk[f][q]);
        kl[q] = f32_to_bf16_bits(kk[f][q] - bf16_to_f32(kh[q]));
        vh[q] = f32_to_bf16_bits(vv[f][q]);
        vl[q] = f32_to_bf16_bits(vv[f][q] - bf16_to_f32(vh[q]));
      }
      if (j < Ck) {
        *reinterpret_cast<u16x4_t*>(a.t_khi + (sidx * Ck + j) * D + d4) = kh;
        *reinterpret_cast<u16x4_t*>(a.t_klo + (sidx * Ck + j) * D + d4) = kl;
        *reinterpret_cast<u16x4_t*>(a.t_vhi + (sidx * Ck + j) * D + d4) = vh;
        *reinterpret_cast<u16x4_t*>(a.t_vlo + (sidx * Ck + j) * D + d4) = vl;
      }
      *reinterpret_cast<u16x4_t*>(sKh + jj * ST + d4) = kh;
      *reinterpret_cast<u16x4_t*>(sKl + jj * ST + d4) = kl;
      *reinterpret_cast<u16x4_t*>(sVh + jj * ST + d4) = vh;
      *reinterpret_cast<u16x4_t*>(sVl + jj * ST + d4) = vl;
    }
    __syncthreads();
    if (a.dipole) {
#pragma unroll
      for (int ks = 0; ks < JC / 16; ++ks) {
        const f32x4_t p0 = *reinterpret_cast<const f32x4_t*>(sP + j0 + 16 * ks + 8 * h);
        const f32x4_t p1 = *reinterpret_cast<const f32x4_t*>(sP + j0 + 16 * ks + 8 * h + 4);
        const float pw[8] = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
          const int ot = wave * TPW + t, dvt = ot / NDT, dkt = ot % NDT;
          const u16x8_t vh = __builtin_bit_cast(u16x8_t, lds_operand_tr(sVh, ST, 16 * ks, 32 * dvt, lane));
          const u16x8_t vl = __builtin_bit_cast(u16x8_t, lds_operand_tr(sVl, ST, 16 * ks, 32 * dvt, lane));
          float av[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) av[e] = (bf16_to_f32(vh[e]) + bf16_to_f32(vl[e])) * pw[e];
          bf16x8_t ah, al;
          split_bf16x8(av, ah, al);
          const bf16x8_t kh = lds_operand_tr(sKh, ST, 16 * ks, 32 * dkt, lane);
          const bf16x8_t kl = lds_operand_tr(sKl, ST, 16 * ks, 32 * dkt, lane);
          acc[t] = mfma32(ah, kh, acc[t]);
          acc[t] = mfma32(ah, kl, acc[t]);
          acc[t] = mfma32(al, kh, acc[t]);
        }
      }
    }
  }
  if (a.dipole) {
    // acc = sum P V K^T - E = -D_i: staged in LDS once every wave is past the last chunk's
    // products, then stored as whole rows with 16-byte stores
    __syncthreads();
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int ot = wave * TPW + t, dvt = ot / NDT, dkt = ot % NDT;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = 32 * dvt + 8 * (v >> 2) + 4 * h + (v & 3);
        sT[row * DST + 32 * dkt + c] = f32_to_bf16_bits(-a.scale * acc[t][v]);
      }
    }
    __syncthreads();
    uint16_t* dip = a.t_dip + sidx * D * D;
    for (int x = tid; x < D * D / 8; x += 256) {
      const int r = x / (D / 8), c8 = x % (D / 8);
      *reinterpret_cast<u16x8_t*>(dip + static_cast<size_t>(r) * D + 8 * c8) =
          *reinterpret_cast<const u16x8_t*>(sT + r * DST + 8 * c8);
    }
  }
}

// Causal tables in one scan over the blocks: one workgroup (8 or 16 waves) per (query
// centroid i, head) walks the blocks in order with the prefix over earlier blocks in
// registers — per key cluster j the log-sum-exp fold (m_j, z_j, sum w k, sum w v) of the
// atoms, and the mass-weighted sum of the block moments — and at every block b >= 1
// writes entry b of the stage-2 tables: log Z_ij, bf16 hi/lo K_ij and V_ij (row-major),
// and  s * D_i = s * (E_i[v k^T] - sum_j P_ij V_ij K_ij^T)  with the sum over j on the
// matrix cores (operands split into bf16 hi + lo, read by the transpose read from LDS
// tiles of 64 clusters). Then block b is folded in.
// Thread mapping: float4 e4 = tid + T r of the [Ck][D] sums, i.e. cluster
// j = e4 / (D/4); the JC-cluster chunk cc holds the thread's float4s r = RPC cc .. RPC cc + RPC - 1.
template <int D>
struct ScanCfg {
  static constexpr int NW = D == 128 ? 16 : 8;
  static constexpr int T = 64 * NW;
  static constexpr int JC = 64;                         // key clusters per LDS chunk
  static constexpr int NE4 = kMaxClusters * D / 4 / T;  // float4s per thread and tensor
  static constexpr int RPC = JC * (D / 4) / T;          // of them per chunk
  static constexpr int NDT = D / 32;
  static constexpr int NT = NDT * NDT;                  // dipole output tiles
  static constexpr int TPW = NT / NW > 0 ? NT / NW : 1;  // per wave
  static constexpr int ST = D + 16;
  static constexpr bool PREF = D == 64;  // atoms requested before the entry is written (registers allow)
};

template <int D>
__global__ void __launch_bounds__(ScanCfg<D>::T) s1_causal_scan_kernel(S1Args a) {
  using Cfg = ScanCfg<D>;
  constexpr int NW = Cfg::NW, T = Cfg::T, NE4 = Cfg::NE4, RPC = Cfg::RPC, NDT = Cfg::NDT, NT = Cfg::NT;
  constexpr int TPW = Cfg::TPW, ST = Cfg::ST, JC = Cfg::JC;
  // the four chunk tiles, one buffer: after an entry's products it stages s * D_i
  __shared__ __align__(16) uint16_t sT[4 * JC * ST];
  uint16_t* const sKh = sT;
  uint16_t* const sKl = sT + JC * ST;
  uint16_t* const sVh = sT + 2 * JC * ST;
  uint16_t* const sVl = sT + 3 * JC * ST;
  constexpr int DST = D + 8;  // row stride of the staged dipole
  static_assert(D * DST <= 4 * JC * ST, "the staged dipole fits in the chunk tiles");
  __shared__ __align__(16) float sP[kMaxClusters];
  __shared__ float sm[kMaxClusters], sz[kMaxClusters], sfo[kMaxClusters], sfn[kMaxClusters], sinv[kMaxClusters];
  __shared__ float red[2 * NW];
  __shared__ float sE[D * D];  // sum over folded ranges of exp(R - Rm) * moment, [dv][dk]
  const int i = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, h = lane >> 5, c = lane & 31;
  const int Cq = a.Cq, Ck = a.Ck, nb = a.nb;
  const int per = a.block / a.mbk;  // moment ranges per block
  auto tile_of = [&](int t, int& dvt, int& dkt) {
    const int ot = wave * TPW + t;
    dvt = ot / NDT;
    dkt = ot % NDT;
    return ot < NT;
  };

  // prefix state
  f32x4_t ks[NE4], vs[NE4];
#pragma unroll
  for (int r = 0; r < NE4; ++r) {
    ks[r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    vs[r] = ks[r];
  }
  if (tid < kMaxClusters) {
    sm[tid] = kNegInf;
    sz[tid] = 0.f;
  }
  for (int e = tid; e < D * D; e += T) sE[e] = 0.f;
  float Rm = kNegInf, W = 0.f;

  for (int b = 0; b < nb; ++b) {
    const bool fold = b + 1 < nb;
    const size_t abase = ((static_cast<size_t>(bh) * nb + b) * Cq + i) * Ck;
    f32x4_t pk[Cfg::PREF ? NE4 : 1], pv[Cfg::PREF ? NE4 : 1];
    auto load_atoms = [&] {
#pragma unroll
      for (int r = 0; r < NE4; ++r) {
        const int e4 = tid + T * r;
        pk[r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        pv[r] = pk[r];
        if (e4 < Ck * D / 4) {
          pk[r] = *reinterpret_cast<const f32x4_t*>(a.at_k + abase * D + 4 * static_cast<size_t>(e4));
          pv[r] = *reinterpret_cast<const f32x4_t*>(a.at_v + abase * D + 4 * static_cast<size_t>(e4));
        }
      }
    };
    // this lane's elements of the block's first moment range (D = 64: requested now, they
    // land while entry b is written; D = 128: requested together at the fold)
    float mpre[TPW][16];
    auto load_moment = [&](int sub) {
      const float* M = a.blk_mom + ((static_cast<size_t>(bh) * a.nmb + b * per + sub) * Cq + i) * D * D;
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        int dvt, dkt;
        if (!tile_of(t, dvt, dkt)) break;
#pragma unroll
        for (int v = 0; v < 16; ++v)
          mpre[t][v] = M[static_cast<size_t>(32 * dvt + 8 * (v >> 2) + 4 * h + (v & 3)) * D + 32 * dkt + c];
      }
    };
    if (Cfg::PREF && fold) {
      load_atoms();
      if (a.dipole) load_moment(0);
    }
    // the block's atom masses and first moment range's log mass, requested now
    float pam = kNegInf, paz = 0.f, pR = kNegInf;
    if (fold) {
      if (tid < Ck) {
        pam = a.at_m[abase + tid];
        paz = a.at_z[abase + tid];
      }
      if (a.dipole) pR = a.blk_lmass[(static_cast<size_t>(bh) * a.nmb + b * per) * Cq + i];
    }
    __syncthreads();  // sm, sz of the prefix are final
    if (b > 0) {
      // ---- entry b: log Z, P, normalised tables ----
      float lz = kNegInf;
      if (tid < Ck) {
        const float z = sz[tid];
        lz = z > 0.f ? sm[tid] + __logf(z) : kNegInf;
        a.s_logz[((static_cast<size_t>(bh) * a.nbS + b) * Cq + i) * Ck + tid] = lz;
        sinv[tid] = z > 0.f ? 1.f / z : 0.f;
      }
      float mx = wave_max(lz);
      if (lane == 0) red[wave] = mx;
      __syncthreads();
      mx = kNegInf;
#pragma unroll
      for (int w = 0; w < NW; ++w) mx = fmaxf(mx, red[w]);
      const float p = (tid < Ck && lz != kNegInf) ? __expf(lz - mx) : 0.f;
      const float ps = wave_sum(p);
      if (lane == 0) red[NW + wave] = ps;
      __syncthreads();
      float psum = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) psum += red[NW + w];
      if (tid < kMaxClusters) sP[tid] = psum > 0.f ? p / psum : 0.f;
      const size_t tbase = ((static_cast<size_t>(bh) * a.nbS + b) * Cq + i) * static_cast<size_t>(Ck) * D;
      f32x16_t dacc[TPW];
      {
        const float winv = W > 0.f ? 1.f / W : 0.f;
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
          int dvt, dkt;
          dacc[t] = zero16();
          if (!tile_of(t, dvt, dkt)) continue;
#pragma unroll
          for (int v = 0; v < 16; ++v)  // -E_i[v k^T] of the prefix
            dacc[t][v] = -sE[(32 * dvt + 8 * (v >> 2) + 4 * h + (v & 3)) * D + 32 * dkt + c] * winv;
        }
      }
#pragma unroll
      for (int cc = 0; cc < kMaxClusters / JC; ++cc) {
        if (cc * JC >= Ck) break;  // uniform
#pragma unroll
        for (int q = 0; q < RPC; ++q) {
          const int r = cc * RPC + q;  // compile-time after unrolling
          const int e4 = tid + T * r, j = e4 / (D / 4), d4 = (e4 % (D / 4)) * 4, jj = j - JC * cc;
          const f32x4_t kf = ks[r], vf = vs[r];
          const float inv = j < Ck ? sinv[j] : 0.f;
          u16x4_t kh, kl, vh, vl;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float kk = kf[e] * inv, vv = vf[e] * inv;
            kh[e] = f32_to_bf16_bits(kk);
            kl[e] = f32_to_bf16_bits(kk - bf16_to_f32(kh[e]));
            vh[e] = f32_to_bf16_bits(vv);
            vl[e] = f32_to_bf16_bits(vv - bf16_to_f32(vh[e]));
          }
          if (j < Ck) {
            *reinterpret_cast<u16x4_t*>(a.t_khi + tbase + 4 * static_cast<size_t>(e4)) = kh;
            *reinterpret_cast<u16x4_t*>(a.t_klo + tbase + 4 * static_cast<size_t>(e4)) = kl;
            *reinterpret_cast<u16x4_t*>(a.t_vhi + tbase + 4 * static_cast<size_t>(e4)) = vh;
            *reinterpret_cast<u16x4_t*>(a.t_vlo + tbase + 4 * static_cast<size_t>(e4)) = vl;
          }
          if (a.dipole) {
            *reinterpret_cast<u16x4_t*>(sKh + jj * ST + d4) = kh;
            *reinterpret_cast<u16x4_t*>(sKl + jj * ST + d4) = kl;
            *reinterpret_cast<u16x4_t*>(sVh + jj * ST + d4) = vh;
            *reinterpret_cast<u16x4_t*>(sVl + jj * ST + d4) = vl;
          }
        }
        if (!a.dipole) continue;
        __syncthreads();
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
          int dvt, dkt;
          if (!tile_of(t, dvt, dkt)) break;
#pragma unroll
          for (int ks2 = 0; ks2 < JC / 16; ++ks2) {
            const f32x4_t p0 = *reinterpret_cast<const f32x4_t*>(sP + JC * cc + 16 * ks2 + 8 * h);
            const f32x4_t p1 = *reinterpret_cast<const f32x4_t*>(sP + JC * cc + 16 * ks2 + 8 * h + 4);
            const float pw[8] = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
            const u16x8_t uh = __builtin_bit_cast(u16x8_t, lds_operand_tr(sVh, ST, 16 * ks2, 32 * dvt, lane));
            const u16x8_t ul = __builtin_bit_cast(u16x8_t, lds_operand_tr(sVl, ST, 16 * ks2, 32 * dvt, lane));
            float av[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) av[e] = (bf16_to_f32(uh[e]) + bf16_to_f32(ul[e])) * pw[e];
            bf16x8_t ah, al;
            split_bf16x8(av, ah, al);
            const bf16x8_t kh8 = lds_operand_tr(sKh, ST, 16 * ks2, 32 * dkt, lane);
            const bf16x8_t kl8 = lds_operand_tr(sKl, ST, 16 * ks2, 32 * dkt, lane);
            dacc[t] = mfma32(ah, kh8, dacc[t]);
            dacc[t] = mfma32(ah, kl8, dacc[t]);
            dacc[t] = mfma32(al, kh8, dacc[t]);
          }
        }
        __syncthreads();  // the next chunk overwrites the tiles
      }
      if (a.dipole) {
        // dacc = sum P V K^T - E = -D_i: staged in LDS (the chunk tiles are free after the
        // last chunk's barrier), then stored as whole rows with 16-byte stores
        uint16_t* dip = a.t_dip + ((static_cast<size_t>(bh) * a.nbS + b) * Cq + i) * D * D;
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
          int dvt, dkt;
          if (!tile_of(t, dvt, dkt)) break;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int row = 32 * dvt + 8 * (v >> 2) + 4 * h + (v & 3);
            sT[row * DST + 32 * dkt + c] = f32_to_bf16_bits(-a.scale * dacc[t][v]);
          }
        }
        __syncthreads();
        for (int x = tid; x < D * D / 8; x += T) {
          const int r = x / (D / 8), c8 = x % (D / 8);
          *reinterpret_cast<u16x8_t*>(dip + static_cast<size_t>(r) * D + 8 * c8) =
              *reinterpret_cast<const u16x8_t*>(sT + r * DST + 8 * c8);
        }
      }
    }
    if (!fold) break;
    // ---- fold block b ----
    if (tid < Ck) {
      const float am = pam, az = paz;
      const float m0 = sm[tid], z0 = sz[tid];
      float fo = 1.f, fn = 0.f;
      if (az > 0.f) {
        const float mn = fmaxf(m0, am);
        fo = z0 > 0.f ? __expf(m0 - mn) : 0.f;
        fn = __expf(am - mn);
        sm[tid] = mn;
        sz[tid] = z0 * fo + az * fn;
      }
      sfo[tid] = fo;
      sfn[tid] = fn;
    }
    if (a.dipole) {
      for (int sub = 0; sub < per; ++sub) {
        const size_t bidx = (static_cast<size_t>(bh) * a.nmb + b * per + sub) * Cq + i;
        // every element of the range in flight at once (the moments are written for every
        // range, also one of zero mass)
        if (!(Cfg::PREF && sub == 0)) load_moment(sub);
        const float R = sub == 0 ? pR : a.blk_lmass[bidx];
        if (R == kNegInf) continue;
        const float Rn = fmaxf(Rm, R);
        const float fo = Rm == kNegInf ? 0.f : __expf(Rm - Rn), fn = __expf(R - Rn);
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
          int dvt, dkt;
          if (!tile_of(t, dvt, dkt)) break;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int row = 32 * dvt + 8 * (v >> 2) + 4 * h + (v & 3);
            float* pe = sE + row * D + 32 * dkt + c;  // this lane's element
            *pe = *pe * fo + mpre[t][v] * fn;
          }
        }
        W = W * fo + fn;
        Rm = Rn;
      }
    }
    __syncthreads();  // sfo, sfn
    if (Cfg::PREF) {
#pragma unroll
      for (int r = 0; r < NE4; ++r) {
        const int e4 = tid + T * r, j = e4 / (D / 4);
        if (j >= Ck) continue;
        const float fo = sfo[j], fn = sfn[j];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          ks[r][q] = ks[r][q] * fo + pk[r][q] * fn;
          vs[r][q] = vs[r][q] * fo + pv[r][q] * fn;
        }
      }
    } else {
      {
        // the block's atoms (both tensors' rows requested together: one wait, and fewer
        // registers spilled than with one tensor at a time)
        f32x4_t prk[NE4], prv[NE4];
#pragma unroll
        for (int r = 0; r < NE4; ++r) {
          const int e4 = tid + T * r;
          prk[r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          prv[r] = prk[r];
          if (e4 < Ck * D / 4) {
            prk[r] = *reinterpret_cast<const f32x4_t*>(a.at_k + abase * D + 4 * static_cast<size_t>(e4));
            prv[r] = *reinterpret_cast<const f32x4_t*>(a.at_v + abase * D + 4 * static_cast<size_t>(e4));
          }
        }
#pragma unroll
        for (int r = 0; r < NE4; ++r) {
          const int e4 = tid + T * r, j = e4 / (D / 4);
          if (j >= Ck) continue;
          const float fo = sfo[j], fn = sfn[j];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            ks[r][q] = ks[r][q] * fo + prk[r][q] * fn;
            vs[r][q] = vs[r][q] * fo + prv[r][q] * fn;
          }
        }
      }
    }
  }
}

// Dipole of one table entry on the general path (causal entries with retrieval or the
// hierarchy), bf16 tables: one workgroup of 4 waves per (i, e, head):
//   D_i = E_i[v k^T] - sum_j P_ij V_ij K_ij^T,  P_ij = softmax_j(log Z_ij),
// with E_i[v k^T] the folded block moments (fp32, [dv][dk]). Key clusters are staged 32 at
// a time: K_ij and V_ij split into bf16 hi + lo (also written out as the stage-2 tables),
// row-major in LDS; on the matrix cores (P V)^T K with both operands split
// (hi.hi + hi.lo + lo.hi) and read through the transpose read, as in the acausal
// finalise. Writes s * D_i in bf16.
template <int D>
__global__ void __launch_bounds__(256) s1_dip_final_mfma_kernel(S1Args a) {
  constexpr int JC = 32, ST = D + 8, NDT = D / 32, TPW = NDT * NDT / 4;
  __shared__ float sP[kMaxClusters];
  __shared__ __align__(16) uint16_t sKh[JC * ST];
  __shared__ __align__(16) uint16_t sKl[JC * ST];
  __shared__ __align__(16) uint16_t sVh[JC * ST];
  __shared__ __align__(16) uint16_t sVl[JC * ST];
  const int i = blockIdx.x, e = blockIdx.y, bh = blockIdx.z;
  const int Cq = a.Cq, Ck = a.Ck, tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, h = lane >> 5, c = lane & 31;
  if (a.causal && e == 0) return;  // block 0 has no far field
  const size_t sidx = (static_cast<size_t>(bh) * a.nbS + e) * Cq + i;
  const int nch = (Ck + JC - 1) / JC;
  if (tid < 64) {
    float mx = kNegInf;
    for (int j = tid; j < Ck; j += 64) mx = fmaxf(mx, a.s_logz[sidx * Ck + j]);
    mx = wave_max(mx);
    float sm = 0.f;
    for (int j = tid; j < Ck; j += 64) {
      const float l = a.s_logz[sidx * Ck + j];
      sm += l == kNegInf ? 0.f : __expf(l - mx);
    }
    sm = wave_sum(sm);
    const float inv = sm > 0.f ? 1.f / sm : 0.f;
    for (int j = tid; j < nch * JC; j += 64) {
      const float l = j < Ck ? a.s_logz[sidx * Ck + j] : kNegInf;
      sP[j] = l == kNegInf ? 0.f : __expf(l - mx) * inv;
    }
  }
  f32x16_t acc[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) acc[t] = zero16();
  for (int ch = 0; ch < nch; ++ch) {
    const int j0 = ch * JC;
    __syncthreads();  // sP written; the previous chunk consumed
    for (int x = tid; x < JC * D / 4; x += 256) {
      const int jj = x / (D / 4), d4 = (x % (D / 4)) * 4, j = j0 + jj;
      f32x4_t k4 = {0.f, 0.f, 0.f, 0.f}, v4 = {0.f, 0.f, 0.f, 0.f};
      if (j < Ck) {
        k4 = *reinterpret_cast<const f32x4_t*>(a.s_k + (sidx * Ck + j) * D + d4);
        v4 = *reinterpret_cast<const f32x4_t*>(a.s_v + (sidx * Ck + j) * D + d4);
      }
      u16x4_t kh, kl, vh, vl;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        kh[q] = f32_to_bf16_bits(k4[q]);
        kl[q] = f32_to_bf16_bits(k4[q] - bf16_to_f32(kh[q]));
        vh[q] = f32_to_bf16_bits(v4[q]);
        vl[q] = f32_to_bf16_bits(v4[q] - bf16_to_f32(vh[q]));
      }
      if (j < Ck) {
        *reinterpret_cast<u16x4_t*>(a.t_khi + (sidx * Ck + j) * D + d4) = kh;
        *reinterpret_cast<u16x4_t*>(a.t_klo + (sidx * Ck + j) * D + d4) = kl;
        *reinterpret_cast<u16x4_t*>(a.t_vhi + (sidx * Ck + j) * D + d4) = vh;
        *reinterpret_cast<u16x4_t*>(a.t_vlo + (sidx * Ck + j) * D + d4) = vl;
      }
      *reinterpret_cast<u16x4_t*>(sKh + jj * ST + d4) = kh;
      *reinterpret_cast<u16x4_t*>(sKl + jj * ST + d4) = kl;
      *reinterpret_cast<u16x4_t*>(sVh + jj * ST + d4) = vh;
      *reinterpret_cast<u16x4_t*>(sVl + jj * ST + d4) = vl;
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < JC / 16; ++ks) {
      const f32x4_t p0 = *reinterpret_cast<const f32x4_t*>(sP + j0 + 16 * ks + 8 * h);
      const f32x4_t p1 = *reinterpret_cast<const f32x4_t*>(sP + j0 + 16 * ks + 8 * h + 4);
      const float pw[8] = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const int ot = wave * TPW + t, dvt = ot / NDT, dkt = ot % NDT;
        const u16x8_t vh = __builtin_bit_cast(u16x8_t, lds_operand_tr(sVh, ST, 16 * ks, 32 * dvt, lane));
        const u16x8_t vl = __builtin_bit_cast(u16x8_t, lds_operand_tr(sVl, ST, 16 * ks, 32 * dvt, lane));
        float av[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) av[q] = (bf16_to_f32(vh[q]) + bf16_to_f32(vl[q])) * pw[q];
        bf16x8_t ah, al;
        split_bf16x8(av, ah, al);
        const bf16x8_t kh = lds_operand_tr(sKh, ST, 16 * ks, 32 * dkt, lane);
        const bf16x8_t kl = lds_operand_tr(sKl, ST, 16 * ks, 32 * dkt, lane);
        acc[t] = mfma32(ah, kh, acc[t]);
        acc[t] = mfma32(ah, kl, acc[t]);
        acc[t] = mfma32(al, kh, acc[t]);
      }
    }
  }
  // lanes (c, h) hold rows dv = 32 dvt + 8 (v / 4) + 4 h + v % 4 of column dk = 32 dkt + c
  const float* E = a.s_dip + sidx * D * D;
  uint16_t* dip = a.t_dip + sidx * D * D;
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int ot = wave * TPW + t, dvt = ot / NDT, dkt = ot % NDT;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const size_t o = static_cast<size_t>(32 * dvt + 8 * (v >> 2) + 4 * h + (v & 3)) * D + 32 * dkt + c;
      dip[o] = f32_to_bf16_bits(a.scale * (E[o] - acc[t][v]));
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
    const int nbC = a.nb * a.Ck;
    const size_t lds = static_cast<size_t>((a.Cq + 31) & ~31) * (D + 8) * 2 * sizeof(uint16_t);
    allow_lds((const void*)s1_atoms_mfma_kernel<D>, lds);  // the dynamic part (s qbar); the row tiles are static
    {
      // items per wave: about items / (16 x resident waves), rounded, 1..16 (measured: 2
      // at 1.3k items per head x 64 heads with D = 64, 4-5 at 5k x 16 with D = 128)
      int dev = 0, cus = 256;
      (void)hipGetDevice(&dev);
      (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
      const long resident = static_cast<long>(cus) * 4 * (D == 64 ? 3 : 1);
      const long items = static_cast<long>(atom_max_items(nbC, a.N)) * a.BH;
      const int ipw = static_cast<int>(std::max<long>(1, std::min<long>(16, (items + 8 * resident) / (16 * resident))));
      const int waves = (atom_max_items(nbC, a.N) + ipw - 1) / ipw;
      ProfScope ps_("s1_atoms_mfma", s);
      hipLaunchKernelGGL((s1_atoms_mfma_kernel<D>), dim3((waves + 3) / 4, a.BH), dim3(256), lds, s, a, ipw);
    }
    // the acausal finalise folds the items itself; the causal scan, retrieval and the
    // fp32-table path read merged atoms
    if (a.causal || a.retr != nullptr || a.tables_f32) {
      ProfScope ps_("s1_atoms_merge", s);
      const dim3 gm(std::min(kMergeGrid, atom_max_multi(a.N)), a.BH);
      if (a.Cq * (D / 2) <= 512) hipLaunchKernelGGL((s1_atoms_merge_kernel<D, 512>), gm, dim3(512), 0, s, a);
      else hipLaunchKernelGGL((s1_atoms_merge_kernel<D, 1024>), gm, dim3(1024), 0, s, a);
    }
  } else if (which == 2) {
    constexpr int G = MomCfg<D>::G;
    ProfScope ps_("s1_moments_f16", s);
    hipLaunchKernelGGL((s1_moments_f16_kernel<D>), dim3(a.nmb, (a.Cq + G - 1) / G, a.BH), dim3(512), 0, s, a);
  } else if (which == 5) {
    ProfScope ps_("s1_dip_final", s);
    hipLaunchKernelGGL((s1_dip_final_mfma_kernel<D>), dim3(a.Cq, a.nbS, a.BH), dim3(256), 0, s, a);
  } else if (which == 3) {
    ProfScope ps_("s1_finalize", s);
    hipLaunchKernelGGL((s1_finalize_acausal_kernel<D>), dim3(a.Cq, a.BH), dim3(256), 0, s, a);
  } else {
    ProfScope ps_("s1_causal_scan", s);
    hipLaunchKernelGGL((s1_causal_scan_kernel<D>), dim3(a.Cq, a.BH), dim3(ScanCfg<D>::T), 0, s, a);
  }
}

// which: 0 scores, 1 atoms, 2 moments, 3 acausal table finalise, 4 causal scan,
// 5 dipole finalise of the general path (bf16 tables)
void launch_stage1_mfma(const S1Args& a, int which, hipStream_t s) {
  if (a.D == 64) launch_t<64>(a, which, s);
  else launch_t<128>(a, which, s);
}

}  // namespace muse
