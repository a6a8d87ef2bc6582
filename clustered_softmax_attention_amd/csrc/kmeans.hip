// Lloyd K-means on queries and on keys, each head separately (gfx950, wave64).
//
// The method clusters queries and keys separately, each in its own space
// (gist.science summary of arXiv 2509.10406, Kernmechanismen 1), with a few
// Euclidean K-means iterations (pith.science review, "Assumptions & free
// parameters": K-means iterations).
//
// Layout: a head's N points are cut into tiles of `tile` consecutive points
// (one workgroup, one thread per point). Tiles never straddle a causal block,
// so a (block, cluster) bucket is a concatenation of per-tile segments.
//
// Per iteration:
//   kmeans_assign : label = argmin_j ||x - c_j||^2 (direct form, fp32, ties to the
//                   lowest j); the tile's points are counting-sorted by label in
//                   LDS (stable) and the tile's per-cluster sums are written out.
//   kmeans_update : c_j = (sum over tiles, in tile order) / count, or unchanged
//                   when the cluster is empty.
// After the last iteration:
//   bucket_offsets / bucket_scatter : stable order of the head's points by
//                   (block, label), i.e. the key (or query) permutation used by
//                   the summary kernels.
//
// bf16 inputs (kmeans_assign_mfma): the scores x.c_j - ||c_j||^2 / 2 (the distance is
// ||x||^2 minus twice the score) come from the matrix cores, with each fp32 centroid
// split into bf16 hi + lo parts (x is exact in bf16). Two scores can swap only within
// E = 1e-4 ||x|| max||c|| + 2e-5 (D / 64) max||c||^2, above twice the worst case of the
// split residual, the fp32 accumulation over 2D + 1 terms, the fp32 norm and the rank
// key's truncation; when a second centroid scores within E of the best, every such
// candidate is re-scored with the exact fp32 direct form sum_d (x_d - c_jd)^2 of the
// fp32 path, so labels are the same as the fp32 path's.
//
// Every sum runs in a fixed order, so labels and centroids are bitwise
// reproducible.
#include "mfma.hpp"
#include "muse_kernels.hpp"

#include <type_traits>

namespace muse {

// Derived forms of centroid j used by the matrix-core assign: bf16 hi/lo split and
// ||c_j||^2 (fp32, fixed reduction order). Called by one whole wave, lanes over d.
__device__ __forceinline__ void write_centroid_tables(const KmTensor& t, int D, size_t row, const float* vals,
                                                      int nper) {
  float n2 = 0.f;
  for (int q = 0; q < nper; ++q) {
    const int d = lane_id() + 64 * q;
    const float cv = vals[q];
    n2 = fmaf(cv, cv, n2);
    if (t.chi != nullptr) {
      const uint16_t hi = f32_to_bf16_bits(cv);
      t.chi[row * D + d] = hi;
      t.clo[row * D + d] = f32_to_bf16_bits(cv - bf16_to_f32(hi));
    }
  }
  n2 = wave_sum(n2);
  if (t.cn2 != nullptr && lane_id() == 0) t.cn2[row] = n2;
}

constexpr int kUpdWaves = 8;  // centroids (one per wave) per init and update workgroup

// One wave per (centroid j, head, tensor): c_j = x[floor(j*N/C)].
template <typename T>
__global__ void __launch_bounds__(64 * kUpdWaves) kmeans_init_kernel(KmArgs a) {
  const KmTensor& t = a.t[blockIdx.z];
  const int j = blockIdx.x * kUpdWaves + (threadIdx.x >> 6), bh = blockIdx.y;
  if (t.labels_in != nullptr || j >= t.C) return;
  const T* x = static_cast<const T*>(t.x) + static_cast<size_t>(bh) * a.N * a.D;
  const long src = (static_cast<long>(j) * a.N) / t.C;
  const size_t row = static_cast<size_t>(bh) * t.C + j;
  float vals[2];
  const int nper = a.D / 64;
  for (int q = 0; q < nper; ++q) {
    const int d = lane_id() + 64 * q;
    vals[q] = Elem<T>::load(x, static_cast<size_t>(src) * a.D + d);
    t.cent[row * a.D + d] = vals[q];
  }
  write_centroid_tables(t, a.D, row, vals, nper);
}

// Stable counting sort of tile tt's points by label (LDS) and the tile's sort info.
// Called by every thread of the workgroup; a thread owns point `pidx` of the tile when
// `valid` (threads that own no point pass lab = C, which sorts nowhere). Points of equal
// label keep the order of their owners (wave, then lane), which is point order.
__device__ void tile_sort(const KmArgs& a, const KmTensor& t, int lab, bool valid, int pidx, int tt, int* s_whist,
                          int* s_cnt, int* s_start, int* s_sorted) {
  const int C = t.C;
  const int bh = blockIdx.y;
  const int nthr = blockDim.x;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int nwaves = nthr >> 6;
  for (int e = tid; e < nwaves * C; e += nthr) s_whist[e] = 0;
  __syncthreads();
  // lanes of this wave with the same label (the sentinel C only matches itself)
  uint64_t peers = __ballot(1);
  for (int b = 0; (1 << b) <= C; ++b) {
    const bool bit = (lab >> b) & 1;
    const uint64_t m = __ballot(bit);
    peers &= bit ? m : ~m;
  }
  const int rank_in_wave = __popcll(peers & lanemask_lt());
  if (valid && rank_in_wave == 0) s_whist[wave * C + lab] = __popcll(peers);
  __syncthreads();
  for (int j = tid; j < C; j += nthr) {
    int run = 0;
    for (int w = 0; w < nwaves; ++w) {
      const int h = s_whist[w * C + j];
      s_whist[w * C + j] = run;  // becomes the wave's base inside the label's segment
      run += h;
    }
    s_cnt[j] = run;
  }
  __syncthreads();
  if (wave == 0) {
    // exclusive scan of the C <= 128 label counts: two per lane, then a wave scan
    const int lane = tid & 63, j0 = 2 * lane;
    const int c0 = j0 < C ? s_cnt[j0] : 0, c1 = j0 + 1 < C ? s_cnt[j0 + 1] : 0;
    int incl = c0 + c1;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    const int excl = incl - c0 - c1;
    if (j0 < C) s_start[j0] = excl;
    if (j0 + 1 < C) s_start[j0 + 1] = excl + c0;
  }
  __syncthreads();
  if (valid) s_sorted[s_start[lab] + s_whist[wave * C + lab] + rank_in_wave] = pidx;
  __syncthreads();

  // ---- outputs: sort info for bucketing ----
  const size_t tix = static_cast<size_t>(bh) * a.ntiles + tt;
  for (int j = tid; j < C; j += nthr) {
    t.tile_cnt[tix * C + j] = s_cnt[j];
    t.tile_start[tix * C + j] = s_start[j];
  }
  for (int pos = tid; pos < a.tile; pos += nthr) t.tile_perm[tix * a.tile + pos] = static_cast<uint16_t>(s_sorted[pos]);
}

// Per-cluster sums of the tile in sorted order (fp32 path).
template <typename T, int D>
__device__ void tile_sums_valu(const KmArgs& a, const KmTensor& t, const int* s_cnt, const int* s_start,
                               const int* s_sorted) {
  const int C = t.C;
  const int bh = blockIdx.y;
  const int tile = blockDim.x;
  const int tid = threadIdx.x;
  const T* x = static_cast<const T*>(t.x) + static_cast<size_t>(bh) * a.N * D;
  const size_t tix = static_cast<size_t>(bh) * a.ntiles + blockIdx.x;
  float* psum = t.psum + tix * C * D;
  const long base = static_cast<long>(blockIdx.x) * tile;
  for (int e = tid; e < C * D; e += tile) {
    const int j = e / D, d = e % D;
    const int st = s_start[j], cnt = s_cnt[j];
    float acc = 0.f;
    for (int r = 0; r < cnt; ++r) acc += Elem<T>::load(x, static_cast<size_t>(base + s_sorted[st + r]) * D + d);
    psum[e] = acc;
  }
}

// One workgroup = one tile of `tile` points (blockDim.x == tile, a multiple of 64).
// Dynamic LDS: centroid chunk [kChunkC][D] f32 | tile labels [tile] | wave histograms
// [tile/64][C] | tile counts [C] | tile starts [C] | sorted order [tile].
template <typename T, int D>
__global__ void __launch_bounds__(kMaxTile) kmeans_assign_kernel(KmArgs a, int iter) {
  extern __shared__ __align__(16) unsigned char smem[];
  const KmTensor& t = a.t[blockIdx.z];
  const int C = t.C;
  const int bh = blockIdx.y;
  const int tile = blockDim.x;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int nwaves = tile >> 6;
  const long n = static_cast<long>(blockIdx.x) * tile + tid;
  const bool valid = n < a.N;
  const T* x = static_cast<const T*>(t.x) + static_cast<size_t>(bh) * a.N * D;

  float* sc = reinterpret_cast<float*>(smem);                       // [kChunkC][D]
  int* s_lab = reinterpret_cast<int*>(sc + kChunkC * D);            // [tile]
  int* s_whist = s_lab + tile;                                      // [nwaves][C]
  int* s_cnt = s_whist + nwaves * C;                                // [C]
  int* s_start = s_cnt + C;                                         // [C]
  int* s_sorted = s_start + C;                                      // [tile]

  int lab = C;  // sentinel for points past the end of the sequence
  if (t.labels_in != nullptr) {
    // caller labels outside [0, C) are clamped so that LDS indexing stays in bounds
    if (valid) lab = min(max(t.labels_in[static_cast<size_t>(bh) * a.N + n], 0), C - 1);
  } else {
    float xr[D];
#pragma unroll
    for (int d = 0; d < D; ++d) xr[d] = valid ? Elem<T>::load(x, static_cast<size_t>(n) * D + d) : 0.f;
    const float* cent = t.cent + static_cast<size_t>(bh) * C * D;
    float best = __builtin_huge_valf();
    int bj = 0;
    for (int j0 = 0; j0 < C; j0 += kChunkC) {
      const int nc = min(kChunkC, C - j0);
      __syncthreads();
      for (int e = tid; e < nc * D; e += tile) sc[e] = cent[static_cast<size_t>(j0) * D + e];
      __syncthreads();
      for (int jj = 0; jj < nc; ++jj) {
        const float* cj = sc + jj * D;
        float dist = 0.f;
#pragma unroll
        for (int d = 0; d < D; ++d) {
          const float diff = xr[d] - cj[d];
          dist = fmaf(diff, diff, dist);
        }
        if (dist < best) {  // strict: an exact tie keeps the lower index
          best = dist;
          bj = j0 + jj;
        }
      }
    }
    if (valid) lab = bj;
  }
  if (valid) {
    t.labels[static_cast<size_t>(bh) * a.N + n] = lab;
    if (t.trace != nullptr) t.trace[(static_cast<size_t>(iter) * a.BH + bh) * a.N + n] = lab;
  }

  tile_sort(a, t, lab, valid, static_cast<int>(threadIdx.x), blockIdx.x, s_whist, s_cnt, s_start, s_sorted);
  tile_sums_valu<T, D>(a, t, s_cnt, s_start, s_sorted);
}

// Matrix-core assign for bf16 inputs. A workgroup of NW waves takes `tpg` consecutive
// tiles of 64*NW points of one head and keeps the centroid tables in LDS across them.
//
// Scores: with the accumulator preset to -||c_j||^2 / 2, the product C X^T gives
// x.c_j - ||c_j||^2/2 = (||x||^2 - ||x - c_j||^2) / 2, so the nearest centroid is the
// largest score. Lane (c, h) of a 32 x 32 tile holds 16 centroid rows of point c; each
// wave scores its 64 points as two 32-point groups that share every centroid fragment.
// Each score is ranked as a key that carries its lane-local slot in the 6 low mantissa
// bits; a running best and second best per lane (max3 / med3 over pairs of keys) are
// merged with the partner lane l^32. The error bound E in distance covers the matrix
// product (bf16 hi + lo centroids, fp32 sums) and the key truncation with a wide
// margin, and is E/2 in score; a second centroid within E of the best (2E in distance)
// sends the point to the exact rescoring, where
// the whole wave computes the fp32 direct-form distance of each candidate (lanes over
// d, fixed-order tree sum).
//
// Cluster sums psum^T [D x C] = X^T onehot run on the matrix cores too: the tile's rows
// sit row-major in LDS and reach the A operand through the transpose read; the one-hot
// B operand is built from the tile's labels with packed 16-bit integer operations, whose
// per-lane tallies of mismatches give the cluster counts as well. Wave w owns a
// fixed set of output tiles (one cluster tile and all D/32 feature tiles when NW = 4),
// accumulated over all tiles of the group and written once.
//
// Dynamic LDS: c_hi, c_lo [Cp][D] bf16 (16-byte chunks XOR-swizzled by row) | bias [Cp] |
// X tile [64 NW][XST] bf16 | labels [64 NW] u16 | counts [C] | sort buffers.
constexpr int kCandMax = 64;  // rescoring candidates listed per wave and round

template <int D, int NW>
struct KmMfmaCfg {
  static constexpr int NKS = D / 16;
  static constexpr int XST = D == 64 ? D + 8 : D + 16;
  static constexpr int NDT = D / 32;
  static constexpr int TILE = 64 * NW;
  // cluster tiles per wave and pass (at most 4 accumulator tiles), output tiles per wave
  static constexpr int CPW = (4 / NDT) < (4 + NW - 1) / NW ? (4 / NDT) : (4 + NW - 1) / NW;
  static constexpr int OPW = CPW * NDT;
  static size_t lds_bytes(int Cmax) {
    const size_t Cp = (Cmax + 31) & ~31;
    return Cp * D * 2 * sizeof(uint16_t) + Cp * sizeof(float) + static_cast<size_t>(TILE) * XST * sizeof(uint16_t) +
           TILE * sizeof(uint16_t) + sizeof(int) * (Cmax + 2 * TILE + NW * Cmax + 2 * Cmax + NW * kCandMax);
  }
  static int passes(int Cmax) { return ((Cmax + 31) / 32 + NW * CPW - 1) / (NW * CPW); }
};

// bf16 one-hot of eight 16-bit labels against label j: per 16-bit half,
// m = min(lab ^ j, 1) is 0 exactly where lab == j, and 0x3F80 - 0x3F80 m is bf16 1.0
// there and 0 elsewhere (labels and j are below 2^15). The m are also summed into the
// packed 16-bit counters `miss` (mismatches per half), from which the cluster counts
// follow.
__device__ __forceinline__ bf16x8_t onehot_bf16x8(const u16x8_t& lab8, uint32_t jj, uint32_t one2, uint32_t neg2,
                                                  uint32_t val2, uint32_t& miss) {
  const uint32_t* p = reinterpret_cast<const uint32_t*>(&lab8);
  uint32_t o[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t m;
    asm volatile(
        "v_xor_b32 %0, %2, %3\n\tv_pk_min_u16 %0, %0, %4\n\tv_pk_add_u16 %1, %1, %0\n\tv_pk_mad_u16 %0, %0, %5, %6"
        : "=&v"(m), "+v"(miss)
        : "v"(p[q]), "v"(jj), "v"(one2), "v"(neg2), "v"(val2));
    o[q] = m;
  }
  return __builtin_bit_cast(bf16x8_t, o);
}

// The same one-hot without the mismatch tallies (counts kept elsewhere): three packed
// operations per pair of labels.
__device__ __forceinline__ bf16x8_t onehot_bf16x8_nc(const u16x8_t& lab8, uint32_t jj, uint32_t one2, uint32_t neg2,
                                                     uint32_t val2) {
  const uint32_t* p = reinterpret_cast<const uint32_t*>(&lab8);
  uint32_t o[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t m;
    asm volatile("v_xor_b32 %0, %1, %2\n\tv_pk_min_u16 %0, %0, %3\n\tv_pk_mad_u16 %0, %0, %4, %5"
                 : "=&v"(m)
                 : "v"(p[q]), "v"(jj), "v"(one2), "v"(neg2), "v"(val2));
    o[q] = m;
  }
  return __builtin_bit_cast(bf16x8_t, o);
}

template <int D, int NW, int NJT>
__device__ __forceinline__ void km_assign_body(const KmArgs& a, int iter, int last, unsigned char* smem) {
  using Cfg = KmMfmaCfg<D, NW>;
  constexpr int NKS = Cfg::NKS, XST = Cfg::XST, NDT = Cfg::NDT, TILE = Cfg::TILE, CPW = Cfg::CPW, OPW = Cfg::OPW;
  constexpr int MAXJT = NJT, njt = NJT;  // centroid tiles of 32
  const KmTensor& t = a.t[blockIdx.z];
  const int C = t.C, Cp = 32 * NJT;
  const int grp = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, h = lane >> 5, c = lane & 31;
  if (grp >= t.ngroups) return;  // this tensor needs fewer workgroups
  const int tt0 = grp * t.tpg, tt1 = min(a.ntiles, tt0 + t.tpg);
  uint16_t* chi = reinterpret_cast<uint16_t*>(smem);
  uint16_t* clo = chi + Cp * D;
  float* bias = reinterpret_cast<float*>(clo + Cp * D);
  uint16_t* sX = reinterpret_cast<uint16_t*>(bias + Cp);
  uint16_t* slab = sX + TILE * XST;
  int* s_gcnt = reinterpret_cast<int*>(slab + TILE);
  int* s_lab = s_gcnt + C;
  int* s_whist = s_lab + TILE;
  int* s_cnt = s_whist + NW * C;
  int* s_start = s_cnt + C;
  int* s_sorted = s_start + C;
  int* s_cand = s_sorted + TILE;  // [NW][kCandMax] rescoring candidates: (tile row << 8) | j
  const uint16_t* X = static_cast<const uint16_t*>(t.x) + static_cast<size_t>(bh) * a.N * D;
  const float* cent = t.cent + static_cast<size_t>(bh) * C * D;
  // this wave's points of tile tt: group gi, lane (c, h) -> point 64 wave + 32 gi + c, dims 16 ks + 8 h
  u16x8_t xf[2][NKS];
  auto load_x = [&](int tt) {
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
      const long p = static_cast<long>(tt) * TILE + wave * 64 + gi * 32 + c;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        xf[gi][ks] = u16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
        if (p < a.N) xf[gi][ks] = *reinterpret_cast<const u16x8_t*>(X + static_cast<size_t>(p) * D + 16 * ks + 8 * h);
      }
    }
  };
  const bool score = t.labels_in == nullptr;
  if (tt0 < tt1) load_x(tt0);  // the first tile's rows travel while the tables are staged

  if (score) {
    const uint16_t* ghi = t.chi + static_cast<size_t>(bh) * C * D;
    const uint16_t* glo = t.clo + static_cast<size_t>(bh) * C * D;
#pragma unroll
    for (int e = tid; e < Cp * (D / 8); e += TILE) {
      const int j = e / (D / 8), c8 = e % (D / 8);
      u16x8_t h8 = {0, 0, 0, 0, 0, 0, 0, 0}, l8 = {0, 0, 0, 0, 0, 0, 0, 0};
      if (j < C) {
        h8 = *reinterpret_cast<const u16x8_t*>(ghi + static_cast<size_t>(j) * D + c8 * 8);
        l8 = *reinterpret_cast<const u16x8_t*>(glo + static_cast<size_t>(j) * D + c8 * 8);
      }
      const int dst = j * D + ((c8 ^ (j & 7)) << 3);
      *reinterpret_cast<u16x8_t*>(chi + dst) = h8;
      *reinterpret_cast<u16x8_t*>(clo + dst) = l8;
    }
    // padding centroids: a finite score far below any real one (their rank keys must
    // not be NaN)
    for (int j = tid; j < Cp; j += TILE) bias[j] = j < C ? -0.5f * t.cn2[static_cast<size_t>(bh) * C + j] : -1e30f;
  }
  __syncthreads();
  float cmax2 = 0.f;
  if (score) {
    for (int j = lane; j < C; j += 64) cmax2 = fmaxf(cmax2, -2.f * bias[j]);
    cmax2 = wave_max(cmax2);
  }
  const float cmax = sqrtf(cmax2);

  f32x16_t acc[OPW];
  uint32_t miss[CPW];  // packed per-half mismatch counts of the one-hot operand
  int nks = 0;         // one-hot steps accumulated (8 labels per lane each)
#pragma unroll
  for (int r = 0; r < OPW; ++r) acc[r] = zero16();
#pragma unroll
  for (int r = 0; r < CPW; ++r) miss[r] = 0u;
  const int npass = (njt + NW * CPW - 1) / (NW * CPW);

  // scores of centroid tile jt for both groups, accumulator preset to the bias
  auto score_tile = [&](int jt, f32x16_t& s0, f32x16_t& s1) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4_t b4 = *reinterpret_cast<const f32x4_t*>(bias + 32 * jt + 8 * q + 4 * h);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s0[4 * q + e] = b4[e];
        s1[4 * q + e] = b4[e];
      }
    }
    const int jr = 32 * jt + c;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int off = jr * D + (((2 * ks + h) ^ (c & 7)) << 3);
      const bf16x8_t ah = as_bf16x8(*reinterpret_cast<const u16x8_t*>(chi + off));
      const bf16x8_t al = as_bf16x8(*reinterpret_cast<const u16x8_t*>(clo + off));
      s0 = mfma32(ah, as_bf16x8(xf[0][ks]), s0);
      s1 = mfma32(ah, as_bf16x8(xf[1][ks]), s1);
      s0 = mfma32(al, as_bf16x8(xf[0][ks]), s0);
      s1 = mfma32(al, as_bf16x8(xf[1][ks]), s1);
    }
  };

  for (int tt = tt0; tt < tt1; ++tt) {
#pragma unroll
    for (int gi = 0; gi < 2; ++gi)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        *reinterpret_cast<u16x8_t*>(sX + (wave * 64 + gi * 32 + c) * XST + 16 * ks + 8 * h) = xf[gi][ks];
    const long n = static_cast<long>(tt) * TILE + tid;
    const bool valid = n < a.N;
    int lab = C;
    if (!score) {
      if (valid) lab = min(max(t.labels_in[static_cast<size_t>(bh) * a.N + n], 0), C - 1);
    } else {
      float xx[2];
#pragma unroll
      for (int gi = 0; gi < 2; ++gi) {
        float s = 0.f;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
          typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const u16x2 uu = {xf[gi][ks][2 * e], xf[gi][ks][2 * e + 1]};
            const bf16x2_t xv = __builtin_bit_cast(bf16x2_t, uu);
            s = __builtin_amdgcn_fdot2_f32_bf16(xv, xv, s, false);
          }
        }
        xx[gi] = s + xor32(s);
      }
      // rank keys: the score with its 6 low mantissa bits replaced by the lane-local
      // slot 16 jt + v (relative change below 2^-17, inside the rescoring window), so
      // that a max carries its slot; top two of a pair of keys per step:
      //   best' = max3(best, k0, k1),  second' = max(second, med3(best, k0, k1))
      const float kLow = -3.0e38f;
      float best[2] = {kLow, kLow}, second[2] = {kLow, kLow};
      auto rkey = [](float x, int slot) {
        return __builtin_bit_cast(float, (__builtin_bit_cast(uint32_t, x) & ~63u) | static_cast<uint32_t>(slot));
      };
      // tile jt + 1 goes to the matrix cores while tile jt is ranked; the centroid-tile
      // loop has compile-time bounds, and a scheduling barrier per step keeps the
      // compiler from hoisting later tiles (register pressure)
      f32x16_t sa0, sa1;
      score_tile(0, sa0, sa1);
#pragma unroll
      for (int jt = 0; jt < NJT; ++jt) {
        f32x16_t sb0, sb1;
        if (jt + 1 < NJT) score_tile(jt + 1, sb0, sb1);
#pragma unroll
        for (int v = 0; v < 16; v += 2) {
          const float a0 = rkey(sa0[v], 16 * jt + v), a1 = rkey(sa0[v + 1], 16 * jt + v + 1);
          const float b0 = rkey(sa1[v], 16 * jt + v), b1 = rkey(sa1[v + 1], 16 * jt + v + 1);
          second[0] = fmaxf(second[0], __builtin_amdgcn_fmed3f(best[0], a0, a1));
          best[0] = fmaxf(best[0], fmaxf(a0, a1));
          second[1] = fmaxf(second[1], __builtin_amdgcn_fmed3f(best[1], b0, b1));
          best[1] = fmaxf(best[1], fmaxf(b0, b1));
        }
        __builtin_amdgcn_sched_barrier(0);
        if (jt + 1 < NJT) {
          sa0 = sb0;
          sa1 = sb1;
        }
      }
      int bj[2];
      bool need[2];
      float E[2];
#pragma unroll
      for (int gi = 0; gi < 2; ++gi) {
        const int sl = static_cast<int>(__builtin_bit_cast(uint32_t, best[gi]) & 63u);
        bj[gi] = 32 * (sl >> 4) + 8 * ((sl >> 2) & 3) + 4 * h + (sl & 3);
        const float ob = xor32(best[gi]);
        const float os = xor32(second[gi]);
        const int oj = xor32(bj[gi]);
        if (ob > best[gi] || (ob == best[gi] && oj < bj[gi])) {
          second[gi] = best[gi] > os ? best[gi] : os;
          best[gi] = ob;
          bj[gi] = oj;
        } else {
          second[gi] = second[gi] > ob ? second[gi] : ob;
        }
        // distance error bound E; scores carry half of it
        E[gi] = 1e-4f * sqrtf(xx[gi]) * cmax + (2e-5f * (D / 64)) * cmax2;  // the max|c|^2 part grows with the 2D + 1 summed terms
        const long p = static_cast<long>(tt) * TILE + wave * 64 + gi * 32 + c;
        need[gi] = p < a.N && second[gi] >= best[gi] - E[gi];
      }
      // a second centroid within the window: re-score every candidate exactly, fp32
      // direct form sum_d (x_d - c_jd)^2 with lanes over d and a fixed-order tree sum
      if (__ballot(need[0] || need[1]) != 0ull) {
        uint64_t cm[2] = {0ull, 0ull};  // candidate slots 16 jt + v of this lane
        for (int jt = 0; jt < njt; ++jt) {
          f32x16_t s0, s1;
          score_tile(jt, s0, s1);
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            if (need[0] && s0[v] >= best[0] - E[0]) cm[0] |= 1ull << (16 * jt + v);
            if (need[1] && s1[v] >= best[1] - E[1]) cm[1] |= 1ull << (16 * jt + v);
          }
        }
        float fb[2] = {__builtin_huge_valf(), __builtin_huge_valf()};
        int fj[2] = {C, C};
        // list the wave's (point, candidate) pairs (uniform loops over the lanes that hold
        // candidates), then evaluate them eight at a time with all centroid-row loads of a
        // batch in flight together
        int* clist = s_cand + wave * kCandMax;
        int tot = 0;
#pragma unroll
        for (int gi = 0; gi < 2; ++gi) {
          uint64_t lanes = __ballot(cm[gi] != 0ull);
          while (lanes != 0ull) {
            const int L = __ffsll(static_cast<unsigned long long>(lanes)) - 1;
            lanes &= lanes - 1;
            const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(cm[gi]), L);
            const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(cm[gi] >> 32), L);
            uint64_t m = (static_cast<uint64_t>(hi) << 32) | lo;
            const int row = wave * 64 + gi * 32 + (L & 31), hL = L >> 5;
            while (m != 0ull) {
              const int sl = __ffsll(static_cast<unsigned long long>(m)) - 1;
              m &= m - 1;
              if (lane == 0 && tot < kCandMax)
                clist[tot] = (row << 8) | (32 * (sl >> 4) + 8 * ((sl >> 2) & 3) + 4 * hL + (sl & 3));
              ++tot;
            }
          }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const int nl = min(tot, kCandMax);
        for (int b0 = 0; b0 < nl; b0 += 8) {
          int ent[8];
          float part[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            ent[q] = b0 + q < nl ? clist[b0 + q] : -1;
            part[q] = 0.f;
          }
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            if (ent[q] < 0) continue;
            const float* cr = cent + static_cast<size_t>(ent[q] & 255) * D;
            const uint16_t* xr = sX + (ent[q] >> 8) * XST;
#pragma unroll
            for (int d = lane; d < D; d += 64) {
              const float diff = bf16_to_f32(xr[d]) - cr[d];
              part[q] = fmaf(diff, diff, part[q]);
            }
          }
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            if (ent[q] < 0) continue;
            const float dist = wave_sum(part[q]);
            const int j = ent[q] & 255, pl = (ent[q] >> 8) - wave * 64;
            if (c == (pl & 31)) {
              const int gq = pl >> 5;
              const float f = gq == 0 ? fb[0] : fb[1];
              const int jj = gq == 0 ? fj[0] : fj[1];
              if (dist < f || (dist == f && j < jj)) {
                if (gq == 0) {
                  fb[0] = dist;
                  fj[0] = j;
                } else {
                  fb[1] = dist;
                  fj[1] = j;
                }
              }
            }
          }
        }
        if (tot > kCandMax) {
          // more candidates than the list holds (rare): one lane's candidates at a time
#pragma unroll
          for (int gi = 0; gi < 2; ++gi) {
            uint64_t lanes = __ballot(cm[gi] != 0ull);
            while (lanes != 0ull) {
              const int L = __ffsll(static_cast<unsigned long long>(lanes)) - 1;
              lanes &= lanes - 1;
              const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(cm[gi]), L);
              const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(cm[gi] >> 32), L);
              uint64_t m = (static_cast<uint64_t>(hi) << 32) | lo;
              const int cL = L & 31, hL = L >> 5;
              const uint16_t* xr = sX + (wave * 64 + gi * 32 + cL) * XST;
              while (m != 0ull) {
                const int sl = __ffsll(static_cast<unsigned long long>(m)) - 1;
                m &= m - 1;
                const int j = 32 * (sl >> 4) + 8 * ((sl >> 2) & 3) + 4 * hL + (sl & 3);
                const float* cr = cent + static_cast<size_t>(j) * D;
                float part = 0.f;
#pragma unroll
                for (int d = lane; d < D; d += 64) {
                  const float diff = bf16_to_f32(xr[d]) - cr[d];
                  part = fmaf(diff, diff, part);
                }
                const float dist = wave_sum(part);
                if (c == cL && (dist < fb[gi] || (dist == fb[gi] && j < fj[gi]))) {
                  fb[gi] = dist;
                  fj[gi] = j;
                }
              }
            }
          }
        }
#pragma unroll
        for (int gi = 0; gi < 2; ++gi)
          if (need[gi] && fj[gi] < C) bj[gi] = fj[gi];
      }
      if (valid) lab = h == 0 ? bj[0] : bj[1];
    }
    // the scores no longer need this tile's fragments: fetch the next tile's now
    if (tt + 1 < tt1) load_x(tt + 1);
    if (valid) {
      t.labels[static_cast<size_t>(bh) * a.N + n] = lab;
      if (t.trace != nullptr) t.trace[(static_cast<size_t>(iter) * a.BH + bh) * a.N + n] = lab;
    }
    slab[tid] = valid ? static_cast<uint16_t>(lab) : static_cast<uint16_t>(0xFFFF);
    if (last) tile_sort(a, t, lab, valid, static_cast<int>(threadIdx.x), tt, s_whist, s_cnt, s_start, s_sorted);
    __syncthreads();  // X tile and labels complete

    for (int pass = 0; pass < npass; ++pass) {
      if (npass > 1) {
#pragma unroll
        for (int r = 0; r < OPW; ++r) acc[r] = zero16();
#pragma unroll
        for (int r = 0; r < CPW; ++r) miss[r] = 0u;
        nks = 0;
      }
      const int ct0 = (pass * NW + wave) * CPW;
      const int nct = min(CPW, njt - ct0);  // uniform; may be <= 0
      if (nct > 0) {
        uint32_t jj[CPW];
#pragma unroll
        for (int rc = 0; rc < CPW; ++rc) jj[rc] = (32u * (ct0 + rc) + c) * 0x10001u;
        const uint32_t one2 = 0x00010001u, neg2 = 0xC080C080u, val2 = 0x3F803F80u;
#pragma unroll 4
        for (int ks = 0; ks < TILE / 16; ++ks) {
          const u16x8_t lab8 = *reinterpret_cast<const u16x8_t*>(slab + 16 * ks + 8 * h);
          bf16x8_t ax[NDT];
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) ax[dt] = lds_operand_tr(sX, XST, 16 * ks, 32 * dt, lane);
#pragma unroll
          for (int rc = 0; rc < CPW; ++rc) {
            if (rc > 0 && rc >= nct) break;
            const bf16x8_t oh = onehot_bf16x8(lab8, jj[rc], one2, neg2, val2, miss[rc]);
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) acc[rc * NDT + dt] = mfma32(ax[dt], oh, acc[rc * NDT + dt]);
          }
        }
      }
      nks += TILE / 16;
      if (npass > 1 || tt + 1 == tt1) {
        // sums and counts of this group (npass > 1 only with one tile per group)
        float* psum = t.psum + (static_cast<size_t>(bh) * a.ntiles + grp) * C * D;
#pragma unroll
        for (int rc = 0; rc < CPW; ++rc) {
          const int j = 32 * (ct0 + rc) + c;
          // lane (c, h) saw 8 nks labels against cluster j
          const int hit = 8 * nks - static_cast<int>((miss[rc] & 0xFFFFu) + (miss[rc] >> 16));
          const int cnt = hit + xor32(hit);
          if (j >= C || nct <= rc) continue;
          if (h == 0) t.gcnt[(static_cast<size_t>(bh) * a.ntiles + grp) * C + j] = cnt;
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const f32x4_t f = {acc[rc * NDT + dt][4 * q], acc[rc * NDT + dt][4 * q + 1], acc[rc * NDT + dt][4 * q + 2],
                                 acc[rc * NDT + dt][4 * q + 3]};
              *reinterpret_cast<f32x4_t*>(psum + static_cast<size_t>(j) * D + 32 * dt + 8 * q + 4 * h) = f;
            }
        }
      }
    }
    __syncthreads();  // the next tile overwrites the X tile and labels
  }
}

// Matrix-core assign for bf16 inputs over 256-point tiles, eight waves of 32 points
// each. Same method as km_assign_body; each wave scores one 32-point group (half the
// registers of the 64-point waves), so that more waves share a SIMD to hide latency:
// two workgroups per compute unit (four waves per SIMD) with D = 64, one (two waves per
// SIMD) with D = 128, whose centroid tables fill most of the LDS. The cluster sums are
// split over (cluster tile, feature tile) outputs: the two waves 2 t, 2 t + 1 of cluster
// tile t take half of its D / 32 feature tiles each, under one one-hot operand. Lane
// (c, h) of wave w holds point 32 w + c (features 16 ks + 8 h); the lanes h = 0 own the
// points for labels and sorting.
constexpr int kW8 = 8;  // waves per workgroup of the 32-point-per-wave assign
template <int D>
struct Km8Cfg {
  static constexpr int NKS = D / 16, XST = D == 64 ? D + 8 : D + 16, NDT = D / 32, NW = kW8, TILE = 32 * kW8,
                       NT = 64 * kW8;
  static constexpr int OPW = NDT / 2;  // cluster-sum outputs (feature tiles) per wave
  static size_t lds_bytes(int Cmax) {
    const size_t Cp = (Cmax + 31) & ~31;
    return Cp * D * 2 * sizeof(uint16_t) + Cp * sizeof(float) + static_cast<size_t>(TILE) * XST * sizeof(uint16_t) +
           TILE * sizeof(uint16_t) + sizeof(int) * (NW * Cmax + 3 * Cmax + TILE);
  }
};

template <int D, int NJT>
__device__ __forceinline__ void km_assign_body8(const KmArgs& a, int iter, int last, unsigned char* smem) {
  using Cfg = Km8Cfg<D>;
  constexpr int NKS = Cfg::NKS, XST = Cfg::XST, NW = Cfg::NW, TILE = Cfg::TILE, NT = Cfg::NT, OPW = Cfg::OPW;
  constexpr int njt = NJT;  // centroid tiles of 32
  const KmTensor& t = a.t[blockIdx.z];
  const int C = t.C, Cp = 32 * NJT;
  const int grp = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, h = lane >> 5, c = lane & 31;
  if (grp >= t.ngroups) return;  // this tensor needs fewer workgroups
  const int tt0 = grp * t.tpg, tt1 = min(a.ntiles, tt0 + t.tpg);
  uint16_t* chi = reinterpret_cast<uint16_t*>(smem);
  uint16_t* clo = chi + Cp * D;
  float* bias = reinterpret_cast<float*>(clo + Cp * D);
  uint16_t* sX = reinterpret_cast<uint16_t*>(bias + Cp);
  uint16_t* slab = sX + TILE * XST;
  int* s_whist = reinterpret_cast<int*>(slab + TILE);
  int* s_cnt = s_whist + NW * C;
  int* s_start = s_cnt + C;
  int* s_sorted = s_start + C;
  int* s_gcnt = s_sorted + TILE;  // [C] members of each cluster in the group's tiles
  const uint16_t* X = static_cast<const uint16_t*>(t.x) + static_cast<size_t>(bh) * a.N * D;
  const float* cent = t.cent + static_cast<size_t>(bh) * C * D;
  const int pw = 32 * wave + c;  // this lane's point within the tile
  u16x8_t xf[NKS];
  auto load_x = [&](int tt) {
    const long p = static_cast<long>(tt) * TILE + pw;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      xf[ks] = u16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
      if (p < a.N) xf[ks] = *reinterpret_cast<const u16x8_t*>(X + static_cast<size_t>(p) * D + 16 * ks + 8 * h);
    }
  };
  const bool score = t.labels_in == nullptr;
  if (tt0 < tt1) load_x(tt0);  // the first tile's rows travel while the tables are staged

  if (score) {
    const uint16_t* ghi = t.chi + static_cast<size_t>(bh) * C * D;
    const uint16_t* glo = t.clo + static_cast<size_t>(bh) * C * D;
#pragma unroll
    for (int e = tid; e < Cp * (D / 8); e += NT) {
      const int j = e / (D / 8), c8 = e % (D / 8);
      u16x8_t h8 = {0, 0, 0, 0, 0, 0, 0, 0}, l8 = {0, 0, 0, 0, 0, 0, 0, 0};
      if (j < C) {
        h8 = *reinterpret_cast<const u16x8_t*>(ghi + static_cast<size_t>(j) * D + c8 * 8);
        l8 = *reinterpret_cast<const u16x8_t*>(glo + static_cast<size_t>(j) * D + c8 * 8);
      }
      const int dst = j * D + ((c8 ^ (j & 7)) << 3);
      *reinterpret_cast<u16x8_t*>(chi + dst) = h8;
      *reinterpret_cast<u16x8_t*>(clo + dst) = l8;
    }
    // padding centroids: a finite score far below any real one (their rank keys must
    // not be NaN)
    for (int j = tid; j < Cp; j += NT) bias[j] = j < C ? -0.5f * t.cn2[static_cast<size_t>(bh) * C + j] : -1e30f;
  }
  for (int j = tid; j < C; j += NT) s_gcnt[j] = 0;
  __syncthreads();
  float cmax2 = 0.f;
  if (score) {
    for (int j = lane; j < C; j += 64) cmax2 = fmaxf(cmax2, -2.f * bias[j]);
    cmax2 = wave_max(cmax2);
  }
  const float cmax = sqrtf(cmax2);

  // cluster sums: wave -> cluster tile wave / 2, feature tiles odt0 .. odt0 + OPW - 1; the
  // counts come from an LDS histogram of the labels (s_gcnt)
  const int oct = wave / 2, odt0 = (wave % 2) * OPW;
  const bool owns = oct < njt;
  f32x16_t acc[OPW];
#pragma unroll
  for (int r = 0; r < OPW; ++r) acc[r] = zero16();

  // scores of centroid tile jt for this wave's group, accumulator preset to the bias
  auto score_tile = [&](int jt, f32x16_t& s0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4_t b4 = *reinterpret_cast<const f32x4_t*>(bias + 32 * jt + 8 * q + 4 * h);
#pragma unroll
      for (int e = 0; e < 4; ++e) s0[4 * q + e] = b4[e];
    }
    const int jr = 32 * jt + c;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int off = jr * D + (((2 * ks + h) ^ (c & 7)) << 3);
      const bf16x8_t ah = as_bf16x8(*reinterpret_cast<const u16x8_t*>(chi + off));
      const bf16x8_t al = as_bf16x8(*reinterpret_cast<const u16x8_t*>(clo + off));
      s0 = mfma32(ah, as_bf16x8(xf[ks]), s0);
      s0 = mfma32(al, as_bf16x8(xf[ks]), s0);
    }
  };

  for (int tt = tt0; tt < tt1; ++tt) {
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) *reinterpret_cast<u16x8_t*>(sX + pw * XST + 16 * ks + 8 * h) = xf[ks];
    const long n = static_cast<long>(tt) * TILE + pw;
    const bool valid = h == 0 && n < a.N;  // the lanes h = 0 own the points
    int lab = C;
    if (!score) {
      if (valid) lab = min(max(t.labels_in[static_cast<size_t>(bh) * a.N + n], 0), C - 1);
    } else {
      float xx;
      {
        float s2 = 0.f;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
          typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const u16x2 uu = {xf[ks][2 * e], xf[ks][2 * e + 1]};
            const bf16x2_t xv = __builtin_bit_cast(bf16x2_t, uu);
            s2 = __builtin_amdgcn_fdot2_f32_bf16(xv, xv, s2, false);
          }
        }
        xx = s2 + xor32(s2);
      }
      // rank keys carry the lane-local slot 16 jt + v in their 6 low mantissa bits
      const float kLow = -3.0e38f;
      float best = kLow, second = kLow;
      auto rkey = [](float x, int slot) {
        return __builtin_bit_cast(float, (__builtin_bit_cast(uint32_t, x) & ~63u) | static_cast<uint32_t>(slot));
      };
      // tile jt + 1 goes to the matrix cores while tile jt is ranked
      f32x16_t sa;
      score_tile(0, sa);
#pragma unroll
      for (int jt = 0; jt < NJT; ++jt) {
        f32x16_t sb;
        if (jt + 1 < NJT) score_tile(jt + 1, sb);
#pragma unroll
        for (int v = 0; v < 16; v += 2) {
          const float a0 = rkey(sa[v], 16 * jt + v), a1 = rkey(sa[v + 1], 16 * jt + v + 1);
          second = fmaxf(second, __builtin_amdgcn_fmed3f(best, a0, a1));
          best = fmaxf(best, fmaxf(a0, a1));
        }
        __builtin_amdgcn_sched_barrier(0);
        if (jt + 1 < NJT) sa = sb;
      }
      int bj;
      bool need;
      float E;
      {
        const int sl = static_cast<int>(__builtin_bit_cast(uint32_t, best) & 63u);
        bj = 32 * (sl >> 4) + 8 * ((sl >> 2) & 3) + 4 * h + (sl & 3);
        const float ob = xor32(best);
        const float os = xor32(second);
        const int oj = xor32(bj);
        if (ob > best || (ob == best && oj < bj)) {
          second = best > os ? best : os;
          best = ob;
          bj = oj;
        } else {
          second = second > ob ? second : ob;
        }
        // distance error bound E; scores carry half of it
        E = 1e-4f * sqrtf(xx) * cmax + (2e-5f * (D / 64)) * cmax2;  // the max|c|^2 part grows with the 2D + 1 summed terms
        need = n < a.N && second >= best - E;
      }
      // a second centroid within the window: every candidate within it is re-scored with
      // the fp32 direct form sum_d (x_d - c_jd)^2 (lanes over d, fixed-order tree sum),
      // one (point, candidate) pair at a time; the smallest distance (then index) wins
      if (__ballot(need) != 0ull) {
        uint64_t cm = 0ull;  // candidate slots 16 jt + v of this lane
        for (int jt = 0; jt < njt; ++jt) {
          f32x16_t s0;
          score_tile(jt, s0);
#pragma unroll
          for (int v = 0; v < 16; ++v)
            if (need && s0[v] >= best - E) cm |= 1ull << (16 * jt + v);
        }
        float fb = __builtin_huge_valf();
        int fj = C;
        uint64_t lanes = __ballot(cm != 0ull);
        while (lanes != 0ull) {
          const int L = __ffsll(static_cast<unsigned long long>(lanes)) - 1;
          lanes &= lanes - 1;
          const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(cm), L);
          const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(cm >> 32), L);
          uint64_t m = (static_cast<uint64_t>(hi) << 32) | lo;
          const int cL = L & 31, hL = L >> 5;
          const uint16_t* xr = sX + (32 * wave + cL) * XST;
          while (m != 0ull) {
            const int sl = __ffsll(static_cast<unsigned long long>(m)) - 1;
            m &= m - 1;
            const int j = 32 * (sl >> 4) + 8 * ((sl >> 2) & 3) + 4 * hL + (sl & 3);
            const float* cr = cent + static_cast<size_t>(j) * D;
            float part = 0.f;
#pragma unroll
            for (int d = lane; d < D; d += 64) {
              const float diff = bf16_to_f32(xr[d]) - cr[d];
              part = fmaf(diff, diff, part);
            }
            const float dist = wave_sum(part);
            if (c == cL && (dist < fb || (dist == fb && j < fj))) {
              fb = dist;
              fj = j;
            }
          }
        }
        if (need && fj < C) bj = fj;
      }
      if (valid) lab = bj;
    }
    // the scores no longer need this tile's fragments: fetch the next tile's now
    if (tt + 1 < tt1) load_x(tt + 1);
    if (valid) {
      t.labels[static_cast<size_t>(bh) * a.N + n] = lab;
      if (t.trace != nullptr) t.trace[(static_cast<size_t>(iter) * a.BH + bh) * a.N + n] = lab;
      atomicAdd(&s_gcnt[lab], 1);  // integer counts: exact in any order
    }
    if (h == 0) slab[pw] = valid ? static_cast<uint16_t>(lab) : static_cast<uint16_t>(0xFFFF);
    if (last) tile_sort(a, t, lab, valid, pw, tt, s_whist, s_cnt, s_start, s_sorted);
    __syncthreads();  // X tile and labels complete

    if (owns) {
      const uint32_t jj = (32u * oct + c) * 0x10001u;
      const uint32_t one2 = 0x00010001u, neg2 = 0xC080C080u, val2 = 0x3F803F80u;
#pragma unroll 4
      for (int ks = 0; ks < TILE / 16; ++ks) {
        const u16x8_t lab8 = *reinterpret_cast<const u16x8_t*>(slab + 16 * ks + 8 * h);
        bf16x8_t ax[OPW];  // requested before the one-hot is built
#pragma unroll
        for (int r = 0; r < OPW; ++r) ax[r] = lds_operand_tr(sX, XST, 16 * ks, 32 * (odt0 + r), lane);
        const bf16x8_t oh = onehot_bf16x8_nc(lab8, jj, one2, neg2, val2);
#pragma unroll
        for (int r = 0; r < OPW; ++r) acc[r] = mfma32(ax[r], oh, acc[r]);
      }
    }
    if (tt + 1 == tt1) {
      // sums and counts of this group
      float* psum = t.psum + (static_cast<size_t>(bh) * a.ntiles + grp) * C * D;
      const int j = 32 * oct + c;
      if (owns && j < C) {
#pragma unroll
        for (int r = 0; r < OPW; ++r)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x4_t f = {acc[r][4 * q], acc[r][4 * q + 1], acc[r][4 * q + 2], acc[r][4 * q + 3]};
            *reinterpret_cast<f32x4_t*>(psum + static_cast<size_t>(j) * D + 32 * (odt0 + r) + 8 * q + 4 * h) = f;
          }
      }
      for (int jc = tid; jc < C; jc += NT) t.gcnt[(static_cast<size_t>(bh) * a.ntiles + grp) * C + jc] = s_gcnt[jc];
    }
    __syncthreads();  // the next tile overwrites the X tile and labels
  }
}

template <int D>
__global__ void __launch_bounds__(64 * kW8, D == 64 ? 4 : 2) kmeans_assign_mfma8_kernel(KmArgs a, int iter, int last) {
  extern __shared__ __align__(16) unsigned char smem[];
  switch ((a.t[blockIdx.z].C + 31) / 32) {
    case 1: km_assign_body8<D, 1>(a, iter, last, smem); break;
    case 2: km_assign_body8<D, 2>(a, iter, last, smem); break;
    case 3: km_assign_body8<D, 3>(a, iter, last, smem); break;
    default: km_assign_body8<D, 4>(a, iter, last, smem); break;
  }
}

// The centroid-tile count is a template parameter of the body so that the score loop
// has no runtime bounds (the two tensors of one launch may differ).
template <int D, int NW>
__global__ void __launch_bounds__(64 * NW, D == 64 && NW == 4 ? 2 : 1) kmeans_assign_mfma_kernel(KmArgs a, int iter, int last) {
  extern __shared__ __align__(16) unsigned char smem[];
  switch ((a.t[blockIdx.z].C + 31) / 32) {
    case 1: km_assign_body<D, NW, 1>(a, iter, last, smem); break;
    case 2: km_assign_body<D, NW, 2>(a, iter, last, smem); break;
    case 3: km_assign_body<D, NW, 3>(a, iter, last, smem); break;
    default: km_assign_body<D, NW, 4>(a, iter, last, smem); break;
  }
}

// One wave per (centroid j, head, tensor), lanes over d: sum the tile-group partials in
// group order; the mean replaces c_j unless the cluster is empty.
template <int D>
__global__ void __launch_bounds__(64 * kUpdWaves) kmeans_update_kernel(KmArgs a) {
  const KmTensor& t = a.t[blockIdx.z];
  const int C = t.C, j = blockIdx.x * kUpdWaves + (threadIdx.x >> 6), bh = blockIdx.y;
  if (j >= C) return;
  const size_t tbase = static_cast<size_t>(bh) * a.ntiles;
  constexpr int nper = D / 64;
  float acc[2] = {0.f, 0.f};
  int cnt = 0;
  // sixteen groups' partials in flight at once, summed in group order
  constexpr int UB = 16;
  for (int t0 = 0; t0 < t.ngroups; t0 += UB) {
    float p0[UB], p1[UB];
    int cn[UB];
#pragma unroll
    for (int q = 0; q < UB; ++q) {
      // unconditional loads (index clamped), so that all of them issue back to back
      const int tt = min(t0 + q, t.ngroups - 1);
      const float* ps = t.psum + ((tbase + tt) * C + j) * D;
      p0[q] = ps[lane_id()];
      p1[q] = nper > 1 ? ps[lane_id() + 64] : 0.f;
      cn[q] = t.gcnt[(tbase + tt) * C + j];
    }
#pragma unroll
    for (int q = 0; q < UB; ++q) {
      if (t0 + q < t.ngroups) {
        acc[0] += p0[q];
        acc[1] += p1[q];
        cnt += cn[q];
      }
    }
  }
  const size_t row = static_cast<size_t>(bh) * C + j;
  float vals[2];
  for (int q = 0; q < nper; ++q) {
    const int d = lane_id() + 64 * q;
    float v;
    if (cnt > 0) v = acc[q] / static_cast<float>(cnt);
    else v = t.labels_in != nullptr ? 0.f : t.cent[row * D + d];  // empty cluster keeps c_j
    t.cent[row * D + d] = v;
    vals[q] = v;
  }
  write_centroid_tables(t, D, row, vals, nper);
}

// One workgroup per (head, tensor): per (block, cluster) the exclusive prefix of the
// tile counts over the block's tiles (written over tile_cnt, which the scatter then
// reads in O(1)), the bucket totals, and their exclusive scan -> offs[nb*C + 1]
// (threads over consecutive buckets, then a scan of the thread totals). With items
// set, the same pass lists the atom work items (runs of at most kAtomSeg positions of
// a bucket), pads the list with empty items, lists the buckets of several items with
// their partial slots, and records per bucket its first partial slot and item count.
// With chunks set (query tensor), it lists the stage-2 chunks: runs of at most kS2Chunk
// positions of one bucket. With a cluster size cap (klen set), each bucket's kept length
// (a prefix of the bucket, since a cluster keeps its earliest members) goes to klen and
// the work items cover the kept prefixes only; the scatter then flags the left-out points.
template <int kBoThreads>
__global__ void __launch_bounds__(kBoThreads) bucket_offsets_kernel(KmArgs a) {
  const KmTensor& t = a.t[blockIdx.z];
  if (t.perm == nullptr) return;
  __shared__ int s_run[5][kBoThreads];
  const int C = t.C, bh = blockIdx.y, tid = threadIdx.x;
  const int nbC = a.nb * C;
  const bool segs = t.items != nullptr, chk = t.chunks != nullptr, capped = t.klen != nullptr;
  const int per = (nbC + kBoThreads - 1) / kBoThreads, e0 = min(nbC, tid * per), e1 = min(nbC, e0 + per);
  int* offs = t.offs + static_cast<size_t>(bh) * (nbC + 1);
  int* klen = capped ? t.klen + static_cast<size_t>(bh) * nbC : nullptr;
  int tot[5] = {0, 0, 0, 0, 0};  // positions, items, partial slots, buckets of several items, chunks
  // Each tile's count is replaced by the members of (b, j) in the block's earlier tiles.
  // Short blocks with many buckets per thread: the thread's (bucket, tile) pairs in order,
  // 32 count loads in flight per batch, with cursors (bucket e = b C + j, tile ti of the block) that advance without
  // divisions.
  const int tpb = a.tiles_per_block;
  const size_t tbase = static_cast<size_t>(bh) * a.ntiles;
  int32_t* tcb = t.tile_cnt + tbase * C;  // this head's [ntiles, C] counts
  // work items of a bucket of `kept` positions
  auto count_items = [&](int kept) {
    const int ni = max(1, (kept + kAtomSeg - 1) / kAtomSeg);
    tot[1] += ni;
    tot[2] += ni > 1 ? ni : 0;
    tot[3] += ni > 1 ? 1 : 0;
  };
  auto finish = [&](int e, int run) {
    offs[e] = run;  // bucket total for now (only this thread touches entry e)
    tot[0] += run;
    if (!capped) count_items(run);
    tot[4] += (run + kS2Chunk - 1) / kS2Chunk;
  };
  // long blocks (32 tiles or more, e.g. one block per head) or few buckets per thread:
  // bucket by bucket, up to 32 tile counts per batch at a fixed stride
  const bool by_bucket = tpb >= 32 || kBoThreads < 1024;
  auto by_bucket_pass = [&](auto width) {
    constexpr int W = decltype(width)::value;
    for (int e = e0; e < e1; ++e) {
      const int b = e / C, j = e % C, t0 = b * tpb, t1 = min(a.ntiles, t0 + tpb);
      int32_t* pc = tcb + static_cast<size_t>(t0) * C + j;
      int run = 0;
      for (int tt = t0; tt < t1; tt += W) {
        int cnt[W];
#pragma unroll
        for (int q = 0; q < W; ++q) cnt[q] = tt + q < t1 ? pc[static_cast<size_t>(tt - t0 + q) * C] : 0;
#pragma unroll
        for (int q = 0; q < W; ++q) {
          if (tt + q < t1) pc[static_cast<size_t>(tt - t0 + q) * C] = run;
          run += cnt[q];
        }
      }
      finish(e, run);
    }
  };
  if (by_bucket) {
    if (tpb >= 32) by_bucket_pass(std::integral_constant<int, 32>{});
    else by_bucket_pass(std::integral_constant<int, 8>{});
  }
  int le = e0, lb = e0 / C, lj = e0 % C, lti = 0;  // load cursor
  int pe = by_bucket ? e1 : e0, pb = lb, pj = lj, pti = 0;  // processing cursor
  int run = 0;
  while (pe < e1) {
    int cnt[32];
#pragma unroll
    for (int q = 0; q < 32; ++q) {
      // unconditional load at a clamped (in-bounds) address, zero when out of range;
      // branch-free cursor step
      const int tt = lb * tpb + lti;
      const bool ok = le < e1 && tt < a.ntiles;
      const int v = tcb[static_cast<uint32_t>(min(tt, a.ntiles - 1) * C + lj)];
      cnt[q] = ok ? v : 0;
      const bool wrap = ++lti == tpb;
      lti = wrap ? 0 : lti;
      le += wrap;
      lj += wrap;
      const bool wrapc = lj == C;
      lj = wrapc ? 0 : lj;
      lb += wrapc;
    }
#pragma unroll
    for (int q = 0; q < 32; ++q) {
      if (pe >= e1) break;
      const int tt = pb * tpb + pti;
      if (pti == 0) run = 0;
      if (tt < a.ntiles) tcb[static_cast<uint32_t>(tt * C + pj)] = run;
      run += cnt[q];
      if (++pti == tpb) {
        finish(pe, run);
        pti = 0;
        ++pe;
        if (++pj == C) {
          pj = 0;
          ++pb;
        }
      }
    }
  }
  if (capped) {
    // kept members: bucket (b, j) keeps what still fits under the cap after the members of
    // cluster j in the blocks before b (a thread per cluster, over the blocks in order,
    // 16 bucket totals in flight per batch)
    __syncthreads();  // every bucket total is in offs
    for (int j = tid; j < C; j += kBoThreads) {
      int seen = 0;
      for (int b0 = 0; b0 < a.nb; b0 += 16) {
        int n[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) n[q] = b0 + q < a.nb ? offs[(b0 + q) * C + j] : 0;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          if (b0 + q < a.nb) klen[(b0 + q) * C + j] = min(n[q], max(0, t.cap - seen));
          seen += n[q];
        }
      }
    }
    __syncthreads();
    for (int e = e0; e < e1; ++e) count_items(klen[e]);
  }
#pragma unroll
  for (int r = 0; r < 5; ++r) s_run[r][tid] = tot[r];
  __syncthreads();
  for (int o = 1; o < kBoThreads; o <<= 1) {
    int x[5];
#pragma unroll
    for (int r = 0; r < 5; ++r) x[r] = tid >= o ? s_run[r][tid - o] : 0;
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 5; ++r) s_run[r][tid] += x[r];
    __syncthreads();
  }
  int pos = s_run[0][tid] - tot[0], it = s_run[1][tid] - tot[1], pt = s_run[2][tid] - tot[2],
      mb = s_run[3][tid] - tot[3], ck = s_run[4][tid] - tot[4];
  int2* chunks = chk ? t.chunks + static_cast<size_t>(bh) * t.max_chunks : nullptr;
  const int max_items = atom_max_items(nbC, a.N);
  int4* items = segs ? t.items + static_cast<size_t>(bh) * max_items : nullptr;
  int4* multi = segs ? t.multi + static_cast<size_t>(bh) * (1 + atom_max_multi(a.N)) : nullptr;
  for (int e = e0; e < e1; ++e) {
    const int cnt = offs[e];
    offs[e] = pos;
    if (segs) {
      const int kept = capped ? klen[e] : cnt;  // the items cover the bucket's kept prefix
      const int ni = max(1, (kept + kAtomSeg - 1) / kAtomSeg);
      for (int q = 0; q < ni; ++q)
        items[it + q] = make_int4(pos + kAtomSeg * q, min(kAtomSeg, kept - kAtomSeg * q), ni > 1 ? pt + q : -1, e);
      if (ni > 1) multi[1 + mb++] = make_int4(e, pt, ni, 0);
      t.bmeta[static_cast<size_t>(bh) * nbC + e] = make_int2(ni > 1 ? pt : -1, ni);
      it += ni;
      pt += ni > 1 ? ni : 0;
    }
    if (chk)
      for (int st = 0; st < cnt; st += kS2Chunk) chunks[ck++] = make_int2(e, pos + st);
    pos += cnt;
  }
  if (tid == kBoThreads - 1) {
    offs[nbC] = s_run[0][kBoThreads - 1];
    if (chk) t.nchunks[bh] = s_run[4][kBoThreads - 1];
  }
  if (segs) {
    const int nit = s_run[1][kBoThreads - 1];
    for (int g = nit + tid; g < max_items; g += kBoThreads) items[g] = make_int4(0, -1, -1, 0);
    if (tid == kBoThreads - 1) multi[0] = make_int4(s_run[3][kBoThreads - 1], 0, 0, 0);
  }
}

// One workgroup per tile: scatter the tile's stably sorted points into the head's
// (block, label) buckets (and, with a cap, flag each point beyond its bucket's kept length).
__global__ void bucket_scatter_kernel(KmArgs a) {
  const KmTensor& t = a.t[blockIdx.z];
  if (t.perm == nullptr) return;
  const int C = t.C, bh = blockIdx.y, tt = blockIdx.x;
  const int b = tt / a.tiles_per_block;
  const size_t tix = static_cast<size_t>(bh) * a.ntiles + tt;
  const int* offs = t.offs + static_cast<size_t>(bh) * (a.nb * C + 1);
  const long tile0 = static_cast<long>(tt) * a.tile;
  const int npts = static_cast<int>(min(static_cast<long>(a.tile), a.N - tile0));
  for (int pos = threadIdx.x; pos < npts; pos += blockDim.x) {
    const int p = t.tile_perm[tix * a.tile + pos];
    const int j = t.labels[static_cast<size_t>(bh) * a.N + tile0 + p];
    const int rank = t.tile_cnt[tix * C + j] + (pos - t.tile_start[tix * C + j]);  // in the bucket
    t.perm[static_cast<size_t>(bh) * a.N + offs[b * C + j] + rank] = static_cast<int>(tile0 + p);
    if (t.kdrop != nullptr)
      t.kdrop[static_cast<size_t>(bh) * a.N + tile0 + p] =
          rank >= t.klen[static_cast<size_t>(bh) * a.nb * C + b * C + j] ? 1 : 0;
  }
}

// ------------------------------------------------------------------ host launchers

template <typename T>
static hipError_t launch_kmeans_t(const KmArgs& a, int iters, hipStream_t s) {
  const int Cmax = max(a.t[0].C, a.ntensors > 1 ? a.t[1].C : 0);
  {
    ProfScope ps_("kmeans_init", s);
    hipLaunchKernelGGL(kmeans_init_kernel<T>, dim3((Cmax + kUpdWaves - 1) / kUpdWaves, a.BH, a.ntensors),
                       dim3(64 * kUpdWaves), 0, s, a);
  }
  const size_t lds = static_cast<size_t>(kChunkC) * a.D * sizeof(float) +
                     sizeof(int) * (2 * a.tile + (a.tile / 64) * Cmax + 2 * Cmax);
  const dim3 g_assign(a.ntiles, a.BH, a.ntensors);
  const dim3 g_update((Cmax + kUpdWaves - 1) / kUpdWaves, a.BH, a.ntensors);
  const bool mf = sizeof(T) == 2;
  const int nw = a.tile / 64;
  KmArgs b = a;
  for (int z = 0; z < a.ntensors; ++z) {
    b.t[z].tpg = 1;
    b.t[z].ngroups = a.ntiles;
  }
  size_t lds_mfma = 0;
  int npass = 1;
#define MUSE_KM_CFG(DD, NN)                               \
  if (a.D == DD && nw == NN) {                            \
    lds_mfma = KmMfmaCfg<DD, NN>::lds_bytes(Cmax);        \
    npass = KmMfmaCfg<DD, NN>::passes(Cmax);              \
  }
  MUSE_KM_CFG(64, 1) MUSE_KM_CFG(64, 2) MUSE_KM_CFG(64, 3) MUSE_KM_CFG(64, 4)
  MUSE_KM_CFG(128, 1) MUSE_KM_CFG(128, 2) MUSE_KM_CFG(128, 3) MUSE_KM_CFG(128, 4)
#undef MUSE_KM_CFG
  if (mf && npass == 1) {
    // several tiles per workgroup amortise the centroid tables. Per tensor, the tiles per
    // workgroup are chosen so that the workgroups of both tensors take about as long
    // (a tile costs about 3 + C/32 units, staging the tables 3 + C/64) while all of them
    // fit on the device at once; when they cannot, about 512 workgroups of up to 8 tiles.
    int dev = 0, cus = 256;
    (void)hipGetDevice(&dev);
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    const long slots = static_cast<long>(cus) * (a.D == 64 && nw == 4 ? 2 : 1);
    const long total = static_cast<long>(a.ntiles) * a.BH * a.ntensors;
    const int tdef = static_cast<int>(std::min<long>(8, std::max<long>(1, total / 512)));
    int best[2] = {tdef, tdef};
    double best_time = 1e30;
    const int tmax = a.ntensors > 1 ? 8 : 1;
    for (int t0 = 1; t0 <= 8; ++t0)
      for (int t1 = 1; t1 <= tmax; ++t1) {
        const int tp[2] = {t0, t1};
        long wgs = 0;
        double tmx = 0.0;
        for (int z = 0; z < a.ntensors; ++z) {
          const double njt = (a.t[z].C + 31) / 32;
          wgs += static_cast<long>(a.BH) * ((a.ntiles + tp[z] - 1) / tp[z]);
          tmx = std::max(tmx, 3.0 + 0.5 * njt + tp[z] * (3.0 + njt));
        }
        if (wgs > slots) continue;
        if (tmx < best_time) {
          best_time = tmx;
          best[0] = t0;
          best[1] = t1;
        }
      }
    for (int z = 0; z < a.ntensors; ++z) {
      b.t[z].tpg = best_time < 1e30 ? best[z] : tdef;
      b.t[z].ngroups = (a.ntiles + b.t[z].tpg - 1) / b.t[z].tpg;
    }
  }
  b.ngroups = 0;
  for (int z = 0; z < a.ntensors; ++z) b.ngroups = std::max(b.ngroups, b.t[z].ngroups);
  const dim3 g_group(b.ngroups, a.BH, a.ntensors);
  // 256-point tiles: the eight-wave variant (32 points per wave)
  const bool w8 = a.tile == Km8Cfg<64>::TILE;
  auto launch_mfma = [&](int it) {
    const int last = it == iters - 1;
    if (w8 && a.D == 64) {
      const size_t lds8 = Km8Cfg<64>::lds_bytes(Cmax);
      allow_lds((const void*)kmeans_assign_mfma8_kernel<64>, lds8);
      hipLaunchKernelGGL((kmeans_assign_mfma8_kernel<64>), g_group, dim3(Km8Cfg<64>::NT), lds8, s, b, it, last);
      return;
    }
    if (w8) {
      const size_t lds8 = Km8Cfg<128>::lds_bytes(Cmax);
      allow_lds((const void*)kmeans_assign_mfma8_kernel<128>, lds8);
      hipLaunchKernelGGL((kmeans_assign_mfma8_kernel<128>), g_group, dim3(Km8Cfg<128>::NT), lds8, s, b, it, last);
      return;
    }
#define MUSE_KM_CASE(DD, NN)                                                                              \
  if (a.D == DD && nw == NN) {                                                                            \
    allow_lds((const void*)kmeans_assign_mfma_kernel<DD, NN>, lds_mfma);                                 \
    hipLaunchKernelGGL((kmeans_assign_mfma_kernel<DD, NN>), g_group, dim3(a.tile), lds_mfma, s, b, it, last); \
  }
    MUSE_KM_CASE(64, 1) MUSE_KM_CASE(64, 2) MUSE_KM_CASE(64, 3) MUSE_KM_CASE(64, 4)
    MUSE_KM_CASE(128, 1) MUSE_KM_CASE(128, 2) MUSE_KM_CASE(128, 3) MUSE_KM_CASE(128, 4)
#undef MUSE_KM_CASE
  };
  for (int it = 0; it < iters; ++it) {
    if (mf) {
      ProfScope ps_("kmeans_assign_mfma", s);
      launch_mfma(it);
    } else {
      ProfScope ps_("kmeans_assign", s);
      if (a.D == 64)
        hipLaunchKernelGGL((kmeans_assign_kernel<T, 64>), g_assign, dim3(a.tile), lds, s, b, it);
      else
        hipLaunchKernelGGL((kmeans_assign_kernel<T, 128>), g_assign, dim3(a.tile), lds, s, b, it);
    }
    {
      ProfScope ps_("kmeans_update", s);
      if (a.D == 64) hipLaunchKernelGGL(kmeans_update_kernel<64>, g_update, dim3(64 * kUpdWaves), 0, s, b);
      else hipLaunchKernelGGL(kmeans_update_kernel<128>, g_update, dim3(64 * kUpdWaves), 0, s, b);
    }
  }
  {
    ProfScope ps_("bucket_offsets", s);
    // threads over consecutive buckets: 1024 when there are thousands of buckets
    if (a.nb * Cmax >= 2048)
      hipLaunchKernelGGL(bucket_offsets_kernel<1024>, dim3(1, a.BH, a.ntensors), dim3(1024), 0, s, a);
    else
      hipLaunchKernelGGL(bucket_offsets_kernel<256>, dim3(1, a.BH, a.ntensors), dim3(256), 0, s, a);
  }
  {
    ProfScope ps_("bucket_scatter", s);
    hipLaunchKernelGGL(bucket_scatter_kernel, dim3(a.ntiles, a.BH, a.ntensors), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_kmeans(const KmArgs& a, int iters, int dtype, hipStream_t s) {
  return dtype == 0 ? launch_kmeans_t<float>(a, iters, s) : launch_kmeans_t<bf16>(a, iters, s);
}

}  // namespace muse
