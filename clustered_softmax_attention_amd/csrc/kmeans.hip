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
// bf16 inputs (kmeans_assign_mfma): the distance scores ||c_j||^2 - 2 x.c_j come from
// the matrix cores, with each fp32 centroid split into bf16 hi + lo parts (x is exact
// in bf16). Their error is bounded by E = 1e-4 ||x|| max||c|| + 2e-5 max||c||^2 (about
// 2.5x the worst case of the split residual 2^-16 and the fp32 accumulation); when a
// second centroid scores within 2E of the best, every such candidate is re-scored with
// the exact fp32 direct form sum_d (x_d - c_jd)^2 of the fp32 path, so labels are the
// same as the fp32 path's.
//
// Every sum runs in a fixed order, so labels and centroids are bitwise
// reproducible.
#include "mfma.hpp"
#include "muse_kernels.hpp"

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

// One wave per (centroid j, head, tensor): c_j = x[floor(j*N/C)].
template <typename T>
__global__ void __launch_bounds__(64) kmeans_init_kernel(KmArgs a) {
  const KmTensor& t = a.t[blockIdx.z];
  const int j = blockIdx.x, bh = blockIdx.y;
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

// Stable counting sort of the tile's points by label (LDS), then the tile's sort info
// and per-cluster sums. Called by every thread of the workgroup.
template <typename T, int D>
__device__ void tile_sort(const KmArgs& a, const KmTensor& t, int lab, bool valid, int* s_lab, int* s_whist,
                          int* s_cnt, int* s_start, int* s_sorted) {
  const int C = t.C;
  const int bh = blockIdx.y;
  const int tile = blockDim.x;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int nwaves = tile >> 6;
  const T* x = static_cast<const T*>(t.x) + static_cast<size_t>(bh) * a.N * D;
  for (int e = tid; e < nwaves * C; e += tile) s_whist[e] = 0;
  s_lab[tid] = lab;
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
  for (int j = tid; j < C; j += tile) {
    int run = 0;
    for (int w = 0; w < nwaves; ++w) {
      const int h = s_whist[w * C + j];
      s_whist[w * C + j] = run;  // becomes the wave's base inside the label's segment
      run += h;
    }
    s_cnt[j] = run;
  }
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int j = 0; j < C; ++j) {
      s_start[j] = run;
      run += s_cnt[j];
    }
  }
  __syncthreads();
  if (valid) s_sorted[s_start[lab] + s_whist[wave * C + lab] + rank_in_wave] = tid;
  __syncthreads();

  // ---- outputs: sort info (for bucketing) and this tile's per-cluster sums ----
  const size_t tix = static_cast<size_t>(bh) * a.ntiles + blockIdx.x;
  for (int j = tid; j < C; j += tile) {
    t.tile_cnt[tix * C + j] = s_cnt[j];
    t.tile_start[tix * C + j] = s_start[j];
  }
  t.tile_perm[tix * a.tile + tid] = static_cast<uint16_t>(s_sorted[tid]);
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

  tile_sort<T, D>(a, t, lab, valid, s_lab, s_whist, s_cnt, s_start, s_sorted);
  tile_sums_valu<T, D>(a, t, s_cnt, s_start, s_sorted);
}

// Matrix-core assign for bf16 inputs; blockDim.x == tile (multiple of 64, <= kMaxTileMfma).
// Wave w scores points w*64 .. w*64+63 in two groups of 32 (lane (c, h) of the product
// holds 16 centroid rows of point c per 32-row tile). Lane l = 32 h + c of the wave
// then owns point w*64 + l for the sort. Dynamic LDS: c_hi, c_lo [Cp][D+8] bf16 |
// ||c||^2 [Cp] | sort buffers | X^T staging [D][64+8] bf16.
template <int D, int NW>
__global__ void __launch_bounds__(64 * NW) kmeans_assign_mfma_kernel(KmArgs a, int iter, int last) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int CST = D + 8;
  constexpr int NKS = D / 16;
  constexpr int MAXJT = kMaxClusters / 32;
  const KmTensor& t = a.t[blockIdx.z];
  const int C = t.C, Cp = (C + 31) & ~31, njt = Cp / 32;
  const int bh = blockIdx.y, tile = blockDim.x, tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, h = lane >> 5, c = lane & 31;
  uint16_t* chi = reinterpret_cast<uint16_t*>(smem);
  uint16_t* clo = chi + Cp * CST;
  float* cn2 = reinterpret_cast<float*>(clo + Cp * CST);
  int* s_lab = reinterpret_cast<int*>(cn2 + Cp);
  int* s_whist = s_lab + tile;
  int* s_cnt = s_whist + (tile >> 6) * C;
  int* s_start = s_cnt + C;
  int* s_sorted = s_start + C;
  const long n = static_cast<long>(blockIdx.x) * tile + tid;
  const bool valid = n < a.N;
  const uint16_t* X = static_cast<const uint16_t*>(t.x) + static_cast<size_t>(bh) * a.N * D;
  const float* cent = t.cent + static_cast<size_t>(bh) * C * D;

  int lab = C;
  if (t.labels_in != nullptr) {
    if (valid) lab = min(max(t.labels_in[static_cast<size_t>(bh) * a.N + n], 0), C - 1);
  } else {
    // the first group of this wave's points, loaded before anything waits on memory
    u16x8_t xraw[NKS];
    auto load_group = [&](int gi) {
      const long p = static_cast<long>(blockIdx.x) * tile + wave * 64 + gi * 32 + c;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        xraw[ks] = u16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
        if (p < a.N) xraw[ks] = *reinterpret_cast<const u16x8_t*>(X + static_cast<size_t>(p) * D + 16 * ks + 8 * h);
      }
    };
    load_group(0);
    const uint16_t* ghi = t.chi + static_cast<size_t>(bh) * C * D;
    const uint16_t* glo = t.clo + static_cast<size_t>(bh) * C * D;
#pragma unroll 4
    for (int e = tid; e < Cp * (D / 8); e += tile) {
      const int j = e / (D / 8), c8 = e % (D / 8);
      u16x8_t h8 = {0, 0, 0, 0, 0, 0, 0, 0}, l8 = {0, 0, 0, 0, 0, 0, 0, 0};
      if (j < C) {
        h8 = *reinterpret_cast<const u16x8_t*>(ghi + static_cast<size_t>(j) * D + c8 * 8);
        l8 = *reinterpret_cast<const u16x8_t*>(glo + static_cast<size_t>(j) * D + c8 * 8);
      }
      *reinterpret_cast<u16x8_t*>(chi + j * CST + c8 * 8) = h8;
      *reinterpret_cast<u16x8_t*>(clo + j * CST + c8 * 8) = l8;
    }
    for (int j = tid; j < Cp; j += tile) cn2[j] = j < C ? t.cn2[static_cast<size_t>(bh) * C + j] : 0.f;
    __syncthreads();
    float cmax2 = 0.f;
    for (int j = lane; j < C; j += 64) cmax2 = fmaxf(cmax2, cn2[j]);
    cmax2 = wave_max(cmax2);
    const float cmax = sqrtf(cmax2);
    int labs[2];
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
      const long p = static_cast<long>(blockIdx.x) * tile + wave * 64 + gi * 32 + c;
      const bool pv = p < a.N;
      bf16x8_t xf[NKS];
      float xx = 0.f;
      if (gi == 1) load_group(1);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const u16x8_t u = xraw[ks];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const float xv = bf16_to_f32(u[r]);
          xx = fmaf(xv, xv, xx);
        }
        xf[ks] = as_bf16x8(u);
      }
      xx += __shfl_xor(xx, 32, 64);
      // scores of one 32-centroid tile: lane (c, h) holds centroids 32 jt + 8 g + 4 h + r
      auto score_tile = [&](int jt, f32x16_t& acc) {
        acc = zero16();
        const int jr = 32 * jt + c;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const bf16x8_t ah = as_bf16x8(*reinterpret_cast<const u16x8_t*>(chi + jr * CST + 16 * ks + 8 * h));
          const bf16x8_t al = as_bf16x8(*reinterpret_cast<const u16x8_t*>(clo + jr * CST + 16 * ks + 8 * h));
          acc = mfma32(ah, xf[ks], acc);
          acc = mfma32(al, xf[ks], acc);
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int j = 32 * jt + 8 * (v >> 2) + 4 * h + (v & 3);
          acc[v] = j < C ? cn2[j] - 2.f * acc[v] : __builtin_huge_valf();
        }
      };
      // running best (lowest index on ties) and second-best score
      float best = __builtin_huge_valf(), second = __builtin_huge_valf();
      int bj = C;
      for (int jt = 0; jt < njt; ++jt) {
        f32x16_t sc;
        score_tile(jt, sc);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int j = 32 * jt + 8 * (v >> 2) + 4 * h + (v & 3);
          const float x = sc[v];
          if (x < best || (x == best && j < bj)) {
            second = best;
            best = x;
            bj = j;
          } else {
            second = fminf(second, x);
          }
        }
      }
      {
        const float ob = __shfl_xor(best, 32, 64);
        const float os = __shfl_xor(second, 32, 64);
        const int oj = __shfl_xor(bj, 32, 64);
        if (ob < best || (ob == best && oj < bj)) {
          second = fminf(best, os);
          best = ob;
          bj = oj;
        } else {
          second = fminf(second, ob);
        }
      }
      const float E = 1e-4f * sqrtf(xx) * cmax + 2e-5f * cmax2;
      const float thr = best + 2.f * E;
      // a second centroid within the window: re-score every candidate exactly
      if (__ballot(pv && second <= thr) != 0ull) {
        const bool need = pv && second <= thr;  // the same for both lanes of the pair
        float fb = __builtin_huge_valf();
        int fj = C;
        const uint16_t* xr = X + static_cast<size_t>(p) * D;
        for (int jt = 0; jt < njt; ++jt) {
          f32x16_t sc;
          score_tile(jt, sc);
          if (need) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              if (sc[v] > thr) continue;
              const int j = 32 * jt + 8 * (v >> 2) + 4 * h + (v & 3);
              const float* cr = cent + static_cast<size_t>(j) * D;
              float dist = 0.f;
              for (int d = 0; d < D; ++d) {
                const float diff = bf16_to_f32(xr[d]) - cr[d];
                dist = fmaf(diff, diff, dist);
              }
              if (dist < fb || (dist == fb && j < fj)) {
                fb = dist;
                fj = j;
              }
            }
          }
        }
        const float ob = __shfl_xor(fb, 32, 64);
        const int oj = __shfl_xor(fj, 32, 64);
        if (ob < fb || (ob == fb && oj < fj)) fj = oj;
        if (need) bj = fj;
      }
      labs[gi] = bj;
    }
    if (valid) lab = h == 0 ? labs[0] : labs[1];
  }
  if (valid) {
    t.labels[static_cast<size_t>(bh) * a.N + n] = lab;
    if (t.trace != nullptr) t.trace[(static_cast<size_t>(iter) * a.BH + bh) * a.N + n] = lab;
  }
  const size_t tix = static_cast<size_t>(bh) * a.ntiles + blockIdx.x;
  if (last) {
    // bucketing after the last iteration needs the stable order
    tile_sort<bf16, D>(a, t, lab, valid, s_lab, s_whist, s_cnt, s_start, s_sorted);
  } else {
    for (int j = tid; j < C; j += tile) s_cnt[j] = 0;
    s_lab[tid] = lab;
    __syncthreads();
    if (valid) atomicAdd(&s_cnt[lab], 1);  // integer counts: order-independent
    __syncthreads();
    for (int j = tid; j < C; j += tile) t.tile_cnt[tix * C + j] = s_cnt[j];
  }
  // cluster sums psum^T [D x C] = X^T onehot over 64-point sub-chunks; wave w owns output
  // tiles w, w + nwaves, ... of the (D/32) x (Cp/32) grid
  constexpr int XST = 64 + 8;
  constexpr int NDT = D / 32;
  constexpr int MAXOT = (NDT * (kMaxClusters / 32) + NW - 1) / NW < 4 ? (NDT * (kMaxClusters / 32) + NW - 1) / NW : 4;
  uint16_t* sXt = reinterpret_cast<uint16_t*>((reinterpret_cast<uintptr_t>(s_sorted + tile) + 15) & ~uintptr_t(15));
  const int nwaves = tile >> 6;
  const int not_ = NDT * njt;
  const uint16_t bf_one = 0x3F80;
  float* psum = t.psum + tix * C * D;
  // a sub-chunk of 64 points is 64*D/8 16-byte pieces; each thread carries kPre of them
  constexpr int kPre = (64 * (D / 8)) / (64 * NW);
  auto load_chunk = [&](int p0, u16x8_t* buf) {
#pragma unroll
    for (int q = 0; q < kPre; ++q) {
      const int x = tid + tile * q;
      buf[q] = u16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
      if (x < 64 * (D / 8)) {
        const int r = x / (D / 8), c8 = x % (D / 8);
        const long pn = static_cast<long>(blockIdx.x) * tile + p0 + r;
        if (pn < a.N) buf[q] = *reinterpret_cast<const u16x8_t*>(X + static_cast<size_t>(pn) * D + c8 * 8);
      }
    }
  };
  for (int ot0 = 0; ot0 < not_; ot0 += nwaves * MAXOT) {
    f32x16_t acc[MAXOT];
#pragma unroll
    for (int r = 0; r < MAXOT; ++r) acc[r] = zero16();
    u16x8_t pre[kPre];
    load_chunk(0, pre);
    for (int p0 = 0; p0 < tile; p0 += 64) {
      __syncthreads();
#pragma unroll
      for (int q = 0; q < kPre; ++q) {
        const int x = tid + tile * q;
        if (x < 64 * (D / 8)) {
          const int r = x / (D / 8), c8 = x % (D / 8);
#pragma unroll
          for (int e = 0; e < 8; ++e) sXt[(c8 * 8 + e) * XST + r] = pre[q][e];
        }
      }
      __syncthreads();
      if (p0 + 64 < tile) load_chunk(p0 + 64, pre);  // next sub-chunk in flight during this one
#pragma unroll
      for (int r = 0; r < MAXOT; ++r) {
        const int ot = ot0 + wave + nwaves * r;
        if (ot >= not_) break;
        const int dt = ot % NDT, ct = ot / NDT;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int kk = 16 * ks + 8 * h;
          const bf16x8_t ax = as_bf16x8(*reinterpret_cast<const u16x8_t*>(sXt + (32 * dt + c) * XST + kk));
          u16x8_t oh;
#pragma unroll
          for (int e = 0; e < 8; ++e) oh[e] = s_lab[p0 + kk + e] == 32 * ct + c ? bf_one : 0;
          acc[r] = mfma32(ax, as_bf16x8(oh), acc[r]);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < MAXOT; ++r) {
      const int ot = ot0 + wave + nwaves * r;
      if (ot >= not_) break;
      const int dt = ot % NDT, ct = ot / NDT;
      const int j = 32 * ct + c;
      if (j >= C) continue;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4_t f = {acc[r][4 * g], acc[r][4 * g + 1], acc[r][4 * g + 2], acc[r][4 * g + 3]};
        *reinterpret_cast<f32x4_t*>(psum + static_cast<size_t>(j) * D + 32 * dt + 8 * g + 4 * h) = f;
      }
    }
  }
}

// One wave per (centroid j, head, tensor), lanes over d: sum the tile partials in tile
// order; the mean replaces c_j unless the cluster is empty.
__global__ void __launch_bounds__(64) kmeans_update_kernel(KmArgs a) {
  const KmTensor& t = a.t[blockIdx.z];
  const int C = t.C, D = a.D, j = blockIdx.x, bh = blockIdx.y;
  if (j >= C) return;
  const size_t tbase = static_cast<size_t>(bh) * a.ntiles;
  const int nper = D / 64;
  float acc[2] = {0.f, 0.f};
  int cnt = 0;
#pragma unroll 8
  for (int tt = 0; tt < a.ntiles; ++tt) {
    const float* ps = t.psum + ((tbase + tt) * C + j) * D;
    acc[0] += ps[lane_id()];
    if (nper > 1) acc[1] += ps[lane_id() + 64];
    cnt += t.tile_cnt[(tbase + tt) * C + j];
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

// One workgroup per (head, tensor): counts per (block, cluster) and their exclusive
// scan -> offs[nb*C + 1].
__global__ void bucket_offsets_kernel(KmArgs a) {
  const KmTensor& t = a.t[blockIdx.z];
  if (t.perm == nullptr) return;
  const int C = t.C, bh = blockIdx.y;
  const int nbC = a.nb * C;
  extern __shared__ int s_tot[];  // [nb*C]
  for (int e = threadIdx.x; e < nbC; e += blockDim.x) {
    const int b = e / C, j = e % C;
    int s = 0;
    for (int tt = b * a.tiles_per_block; tt < min(a.ntiles, (b + 1) * a.tiles_per_block); ++tt)
      s += t.tile_cnt[(static_cast<size_t>(bh) * a.ntiles + tt) * C + j];
    s_tot[e] = s;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int* offs = t.offs + static_cast<size_t>(bh) * (nbC + 1);
    int run = 0;
    for (int e = 0; e < nbC; ++e) {
      offs[e] = run;
      run += s_tot[e];
    }
    offs[nbC] = run;
  }
}

// One workgroup per tile: scatter the tile's stably sorted points into the head's
// (block, label) buckets.
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
    // members of (b, j) in earlier tiles of the same block come first
    int before = 0;
    for (int t2 = b * a.tiles_per_block; t2 < tt; ++t2)
      before += t.tile_cnt[(static_cast<size_t>(bh) * a.ntiles + t2) * C + j];
    const int dst = offs[b * C + j] + before + (pos - t.tile_start[tix * C + j]);
    t.perm[static_cast<size_t>(bh) * a.N + dst] = static_cast<int>(tile0 + p);
  }
}

// ------------------------------------------------------------------ host launchers

template <typename T>
static hipError_t launch_kmeans_t(const KmArgs& a, int iters, hipStream_t s) {
  const int Cmax = max(a.t[0].C, a.ntensors > 1 ? a.t[1].C : 0);
  {
    ProfScope ps_("kmeans_init", s);
    hipLaunchKernelGGL(kmeans_init_kernel<T>, dim3(Cmax, a.BH, a.ntensors), dim3(64), 0, s, a);
  }
  const size_t lds = static_cast<size_t>(kChunkC) * a.D * sizeof(float) +
                     sizeof(int) * (2 * a.tile + (a.tile / 64) * Cmax + 2 * Cmax);
  const dim3 g_assign(a.ntiles, a.BH, a.ntensors);
  const dim3 g_update(Cmax, a.BH, a.ntensors);
  const int Cp = (Cmax + 31) & ~31;
  const size_t lds_mfma = static_cast<size_t>(Cp) * (a.D + 8) * 2 * sizeof(uint16_t) + Cp * sizeof(float) +
                          sizeof(int) * (2 * a.tile + (a.tile / 64) * Cmax + 2 * Cmax) +
                          static_cast<size_t>(a.D) * (64 + 8) * sizeof(uint16_t) + 16;
  const bool mf = sizeof(T) == 2;
  auto launch_mfma = [&](int it) {
    const int last = it == iters - 1;
    const int nw = a.tile / 64;
#define MUSE_KM_CASE(DD, NN)                                                                            \
  if (a.D == DD && nw == NN) {                                                                          \
    allow_lds((const void*)kmeans_assign_mfma_kernel<DD, NN>, lds_mfma);                               \
    hipLaunchKernelGGL((kmeans_assign_mfma_kernel<DD, NN>), g_assign, dim3(a.tile), lds_mfma, s, a, it, last); \
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
        hipLaunchKernelGGL((kmeans_assign_kernel<T, 64>), g_assign, dim3(a.tile), lds, s, a, it);
      else
        hipLaunchKernelGGL((kmeans_assign_kernel<T, 128>), g_assign, dim3(a.tile), lds, s, a, it);
    }
    {
      ProfScope ps_("kmeans_update", s);
      hipLaunchKernelGGL(kmeans_update_kernel, g_update, dim3(64), 0, s, a);
    }
  }
  const size_t lds_off = sizeof(int) * static_cast<size_t>(a.nb) * Cmax;
  {
    ProfScope ps_("bucket_offsets", s);
    hipLaunchKernelGGL(bucket_offsets_kernel, dim3(1, a.BH, a.ntensors), dim3(256), lds_off, s, a);
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
