// C ABI of the MuSe forward pass: argument validation, workspace plan and the fixed
// launch sequence on the caller's stream. Declarations and conventions: include/muse.h.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/muse.h"
#include "muse_kernels.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(MUSE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Bump allocator over one device buffer; every region is 256-byte aligned.
struct Layout {
  size_t bytes = 0;
  size_t take(size_t n) {
    const size_t at = bytes;
    bytes += (n + 255) & ~static_cast<size_t>(255);
    return at;
  }
};

struct Shape {
  int B, H, N, D, Cq, Ck, iters, causal, block, dtype;
  int BH, nb, nbS, tile, ntiles, tiles_per_block;
  int nmb, mbk;  // dipole-moment sub-blocks
};

// Largest multiple of 64 that divides `block` and is at most max_tile.
int tile_for_block(int block, int max_tile) {
  const int k = block / 64;
  for (int t = max_tile / 64; t >= 1; --t)
    if (k % t == 0) return 64 * t;
  return 64;
}

int validate(Shape& s, const muse_fwd_params* p) {
  if (s.B < 1 || s.H < 1 || s.N < 1) return fail(MUSE_ERR_INVALID_ARG, "B, H, N must be >= 1 (got %d, %d, %d)", s.B, s.H, s.N);
  if (s.dtype != MUSE_F32 && s.dtype != MUSE_BF16) return fail(MUSE_ERR_INVALID_ARG, "dtype %d is not MUSE_F32 or MUSE_BF16", s.dtype);
  if (s.D != 64 && s.D != 128) return fail(MUSE_ERR_UNSUPPORTED, "head dim D=%d unsupported (64 or 128)", s.D);
  if (static_cast<long>(s.B) * s.H * s.N > (1l << 31) / 256) return fail(MUSE_ERR_UNSUPPORTED, "B*H*N too large");
  if (s.causal != 0 && s.causal != 1) return fail(MUSE_ERR_INVALID_ARG, "causal must be 0 or 1");
  s.BH = s.B * s.H;
  const int max_tile = s.dtype == MUSE_BF16 ? muse::kMaxTileMfma : muse::kMaxTile;
  if (s.causal) {
    if (s.block < 1 || s.block > s.N || s.N % s.block != 0)
      return fail(MUSE_ERR_INVALID_ARG, "causal block=%d must lie in [1, N=%d] and divide N", s.block, s.N);
    if (s.block < 64 || s.block % 64 != 0)
      return fail(MUSE_ERR_UNSUPPORTED, "causal block=%d: blocks of at least 64 tokens, multiples of 64, are implemented",
                  s.block);
    s.nb = s.N / s.block;
    s.nbS = s.nb;
    s.tile = tile_for_block(s.block, max_tile);
    s.tiles_per_block = s.block / s.tile;
  } else {
    s.block = s.N;
    s.nb = 1;
    s.nbS = 1;
    s.tile = max_tile;
    s.tiles_per_block = (s.N + s.tile - 1) / s.tile;
  }
  s.ntiles = (s.N + s.tile - 1) / s.tile;
  // moment key ranges: a causal block (split into equal ranges of at most kMaxMomKeys
  // positions for the matrix-core kernel); for an acausal bf16 call, slices sized so that
  // the moment kernel has about 256 workgroups (multiples of its 128-key chunk)
  if (s.dtype == MUSE_BF16 && !s.causal) {
    const int groups = (s.Cq + muse::moments_group(s.D) - 1) / muse::moments_group(s.D);
    const int want = std::max(1, (256 + groups * s.BH - 1) / (groups * s.BH));
    int slice = (s.N + want - 1) / want;
    slice = (slice + 127) / 128 * 128;
    s.mbk = std::min(slice, muse::kMaxMomKeys);
  } else {
    s.mbk = s.block;
    if (s.dtype == MUSE_BF16)
      for (int k = s.block / 64; k >= 1; --k)
        if ((s.block / 64) % k == 0 && 64 * k <= muse::kMaxMomKeys) {
          s.mbk = 64 * k;
          break;
        }
  }
  s.nmb = (s.N + s.mbk - 1) / s.mbk;
  if (p != nullptr) {
    if (p->out_dtype != -1 && p->out_dtype != MUSE_F32 && p->out_dtype != MUSE_BF16)
      return fail(MUSE_ERR_INVALID_ARG, "out_dtype %d invalid", p->out_dtype);
    if (p->dipole != MUSE_DIPOLE_NONE && p->dipole != MUSE_DIPOLE_TILTED && p->dipole != MUSE_DIPOLE_UNTILTED)
      return fail(MUSE_ERR_INVALID_ARG, "dipole mode %d invalid", p->dipole);
    if (p->dipole == MUSE_DIPOLE_UNTILTED && s.causal && (p->topk_clusters > 0 || p->hierarchy))
      return fail(MUSE_ERR_UNSUPPORTED,
                  "the untilted dipole is not combined with retrieval or the hierarchical decomposition");
    if (p->topk_clusters < 0 || p->topk_blocks < 0) return fail(MUSE_ERR_INVALID_ARG, "retrieval top-k must be >= 0");
    if (p->topk_clusters > 0 && !s.causal) return fail(MUSE_ERR_INVALID_ARG, "retrieval requires causal=1");
    if (p->topk_clusters > 0 && p->topk_blocks < 1) return fail(MUSE_ERR_INVALID_ARG, "retrieval needs topk_blocks >= 1");
    if (p->topk_clusters > 0 && p->topk_clusters * (1 + p->topk_blocks) > muse::kMaxRetrRow)
      return fail(MUSE_ERR_UNSUPPORTED, "topk_clusters * (1 + topk_blocks) must be at most %d", muse::kMaxRetrRow);
    if (p->hierarchy != 0 && p->hierarchy != 1) return fail(MUSE_ERR_INVALID_ARG, "hierarchy must be 0 or 1");
    if (p->single_stream != 0 && p->single_stream != 1) return fail(MUSE_ERR_INVALID_ARG, "single_stream must be 0 or 1");
    if (p->hierarchy && !s.causal) return fail(MUSE_ERR_INVALID_ARG, "the hierarchical decomposition requires causal=1");
    if (p->hierarchy && p->topk_clusters > 0)
      return fail(MUSE_ERR_UNSUPPORTED, "retrieval is not combined with the hierarchical decomposition");
    if (p->topk_clusters > 0 && s.nb > muse::kMaxRetrBlocks)
      return fail(MUSE_ERR_UNSUPPORTED, "retrieval supports at most %d blocks", muse::kMaxRetrBlocks);
    if (!(p->cap_ratio >= 0.0)) return fail(MUSE_ERR_INVALID_ARG, "cap_ratio must be >= 0 (0: no cap)");
    if (p->cap_ratio > 0.0 && p->topk_clusters > 0)
      return fail(MUSE_ERR_UNSUPPORTED, "the cluster size cap is not combined with retrieval");
  }
  return MUSE_OK;
}

// Members kept per key cluster under the cap, ceil(cap_ratio * N / Ck) (at most N), or 0
// for no cap.
int cap_members(const Shape& s, const muse_fwd_params* p) {
  if (p == nullptr || !(p->cap_ratio > 0.0)) return 0;
  const double u = ceil(p->cap_ratio * s.N / s.Ck);
  return u >= static_cast<double>(s.N) ? s.N : static_cast<int>(u);
}

int validate_muse(Shape& s, const muse_fwd_params* p) {
  const int r = validate(s, p);
  if (r != MUSE_OK) return r;
  if (s.Cq < 1 || s.Ck < 1 || s.Cq > s.N || s.Ck > s.N)
    return fail(MUSE_ERR_INVALID_ARG, "clusters Cq=%d Ck=%d must lie in [1, N=%d]", s.Cq, s.Ck, s.N);
  if (s.Cq > muse::kMaxClusters || s.Ck > muse::kMaxClusters)
    return fail(MUSE_ERR_UNSUPPORTED, "at most %d clusters per tensor (Cq=%d Ck=%d)", muse::kMaxClusters, s.Cq, s.Ck);
  if (s.iters < 1) return fail(MUSE_ERR_INVALID_ARG, "kmeans_iters=%d must be >= 1", s.iters);
  return MUSE_OK;
}

struct Plan {
  size_t chi_q, clo_q, cn2_q, chi_k, clo_k, cn2_k;
  size_t cent_q, cent_k, lab_q, lab_k, tperm_q, tperm_k, tcnt_q, tcnt_k, tst_q, tst_k, psum_q, psum_k;
  size_t gcnt_q, gcnt_k;
  size_t perm_k, offs_k, perm_q, offs_q;
  size_t items_k, multi_k, bmeta_k, pt_m, pt_z, pt_k, pt_v;
  size_t t_khi, t_klo, t_vhi, t_vlo, t_dip, tiles, ntiles;
  int max_tiles;
  size_t at_m, at_z, at_k, at_v, blk_lmass, blk_mom, scores, tmax, cov_k;
  size_t ub_n, ub_mk, ub_mv, ub_c, up_n, up_mk, up_mv;
  size_t klen, kdrop;
  size_t s_logz, s_k, s_v, s_dip;
  size_t o_far, l_far, retr_sel;
  size_t total;
};

Plan make_plan(const Shape& s, const muse_fwd_params* p) {
  Layout L;
  Plan P{};
  const size_t BH = s.BH, N = s.N, D = s.D, Cq = s.Cq, Ck = s.Ck, nb = s.nb, nbS = s.nbS;
  const size_t nt = s.ntiles, tile = s.tile;
  const size_t f = sizeof(float), i4 = sizeof(int32_t);
  P.cent_q = L.take(BH * Cq * D * f);
  P.cent_k = L.take(BH * Ck * D * f);
  if (s.dtype == MUSE_BF16) {
    P.chi_q = L.take(BH * Cq * D * 2);
    P.clo_q = L.take(BH * Cq * D * 2);
    P.chi_k = L.take(BH * Ck * D * 2);
    P.clo_k = L.take(BH * Ck * D * 2);
  }
  P.cn2_q = L.take(BH * Cq * f);
  P.cn2_k = L.take(BH * Ck * f);
  P.lab_q = L.take(BH * N * i4);
  P.lab_k = L.take(BH * N * i4);
  P.tperm_q = L.take(BH * nt * tile * sizeof(uint16_t));
  P.tperm_k = L.take(BH * nt * tile * sizeof(uint16_t));
  P.tcnt_q = L.take(BH * nt * Cq * i4);
  P.tcnt_k = L.take(BH * nt * Ck * i4);
  P.tst_q = L.take(BH * nt * Cq * i4);
  P.tst_k = L.take(BH * nt * Ck * i4);
  P.psum_q = L.take(BH * nt * Cq * D * f);
  P.psum_k = L.take(BH * nt * Ck * D * f);
  if (s.dtype == MUSE_BF16) {
    P.gcnt_q = L.take(BH * nt * Cq * i4);
    P.gcnt_k = L.take(BH * nt * Ck * i4);
  }
  P.perm_k = L.take(BH * N * i4);
  P.offs_k = L.take(BH * (nb * Ck + 1) * i4);
  P.perm_q = L.take(BH * N * i4);
  P.offs_q = L.take(BH * (nb * Cq + 1) * i4);
  if (cap_members(s, p) > 0) {
    P.klen = L.take(BH * nb * Ck * i4);
    P.kdrop = L.take(BH * N);
  }
  if (s.dtype == MUSE_BF16) {
    const size_t ni = muse::atom_max_items(static_cast<int>(nb * Ck), static_cast<int>(N));
    const size_t np = muse::atom_max_partials(static_cast<int>(N));
    P.items_k = L.take(BH * ni * 4 * i4);
    P.multi_k = L.take(BH * (1 + muse::atom_max_multi(static_cast<int>(N))) * 4 * i4);
    P.bmeta_k = L.take(BH * nb * Ck * 2 * i4);
    P.pt_m = L.take(BH * np * Cq * f);
    P.pt_z = L.take(BH * np * Cq * f);
    P.pt_k = L.take(BH * np * Cq * D * f);
    P.pt_v = L.take(BH * np * Cq * D * f);
  }
  P.at_m = L.take(BH * nb * Cq * Ck * f);
  P.at_z = L.take(BH * nb * Cq * Ck * f);
  P.at_k = L.take(BH * nb * Cq * Ck * D * f);
  P.at_v = L.take(BH * nb * Cq * Ck * D * f);
  P.scores = s.dtype == MUSE_BF16 ? L.take(BH * Cq * N * f) : 0;
  P.tmax = s.dtype == MUSE_BF16 ? L.take(BH * Cq * ((N + 31) / 32) * f) : 0;
  P.blk_lmass = L.take(BH * static_cast<size_t>(s.nmb) * Cq * f);
  P.blk_mom = L.take(BH * static_cast<size_t>(s.nmb) * Cq * D * D * f);
  const bool untilted = p != nullptr && p->dipole == MUSE_DIPOLE_UNTILTED;
  P.cov_k = (untilted && !s.causal) ? L.take(BH * static_cast<size_t>(Ck) * D * D * f) : 0;
  if (untilted && s.causal) {
    // per (key block, key cluster) bucket statistics and their prefix over the blocks
    P.ub_n = L.take(BH * nb * Ck * f);
    P.ub_mk = L.take(BH * nb * Ck * D * f);
    P.ub_mv = L.take(BH * nb * Ck * D * f);
    P.ub_c = L.take(BH * nb * Ck * D * D * f);
    P.up_n = L.take(BH * nb * Ck * f);
    P.up_mk = L.take(BH * nb * Ck * D * f);
    P.up_mv = L.take(BH * nb * Ck * D * f);
  }
  P.s_logz = L.take(BH * nbS * Cq * Ck * f);
  P.s_k = L.take(BH * nbS * Cq * Ck * D * f);
  P.s_v = L.take(BH * nbS * Cq * Ck * D * f);
  P.s_dip = L.take(BH * nbS * Cq * D * D * f);
  if (s.causal) {
    P.o_far = L.take(BH * N * D * f);
    P.l_far = L.take(BH * N * f);
  }
  if (p != nullptr && p->topk_clusters > 0)
    P.retr_sel = L.take(BH * nb * Cq * static_cast<size_t>(p->topk_clusters) * (1 + p->topk_blocks) * i4);
  if (s.dtype == MUSE_BF16) {
    const size_t h2 = sizeof(uint16_t);
    P.t_khi = L.take(BH * nbS * Cq * Ck * D * h2);
    P.t_klo = L.take(BH * nbS * Cq * Ck * D * h2);
    P.t_vhi = L.take(BH * nbS * Cq * Ck * D * h2);
    P.t_vlo = L.take(BH * nbS * Cq * Ck * D * h2);
    P.t_dip = L.take(BH * nbS * Cq * D * D * h2);
    // stage-2 chunks of the query buckets: at most ceil(N / kS2Chunk) + nb*Cq per head
    P.max_tiles = static_cast<int>((N + muse::kS2Chunk - 1) / muse::kS2Chunk + nb * Cq);
    P.tiles = L.take(BH * P.max_tiles * 2 * i4);
    P.ntiles = L.take(BH * i4);
  }
  P.total = L.bytes;
  return P;
}

template <typename T>
T* at(void* base, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(base) + off);
}

float scale_of(const Shape& s, const muse_fwd_params* p) {
  return (p != nullptr && p->scale > 0.f) ? p->scale : 1.0f / sqrtf(static_cast<float>(s.D));
}

int out_is_bf16(const Shape& s, const muse_fwd_params* p) {
  const int od = (p != nullptr && p->out_dtype != -1) ? p->out_dtype : s.dtype;
  return od == MUSE_BF16;
}

// K-means arguments of one call: both tensors, their tables and buckets in the workspace.
muse::KmArgs kmeans_args(const void* q, const void* k, const Shape& s, const Plan& P, void* ws) {
  using namespace muse;
  const bool mf = s.dtype == MUSE_BF16;
  KmArgs km{};
  km.ntensors = 2;
  km.BH = s.BH;
  km.N = s.N;
  km.D = s.D;
  km.tile = s.tile;
  km.ntiles = s.ntiles;
  km.nb = s.nb;
  km.tiles_per_block = s.tiles_per_block;
  KmTensor& tq = km.t[0];
  tq.x = q;
  tq.C = s.Cq;
  tq.cent = at<float>(ws, P.cent_q);
  tq.chi = mf ? at<uint16_t>(ws, P.chi_q) : nullptr;
  tq.clo = mf ? at<uint16_t>(ws, P.clo_q) : nullptr;
  tq.cn2 = at<float>(ws, P.cn2_q);
  tq.labels = at<int32_t>(ws, P.lab_q);
  tq.tile_perm = at<uint16_t>(ws, P.tperm_q);
  tq.tile_cnt = at<int32_t>(ws, P.tcnt_q);
  tq.tile_start = at<int32_t>(ws, P.tst_q);
  tq.psum = at<float>(ws, P.psum_q);
  tq.gcnt = mf ? at<int32_t>(ws, P.gcnt_q) : tq.tile_cnt;
  if (mf) {
    tq.chunks = at<int2>(ws, P.tiles);
    tq.nchunks = at<int32_t>(ws, P.ntiles);
    tq.max_chunks = P.max_tiles;
  }
  KmTensor& tk = km.t[1];
  tk.x = k;
  tk.C = s.Ck;
  tk.cent = at<float>(ws, P.cent_k);
  tk.chi = mf ? at<uint16_t>(ws, P.chi_k) : nullptr;
  tk.clo = mf ? at<uint16_t>(ws, P.clo_k) : nullptr;
  tk.cn2 = at<float>(ws, P.cn2_k);
  tk.labels = at<int32_t>(ws, P.lab_k);
  tk.tile_perm = at<uint16_t>(ws, P.tperm_k);
  tk.tile_cnt = at<int32_t>(ws, P.tcnt_k);
  tk.tile_start = at<int32_t>(ws, P.tst_k);
  tk.psum = at<float>(ws, P.psum_k);
  tk.gcnt = mf ? at<int32_t>(ws, P.gcnt_k) : tk.tile_cnt;
  tk.perm = at<int32_t>(ws, P.perm_k);
  tk.offs = at<int32_t>(ws, P.offs_k);
  tk.items = mf ? at<int4>(ws, P.items_k) : nullptr;
  tk.multi = mf ? at<int4>(ws, P.multi_k) : nullptr;
  tk.bmeta = mf ? at<int2>(ws, P.bmeta_k) : nullptr;
  return km;
}

// Stage-1 arguments of one call (tables in the workspace; the caller sets the options).
muse::S1Args stage1_args(const void* k, const void* v, const Shape& s, const Plan& P, void* ws,
                         const muse::KmArgs& km, float scale, int dipole) {
  using namespace muse;
  const bool mf = s.dtype == MUSE_BF16;
  const KmTensor& tq = km.t[0];
  const KmTensor& tk = km.t[1];
  S1Args a1{};
  a1.k = k;
  a1.v = v;
  a1.BH = s.BH;
  a1.N = s.N;
  a1.D = s.D;
  a1.Cq = s.Cq;
  a1.Ck = s.Ck;
  a1.nb = s.nb;
  a1.block = s.block;
  a1.causal = s.causal;
  a1.nbS = s.nbS;
  a1.scale = scale;
  a1.dipole = dipole;
  a1.qbar = tq.cent;
  a1.perm_k = tk.perm;
  a1.offs_k = tk.offs;
  a1.items_k = tk.items;
  a1.multi_k = tk.multi;
  a1.bmeta_k = tk.bmeta;
  a1.klen = tk.klen;
  a1.kdrop = tk.kdrop;
  if (mf) {
    a1.pt_m = at<float>(ws, P.pt_m);
    a1.pt_z = at<float>(ws, P.pt_z);
    a1.pt_k = at<float>(ws, P.pt_k);
    a1.pt_v = at<float>(ws, P.pt_v);
  }
  a1.at_m = at<float>(ws, P.at_m);
  a1.at_z = at<float>(ws, P.at_z);
  a1.at_k = at<float>(ws, P.at_k);
  a1.at_v = at<float>(ws, P.at_v);
  a1.scores = mf ? at<float>(ws, P.scores) : nullptr;
  a1.tmax = mf ? at<float>(ws, P.tmax) : nullptr;
  a1.nmb = s.nmb;
  a1.mbk = s.mbk;
  a1.blk_lmass = at<float>(ws, P.blk_lmass);
  a1.blk_mom = at<float>(ws, P.blk_mom);
  a1.cov_k = (dipole == MUSE_DIPOLE_UNTILTED && !s.causal) ? at<float>(ws, P.cov_k) : nullptr;
  if (dipole == MUSE_DIPOLE_UNTILTED && s.causal) {
    a1.ub_n = at<float>(ws, P.ub_n);
    a1.ub_mk = at<float>(ws, P.ub_mk);
    a1.ub_mv = at<float>(ws, P.ub_mv);
    a1.ub_c = at<float>(ws, P.ub_c);
    a1.up_n = at<float>(ws, P.up_n);
    a1.up_mk = at<float>(ws, P.up_mk);
    a1.up_mv = at<float>(ws, P.up_mv);
  }
  a1.s_logz = at<float>(ws, P.s_logz);
  a1.s_k = at<float>(ws, P.s_k);
  a1.s_v = at<float>(ws, P.s_v);
  a1.s_dip = at<float>(ws, P.s_dip);
  if (mf) {
    a1.t_khi = at<uint16_t>(ws, P.t_khi);
    a1.t_klo = at<uint16_t>(ws, P.t_klo);
    a1.t_vhi = at<uint16_t>(ws, P.t_vhi);
    a1.t_vlo = at<uint16_t>(ws, P.t_vlo);
    a1.t_dip = at<uint16_t>(ws, P.t_dip);
  }
  return a1;
}

int run_muse(const void* q, const void* k, const void* v, void* out, const Shape& s,
             const muse_fwd_params* p, hipStream_t stream, void* ws, bool one_stream = false) {
  using namespace muse;
  const Plan P = make_plan(s, p);
  const float scale = scale_of(s, p);
  const int dipole = p ? p->dipole : MUSE_DIPOLE_TILTED;
  const bool mf = s.dtype == MUSE_BF16;
  const bool retr = p != nullptr && p->topk_clusters > 0;

  KmArgs km = kmeans_args(q, k, s, P, ws);
  KmTensor& tq = km.t[0];
  KmTensor& tk = km.t[1];
  tq.trace = p ? p->labels_q_trace : nullptr;
  tq.labels_in = p ? p->labels_q_in : nullptr;
  tk.trace = p ? p->labels_k_trace : nullptr;
  tk.labels_in = p ? p->labels_k_in : nullptr;
  // the matrix-core stage 2 and retrieval need the query buckets
  const bool want_qb = p != nullptr && (p->perm_q_out != nullptr || p->offs_q_out != nullptr);
  tq.perm = (mf || retr || want_qb) ? at<int32_t>(ws, P.perm_q) : nullptr;
  tq.offs = (mf || retr || want_qb) ? at<int32_t>(ws, P.offs_q) : nullptr;
  tk.cap = cap_members(s, p);
  tk.klen = tk.cap > 0 ? at<int32_t>(ws, P.klen) : nullptr;
  tk.kdrop = tk.cap > 0 ? at<uint8_t>(ws, P.kdrop) : nullptr;
  hipError_t e = launch_kmeans(km, s.iters, s.dtype, stream);
  if (e != hipSuccess) return hip_fail(e, "K-means launch");

  S1Args a1 = stage1_args(k, v, s, P, ws, km, scale, dipole);
  a1.hier = (p != nullptr && p->hierarchy) ? 1 : 0;
  a1.one_stream = (one_stream || (p != nullptr && p->single_stream != 0)) ? 1 : 0;
  RetrArgs ra{};
  if (retr) {
    ra.q = q;
    ra.k = k;
    ra.v = v;
    ra.BH = s.BH;
    ra.N = s.N;
    ra.D = s.D;
    ra.Cq = s.Cq;
    ra.Ck = s.Ck;
    ra.nb = s.nb;
    ra.k1 = p->topk_clusters;
    ra.k2 = p->topk_blocks;
    ra.dipole = dipole;
    ra.scale = scale;
    ra.qbar = tq.cent;
    ra.perm_k = tk.perm;
    ra.offs_k = tk.offs;
    ra.perm_q = tq.perm;
    ra.offs_q = tq.offs;
    ra.at_m = a1.at_m;
    ra.at_z = a1.at_z;
    ra.at_k = a1.at_k;
    ra.at_v = a1.at_v;
    ra.s_logz = a1.s_logz;
    ra.s_k = a1.s_k;
    ra.s_v = a1.s_v;
    ra.s_dip = a1.s_dip;
    ra.sel = at<int32_t>(ws, P.retr_sel);
    ra.trace = p->retrieval_trace;
    ra.o_far = at<float>(ws, P.o_far);
    ra.l_far = at<float>(ws, P.l_far);
    if (mf) {
      ra.tiles = at<int2>(ws, P.tiles);
      ra.ntiles = at<int32_t>(ws, P.ntiles);
      ra.max_tiles = P.max_tiles;
    }
    a1.retr = &ra;
  }
  e = launch_stage1(a1, s.dtype, stream);
  if (e != hipSuccess) return hip_fail(e, "stage-1 launch");

  S2Args a2{};
  a2.q = q;
  a2.out = out;
  a2.lse_out = p ? p->lse_out : nullptr;
  a2.BH = s.BH;
  a2.N = s.N;
  a2.D = s.D;
  a2.Cq = s.Cq;
  a2.Ck = s.Ck;
  a2.causal = s.causal;
  a2.block = s.block;
  a2.nbS = s.nbS;
  a2.scale = scale;
  a2.dipole = dipole;
  a2.hier = a1.hier;
  a2.out_bf16 = out_is_bf16(s, p);
  a2.labels_q = tq.labels;
  a2.qbar = tq.cent;
  a2.s_logz = a1.s_logz;
  a2.s_k = a1.s_k;
  a2.s_v = a1.s_v;
  a2.s_dip = a1.s_dip;
  a2.t_khi = a1.t_khi;
  a2.t_klo = a1.t_klo;
  a2.t_vhi = a1.t_vhi;
  a2.t_vlo = a1.t_vlo;
  a2.t_dip = a1.t_dip;
  a2.perm_q = tq.perm;
  a2.offs_q = tq.offs;
  a2.nb = s.nb;
  if (mf) {
    a2.tiles = at<int2>(ws, P.tiles);
    a2.ntiles = at<int32_t>(ws, P.ntiles);
    a2.max_tiles = P.max_tiles;
  }
  if (s.causal) {
    a2.o_far = at<float>(ws, P.o_far);
    a2.l_far = at<float>(ws, P.l_far);
  }
  e = launch_stage2(a2, s.dtype, stream);
  if (e != hipSuccess) return hip_fail(e, "stage-2 launch");
  if (retr) {
    e = launch_retrieval(ra, 1, s.dtype, stream);
    if (e != hipSuccess) return hip_fail(e, "retrieval launch");
  }

  if (s.causal) {
    ExactArgs ax{};
    ax.q = q;
    ax.k = k;
    ax.v = v;
    ax.out = out;
    ax.lse_out = p ? p->lse_out : nullptr;
    ax.o_far = a2.o_far;
    ax.l_far = a2.l_far;
    ax.BH = s.BH;
    ax.N = s.N;
    ax.D = s.D;
    ax.causal = 1;
    ax.block = s.block;
    ax.scale = scale;
    ax.out_bf16 = a2.out_bf16;
    e = launch_exact(ax, s.dtype, stream);
    if (e != hipSuccess) return hip_fail(e, "local block launch");
  }
  if (p != nullptr) {
    // copies of the bucket order (position permutation and offsets) for the caller
    const size_t nq = static_cast<size_t>(s.nb) * s.Cq + 1, nk = static_cast<size_t>(s.nb) * s.Ck + 1;
    const struct {
      int32_t* dst;
      const int32_t* src;
      size_t n;
    } cp[4] = {{p->perm_q_out, tq.perm, static_cast<size_t>(s.N)}, {p->offs_q_out, tq.offs, nq},
               {p->perm_k_out, tk.perm, static_cast<size_t>(s.N)}, {p->offs_k_out, tk.offs, nk}};
    for (const auto& c : cp) {
      if (c.dst == nullptr) continue;
      e = hipMemcpyAsync(c.dst, c.src, sizeof(int32_t) * s.BH * c.n, hipMemcpyDeviceToDevice, stream);
      if (e != hipSuccess) return hip_fail(e, "bucket order copy");
    }
  }
  if (p != nullptr && p->centroids_q_out != nullptr) {
    e = hipMemcpyAsync(p->centroids_q_out, tq.cent, sizeof(float) * s.BH * s.Cq * s.D, hipMemcpyDeviceToDevice, stream);
    if (e != hipSuccess) return hip_fail(e, "centroid copy");
  }
  if (p != nullptr && p->centroids_k_out != nullptr) {
    e = hipMemcpyAsync(p->centroids_k_out, tk.cent, sizeof(float) * s.BH * s.Ck * s.D, hipMemcpyDeviceToDevice, stream);
    if (e != hipSuccess) return hip_fail(e, "centroid copy");
  }
  return MUSE_OK;
}

// ---------------------------------------------------------------- backward pass

int validate_bwd(Shape& s, const muse_fwd_params* p) {
  const int r = validate_muse(s, p);
  if (r != MUSE_OK) return r;
  if (s.D != muse::kBwD) return fail(MUSE_ERR_UNSUPPORTED, "the backward pass is implemented for D=%d", muse::kBwD);
  if (s.causal && p != nullptr && p->dipole == MUSE_DIPOLE_UNTILTED)
    return fail(MUSE_ERR_UNSUPPORTED, "the causal backward pass takes the tilted dipole or none");
  if (p != nullptr) {
    if (p->topk_clusters > 0 || p->hierarchy)
      return fail(MUSE_ERR_UNSUPPORTED, "the backward pass takes no retrieval or hierarchy");
    if (p->labels_q_in != nullptr || p->labels_k_in != nullptr || p->labels_q_trace != nullptr ||
        p->labels_k_trace != nullptr || p->centroids_q_out != nullptr || p->centroids_k_out != nullptr ||
        p->lse_out != nullptr || p->retrieval_trace != nullptr || p->perm_q_out != nullptr ||
        p->offs_q_out != nullptr || p->perm_k_out != nullptr || p->offs_k_out != nullptr)
      return fail(MUSE_ERR_INVALID_ARG, "the backward pass takes the labels as arguments and returns no forward outputs");
  }
  return MUSE_OK;
}

struct BwPlan {
  Plan f;  // the forward's regions (clustering with the fixed labels, stage-1 tables, far field)
  size_t g_logz, g_k, g_v, g_dip, P, lz, gd, dKp, dVp, vgk, dP, dlogz, sij, A, Q, WQ, dcov, kmean, vmean;
  size_t dqbar1, dqbar2, dqbar_part;
  size_t o_loc, l_loc, delta_loc, sdk, sdv, st;  // causal
  int ntb;
  size_t total;
};

BwPlan make_bwd_plan(const Shape& s, const muse_fwd_params* p) {
  BwPlan B{};
  B.f = make_plan(s, p);
  Layout L;
  L.bytes = B.f.total;
  const size_t BH = s.BH, N = s.N, D = s.D, Cq = s.Cq, Ck = s.Ck, f = sizeof(float);
  const size_t E = s.causal ? s.nb : 1;  // table entries
  const int dipole = p ? p->dipole : MUSE_DIPOLE_TILTED;
  B.ntb = (s.N + muse::kBwKeyTile - 1) / muse::kBwKeyTile;
  B.g_logz = L.take(BH * E * Cq * Ck * f);
  B.g_k = L.take(BH * E * Cq * Ck * D * f);
  B.g_v = L.take(BH * E * Cq * Ck * D * f);
  B.g_dip = L.take(BH * E * Cq * D * D * f);
  B.P = L.take(BH * E * Cq * Ck * f);
  B.lz = L.take(BH * E * Cq * f);
  B.dKp = L.take(BH * E * Cq * Ck * D * f);
  B.dVp = L.take(BH * E * Cq * Ck * D * f);
  B.dlogz = L.take(BH * E * Cq * Ck * f);
  if (!s.causal) {
    B.dP = L.take(BH * Cq * Ck * f);
    B.sij = L.take(BH * Cq * Ck * f);
  } else {
    B.sdk = L.take(BH * E * Cq * Ck * D * f);
    B.sdv = L.take(BH * E * Cq * Ck * D * f);
    B.st = L.take(BH * E * Cq * Ck * f);
    B.o_loc = L.take(BH * N * D * f);
    B.l_loc = L.take(BH * N * f);
    B.delta_loc = L.take(BH * N * f);
  }
  if (dipole == MUSE_DIPOLE_TILTED) {
    B.gd = L.take(BH * E * Cq * 4 * D * D * sizeof(uint16_t));
    B.vgk = L.take(BH * E * Cq * Ck * f);
    B.A = L.take(BH * Cq * N * f);
    B.Q = L.take(BH * Cq * N * f);
    if (!s.causal) B.WQ = L.take(BH * Cq * N * f);
  }
  if (dipole == MUSE_DIPOLE_UNTILTED) {
    B.dcov = L.take(BH * Ck * D * D * f);
    B.kmean = L.take(BH * Ck * D * f);
    B.vmean = L.take(BH * Ck * D * f);
  }
  B.dqbar1 = L.take(BH * Cq * D * f);
  B.dqbar2 = L.take(BH * E * Cq * D * f);
  B.dqbar_part = L.take(BH * static_cast<size_t>(B.ntb) * Cq * D * f);
  B.total = L.bytes;
  return B;
}

int run_muse_bwd(const void* q, const void* k, const void* v, const void* dout, const int32_t* labels_q,
                 const int32_t* labels_k, float* dq, float* dk, float* dv, const Shape& s,
                 const muse_fwd_params* p, hipStream_t stream, void* ws) {
  using namespace muse;
  const BwPlan B = make_bwd_plan(s, p);
  const Plan& P = B.f;
  const float scale = scale_of(s, p);
  const int dipole = p ? p->dipole : MUSE_DIPOLE_TILTED;
  // the clustering with the labels held fixed: member-mean centroids and the buckets
  KmArgs km = kmeans_args(q, k, s, P, ws);
  km.t[0].labels_in = labels_q;
  km.t[1].labels_in = labels_k;
  km.t[0].perm = at<int32_t>(ws, P.perm_q);
  km.t[0].offs = at<int32_t>(ws, P.offs_q);
  // the cluster size cap, as in the forward: kept lengths and flags of the key buckets
  km.t[1].cap = cap_members(s, p);
  km.t[1].klen = km.t[1].cap > 0 ? at<int32_t>(ws, P.klen) : nullptr;
  km.t[1].kdrop = km.t[1].cap > 0 ? at<uint8_t>(ws, P.kdrop) : nullptr;
  hipError_t e = launch_kmeans(km, 1, s.dtype, stream);
  if (e != hipSuccess) return hip_fail(e, "K-means launch");
  // the forward's stage-1 summaries as fp32 tables
  S1Args a1 = stage1_args(k, v, s, P, ws, km, scale, dipole);
  a1.one_stream = 1;
  a1.tables_f32 = 1;
  a1.t_khi = a1.t_klo = a1.t_vhi = a1.t_vlo = a1.t_dip = nullptr;
  e = launch_stage1(a1, s.dtype, stream);
  if (e != hipSuccess) return hip_fail(e, "stage-1 launch");
  // causal calls: the forward's far field and in-block exact part, kept apart for the
  // merge's backward; bf16 inputs take the forward's own matrix-core kernels (the far field
  // from bf16 hi/lo copies of the fp32 tables), fp32 inputs the vector-ALU ones
  const bool mf = s.dtype == MUSE_BF16;
  if (s.causal && mf) {
    a1.t_khi = at<uint16_t>(ws, P.t_khi);
    a1.t_klo = at<uint16_t>(ws, P.t_klo);
    a1.t_vhi = at<uint16_t>(ws, P.t_vhi);
    a1.t_vlo = at<uint16_t>(ws, P.t_vlo);
    a1.t_dip = at<uint16_t>(ws, P.t_dip);
    e = launch_stage1_pack(a1, stream);
    if (e != hipSuccess) return hip_fail(e, "table packing launch");
  }
  if (s.causal) {
    S2Args a2{};
    a2.q = q;
    a2.BH = s.BH;
    a2.N = s.N;
    a2.D = s.D;
    a2.Cq = s.Cq;
    a2.Ck = s.Ck;
    a2.causal = 1;
    a2.block = s.block;
    a2.nbS = s.nbS;
    a2.scale = scale;
    a2.dipole = dipole;
    a2.labels_q = km.t[0].labels;
    a2.qbar = km.t[0].cent;
    a2.s_logz = a1.s_logz;
    a2.s_k = a1.s_k;
    a2.s_v = a1.s_v;
    a2.s_dip = a1.s_dip;
    a2.t_khi = a1.t_khi;
    a2.t_klo = a1.t_klo;
    a2.t_vhi = a1.t_vhi;
    a2.t_vlo = a1.t_vlo;
    a2.t_dip = a1.t_dip;
    a2.perm_q = km.t[0].perm;
    a2.offs_q = km.t[0].offs;
    a2.nb = s.nb;
    if (mf) {
      a2.tiles = at<int2>(ws, P.tiles);
      a2.ntiles = at<int32_t>(ws, P.ntiles);
      a2.max_tiles = P.max_tiles;
    }
    a2.o_far = at<float>(ws, P.o_far);
    a2.l_far = at<float>(ws, P.l_far);
    e = launch_stage2(a2, s.dtype, stream);
    if (e != hipSuccess) return hip_fail(e, "stage-2 launch");
    ExactArgs ax{};
    ax.q = q;
    ax.k = k;
    ax.v = v;
    ax.out = at<float>(ws, B.o_loc);
    ax.lse_out = at<float>(ws, B.l_loc);
    ax.BH = s.BH;
    ax.N = s.N;
    ax.D = s.D;
    ax.causal = 1;
    ax.block = s.block;
    ax.scale = scale;
    ax.out_bf16 = 0;
    ax.exact_p = 1;
    e = launch_exact(ax, s.dtype, stream);
    if (e != hipSuccess) return hip_fail(e, "local block launch");
  }
  BwArgs b{};
  b.q = q;
  b.k = k;
  b.v = v;
  b.dout = dout;
  b.dq = dq;
  b.dk = dk;
  b.dv = dv;
  b.BH = s.BH;
  b.N = s.N;
  b.D = s.D;
  b.Cq = s.Cq;
  b.Ck = s.Ck;
  b.scale = scale;
  b.dipole = dipole;
  b.labels_k = labels_k;
  b.kdrop = km.t[1].kdrop;
  b.klen = km.t[1].klen;
  b.qbar = km.t[0].cent;
  b.perm_q = km.t[0].perm;
  b.offs_q = km.t[0].offs;
  b.perm_k = km.t[1].perm;
  b.offs_k = km.t[1].offs;
  b.logz = a1.s_logz;
  b.tk = a1.s_k;
  b.tv = a1.s_v;
  b.dip = a1.s_dip;
  b.cov = a1.cov_k;
  b.g_logz = at<float>(ws, B.g_logz);
  b.g_k = at<float>(ws, B.g_k);
  b.g_v = at<float>(ws, B.g_v);
  b.g_dip = at<float>(ws, B.g_dip);
  b.P = at<float>(ws, B.P);
  b.lz = at<float>(ws, B.lz);
  b.dKp = at<float>(ws, B.dKp);
  b.dVp = at<float>(ws, B.dVp);
  b.dlogz = at<float>(ws, B.dlogz);
  if (!s.causal) {
    b.dP = at<float>(ws, B.dP);
    b.sij = at<float>(ws, B.sij);
  } else {
    b.causal = 1;
    b.nb = s.nb;
    b.block = s.block;
    b.o_loc = at<float>(ws, B.o_loc);
    b.l_loc = at<float>(ws, B.l_loc);
    b.delta_loc = at<float>(ws, B.delta_loc);
    b.o_far = at<float>(ws, P.o_far);
    b.l_far = at<float>(ws, P.l_far);
    b.sdk = at<float>(ws, B.sdk);
    b.sdv = at<float>(ws, B.sdv);
    b.st = at<float>(ws, B.st);
  }
  if (dipole == MUSE_DIPOLE_TILTED) {
    b.gd = at<uint16_t>(ws, B.gd);
    b.vgk = at<float>(ws, B.vgk);
    b.A = at<float>(ws, B.A);
    b.Q = at<float>(ws, B.Q);
    if (!s.causal) b.WQ = at<float>(ws, B.WQ);
  }
  if (dipole == MUSE_DIPOLE_UNTILTED) {
    b.dcov = at<float>(ws, B.dcov);
    b.kmean = at<float>(ws, B.kmean);
    b.vmean = at<float>(ws, B.vmean);
  }
  b.dqbar1 = at<float>(ws, B.dqbar1);
  b.dqbar2 = at<float>(ws, B.dqbar2);
  b.dqbar_part = at<float>(ws, B.dqbar_part);
  b.ntb = B.ntb;
  e = launch_backward(b, s.dtype, stream);
  if (e != hipSuccess) return hip_fail(e, "backward launch");
  return MUSE_OK;
}

// ---------------------------------------------------------------- allocation-free scratch

}  // namespace

// Scratch of muse_attn_fwd_noalloc: device memory that is part of the library's code
// object, so no call allocates it. Each device holds its own copy from the library's
// load until the process ends. In host code `scratch` names a host-side shadow, not the
// device memory: kernels only ever receive the address hipGetSymbolAddress returns for
// the current device (scratch_address below).
static __device__ __align__(256) unsigned char scratch[MUSE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 64;

// Device address of `scratch` on the current device, looked up once per device (with
// that device current) and kept; MUSE_ERR_HIP when the lookup fails.
int scratch_address(void** out) {
  static std::mutex mu;
  static void* addr[kMaxScratchDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(MUSE_ERR_UNSUPPORTED, "device %d: the allocation-free entry serves devices 0..%d", dev,
                kMaxScratchDevices - 1);
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (ptr == nullptr) return fail(MUSE_ERR_HIP, "hipGetSymbolAddress(scratch) returned a null address");
    addr[dev] = ptr;
  }
  *out = addr[dev];
  return MUSE_OK;
}

// ---------------------------------------------------------------- per-kernel timing

struct ProfRec {
  const char* name;
  hipEvent_t e0, e1;
};

struct ProfState {
  std::mutex mu;
  bool on = false;
  std::vector<hipEvent_t> pool;
  std::vector<ProfRec> pending;
  std::vector<std::string> names;
  std::vector<double> total_ms;
  std::vector<long> launches;
};

ProfState& prof() {
  static ProfState* p = new ProfState();  // never destroyed: events may outlive static teardown
  return *p;
}

hipEvent_t prof_event(ProfState& P) {
  if (!P.pool.empty()) {
    hipEvent_t e = P.pool.back();
    P.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

namespace muse {

ProfScope::ProfScope(const char* name, hipStream_t s) : name_(name), s_(s), e0_(nullptr), e1_(nullptr) {
  ProfState& P = prof();
  std::lock_guard<std::mutex> g(P.mu);
  if (!P.on) return;
  e0_ = prof_event(P);
  e1_ = prof_event(P);
  if (e0_ != nullptr) (void)hipEventRecord(e0_, s_);
}

ProfScope::~ProfScope() {
  if (e0_ == nullptr || e1_ == nullptr) return;
  ProfState& P = prof();
  std::lock_guard<std::mutex> g(P.mu);
  (void)hipEventRecord(e1_, s_);
  P.pending.push_back({name_, e0_, e1_});
}

}  // namespace muse

extern "C" {

void muse_prof_enable(int on) {
  ProfState& P = prof();
  std::lock_guard<std::mutex> g(P.mu);
  P.on = on != 0;
}

int muse_prof_collect(void) {
  ProfState& P = prof();
  std::lock_guard<std::mutex> g(P.mu);
  for (const ProfRec& r : P.pending) {
    float ms = 0.f;
    if (hipEventSynchronize(r.e1) == hipSuccess && hipEventElapsedTime(&ms, r.e0, r.e1) == hipSuccess) {
      size_t i = 0;
      while (i < P.names.size() && P.names[i] != r.name) ++i;
      if (i == P.names.size()) {
        P.names.emplace_back(r.name);
        P.total_ms.push_back(0.0);
        P.launches.push_back(0);
      }
      P.total_ms[i] += ms;
      P.launches[i] += 1;
    }
    P.pool.push_back(r.e0);
    P.pool.push_back(r.e1);
  }
  P.pending.clear();
  return static_cast<int>(P.names.size());
}

const char* muse_prof_name(int i) {
  ProfState& P = prof();
  return (i >= 0 && i < static_cast<int>(P.names.size())) ? P.names[i].c_str() : "";
}

double muse_prof_total_ms(int i) {
  ProfState& P = prof();
  return (i >= 0 && i < static_cast<int>(P.total_ms.size())) ? P.total_ms[i] : 0.0;
}

long muse_prof_launches(int i) {
  ProfState& P = prof();
  return (i >= 0 && i < static_cast<int>(P.launches.size())) ? P.launches[i] : 0;
}

void muse_prof_reset(void) {
  (void)muse_prof_collect();
  ProfState& P = prof();
  std::lock_guard<std::mutex> g(P.mu);
  P.names.clear();
  P.total_ms.clear();
  P.launches.clear();
}

void muse_fwd_params_init(muse_fwd_params* p) {
  if (p == nullptr) return;
  memset(p, 0, sizeof(*p));
  p->scale = 0.f;
  p->out_dtype = -1;
  p->dipole = MUSE_DIPOLE_TILTED;
}

const char* muse_last_error(void) { return g_last_error.c_str(); }

int muse_version(void) { return 102; }

size_t muse_attn_fwd_workspace_bytes(int B, int H, int N, int D, int Cq, int Ck, int causal, int block,
                                     int dtype, const muse_fwd_params* p) {
  Shape s{B, H, N, D, Cq, Ck, 1, causal, block, dtype};
  if (validate_muse(s, p) != MUSE_OK) return 0;
  return make_plan(s, p).total;
}

int muse_attn_fwd_ex(const void* q, const void* k, const void* v, void* out, int B, int H, int N, int D,
                     int Cq, int Ck, int kmeans_iters, int causal, int block, int dtype, void* hip_stream,
                     const muse_fwd_params* p) {
  g_last_error.clear();
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr)
    return fail(MUSE_ERR_INVALID_ARG, "q, k, v and out must be non-null device pointers");
  Shape s{B, H, N, D, Cq, Ck, kmeans_iters, causal, block, dtype};
  int r = validate_muse(s, p);
  if (r != MUSE_OK) return r;
  if (out == q || out == k || out == v) return fail(MUSE_ERR_INVALID_ARG, "out must not alias an input");
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  const size_t need = make_plan(s, p).total;
  void* ws = p ? p->workspace : nullptr;
  bool owned = false;
  if (ws != nullptr) {
    if (p->workspace_bytes < need)
      return fail(MUSE_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", p->workspace_bytes, need);
  } else {
    const hipError_t e = hipMallocAsync(&ws, need, stream);
    if (e != hipSuccess) return fail(MUSE_ERR_NO_MEMORY, "hipMallocAsync(%zu): %s", need, hipGetErrorString(e));
    owned = true;
  }
  r = run_muse(q, k, v, out, s, p, stream, ws);
  if (owned) {
    const hipError_t e = hipFreeAsync(ws, stream);
    if (e != hipSuccess && r == MUSE_OK) r = hip_fail(e, "hipFreeAsync");
  }
  if (r == MUSE_OK && getenv("MUSE_DEBUG_SYNC") != nullptr) {
    const hipError_t e = hipStreamSynchronize(stream);
    if (e != hipSuccess) r = hip_fail(e, "debug sync");
  }
  return r;
}

int muse_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* out, int B, int H, int N, int D,
                          int Cq, int Ck, int kmeans_iters, int causal, int block, int dtype, void* hip_stream,
                          const muse_fwd_params* p) {
  g_last_error.clear();
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr)
    return fail(MUSE_ERR_INVALID_ARG, "q, k, v and out must be non-null device pointers");
  Shape s{B, H, N, D, Cq, Ck, kmeans_iters, causal, block, dtype};
  int r = validate_muse(s, p);
  if (r != MUSE_OK) return r;
  if (out == q || out == k || out == v) return fail(MUSE_ERR_INVALID_ARG, "out must not alias an input");
  if (p != nullptr && p->workspace != nullptr)
    return fail(MUSE_ERR_INVALID_ARG, "the allocation-free entry uses the library's own scratch: workspace must be NULL");
  const size_t need = make_plan(s, p).total;
  if (need > static_cast<size_t>(MUSE_NOALLOC_SCRATCH_BYTES))
    return fail(MUSE_ERR_WORKSPACE, "this call needs %zu bytes of scratch, more than the %zu the allocation-free entry holds",
                need, static_cast<size_t>(MUSE_NOALLOC_SCRATCH_BYTES));
  void* ws = nullptr;
  r = scratch_address(&ws);
  if (r != MUSE_OK) return r;
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  r = run_muse(q, k, v, out, s, p, stream, ws, /*one_stream=*/true);
  if (r == MUSE_OK && getenv("MUSE_DEBUG_SYNC") != nullptr) {
    const hipError_t e = hipStreamSynchronize(stream);
    if (e != hipSuccess) r = hip_fail(e, "debug sync");
  }
  return r;
}

size_t muse_attn_bwd_workspace_bytes(int B, int H, int N, int D, int Cq, int Ck, int causal, int block,
                                     int dtype, const muse_fwd_params* p) {
  Shape s{B, H, N, D, Cq, Ck, 1, causal, block, dtype};
  if (validate_bwd(s, p) != MUSE_OK) return 0;
  return make_bwd_plan(s, p).total;
}

int muse_attn_bwd(const void* q, const void* k, const void* v, const void* dout, const int32_t* labels_q,
                  const int32_t* labels_k, float* dq, float* dk, float* dv, int B, int H, int N, int D, int Cq,
                  int Ck, int causal, int block, int dtype, void* hip_stream, const muse_fwd_params* p) {
  g_last_error.clear();
  if (q == nullptr || k == nullptr || v == nullptr || dout == nullptr)
    return fail(MUSE_ERR_INVALID_ARG, "q, k, v and dout must be non-null device pointers");
  if (labels_q == nullptr || labels_k == nullptr)
    return fail(MUSE_ERR_INVALID_ARG, "labels_q and labels_k (the forward's final labels) are required");
  if (dq == nullptr || dk == nullptr || dv == nullptr)
    return fail(MUSE_ERR_INVALID_ARG, "dq, dk and dv must be non-null device pointers");
  Shape s{B, H, N, D, Cq, Ck, 1, causal, block, dtype};
  int r = validate_bwd(s, p);
  if (r != MUSE_OK) return r;
  const void* ins[] = {q, k, v, dout, labels_q, labels_k};
  const void* outs[] = {dq, dk, dv};
  for (const void* o : outs)
    for (const void* in : ins)
      if (o == in) return fail(MUSE_ERR_INVALID_ARG, "dq, dk and dv must not alias an input");
  if (dq == dk || dq == dv || dk == dv) return fail(MUSE_ERR_INVALID_ARG, "dq, dk and dv must be distinct");
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  const size_t need = make_bwd_plan(s, p).total;
  void* ws = p ? p->workspace : nullptr;
  bool owned = false;
  if (ws != nullptr) {
    if (p->workspace_bytes < need)
      return fail(MUSE_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", p->workspace_bytes, need);
  } else {
    const hipError_t e = hipMallocAsync(&ws, need, stream);
    if (e != hipSuccess) return fail(MUSE_ERR_NO_MEMORY, "hipMallocAsync(%zu): %s", need, hipGetErrorString(e));
    owned = true;
  }
  r = run_muse_bwd(q, k, v, dout, labels_q, labels_k, dq, dk, dv, s, p, stream, ws);
  if (owned) {
    const hipError_t e = hipFreeAsync(ws, stream);
    if (e != hipSuccess && r == MUSE_OK) r = hip_fail(e, "hipFreeAsync");
  }
  if (r == MUSE_OK && getenv("MUSE_DEBUG_SYNC") != nullptr) {
    const hipError_t e = hipStreamSynchronize(stream);
    if (e != hipSuccess) r = hip_fail(e, "debug sync");
  }
  return r;
}

int muse_attn_fwd(const void* q, const void* k, const void* v, void* out, int B, int H, int N, int D, int Cq,
                  int Ck, int kmeans_iters, int causal, int block, int dtype, void* hip_stream) {
  return muse_attn_fwd_ex(q, k, v, out, B, H, N, D, Cq, Ck, kmeans_iters, causal, block, dtype, hip_stream,
                          nullptr);
}

int muse_exact_attn_fwd(const void* q, const void* k, const void* v, void* out, int B, int H, int N, int D,
                        int causal, int dtype, void* hip_stream) {
  g_last_error.clear();
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr)
    return fail(MUSE_ERR_INVALID_ARG, "q, k, v and out must be non-null device pointers");
  Shape s{B, H, N, D, 1, 1, 1, causal, 0, dtype};
  if (causal != 0 && causal != 1) return fail(MUSE_ERR_INVALID_ARG, "causal must be 0 or 1");
  s.causal = 0;  // validate the shape without the block checks of causal MuSe
  const int r = validate(s, nullptr);
  if (r != MUSE_OK) return r;
  if (out == q || out == k || out == v) return fail(MUSE_ERR_INVALID_ARG, "out must not alias an input");
  muse::ExactArgs ax{};
  ax.q = q;
  ax.k = k;
  ax.v = v;
  ax.out = out;
  ax.BH = s.BH;
  ax.N = N;
  ax.D = D;
  ax.causal = causal;
  ax.block = 0;
  ax.scale = 1.0f / sqrtf(static_cast<float>(D));
  ax.out_bf16 = dtype == MUSE_BF16;
  const hipError_t e = muse::launch_exact(ax, dtype, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return hip_fail(e, "exact attention launch");
  return MUSE_OK;
}

}  // extern "C"
