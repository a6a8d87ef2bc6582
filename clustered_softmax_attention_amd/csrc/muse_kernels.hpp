// Kernel argument blocks and launcher declarations of the MuSe HIP library.
#pragma once

#include "muse_common.hpp"

namespace muse {

constexpr int kChunkC = 32;    // centroids staged in LDS at a time by the fp32 assign kernel
constexpr int kMaxTile = 512;  // K-means tile (points per workgroup) upper bound, fp32 path
constexpr int kMaxTileMfma = 256;  // the same for the matrix-core (bf16) path
constexpr int kMaxClusters = 128;
constexpr int kMaxMomKeys = 8192;  // positions per block-moment range (matrix-core path)
// query centroids per workgroup of the matrix-core moment kernel
constexpr int moments_group(int D) { return D == 64 ? 16 : 4; }
// Key buckets are cut into atom work items of at most kAtomSeg positions, so that one
// large cluster does not serialise the atoms; a bucket of n keys gives max(1, ceil(n /
// kAtomSeg)) items, hence at most nb*Ck + ceil(N / kAtomSeg) per head. Buckets of more
// than one item (fewer than ceil(N / kAtomSeg) of them) hold fewer than 2 ceil(N /
// kAtomSeg) items together, each with a partial-atom slot.
constexpr int kAtomSeg = 64;
constexpr int kS2Chunk = 128;  // queries per matrix-core stage-2 workgroup (a run of one query bucket)
__host__ __device__ constexpr int atom_max_items(int nbC, int N) { return nbC + (N + kAtomSeg - 1) / kAtomSeg; }
__host__ __device__ constexpr int atom_max_multi(int N) { return (N + kAtomSeg - 1) / kAtomSeg; }
__host__ __device__ constexpr int atom_max_partials(int N) { return 2 * atom_max_multi(N); }

// ------------------------------------------------------------------ K-means

struct KmTensor {
  const void* x;               // [BH, N, D] input (dtype of the call)
  int C;                       // clusters
  float* cent;                 // [BH, C, D] current centroids
  uint16_t* chi;               // [BH, C, D] bf16 hi part of cent (matrix-core path) or null
  uint16_t* clo;               // [BH, C, D] bf16 lo part: cent = hi + lo up to 2^-16
  float* cn2;                  // [BH, C] ||c_j||^2 in fp32
  int32_t* labels;             // [BH, N] labels of the latest assign step
  int32_t* trace;              // [iters, BH, N] or null
  const int32_t* labels_in;    // [BH, N] caller-fixed labels or null
  uint16_t* tile_perm;         // [BH, ntiles, tile] tile-local stable order by label
  int32_t* tile_cnt;           // [BH, ntiles, C] (last iteration: per-tile counts for bucketing)
  int32_t* tile_start;         // [BH, ntiles, C]
  float* psum;                 // [BH, ntiles, C, D] cluster sums, one slab per tile group
  int32_t* gcnt;               // [BH, ntiles, C] cluster counts, one row per tile group
  int32_t* perm;               // [BH, N] points ordered by (block, label, position), or null
  int32_t* offs;               // [BH, nb*C + 1] bucket offsets into perm
  int tpg, ngroups;             // tiles per assign workgroup and workgroups per head (set by the launcher)
  // atom work items (key tensor, matrix-core path; null otherwise):
  int4* items;                 // [BH, atom_max_items] (first position, positions (-1: none), partial slot or -1, bucket)
  int4* multi;                 // [BH, 1 + atom_max_multi]: (count), then (bucket, first partial slot, items) per
                               // bucket of several items
  int2* bmeta;                 // [BH, nb*C]: per bucket (first partial slot or -1, items)
  // stage-2 chunks (query tensor, matrix-core path; null otherwise): runs of at most
  // kS2Chunk positions of one bucket
  int2* chunks;                // [BH, max_chunks] (bucket, first position)
  int32_t* nchunks;            // [BH]
  int max_chunks;
  // cluster size cap (key tensor; null: no cap): a cluster keeps its first `cap` members
  // in position order, so bucket (b, j) keeps a prefix of its positions
  int cap;
  int32_t* klen;               // [BH, nb*C] kept members of every bucket (items cover only these)
  uint8_t* kdrop;              // [BH, N] 1 for a point left out (by position in the input)
};

struct KmArgs {
  KmTensor t[2];
  int ntensors;
  int BH, N, D;
  int tile, ntiles;            // points per tile, tiles per head
  int nb, tiles_per_block;     // spatial blocks (1 when acausal) and tiles in one
  int ngroups;                 // assign workgroups per head: the largest of the tensors' (set by the launcher)
};

hipError_t launch_kmeans(const KmArgs& a, int iters, int dtype, hipStream_t s);

// ------------------------------------------------------------------ retrieval

constexpr int kMaxRetrBlocks = 4096;  // spatial blocks per head with retrieval on
constexpr int kMaxRetrRow = 256;      // k1 * (1 + k2)

struct RetrArgs {
  const void* q;
  const void* k;
  const void* v;
  int BH, N, D, Cq, Ck, nb;
  int k1, k2, dipole;
  float scale;
  const float* qbar;           // [BH, Cq, D]
  const int32_t* perm_k;       // [BH, N]
  const int32_t* offs_k;       // [BH, nb*Ck + 1]
  const int32_t* perm_q;       // [BH, N]
  const int32_t* offs_q;       // [BH, nb*Cq + 1]
  const float* at_m;           // atoms [BH, nb, Cq, Ck(, D)]
  const float* at_z;
  const float* at_k;
  const float* at_v;
  float* s_logz;               // tables [BH, nb, Cq, ...], entry (b, i) rewritten in place
  float* s_k;
  float* s_v;
  float* s_dip;               // entry (b, i) holds E[v k^T] before the dipole finalise
  int32_t* sel;                // [BH, nb, Cq, k1*(1+k2)] selection
  int32_t* trace;              // copy of sel for the caller, or null
  float* o_far;                // [BH, N, D] far-field partial result (merged in place)
  float* l_far;                // [BH, N]
  // matrix-core exact part (bf16 inputs): the stage-2 query chunks
  const int2* tiles;           // [BH, max_tiles] (bucket, first position)
  const int32_t* ntiles;       // [BH]
  int max_tiles;
};

hipError_t launch_retrieval(const RetrArgs& a, int phase, int dtype, hipStream_t s);  // 0 tables, 1 exact

// ------------------------------------------------------------------ stage 1

struct S1Args {
  const void* k;               // [BH, N, D]
  const void* v;               // [BH, N, D]
  int BH, N, D, Cq, Ck;
  int nb, block;               // key blocks (1 and N when acausal)
  int causal;                  // table entry b holds blocks < b (causal) or all keys (acausal)
  int nbS;                     // table entries: nb when causal, 1 when acausal
  float scale;
  int dipole;                  // 0 none, 1 tilted, 2 untilted (acausal only)
  int hier;                    // causal: table entry e covers key blocks [e - lowbit(e), e)
                               // (hierarchical squares) instead of [0, e)
  const float* qbar;           // [BH, Cq, D] query centroids
  const int32_t* perm_k;       // [BH, N] keys by (block, label)
  const int32_t* offs_k;       // [BH, nb*Ck + 1]
  const int4* items_k;         // [BH, atom_max_items] atom work items (matrix-core path)
  const int4* multi_k;         // [BH, 1 + atom_max_multi] buckets of several items
  const int2* bmeta_k;         // [BH, nb*Ck] per bucket (first partial slot or -1, items)
  // partial atoms of buckets with several work items: [BH, atom_max_partials, Cq(, D)]
  float* pt_m;
  float* pt_z;
  float* pt_k;
  float* pt_v;
  // atoms: one (query cluster i, key cluster j, key block b') each
  float* at_m;                 // [BH, nb, Cq, Ck] max logit
  float* at_z;                 // [BH, nb, Cq, Ck] sum exp(a - m)
  float* at_k;                 // [BH, nb, Cq, Ck, D] sum exp(a - m) k
  float* at_v;                 // [BH, nb, Cq, Ck, D] sum exp(a - m) v
  int nmb, mbk;                // moment sub-blocks: count and keys per sub-block (divides block)
  float* scores;               // [BH, Cq, N] s qbar_i . k_m (matrix-core path) or null
  float* tmax;                 // [BH, Cq, ceil(N / 32)] max of the scores of every 32 positions
  float* blk_lmass;            // [BH, nmb, Cq] log mass of a sub-block seen by centroid i
  float* blk_mom;              // [BH, nmb, Cq, D, D] sub-block-normalised sum w v k^T (v index first)
  // summary tables
  float* s_logz;               // [BH, nbS, Cq, Ck]
  float* s_k;                  // [BH, nbS, Cq, Ck, D] tilted key means
  float* s_v;                  // [BH, nbS, Cq, Ck, D] tilted value means
  float* s_dip;                // [BH, nbS, Cq, D(v), D(k)] aggregated dipole, value index first
  // bf16 copies for the matrix-core stage 2 (null on the fp32 path)
  uint16_t* t_khi;             // [BH, nbS, Cq, Ck, D]  K_ij = hi + lo
  uint16_t* t_klo;
  uint16_t* t_vhi;             // [BH, nbS, Cq, Ck, D]  V_ij = hi + lo (row-major like K)
  uint16_t* t_vlo;
  uint16_t* t_dip;             // [BH, nbS, Cq, D(v), D(k)]  s * D_i, value index first
  const RetrArgs* retr;        // retrieval: rewrites table entries before the dipole finalise
  int one_stream;              // 1: every kernel on the caller's stream (no side stream, no events)
  float* cov_k;                // [BH, Ck, D(v), D(k)] untilted dipole: per key cluster covariance
  // untilted dipole, causal: statistics of every (key block, key cluster) bucket and
  // their prefix over the blocks (entry b: the keys of blocks < b)
  float* ub_n;                 // [BH, nb*Ck] keys in the bucket
  float* ub_mk;                // [BH, nb*Ck, D] their key mean
  float* ub_mv;                // [BH, nb*Ck, D] their value mean
  float* ub_c;                 // [BH, nb*Ck, D(v), D(k)] centred sum of (v - mv)(k - mk)^T
  float* up_n;                 // [BH, nb, Ck] keys of cluster j in the blocks before b
  float* up_mk;                // [BH, nb, Ck, D] their key mean
  float* up_mv;                // [BH, nb, Ck, D] their value mean
  // cluster size cap (null: none): kept keys of every bucket (a prefix of it) and a flag
  // per key (input position) that is 1 when the key is left out of the summaries
  const int32_t* klen;         // [BH, nb*Ck]
  const uint8_t* kdrop;        // [BH, N]
  // 1: fp32 tables only (s_logz, s_k, s_v, s_dip; no bf16 packing), on the general path
  // for either dtype (used by the backward pass)
  int tables_f32;
};

hipError_t launch_stage1(const S1Args& a, int dtype, hipStream_t s);
// bf16 hi/lo copies (t_*) of fp32 tables already built (s_logz, s_k, s_v, s_dip)
hipError_t launch_stage1_pack(const S1Args& a, hipStream_t s);
void launch_stage1_mfma(const S1Args& a, int which, hipStream_t s);  // 0 scores, 1 atoms (+ merge), 2 moments, 3 finalise, 4 scan, 5 general-path dipole

// ------------------------------------------------------------------ stage 2

struct S2Args {
  const void* q;               // [BH, N, D]
  void* out;                   // [BH, N, D] (acausal) in out dtype
  float* o_far;                // [BH, N, D] f32 (causal far field) or null
  float* l_far;                // [BH, N] (causal) or null
  float* lse_out;              // [BH, N] (acausal) or null
  int BH, N, D, Cq, Ck;
  int causal, block, nbS;
  float scale;
  int dipole;
  int hier;                    // causal: merge the entries b, b & (b - 1), ... > 0
  int level;                   // matrix-core path with hier: the chain entry of this launch
  int out_bf16;
  const int32_t* labels_q;     // [BH, N]
  const float* qbar;           // [BH, Cq, D]
  const float* s_logz;
  const float* s_k;
  const float* s_v;
  const float* s_dip;
  // matrix-core path (bf16 inputs)
  const uint16_t* t_khi;
  const uint16_t* t_klo;
  const uint16_t* t_vhi;
  const uint16_t* t_vlo;
  const uint16_t* t_dip;
  const int32_t* perm_q;       // [BH, N] queries by (block, label)
  const int32_t* offs_q;       // [BH, nb*Cq + 1]
  int nb;                      // query blocks (1 when acausal)
  const int2* tiles;           // [BH, max_tiles] (bucket, first position) of kS2Chunk-query chunks
  const int32_t* ntiles;       // [BH] (both listed by the query tensor's bucket pass)
  int max_tiles;
};

hipError_t launch_stage2(const S2Args& a, int dtype, hipStream_t s);

// ------------------------------------------------------------------ exact attention

struct ExactArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;                   // [BH, N, D] in out dtype
  float* lse_out;              // [BH, N] or null
  const float* o_far;          // far-field partial result to merge, or null
  const float* l_far;
  int BH, N, D;
  int causal;
  int block;                   // > 0: keys restricted to the query's own block (local)
  float scale;
  int out_bf16;
  int exact_p;                 // bf16 path: weights as bf16 hi + lo in the product with V
};

hipError_t launch_exact(const ExactArgs& a, int dtype, hipStream_t s);

// ------------------------------------------------------------------ backward

constexpr int kBwD = 64;       // head dimension of the backward kernels
constexpr int kBwKeyTile = 64; // keys per tile of the per-key backward pass

struct BwArgs {
  const void* q;               // [BH, N, D] inputs of the forward (dtype of the call)
  const void* k;
  const void* v;
  const void* dout;            // [BH, N, D] upstream gradient (dtype of the call)
  float* dq;                   // [BH, N, D] outputs
  float* dk;
  float* dv;
  int BH, N, D, Cq, Ck;
  float scale;
  int dipole;                  // 0 none, 1 tilted, 2 untilted
  const int32_t* labels_k;     // [BH, N] fixed key labels (clamped to [0, Ck) on read)
  const float* qbar;           // [BH, Cq, D] query centroids (member means)
  const int32_t* perm_q;       // [BH, N] / [BH, Cq + 1] query buckets
  const int32_t* offs_q;
  const int32_t* perm_k;       // [BH, N] / [BH, Ck + 1] key buckets
  const int32_t* offs_k;
  // forward summaries (fp32, the single acausal entry)
  const float* logz;           // [BH, Cq, Ck]
  const float* tk;             // [BH, Cq, Ck, D] K_ij
  const float* tv;             // [BH, Cq, Ck, D] V_ij
  const float* dip;            // [BH, Cq, D(v), D(k)] D_i
  const float* cov;            // [BH, Ck, D(v), D(k)] untilted: Cov_j
  // gradients with respect to the summaries and intermediates
  float* g_logz;               // [BH, Cq, Ck]
  float* g_k;                  // [BH, Cq, Ck, D]
  float* g_v;                  // [BH, Cq, Ck, D]
  float* g_dip;                // [BH, Cq, D(v), D(k)]
  float* P;                    // [BH, Cq, Ck] softmax_j log Z_ij
  float* lz;                   // [BH, Cq] log sum_j Z_ij
  uint16_t* gd;                // [BH, Cq, 4, D, D] bf16: hi, lo of G_Dip (row v), hi, lo of its transpose
  float* dKp;                  // [BH, Cq, Ck, D] dL/dK_ij after the dipole's dependence on K_ij
  float* dVp;                  // [BH, Cq, Ck, D]
  float* vgk;                  // [BH, Cq, Ck] V_ij^T G_Dip_i K_ij
  float* dP;                   // [BH, Cq, Ck] dL/dP_ij
  float* dlogz;                // [BH, Cq, Ck] total dL/dlog Z_ij
  float* sij;                  // [BH, Cq, Ck] sum over the cluster's keys of w dL/dw
  float* A;                    // [BH, Cq, N] s qbar_i . k at key positions in bucket order
  float* Q;                    // [BH, Cq, N] v^T G_Dip_i k
  float* WQ;                   // [BH, Cq, N] w Q
  float* dcov;                 // [BH, Ck, D, D] untilted: sum_i P_ij G_Dip_i
  float* kmean;                // [BH, Ck, D] untilted: cluster means
  float* vmean;
  float* dqbar1;               // [BH, Cq, D] stage-1 part of dL/dqbar through K_ij
  float* dqbar2;               // [BH, Cq, D] stage-2 part
  float* dqbar_part;           // [BH, ntb, Cq, D] per key tile: s sum_m w dL/dw k_m
  int ntb;                     // key tiles of kBwKeyTile positions
  // causal calls: table entry b (b >= 1) covers the key blocks before b; the summary
  // arrays above then hold one entry per block ([BH, nb, Cq, ...]); the far field is
  // merged with the exact attention inside each block by log-sum-exp
  int causal, nb, block;
  float* o_loc;                // [BH, N, D] exact in-block output (fp32), then dL/d(it) in place
  float* l_loc;                // [BH, N] its log normaliser
  float* delta_loc;            // [BH, N] dL/do_loc . o_loc - dL/dl_loc
  float* o_far;                // [BH, N, D] far-field output (fp32), then dL/d(it) in place
  float* l_far;                // [BH, N] its log normaliser, then dL/d(it) in place
  // suffix tables over the entries after block b' (scaled relative to entry b' + 1)
  float* sdk;                  // [BH, nb, Cq, Ck, D] sum_{b > b'} exp(logZ^{b'+1} - logZ^b) dK'^b
  float* sdv;                  // [BH, nb, Cq, Ck, D]
  float* st;                   // [BH, nb, Cq, Ck] the same of dL/dlog Z^b - S^b
  // (tilted) gd then holds, per (b', i), sh = sum_{b > b'} exp(lz^{b'+1} - lz^b) G_Dip^b
  // in the same four bf16 layouts ([BH, nb, Cq, 4, D, D])
  // cluster size cap (null: none): keys left out of the summaries take no gradient
  // through them; per bucket the kept members are a prefix of its positions
  const uint8_t* kdrop;        // [BH, N] by input position
  const int32_t* klen;         // [BH, nb*Ck] kept members per bucket
};

hipError_t launch_backward(const BwArgs& a, int dtype, hipStream_t s);

}  // namespace muse
