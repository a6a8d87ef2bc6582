/*
 * muse.h - C ABI of the MI355X (gfx950) Multipole Semantic Attention forward pass.
 *
 * Method (arXiv 2509.10406, R. Mitchell and K. Kersting, known here from the
 * pith.science review page, the pith.science verdict record, the gist.science
 * technical summary and the fugumt.com v2 abstract):
 *   - queries and keys are clustered separately with K-means (gist.science,
 *     Kernmechanismen 1; pith.science review, "Core claim");
 *   - stage 1: coarse query centroids attend to fine key clusters and form
 *     exponentially tilted key/value means, log-normalisers and a tilted
 *     value-key covariance (pith.science review, "What carries the argument");
 *   - stage 2: every query refines its cluster's summaries with its residual:
 *     monopole plus dipole (gist.science, Kernmechanismen 2);
 *   - causal: exact attention inside each diagonal block plus summaries of all
 *     preceding blocks (pith.science review, caption of Figure 2; gist.science,
 *     Kernmechanismen 3), optionally with retrieval of the top (cluster, block)
 *     pairs attended exactly (gist.science, Kernmechanismen 4).
 *
 * Conventions shared by every entry point
 *   - q, k, v, out: DEVICE pointers to contiguous [B, H, N, D] tensors, row-major
 *     with D fastest, 16-byte aligned, owned by the caller. out must not alias an
 *     input. Every element of out is written; nothing is accumulated into it.
 *   - dtype: MUSE_F32 or MUSE_BF16 (storage type of q, k, v; bfloat16 as raw
 *     16-bit patterns). All arithmetic accumulates in fp32.
 *   - hip_stream: a hipStream_t (NULL = the default stream). Calls only enqueue
 *     work on it and return; there is no host synchronisation inside. Pointers
 *     must stay valid until that work completes. Part of a bf16 call (the stage-1
 *     atoms) runs on a stream the library keeps per device, forked from and joined
 *     back into hip_stream by events recorded in the call, so the whole call is
 *     still ordered after earlier work on hip_stream and before later work on it
 *     (a graph capture of hip_stream captures both branches). Concurrent calls on
 *     several caller streams of one device serialise on that stream's share.
 *   - Errors: arguments are validated on the host before anything is launched; a
 *     negative status is returned and muse_last_error() describes it. A launch
 *     failure returns MUSE_ERR_HIP. Faults during execution surface at the
 *     caller's next synchronisation. No exception or abort crosses the ABI.
 *   - Determinism: identical inputs on the same device give bitwise identical
 *     outputs (no floating-point atomics anywhere).
 *   - Valid shapes: B, H, N >= 1; 1 <= Cq, Ck <= N; kmeans_iters >= 1; causal:
 *     1 <= block <= N with N % block == 0. A valid shape outside what the kernels
 *     implement returns MUSE_ERR_UNSUPPORTED: D not in {64, 128}, Cq or Ck above
 *     128, a causal block below 64 or not a multiple of 64.
 *   - Value range (bf16 inputs): the block second moments take keys and values as
 *     fp16 operands, so every |k| and |v| element must stay below 65504 (larger ones
 *     give infinite or NaN outputs). bf16 converts to fp16 exactly for magnitudes from
 *     2^-14 up; smaller ones keep fewer bits (fp16 subnormals) or become zero below
 *     2^-25, a change far below the stated tolerances.
 */
#ifndef MUSE_H_
#define MUSE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { MUSE_F32 = 0, MUSE_BF16 = 1 } muse_dtype_t;

enum {
  MUSE_OK = 0,
  MUSE_ERR_INVALID_ARG = -1, /* a pointer, size or flag is out of range         */
  MUSE_ERR_UNSUPPORTED = -2, /* valid, but not a shape the library implements  */
  MUSE_ERR_HIP = -3,         /* a HIP runtime call or kernel launch failed      */
  MUSE_ERR_NO_MEMORY = -4,   /* workspace allocation failed                     */
  MUSE_ERR_WORKSPACE = -5    /* caller workspace too small                      */
};

/*
 * Dipole modes (muse_fwd_params.dipole). TILTED: D_i = sum_j P_ij C_ij with C_ij the
 * value-key covariance of key cluster j under the weights exp(s qbar_i . k) (the
 * exponentially tilted distribution; gist.science, Kernmechanismen 2). UNTILTED: C_ij
 * replaced by the plain within-cluster covariance Cov_j of key cluster j, the same for
 * every query cluster (the paper's partially specialised dipole; pith.science review,
 * referee's minor comment on Algorithm 3). In causal calls Cov_j covers the keys of
 * cluster j in the blocks before the query's block and P_ij the same keys' log masses
 * (the prefix tables); it is not combined with retrieval or the hierarchical
 * decomposition (MUSE_ERR_UNSUPPORTED). NONE: monopole terms only.
 */
enum { MUSE_DIPOLE_NONE = 0, MUSE_DIPOLE_TILTED = 1, MUSE_DIPOLE_UNTILTED = 2 };

/*
 * MuSe forward pass (acausal when causal == 0).
 *
 * Cq, Ck       number of query / key clusters per (b, h) head, fitted over the
 *              whole sequence of that head (also when causal).
 * kmeans_iters Lloyd iterations: strided init c_j = x[floor(j*N/C)], then
 *              kmeans_iters x (assign to the nearest centroid in Euclidean
 *              distance, ties to the lowest index; update to member means, an
 *              empty cluster keeps its centroid). pith.science review,
 *              "Assumptions & free parameters": K-means iterations.
 * causal,block causal = 1: spatial blocks of `block` tokens; exact causal
 *              attention inside each block, merged by log-sum-exp with the
 *              two-stage approximation over all keys of earlier blocks.
 * Softmax scale 1/sqrt(D); output dtype = input dtype; tilted dipole on.
 */
int muse_attn_fwd(const void* q, const void* k, const void* v, void* out,
                  int B, int H, int N, int D, int Cq, int Ck,
                  int kmeans_iters, int causal, int block,
                  int dtype, void* hip_stream);

/*
 * Exact softmax attention softmax(s q k^T) v (causal: key m <= query n), the
 * quantity MuSe approximates (gist.science, "Probleemstelling"); the in-library
 * comparator. Same tensor conventions; scale 1/sqrt(D); out dtype = dtype.
 */
int muse_exact_attn_fwd(const void* q, const void* k, const void* v, void* out,
                        int B, int H, int N, int D, int causal,
                        int dtype, void* hip_stream);

/* Optional controls of muse_attn_fwd_ex. Fill with muse_fwd_params_init(). */
typedef struct muse_fwd_params {
  float scale;          /* softmax scale; <= 0 means 1/sqrt(D)                        */
  int out_dtype;        /* -1: same as input; else MUSE_F32 or MUSE_BF16              */
  int dipole;           /* MUSE_DIPOLE_TILTED (default), _UNTILTED or _NONE           */
  int topk_clusters;    /* retrieval k1 (causal only); 0 = off. Per (block b >= 1,
                           query cluster i): the k1 key clusters of largest log Z^{<b}_ij,
                           then inside each the k2 earlier blocks of largest atom log
                           mass; their keys are attended exactly, the summaries cover the
                           rest (gist.science, Kernmechanismen 4)                       */
  int topk_blocks;      /* retrieval k2 (>= 1 when k1 > 0); k1*(1+k2) <= 256          */
  const int32_t* labels_q_in;  /* device [B,H,N]: fixed query clusters, skips Q K-means */
  const int32_t* labels_k_in;  /* device [B,H,N]: fixed key clusters, skips K K-means   */
  int32_t* labels_q_trace;     /* device [iters,B,H,N]: labels of every assign step      */
  int32_t* labels_k_trace;     /* device [iters,B,H,N]                                   */
  float* centroids_q_out;      /* device [B,H,Cq,D]: final query centroids               */
  float* centroids_k_out;      /* device [B,H,Ck,D]: final key centroids                 */
  float* lse_out;              /* device [B,H,N]: log of each row's softmax normaliser
                                  (bf16 inputs: requesting it adds an fp32 sum of the
                                  in-block weights beside the sum of their bf16-rounded
                                  values that normalises the output)                      */
  void* workspace;             /* device scratch; NULL = stream-ordered allocation       */
  size_t workspace_bytes;      /* size of `workspace`                                     */
  int32_t* retrieval_trace;    /* device [B,H,N/block,Cq,k1*(1+k2)]: per (block, query
                                  cluster) the k1 chosen key clusters, each followed by
                                  its k2 chosen earlier blocks; -1 = none (block 0: all -1) */
  int hierarchy;               /* causal far field. 0 (default): one two-stage approximation
                                  over all keys of the earlier blocks (summaries accumulated
                                  block by block; gist.science, Kernmechanismen 3). 1: the
                                  hierarchical block decomposition (pith.science review,
                                  Figure 2 caption and "invented entities": exact diagonal
                                  blocks, MuSe on the squares below the diagonal, N C D log N):
                                  the block grid, padded to a power of two, is split
                                  recursively into two diagonal halves and the square below
                                  the diagonal; block b >= 1 sees the earlier keys through
                                  popcount(b) squares, the one covering key blocks
                                  [e - lowbit(e), e) for e = b, b & (b - 1), ... > 0, each a
                                  two-stage approximation over its own keys (clusters fitted
                                  once per head), merged by log-sum-exp. Needs causal = 1
                                  (else MUSE_ERR_INVALID_ARG); not combined with retrieval
                                  (MUSE_ERR_UNSUPPORTED)                                    */
  /* Bucket order of the last K-means assignment (optional copies, device memory). The
     library replaces the paper's ragged cluster tensors, padded per cluster
     (pith.science review, "Assumptions & free parameters": cluster size cap), by a
     stable counting sort of each head's positions by (block, cluster): perm lists the
     positions of bucket (b, j) = (block b, cluster j) in ascending position order,
     buckets in ascending b * C + j; offs[b * C + j] is the bucket's first index in
     perm and offs[nb * C] = N (nb = N / block when causal, else 1).                    */
  int32_t* perm_q_out;         /* device [B,H,N]          query positions in bucket order */
  int32_t* offs_q_out;         /* device [B,H,nb*Cq + 1]  query bucket offsets            */
  int32_t* perm_k_out;         /* device [B,H,N]          key positions in bucket order   */
  int32_t* offs_k_out;         /* device [B,H,nb*Ck + 1]  key bucket offsets              */
  int single_stream;           /* 1: every kernel on hip_stream, one after the other (no
                                  side stream, no events; e.g. to time each kernel alone);
                                  0 (default): the stage-1 atoms run beside the scores and
                                  block moments on the library's second stream             */
  double cap_ratio;            /* key cluster size cap (pith.science review, "Assumptions &
                                  free parameters": ratio 1.5, 1.25 to 4.0 explored, the
                                  row length of the padded per-cluster tensors). 0 (default):
                                  no cap. > 0: key cluster j takes part in the stage-1
                                  summaries (log Z_ij, K_ij, V_ij, dipole) with its first
                                  U = ceil(cap_ratio * N / Ck) members in position order only;
                                  the others are left out of them (causal: counted over the
                                  whole sequence, so a bucket (b, j) keeps the members that
                                  still fit after the blocks before b; every key is still
                                  attended exactly inside its own block). Not combined with
                                  retrieval (MUSE_ERR_UNSUPPORTED); negative or NaN:
                                  MUSE_ERR_INVALID_ARG                                       */
} muse_fwd_params;

/* Defaults: scale 0, out_dtype -1, dipole tilted, retrieval off, hierarchy 0, single_stream 0,
 * cap_ratio 0, all pointers NULL. */
void muse_fwd_params_init(muse_fwd_params* p);

/* muse_attn_fwd with optional controls; p == NULL means defaults. With fixed
 * labels (labels_*_in) the centroids are the member means of those labels. */
int muse_attn_fwd_ex(const void* q, const void* k, const void* v, void* out,
                     int B, int H, int N, int D, int Cq, int Ck,
                     int kmeans_iters, int causal, int block,
                     int dtype, void* hip_stream, const muse_fwd_params* p);

/* Device scratch bytes muse_attn_fwd_ex needs for this shape (0 on invalid
 * arguments, with muse_last_error() set). */
size_t muse_attn_fwd_workspace_bytes(int B, int H, int N, int D, int Cq, int Ck,
                                     int causal, int block, int dtype,
                                     const muse_fwd_params* p);

/*
 * muse_attn_fwd_ex that allocates nothing, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. Same arguments, semantics and outputs as muse_attn_fwd_ex (p == NULL means
 * defaults; p->workspace must be NULL). Instead of a caller or stream-ordered workspace
 * the call uses a fixed scratch array inside the library's device code,
 * MUSE_NOALLOC_SCRATCH_BYTES per device, held by every device the library runs on from
 * the library's load until the process ends. A shape whose workspace
 * (muse_attn_fwd_workspace_bytes) exceeds it returns MUSE_ERR_WORKSPACE before anything
 * is launched; 64 MiB holds, e.g., one 8k head (D 64, Cq 32, Ck 128) or one causal 16k
 * head (block 1024, Cq 16, Ck 64). All work runs on hip_stream (no side stream, no
 * events), and the call makes no allocation (with muse_prof_enable on, the timing hooks
 * still create their HIP events). Nothing in the scratch has to start at zero. Every
 * call on a device shares that device's scratch: calls that overlap in time on one
 * device (on different streams, or from several threads) race and give wrong results;
 * order them on one stream.
 */
#define MUSE_NOALLOC_SCRATCH_BYTES (64u << 20)
int muse_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* out,
                          int B, int H, int N, int D, int Cq, int Ck,
                          int kmeans_iters, int causal, int block,
                          int dtype, void* hip_stream, const muse_fwd_params* p);

/*
 * Backward pass of the MuSe forward: the vector-Jacobian products dq, dk, dv of
 * muse_attn_fwd_ex's output o(q, k, v) for an upstream gradient dout = dLoss/do. The
 * reviews note that the method's backward pass uses the same approximations as its
 * forward and that its gradient error was never measured (pith.science review, "Reading
 * between the lines"; Referee Report, Section 7.2 / Q4). Differentiated: the forward with
 * the K-means labels held fixed (the clustering is piecewise constant in q and k, so it
 * has no gradient). The query centroids are the member means of labels_q and pass their
 * gradient to every member; stage 1 (log Z_ij, the tilted means K_ij and V_ij, P_ij and
 * the dipole D_i, tilted or untilted as p->dipole says) and stage 2 (the refinement) are
 * differentiated exactly; the no-dipole mode drops D_i from both. Causal calls (the
 * prefix form: block b's far field summarises the keys of blocks < b, merged by
 * log-sum-exp with exact attention inside the block; gist.science summary,
 * Kernmechanismen 3; pith.science review, caption of Figure 2) differentiate the merge,
 * the exact in-block attention, and every block's table entry, whose gradients reach the
 * keys of the earlier blocks.
 *   q, k, v, dout   device [B,H,N,D] in dtype (MUSE_F32 or MUSE_BF16), as in the forward
 *   labels_q/_k     device int32 [B,H,N]: the forward call's final labels (the last row
 *                   of labels_*_trace, or the labels_*_in it was given); values outside
 *                   [0, C) are clamped like labels_*_in
 *   dq, dk, dv      device float32 [B,H,N,D], written (not accumulated); distinct from
 *                   each other and from every input
 *   p               scale, dipole and cap_ratio as in the forward call (NULL: defaults); workspace
 *                   and workspace_bytes as in muse_attn_fwd_ex, sized by
 *                   muse_attn_bwd_workspace_bytes. Every other field keeps its default
 *                   (MUSE_ERR_INVALID_ARG for the forward's output pointers).
 * Implemented for D = 64, acausal (every dipole mode) and causal (tilted dipole or none)
 * with the forward's block rules, with or without the cluster size cap (p->cap_ratio as
 * in the forward: keys left out of the summaries take no gradient through them); other
 * head sizes, the untilted dipole with causal = 1, retrieval and the hierarchy return
 * MUSE_ERR_UNSUPPORTED before any launch. All
 * arithmetic in fp32 (bf16 inputs are exact in it); results are deterministic (fixed
 * summation orders, no floating-point atomics). Work is queued on hip_stream.
 */
int muse_attn_bwd(const void* q, const void* k, const void* v, const void* dout,
                  const int32_t* labels_q, const int32_t* labels_k,
                  float* dq, float* dk, float* dv,
                  int B, int H, int N, int D, int Cq, int Ck,
                  int causal, int block, int dtype, void* hip_stream,
                  const muse_fwd_params* p);

/* Device scratch bytes muse_attn_bwd needs for this shape (0 on invalid or unsupported
 * arguments, with muse_last_error() set). */
size_t muse_attn_bwd_workspace_bytes(int B, int H, int N, int D, int Cq, int Ck,
                                     int causal, int block, int dtype,
                                     const muse_fwd_params* p);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* muse_last_error(void);

/*
 * Per-kernel timing (tracing aid; not part of the method). While enabled, every
 * kernel the library launches is bracketed by a pair of HIP events recorded on
 * the caller's stream, which adds a little launch overhead. muse_prof_collect()
 * waits for the recorded events and folds them into per-kernel totals; it returns
 * the number of distinct kernel names, which muse_prof_name / muse_prof_total_ms /
 * muse_prof_launches index (0 .. count-1; out-of-range gives "" / 0). The state is
 * process-wide and guarded by a mutex; the strings stay valid until the next
 * muse_prof_collect or muse_prof_reset.
 */
void muse_prof_enable(int on);
int muse_prof_collect(void);
const char* muse_prof_name(int i);
double muse_prof_total_ms(int i);
long muse_prof_launches(int i);
void muse_prof_reset(void);

/* ABI version: major * 10000 + minor * 100 + patch. */
int muse_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MUSE_H_ */
