"""GPU parity of the HIP path against the CPU oracle, through the C-ABI binding.

Every case runs the library on the GPU and compares with the float64 oracle on the same
seeded inputs: K-means labels must match except at documented near-ties (relative gap
< 1e-5, where the oracle adopts the GPU label), outputs to relative L2 <= 1e-5 (fp32
inputs) or <= 3e-3 (bf16 inputs, fp32 accumulation).
"""

import numpy as np
import pytest
import torch

from oracle import exact_attention
from parity_util import TOL, check_config, log, rel_l2, run_gpu, to_device
from workloads import CONFIGS, make_inputs, scaled_config

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------ small cases: whole tensors

def test_acausal_1k_f32_full(muse_lib):
    check_config(CONFIGS["acausal_1k_f32"], [(0, 0)])


@pytest.mark.parametrize("N", [1000, 1536])
def test_acausal_bf16_ragged(muse_lib, N):
    # several 256-point K-means tiles plus a ragged tail (N=1000)
    cfg = scaled_config("acausal_8k", B=1, H=2, N=N)
    check_config(cfg, [(0, 0), (0, 1)])


@pytest.mark.parametrize("causal", [False, True])
def test_bf16_odd_cluster_counts_long_buckets(muse_lib, causal):
    # cluster counts off the 32-centroid tiles, a ragged tail, and key buckets longer
    # than one 64-key atom work item (folded by the finalise, or merged when causal)
    if causal:
        cfg = scaled_config("causal_16k", B=1, H=2, N=3072, block=1024, Cq=12, Ck=20)
    else:
        cfg = scaled_config("acausal_8k", B=1, H=2, N=3000, Cq=20, Ck=40)
    check_config(cfg, [(0, 0), (0, 1)])


@pytest.mark.parametrize("name,over", [
    # fewer points than one 256-point K-means tile, one cluster of each kind
    ("acausal_8k", {"B": 1, "H": 1, "N": 200, "Cq": 1, "Ck": 1}),
    # the largest cluster counts, many of them small or empty
    ("acausal_8k", {"B": 1, "H": 1, "N": 700, "Cq": 128, "Ck": 128}),
    # one query cluster against the largest key count, 64-token causal blocks (64-point tiles)
    ("causal_16k", {"B": 1, "H": 1, "N": 1024, "block": 64, "Cq": 1, "Ck": 128}),
    # fp32, and D = 128 with one key cluster
    ("acausal_1k_f32", {"N": 300, "Cq": 3, "Ck": 128}),
    ("causal_64k_d128", {"B": 1, "H": 1, "N": 256, "causal": False, "block": 0, "Cq": 128, "Ck": 1}),
    # D = 128 with the largest query cluster count (the atoms' centroid tables exceed 64 KB
    # of LDS), fp32 and causal bf16
    ("acausal_1k_f32", {"N": 512, "D": 128, "Cq": 128, "Ck": 128}),
    ("causal_64k_d128", {"B": 1, "H": 1, "N": 2048, "block": 512, "Cq": 128, "Ck": 64}),
])
def test_cluster_count_extremes(muse_lib, name, over):
    check_config(scaled_config(name, **over), [(0, 0)])


@pytest.mark.parametrize("name,over", [
    ("acausal_8k", {"B": 1, "H": 1, "N": 1024, "iters": 1}),           # one Lloyd iteration
    ("causal_16k", {"B": 1, "H": 1, "N": 1536, "block": 192, "iters": 3}),  # 192-point tiles
    ("causal_16k", {"B": 1, "H": 1, "N": 1024, "block": 1024}),          # one block: no far field
    ("retrieval_16k", {"B": 1, "H": 1, "N": 2048, "D": 128, "block": 512}),  # retrieval at D = 128
    ("acausal_8k", {"B": 8, "H": 8, "N": 256, "Cq": 4, "Ck": 16}),       # many short heads
])
def test_shapes(muse_lib, name, over):
    cfg = scaled_config(name, **over)
    check_config(cfg, [(0, 0)] if cfg.B * cfg.H == 1 else [(0, 0), (cfg.B - 1, cfg.H - 1)])


@pytest.mark.parametrize("causal", [False, True])
def test_bf16_d128_odd_cluster_counts(muse_lib, causal):
    # D = 128: cluster counts off the 32-centroid tiles (one to three tiles of them, so
    # that some cluster-sum waves own no output) and a ragged tail
    if causal:
        cfg = scaled_config("causal_64k_d128", B=1, H=2, N=3072, block=1024, Cq=12, Ck=40)
    else:
        cfg = scaled_config("causal_64k_d128", B=1, H=2, N=3000, causal=False, block=0, Cq=20, Ck=72)
    check_config(cfg, [(0, 0), (0, 1)])


@pytest.mark.parametrize("name,over", [
    ("acausal_1k_f32", {}),
    ("acausal_8k", {"B": 1, "H": 2, "N": 1536}),
    ("causal_64k_d128", {"B": 1, "H": 2, "N": 1000, "causal": False, "block": 0, "Cq": 12, "Ck": 40}),
])
def test_untilted_dipole(muse_lib, name, over):
    # the partially specialised (untilted) dipole: per key cluster covariances, fp32 and
    # bf16 inputs, D = 64 and 128, a ragged tail and cluster counts off the 32-tiles
    cfg = scaled_config(name, **over) if over else CONFIGS[name]
    check_config(cfg, [(0, 0)] if cfg.H == 1 else [(0, 0), (0, 1)], dipole="untilted")


@pytest.mark.parametrize("name,over", [
    ("causal_16k", {"B": 1, "H": 2, "N": 4096, "block": 1024}),
    # D = 128, cluster counts off the 32-tiles, 8 blocks
    ("causal_64k_d128", {"B": 1, "H": 1, "N": 4096, "block": 512, "Cq": 12, "Ck": 40}),
    # fp32 inputs (the general causal path), 4 blocks
    ("acausal_1k_f32", {"H": 2, "N": 1024, "causal": True, "block": 256, "Cq": 8, "Ck": 32}),
    # 64-token blocks: many small buckets, some empty
    ("causal_16k", {"B": 1, "H": 1, "N": 1024, "block": 64, "Cq": 8, "Ck": 24}),
])
def test_untilted_dipole_causal(muse_lib, name, over):
    # the untilted dipole in causal calls: per block, the plain covariance of every key
    # cluster over the keys of the earlier blocks, aggregated with the prefix weights P_ij
    cfg = scaled_config(name, **over)
    check_config(cfg, [(0, 0)] if cfg.H == 1 else [(0, 0), (0, 1)], dipole="untilted")


def test_untilted_dipole_causal_64k_full_size_sampled_blocks(muse_lib):
    check_config(CONFIGS["causal_64k_d128"], [(0, 3)], blocks=[1, 16, 31], dipole="untilted")


def test_untilted_dipole_refused_with_retrieval_or_hierarchy(muse_lib):
    from clustered_softmax_attention_amd import binding
    cfg = scaled_config("retrieval_16k", B=1, H=1, N=2048, block=256)
    q, k, v = (to_device(t, cfg.dtype) for t in make_inputs(cfg))
    for kw in ({"topk_clusters": 2, "topk_blocks": 1}, {"hierarchy": True}):
        with pytest.raises(binding.MuseError, match="untilted") as err:
            binding.attn_fwd(q, k, v, cfg.Cq, cfg.Ck, cfg.iters, causal=True, block=cfg.block, dipole="untilted", **kw)
        assert err.value.code == -2  # MUSE_ERR_UNSUPPORTED


def test_acausal_bf16_d128(muse_lib):
    cfg = scaled_config("causal_64k_d128", B=1, H=2, N=2048, causal=False, block=0)
    check_config(cfg, [(0, 0), (0, 1)])


def test_acausal_fp32_d128_monopole(muse_lib):
    cfg = scaled_config("acausal_1k_f32", H=2, N=777, D=128, Cq=5, Ck=17)
    check_config(cfg, [(0, 0), (0, 1)], dipole=False)


def test_causal_bf16_small_blocks(muse_lib):
    cfg = scaled_config("causal_16k", B=1, H=2, N=2048, block=256)
    check_config(cfg, [(0, 0), (0, 1)])


def test_causal_bf16_block64(muse_lib):
    # one-wave K-means tiles and 64-token diagonal blocks
    cfg = scaled_config("causal_16k", B=1, H=1, N=512, block=64, Cq=8, Ck=16)
    check_config(cfg, [(0, 0)])


def test_causal_16k_shape_reduced(muse_lib):
    cfg = scaled_config("causal_16k", B=1, H=2, N=4096)
    check_config(cfg, [(0, 0), (0, 1)])


def test_causal_64k_d128_shape_reduced(muse_lib):
    cfg = scaled_config("causal_64k_d128", B=1, H=2, N=8192)
    check_config(cfg, [(0, 1)])


def test_causal_fp32(muse_lib):
    cfg = scaled_config("acausal_1k_f32", H=2, N=1024, causal=True, block=256, Cq=8, Ck=32)
    check_config(cfg, [(0, 0), (0, 1)])


@pytest.mark.parametrize("name,over,dipole", [
    # 7 blocks (not a power of two: blocks 3, 5, 6 see two squares, block 6 [0,4) and [4,6))
    ("causal_16k", {"B": 1, "H": 2, "N": 1792, "block": 256}, True),
    # 16 blocks of 128 tokens, up to four squares per block, monopole only
    ("causal_16k", {"B": 1, "H": 1, "N": 2048, "block": 128, "Cq": 8, "Ck": 24}, False),
    # D = 128, 12 blocks
    ("causal_64k_d128", {"B": 1, "H": 2, "N": 3072, "block": 256}, True),
    # fp32 inputs, 5 blocks, cluster counts off the 32-tiles
    ("acausal_1k_f32", {"H": 2, "N": 1280, "causal": True, "block": 256, "Cq": 7, "Ck": 29}, True),
    # two blocks: the single-level instance (one exact diagonal block, one MuSe square)
    ("causal_16k", {"B": 1, "H": 1, "N": 2048, "block": 1024}, True),
])
def test_hierarchical_causal(muse_lib, name, over, dipole):
    # the hierarchical block decomposition: a block's far field merges one two-stage
    # approximation per square below the diagonal (log-sum-exp), squares from the oracle's
    # recursive split, entries e = b, b & (b - 1), ... on the GPU
    cfg = scaled_config(name, **over)
    check_config(cfg, [(0, 0)] if cfg.H == 1 else [(0, 0), (0, 1)], dipole=dipole, hierarchy=True)


def test_hierarchical_many_blocks(muse_lib):
    # 2048 blocks of 64 tokens: the stage-1 folds build each square directly from its
    # blocks instead of by the binary counter over the blocks; block 2047 sees 11 squares
    cfg = scaled_config("causal_16k", B=1, H=1, N=131072, block=64, Cq=8, Ck=16)
    check_config(cfg, [(0, 0)], blocks=[1, 1024, 2047], hierarchy=True)


def test_hierarchical_refusals(muse_lib):
    from clustered_softmax_attention_amd import binding
    cfg = scaled_config("retrieval_16k", B=1, H=1, N=2048, block=256)
    q, k, v = (to_device(t, cfg.dtype) for t in make_inputs(cfg))
    with pytest.raises(binding.MuseError, match="retrieval") as err:
        binding.attn_fwd(q, k, v, cfg.Cq, cfg.Ck, cfg.iters, causal=True, block=cfg.block, topk_clusters=2,
                         topk_blocks=1, hierarchy=True)
    assert err.value.code == -2  # MUSE_ERR_UNSUPPORTED
    with pytest.raises(binding.MuseError, match="causal") as err:
        binding.attn_fwd(q, k, v, cfg.Cq, cfg.Ck, cfg.iters, hierarchy=True)
    assert err.value.code == -1  # MUSE_ERR_INVALID_ARG


def test_retrieval_16k_shape_reduced(muse_lib):
    cfg = scaled_config("retrieval_16k", B=1, H=2, N=4096)
    check_config(cfg, [(0, 0), (0, 1)])


def test_retrieval_small_blocks_fp32(muse_lib):
    cfg = scaled_config("retrieval_16k", B=1, H=1, N=2048, block=256, dtype="f32", Cq=8, Ck=16, topk_clusters=3,
                        topk_blocks=2)
    check_config(cfg, [(0, 0)])


def test_retrieval_bf16_d128(muse_lib):
    # D = 128: the matrix-core exact part on retrieved keys (several 32-key chunks per
    # bucket) and the retrieval tables, cluster counts off the 32-tiles
    cfg = scaled_config("causal_64k_d128", B=1, H=2, N=4096, block=512, Cq=12, Ck=40, topk_clusters=3,
                        topk_blocks=2)
    check_config(cfg, [(0, 0), (0, 1)])


def _bucket_sizes(cfg, q, k, v):
    """Queries per (block, query cluster) bucket of blocks b >= 1 (head (0, 0))."""
    _, ex = run_gpu(cfg, q, k, v, extra_returns=True)
    offs = ex["offs_q"][0, 0].cpu().numpy().astype(np.int64)
    return np.diff(offs)[cfg.Cq:]


def test_retrieval_wide_and_narrow_buckets(muse_lib):
    # four query clusters per block of 512: buckets of more than 64 queries (each of the
    # exact part's waves takes its own 32 queries and every retrieved key) beside chunk
    # remainders of at most 64 (wave pairs split the keys and merge their halves); about
    # 128 retrieved keys per entry: two 64-key staging steps
    cfg = scaled_config("retrieval_16k", B=1, H=1, N=2048, block=512, Cq=4, Ck=16, topk_clusters=2, topk_blocks=2)
    q, k, v = make_inputs(cfg)
    sizes = _bucket_sizes(cfg, q, k, v)
    chunks = np.concatenate([np.minimum(128, np.maximum(0, sizes - 128 * c)) for c in range(4)])
    assert (chunks > 64).any() and ((chunks > 0) & (chunks <= 64)).any(), sizes
    check_config(cfg, [(0, 0)], inputs=(q, k, v))


def test_retrieval_few_keys(muse_lib):
    # one cluster and one block retrieved out of 64 clusters: about eight keys per entry,
    # so the second key half of every staging step is empty
    cfg = scaled_config("retrieval_16k", B=1, H=1, N=2048, block=512, Cq=16, Ck=64, topk_clusters=1, topk_blocks=1)
    check_config(cfg, [(0, 0)])


def test_retrieval_of_everything_is_exact_d128(muse_lib):
    cfg = scaled_config("causal_64k_d128", B=1, H=1, N=2048, block=256, Cq=8, Ck=16, topk_clusters=16,
                        topk_blocks=8)
    q, k, v = make_inputs(cfg)
    out, _ = run_gpu(cfg, q, k, v)
    o, _ = exact_attention(q[0, 0], k[0, 0], v[0, 0], causal=True)
    rel = rel_l2(out.float().cpu().numpy()[0, 0], o)
    log(f"[retrieval everything, D=128] rel-L2 vs exact {rel:.3e}")
    assert rel <= TOL["bf16"]


def test_retrieval_of_everything_is_exact(muse_lib):
    # k1 = Ck and k2 = number of blocks: every earlier key is attended exactly
    cfg = scaled_config("retrieval_16k", B=1, H=1, N=2048, block=256, Cq=8, Ck=16, topk_clusters=16, topk_blocks=8)
    q, k, v = make_inputs(cfg)
    out, _ = run_gpu(cfg, q, k, v)
    o, _ = exact_attention(q[0, 0], k[0, 0], v[0, 0], causal=True)
    rel = rel_l2(out.float().cpu().numpy()[0, 0], o)
    log(f"retrieval of everything vs exact causal: rel-L2 {rel:.3e}")
    assert rel <= TOL["bf16"]


def test_bf16_output_within_tolerance(muse_lib):
    cfg = scaled_config("acausal_8k", B=1, H=1, N=2048)
    check_config(cfg, [(0, 0)], out_dtype=torch.bfloat16)


def test_fixed_labels_path(muse_lib):
    # caller-fixed labels: the library uses member means as centroids and skips K-means
    from oracle import muse_acausal
    cfg = scaled_config("acausal_8k", B=1, H=1, N=1024, Cq=8, Ck=16)
    q, k, v = make_inputs(cfg)
    rng = np.random.default_rng(5)
    lq = rng.integers(0, cfg.Cq, size=(1, 1, cfg.N)).astype(np.int32)
    lk = rng.integers(0, cfg.Ck, size=(1, 1, cfg.N)).astype(np.int32)
    lk[0, 0, lk[0, 0] == 3] = 4  # one empty key cluster
    out, ex = run_gpu(cfg, q, k, v, labels_q_in=torch.from_numpy(lq), labels_k_in=torch.from_numpy(lk))
    r = muse_acausal(q[0, 0], k[0, 0], v[0, 0], cfg.Cq, cfg.Ck, 1, labels_q=lq[0, 0], labels_k=lk[0, 0])
    rel = rel_l2(out.float().cpu().numpy()[0, 0], r.o)
    log(f"fixed labels rel-L2 {rel:.3e}")
    assert rel <= TOL["bf16"]


def test_fixed_labels_hierarchical(muse_lib):
    # caller-fixed labels with the hierarchical decomposition (6 blocks: blocks 3 and 5 see
    # two squares) and an empty key cluster
    from oracle import muse_causal
    cfg = scaled_config("causal_16k", B=1, H=1, N=1536, block=256, Cq=6, Ck=20)
    q, k, v = make_inputs(cfg)
    rng = np.random.default_rng(6)
    lq = rng.integers(0, cfg.Cq, size=(1, 1, cfg.N)).astype(np.int32)
    lk = rng.integers(0, cfg.Ck, size=(1, 1, cfg.N)).astype(np.int32)
    lk[0, 0, lk[0, 0] == 7] = 8
    out, _ = run_gpu(cfg, q, k, v, labels_q_in=torch.from_numpy(lq), labels_k_in=torch.from_numpy(lk),
                     hierarchy=True)
    r = muse_causal(q[0, 0], k[0, 0], v[0, 0], cfg.Cq, cfg.Ck, 1, cfg.block, labels_q=lq[0, 0],
                    labels_k=lk[0, 0], hierarchical=True)
    rel = rel_l2(out.float().cpu().numpy()[0, 0], r.o)
    log(f"fixed labels, hierarchy: rel-L2 {rel:.3e}")
    assert rel <= TOL["bf16"]


def test_deterministic_bitwise(muse_lib):
    cfg = scaled_config("causal_16k", B=1, H=2, N=2048, block=512)
    q, k, v = make_inputs(cfg)
    a, _ = run_gpu(cfg, q, k, v)
    b, _ = run_gpu(cfg, q, k, v)
    assert torch.equal(a, b)


# ------------------------------------------------------------ exact attention comparator

@pytest.mark.parametrize("dtype,D,causal", [("f32", 64, False), ("f32", 128, True), ("bf16", 64, True),
                                            ("bf16", 128, False)])
def test_exact_attention(muse_lib, dtype, D, causal):
    from clustered_softmax_attention_amd import exact_attn_fwd
    rng = np.random.default_rng(7)
    B, H, N = 1, 2, 1000
    q, k, v = (rng.standard_normal((B, H, N, D)).astype(np.float32) for _ in range(3))
    Q, K, V = (to_device(t, dtype) for t in (q, k, v))
    out = exact_attn_fwd(Q, K, V, causal=causal).float().cpu().numpy()
    q64, k64, v64 = (t.float().cpu().numpy() for t in (Q, K, V))
    for h in range(H):
        o, _ = exact_attention(q64[0, h], k64[0, h], v64[0, h], causal=causal)
        rel = rel_l2(out[0, h], o)
        log(f"exact {dtype} D={D} causal={causal} head {h}: rel-L2 {rel:.3e}")
        assert rel <= TOL[dtype]


# ------------------------------------------------------------ full-size configurations (sampled)

@pytest.mark.parametrize("dipole", [True, "untilted"])
def test_acausal_8k_full_size_sampled_heads(muse_lib, dipole):
    cfg = CONFIGS["acausal_8k"]
    check_config(cfg, [(0, 0), (3, 7)], dipole=dipole)


def test_causal_16k_full_size_sampled_blocks(muse_lib):
    cfg = CONFIGS["causal_16k"]
    check_config(cfg, [(7, 5)], blocks=[1, 15])


def test_causal_16k_hierarchical_full_size_sampled_blocks(muse_lib):
    # block 15 sees four squares ([0,8), [8,12), [12,14), [14,15) in blocks), block 8 one
    cfg = CONFIGS["causal_16k"]
    check_config(cfg, [(5, 2)], blocks=[8, 15], hierarchy=True)


def test_retrieval_16k_full_size_sampled_blocks(muse_lib):
    cfg = CONFIGS["retrieval_16k"]
    check_config(cfg, [(1, 6)], blocks=[1, 15])


def test_causal_64k_d128_full_size_sampled_blocks(muse_lib):
    cfg = CONFIGS["causal_64k_d128"]
    check_config(cfg, [(0, 9)], blocks=[1, 31])
