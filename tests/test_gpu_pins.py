"""GPU parity at the cases the pages single out, through the C-ABI binding.

* the peaked regime s = 1 (the pages' logits exp(q.k), gist.science Kernmechanismen 2),
  acausal, causal, hierarchical and retrieval, fp32 and bf16, D = 64 and 128;
* translation of every key by a constant vector: attention is invariant to it
  (gist.science, Kernmechanismen 1), and so are the K-means labels;
* singleton clusters and keys (or queries) equal to their centroids reduce MuSe to
  exact attention (pith.science review, "Circularity Check");
* the timed configuration with bf16 output at full size (8k acausal, 64k causal);
* the plain muse_attn_fwd entry point (defaults only) against muse_attn_fwd_ex.
Tolerances as everywhere: relative L2 <= 1e-5 (fp32 inputs), <= 3e-3 (bf16 inputs).
"""

import numpy as np
import pytest
import torch

from oracle import exact_attention, lloyd_kmeans
from parity_util import TOL, check_config, log, rel_l2, run_gpu, to_device
from workloads import CONFIGS, make_inputs, scaled_config
from workloads.gaussian_mixture import bf16_bits_to_f32, f32_to_bf16_bits

pytestmark = pytest.mark.gpu


def _heads(cfg):
    return [(0, 0)] if cfg.B * cfg.H == 1 else [(0, 0), (cfg.B - 1, cfg.H - 1)]


# ------------------------------------------------------------ peaked attention, s = 1

@pytest.mark.parametrize("name,over,hier", [
    ("acausal_8k", {"B": 1, "H": 2, "N": 2048}, False),
    ("acausal_1k_f32", {}, False),
    ("causal_16k", {"B": 1, "H": 1, "N": 4096, "block": 1024}, False),
    ("causal_64k_d128", {"B": 1, "H": 1, "N": 4096, "block": 1024}, False),
    ("causal_16k", {"B": 1, "H": 1, "N": 2048, "block": 256}, True),
    ("retrieval_16k", {"B": 1, "H": 1, "N": 4096}, False),
    ("acausal_1k_f32", {"N": 1024, "causal": True, "block": 256}, False),
])
def test_scale_one(muse_lib, name, over, hier):
    cfg = scaled_config(name, **over) if over else CONFIGS[name]
    check_config(cfg, _heads(cfg), scale=1.0, hierarchy=hier)


@pytest.mark.parametrize("name,over", [
    ("acausal_8k", {"B": 1, "H": 1, "N": 2048}),
    ("causal_16k", {"B": 1, "H": 1, "N": 4096, "block": 1024}),
])
def test_scale_one_untilted(muse_lib, name, over):
    cfg = scaled_config(name, **over)
    check_config(cfg, _heads(cfg), scale=1.0, dipole="untilted")


# ------------------------------------------------------------ key translation

def _translate_exactly(k: np.ndarray, c: float, dtype: str):
    """(k_base, k_moved) with k_moved = k_base + c exactly in the storage dtype: k_moved is
    k + c rounded to the dtype, k_base = k_moved - c (exact for every element here)."""
    k = np.asarray(k, np.float32)
    moved = (k + np.float32(c)).astype(np.float32)
    if dtype == "bf16":
        moved = bf16_bits_to_f32(f32_to_bf16_bits(moved))
    base = (moved - np.float32(c)).astype(np.float32)
    if dtype == "bf16":
        assert np.array_equal(bf16_bits_to_f32(f32_to_bf16_bits(base)), base)
    assert np.array_equal((base + np.float32(c)).astype(np.float32), moved)
    return base, moved


@pytest.mark.parametrize("name,over", [
    ("acausal_8k", {"B": 1, "H": 2, "N": 2048}),
    ("causal_16k", {"B": 1, "H": 1, "N": 4096, "block": 1024}),
    ("acausal_1k_f32", {}),
    ("causal_64k_d128", {"B": 1, "H": 1, "N": 2048, "causal": False, "block": 0}),
])
def test_key_translation(muse_lib, name, over):
    # every key moved by c = 4 in each coordinate (norms grow from ~3 to ~32 at D = 64)
    cfg = scaled_config(name, **over) if over else CONFIGS[name]
    q, k, v = make_inputs(cfg)
    k_base, k_moved = _translate_exactly(k, 4.0, cfg.dtype)
    out_b, ex_b = run_gpu(cfg, q, k_base, v)
    out_m, ex_m = run_gpu(cfg, q, k_moved, v)
    tk_b = ex_b["labels_k_trace"].cpu().numpy()
    tk_m = ex_m["labels_k_trace"].cpu().numpy()
    for b, h in _heads(cfg):
        # the translated run's labels are valid for the untranslated keys up to near-ties
        # (relative gap <= 1e-5 in float64 distances), and the other way round
        fb = lloyd_kmeans(k_base[b, h], cfg.Ck, cfg.iters, follow_trace=tk_m[:, b, h])
        fm = lloyd_kmeans(k_moved[b, h], cfg.Ck, cfg.iters, follow_trace=tk_b[:, b, h])
        ndiff = int((tk_b[:, b, h] != tk_m[:, b, h]).sum())
        log(f"[{cfg.name} translated keys] head ({b},{h}): label differences {ndiff}, "
            f"near-ties {fb.near_ties}/{fm.near_ties}")
        assert fb.mismatches == 0 and fm.mismatches == 0
        rel = rel_l2(out_m.float().cpu().numpy()[b, h], out_b.float().cpu().numpy()[b, h])
        log(f"[{cfg.name} translated keys] head ({b},{h}): rel-L2 moved vs base {rel:.3e}")
        assert rel <= TOL[cfg.dtype]
    # and the translated run against the oracle (labels, centroids, bucket order, output)
    check_config(cfg, _heads(cfg), inputs=(q, k_moved, v))


# ------------------------------------------------------------ reductions to exact attention

@pytest.mark.parametrize("name,over", [
    ("acausal_8k", {"B": 1, "H": 1, "N": 128, "Cq": 128, "Ck": 128}),
    ("acausal_1k_f32", {"N": 128, "Cq": 128, "Ck": 128}),
    ("causal_64k_d128", {"B": 1, "H": 1, "N": 128, "causal": False, "block": 0, "Cq": 128, "Ck": 128}),
    ("causal_16k", {"B": 1, "H": 1, "N": 128, "block": 64, "Cq": 128, "Ck": 128}),
])
def test_singleton_clusters_are_exact(muse_lib, name, over):
    # as many clusters as points: the strided init puts one centroid on every point, so
    # every cluster is a singleton and both residuals vanish
    cfg = scaled_config(name, **over)
    q, k, v = make_inputs(cfg)
    out, ex = run_gpu(cfg, q, k, v)
    assert np.array_equal(ex["labels_k_trace"].cpu().numpy()[-1, 0, 0], np.arange(cfg.N))
    assert np.array_equal(ex["labels_q_trace"].cpu().numpy()[-1, 0, 0], np.arange(cfg.N))
    o, _ = exact_attention(q[0, 0], k[0, 0], v[0, 0], causal=cfg.causal)
    rel = rel_l2(out.float().cpu().numpy()[0, 0], o)
    log(f"[{cfg.name} singletons] rel-L2 vs exact attention {rel:.3e}")
    assert rel <= TOL[cfg.dtype]


def _runs(x: np.ndarray, C: int) -> np.ndarray:
    """Replace the rows of x [N, D] by C distinct rows, each repeated over a contiguous
    run of N / C positions, so the strided K-means init lands on every distinct row."""
    N = x.shape[0]
    idx = (np.arange(N) * C) // N
    return np.ascontiguousarray(x[(np.arange(C) * N) // C][idx])


@pytest.mark.parametrize("which,name,over", [
    ("k", "acausal_8k", {"B": 1, "H": 1, "N": 1024, "Cq": 8, "Ck": 32}),
    ("k", "causal_16k", {"B": 1, "H": 1, "N": 2048, "block": 512, "Cq": 8, "Ck": 16}),
    ("q", "causal_16k", {"B": 1, "H": 1, "N": 2048, "block": 512, "Cq": 16, "Ck": 32}),
    ("q", "acausal_1k_f32", {"N": 1024, "Cq": 8, "Ck": 32}),
    ("k", "causal_64k_d128", {"B": 1, "H": 1, "N": 1024, "causal": False, "block": 0, "Cq": 8, "Ck": 32}),
])
def test_centroid_equal_inputs_are_exact(muse_lib, which, name, over):
    # keys (or queries) equal to their cluster centroids: the residual-residual term
    # q~.k~ vanishes and MuSe equals exact attention
    cfg = scaled_config(name, **over)
    q, k, v = make_inputs(cfg)
    if which == "k":
        k[0, 0] = _runs(k[0, 0], cfg.Ck)
    else:
        q[0, 0] = _runs(q[0, 0], cfg.Cq)
    out, _ = run_gpu(cfg, q, k, v)
    o, _ = exact_attention(q[0, 0], k[0, 0], v[0, 0], causal=cfg.causal)
    rel = rel_l2(out.float().cpu().numpy()[0, 0], o)
    log(f"[{cfg.name} {which} = centroids] rel-L2 vs exact attention {rel:.3e}")
    assert rel <= TOL[cfg.dtype]


# ------------------------------------------------------------ the timed path: bf16 output at full size

def test_acausal_8k_full_size_bf16_output(muse_lib):
    check_config(CONFIGS["acausal_8k"], [(1, 3)], out_dtype=torch.bfloat16)


def test_causal_64k_d128_full_size_bf16_output(muse_lib):
    check_config(CONFIGS["causal_64k_d128"], [(0, 5)], blocks=[1, 17, 31], out_dtype=torch.bfloat16)


# ------------------------------------------------------------ plain entry point

@pytest.mark.parametrize("name,over", [
    ("acausal_8k", {"B": 1, "H": 2, "N": 2048}),
    ("causal_16k", {"B": 1, "H": 1, "N": 2048, "block": 512}),
    ("acausal_1k_f32", {}),
])
def test_plain_entry_point(muse_lib, name, over):
    # muse_attn_fwd (no parameter block) equals muse_attn_fwd_ex with defaults bitwise,
    # and matches the oracle with output in the input dtype
    from clustered_softmax_attention_amd import attn_fwd, attn_fwd_plain
    cfg = scaled_config(name, **over) if over else CONFIGS[name]
    q, k, v = make_inputs(cfg)
    Q, K, V = (to_device(t, cfg.dtype) for t in (q, k, v))
    a = attn_fwd_plain(Q, K, V, cfg.Cq, cfg.Ck, cfg.iters, causal=cfg.causal, block=cfg.block)
    b = attn_fwd(Q, K, V, cfg.Cq, cfg.Ck, cfg.iters, causal=cfg.causal, block=cfg.block)
    torch.cuda.synchronize()
    assert a.dtype == Q.dtype and torch.equal(a, b)
    check_config(cfg, _heads(cfg), out_dtype=Q.dtype)
