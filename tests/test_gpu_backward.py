"""GPU parity of the backward pass (muse_attn_bwd) through the C-ABI binding.

The library's dq, dk, dv for the labels of a GPU forward call are compared with the
float64 oracle backward (oracle/muse_bwd_ref.muse_acausal_bwd and muse_causal_bwd, pinned
by finite differences) on the same labels: acausal with the tilted, untilted and no
dipole, causal with the tilted and no dipole; fp32 and bf16 inputs; s = 1/sqrt(D) and the
peaked s = 1; blocks of 64 to 1024 keys, one whose tiles straddle the per-key pass's
128-key workgroups, and a single block; the full 8k acausal shape and the full 16k causal
sequence on sampled heads. Singleton clusters reduce the gradients to exact attention's
(pith.science review, "Circularity Check"), and so does a causal call with one block (the
far field is empty), both checked against the oracle's exact-attention backward. The
gradient error of MuSe against exact attention, which the reviews note was never measured
("Reading between the lines"), is logged for the workload shapes.

Tolerances on relative L2 per gradient: 1e-4 for fp32 inputs (the dipole's matrix-core
products split G_Dip into bf16 hi + lo, about 2^-17 relative, and the forward tables
enter through exponentials of logits of size up to ~10); 3e-3 for bf16 inputs, as for
the forward (the recomputed forward summaries use fp16 second moments).
"""

import numpy as np
import pytest
import torch

from oracle import exact_attention
from oracle.muse_bwd_ref import exact_attention_bwd, muse_acausal_bwd, muse_causal_bwd
from parity_util import TOL, log, rel_l2, run_gpu, to_device
from workloads import CONFIGS, make_inputs, scaled_config
from workloads.gaussian_mixture import bf16_bits_to_f32, f32_to_bf16_bits

pytestmark = pytest.mark.gpu

BWD_TOL = {"f32": 1e-4, "bf16": 3e-3}


def _dout(cfg, seed=7):
    """Seeded upstream gradient [B,H,N,D], exact in the input dtype."""
    g = np.random.default_rng(seed).standard_normal((cfg.B, cfg.H, cfg.N, cfg.D)).astype(np.float32)
    if cfg.dtype == "bf16":
        g = bf16_bits_to_f32(f32_to_bf16_bits(g))
    return g


def _gpu_grads(cfg, q, k, v, dO, dipole, scale=0.0, cap_ratio=0.0):
    from clustered_softmax_attention_amd import attn_bwd
    _, ex = run_gpu(cfg, q, k, v, dipole=dipole, scale=scale, cap_ratio=cap_ratio)
    lq = ex["labels_q_trace"][-1].contiguous()
    lk = ex["labels_k_trace"][-1].contiguous()
    Q, K, V, G = (to_device(t, cfg.dtype) for t in (q, k, v, dO))
    dq, dk, dv = attn_bwd(Q, K, V, G, lq, lk, cfg.Cq, cfg.Ck, causal=cfg.causal, block=cfg.block, scale=scale,
                          dipole=dipole, cap_ratio=cap_ratio)
    torch.cuda.synchronize()
    return (dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy()), lq.cpu().numpy(), lk.cpu().numpy()


def _oracle_dipole(dipole):
    return {True: "tilted", False: "none"}.get(dipole, dipole)


def check_bwd(cfg, heads, dipole=True, scale=None, cap_ratio=None):
    q, k, v = make_inputs(cfg)
    dO = _dout(cfg)
    grads, lq, lk = _gpu_grads(cfg, q, k, v, dO, dipole, 0.0 if scale is None else scale,
                               0.0 if cap_ratio is None else cap_ratio)
    tol = BWD_TOL[cfg.dtype]
    for b, h in heads:
        if cfg.causal:
            ref = muse_causal_bwd(q[b, h], k[b, h], v[b, h], cfg.Cq, cfg.Ck, cfg.block, lq[b, h], lk[b, h],
                                  dO[b, h], scale=scale, dipole=_oracle_dipole(dipole), cap_ratio=cap_ratio)
        else:
            ref = muse_acausal_bwd(q[b, h], k[b, h], v[b, h], cfg.Cq, cfg.Ck, lq[b, h], lk[b, h], dO[b, h],
                                   scale=scale, dipole=_oracle_dipole(dipole), cap_ratio=cap_ratio)
        for name, g, r in zip(("dq", "dk", "dv"), grads, ref):
            rel = rel_l2(g[b, h], r)
            log(f"[{cfg.name} bwd {_oracle_dipole(dipole)}] head ({b},{h}) {name}: rel-L2 {rel:.3e} (tol {tol:.0e})")
            assert rel <= tol, f"{name} rel-L2 {rel} > {tol}"


def _heads(cfg):
    return [(0, 0)] if cfg.B * cfg.H == 1 else [(0, 0), (cfg.B - 1, cfg.H - 1)]


@pytest.mark.parametrize("dipole", [True, "untilted", False])
def test_acausal_f32(muse_lib, dipole):
    cfg = CONFIGS["acausal_1k_f32"]
    check_bwd(cfg, _heads(cfg), dipole)


@pytest.mark.parametrize("dipole", [True, "untilted", False])
def test_acausal_bf16(muse_lib, dipole):
    cfg = scaled_config("acausal_8k", B=1, H=2, N=2048)
    check_bwd(cfg, _heads(cfg), dipole)


@pytest.mark.parametrize("name,over", [
    ("acausal_8k", {"B": 1, "H": 1, "N": 1000}),                # ragged key tiles and query tiles
    ("acausal_8k", {"B": 2, "H": 1, "N": 1536, "Cq": 17, "Ck": 45}),  # odd cluster counts
    ("acausal_1k_f32", {"N": 768, "Cq": 128, "Ck": 128}),       # the largest cluster counts
])
def test_shapes(muse_lib, name, over):
    cfg = scaled_config(name, **over)
    check_bwd(cfg, _heads(cfg))


@pytest.mark.parametrize("name,over", [("acausal_8k", {"B": 1, "H": 1, "N": 2048}), ("acausal_1k_f32", {})])
def test_scale_one(muse_lib, name, over):
    cfg = scaled_config(name, **over) if over else CONFIGS[name]
    check_bwd(cfg, _heads(cfg), scale=1.0)


def test_acausal_8k_full_size_sampled_head(muse_lib):
    cfg = CONFIGS["acausal_8k"]
    check_bwd(cfg, [(1, 5)])


@pytest.mark.parametrize("name", ["acausal_8k", "acausal_1k_f32"])
def test_singleton_clusters_give_exact_gradients(muse_lib, name):
    # as many clusters as points, labels 0..N-1: MuSe is exact attention, and so are its
    # gradients
    from clustered_softmax_attention_amd import attn_bwd
    cfg = scaled_config(name, B=1, H=1, N=128, Cq=128, Ck=128)
    q, k, v = make_inputs(cfg)
    dO = _dout(cfg)
    lab = torch.arange(cfg.N, dtype=torch.int32, device="cuda").reshape(1, 1, cfg.N)
    Q, K, V, G = (to_device(t, cfg.dtype) for t in (q, k, v, dO))
    grads = attn_bwd(Q, K, V, G, lab, lab, cfg.Cq, cfg.Ck)
    torch.cuda.synchronize()
    ref = exact_attention_bwd(q[0, 0], k[0, 0], v[0, 0], dO[0, 0])
    for name_, g, r in zip(("dq", "dk", "dv"), grads, ref):
        rel = rel_l2(g.cpu().numpy()[0, 0], r)
        log(f"[{cfg.name} singletons bwd] {name_}: rel-L2 vs exact attention {rel:.3e}")
        assert rel <= BWD_TOL[cfg.dtype]


@pytest.mark.parametrize("name,over", [("acausal_8k", {"B": 1, "H": 1}), ("acausal_1k_f32", {})])
def test_gradient_error_against_exact_attention(muse_lib, name, over):
    # the measurement the reviews ask for: relative squared error of MuSe's gradients (and
    # output) against exact attention's, one head of the workload shape
    cfg = scaled_config(name, **over) if over else CONFIGS[name]
    q, k, v = make_inputs(cfg)
    dO = _dout(cfg)
    grads, _, _ = _gpu_grads(cfg, q, k, v, dO, True)
    ref = exact_attention_bwd(q[0, 0], k[0, 0], v[0, 0], dO[0, 0])
    o_ref, _ = exact_attention(q[0, 0], k[0, 0], v[0, 0])
    out, _ = run_gpu(cfg, q, k, v)
    rse_o = rel_l2(out.float().cpu().numpy()[0, 0], o_ref) ** 2
    rses = [rel_l2(g[0, 0], r) ** 2 for g, r in zip(grads, ref)]
    log(f"[{cfg.name}] RSE vs exact attention: output {rse_o:.3e}, dq {rses[0]:.3e}, dk {rses[1]:.3e}, "
        f"dv {rses[2]:.3e}")
    assert all(np.isfinite(r) and r < 1.0 for r in rses)


@pytest.mark.parametrize("dipole", [True, False])
def test_causal_f32(muse_lib, dipole):
    cfg = scaled_config("acausal_1k_f32", causal=True, block=256)
    check_bwd(cfg, _heads(cfg), dipole)


@pytest.mark.parametrize("dipole", [True, False])
def test_causal_bf16(muse_lib, dipole):
    cfg = scaled_config("causal_16k", B=1, H=2, N=2048, block=512)
    check_bwd(cfg, _heads(cfg), dipole)


@pytest.mark.parametrize("name,over", [
    ("causal_16k", {"B": 1, "H": 1, "N": 1024, "block": 64}),             # 16 blocks of one key tile
    ("causal_16k", {"B": 2, "H": 1, "N": 1536, "block": 192, "Cq": 11, "Ck": 37}),  # tiles across 128-key groups
    ("acausal_1k_f32", {"N": 768, "causal": True, "block": 128, "Cq": 128, "Ck": 128}),  # the largest counts
])
def test_causal_shapes(muse_lib, name, over):
    cfg = scaled_config(name, **over)
    check_bwd(cfg, _heads(cfg))


@pytest.mark.parametrize("name,over,dipole", [
    ("acausal_8k", {"B": 1, "H": 2, "N": 2048, "iters": 1}, True),
    ("acausal_8k", {"B": 1, "H": 1, "N": 2048, "iters": 1}, "untilted"),
    ("acausal_1k_f32", {"iters": 1}, True),
    ("causal_16k", {"B": 1, "H": 2, "N": 2048, "block": 512, "iters": 1}, True),
    ("causal_16k", {"B": 1, "H": 1, "N": 2048, "block": 256, "iters": 1}, False),
])
def test_cap_one_iteration(muse_lib, name, over, dipole):
    # the paper's speed setting: key clusters capped at 1.5 N / Ck members, one Lloyd
    # iteration; the keys left out of the summaries get gradients only through their own
    # block's exact attention (causal) or none (acausal)
    cfg = scaled_config(name, **over)
    check_bwd(cfg, _heads(cfg), dipole, cap_ratio=1.5)


def test_causal_scale_one(muse_lib):
    check_bwd(scaled_config("causal_16k", B=1, H=1, N=1024, block=256), [(0, 0)], scale=1.0)


def test_causal_16k_full_sequence_sampled_head(muse_lib):
    cfg = scaled_config("causal_16k", B=1, H=2)
    check_bwd(cfg, [(0, 1)])


@pytest.mark.parametrize("name", ["causal_16k", "acausal_1k_f32"])
def test_causal_single_block_gives_exact_gradients(muse_lib, name):
    # block = N: no earlier block, so the far field is empty and the output is causal exact
    # attention, and so are its gradients
    cfg = scaled_config(name, B=1, H=1, N=512, causal=True, block=512)
    q, k, v = make_inputs(cfg)
    dO = _dout(cfg)
    grads, _, _ = _gpu_grads(cfg, q, k, v, dO, True)
    ref = exact_attention_bwd(q[0, 0], k[0, 0], v[0, 0], dO[0, 0], causal=True)
    for name_, g, r in zip(("dq", "dk", "dv"), grads, ref):
        rel = rel_l2(g[0, 0], r)
        log(f"[{cfg.name} one block bwd] {name_}: rel-L2 vs causal exact attention {rel:.3e}")
        assert rel <= BWD_TOL[cfg.dtype]


def test_causal_gradient_error_against_exact_attention(muse_lib):
    cfg = scaled_config("causal_16k", B=1, H=1, N=4096)
    q, k, v = make_inputs(cfg)
    dO = _dout(cfg)
    grads, _, _ = _gpu_grads(cfg, q, k, v, dO, True)
    ref = exact_attention_bwd(q[0, 0], k[0, 0], v[0, 0], dO[0, 0], causal=True)
    rses = [rel_l2(g[0, 0], r) ** 2 for g, r in zip(grads, ref)]
    log(f"[{cfg.name} N={cfg.N}] RSE vs causal exact attention: dq {rses[0]:.3e}, dk {rses[1]:.3e}, dv {rses[2]:.3e}")
    assert all(np.isfinite(r) and r < 1.0 for r in rses)


def test_unsupported_calls_are_refused(muse_lib):
    from clustered_softmax_attention_amd import MuseError, attn_bwd
    cfg = scaled_config("causal_16k", B=1, H=1, N=2048, block=512)
    q, k, v = make_inputs(cfg)
    Q, K, V = (to_device(t, cfg.dtype) for t in (q, k, v))
    lab = torch.zeros((1, 1, cfg.N), dtype=torch.int32, device="cuda")
    with pytest.raises(MuseError, match="UNSUPPORTED"):
        attn_bwd(Q, K, V, Q.clone(), lab, lab, cfg.Cq, cfg.Ck, causal=True, block=cfg.block, dipole="untilted")
    cfg = scaled_config("causal_64k_d128", B=1, H=1, N=1024, causal=False, block=0)
    q, k, v = make_inputs(cfg)
    Q, K, V = (to_device(t, cfg.dtype) for t in (q, k, v))
    with pytest.raises(MuseError, match="UNSUPPORTED"):
        attn_bwd(Q, K, V, Q.clone(), lab[..., :1024].contiguous(), lab[..., :1024].contiguous(), cfg.Cq, cfg.Ck)
