"""A MuSe call (forward, or backward with a workspace) captured into a HIP graph (through torch's graph capture on a side stream)
replays to the eager result, bitwise, every time: the library's event fork/join with its
internal stream is captured as graph dependencies, and nothing in a call records a memset."""

import pytest
import torch

from parity_util import to_device
from workloads import make_inputs, scaled_config

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,over,hier", [
    ("acausal_8k", {"B": 1, "H": 2, "N": 1536}, False),
    ("causal_16k", {"B": 1, "H": 2, "N": 2048, "block": 512}, False),
    # the general stage-1 path: the hierarchical squares, and retrieval
    ("causal_16k", {"B": 1, "H": 2, "N": 3072, "block": 512}, True),
    ("retrieval_16k", {"B": 1, "H": 2, "N": 2048, "block": 256}, False),
])
def test_graph_replay_matches_eager(muse_lib, name, over, hier):
    from clustered_softmax_attention_amd import binding
    cfg = scaled_config(name, **over)
    q, k, v = (to_device(t, cfg.dtype) for t in make_inputs(cfg))
    ws = torch.empty(binding.workspace_bytes(cfg.B, cfg.H, cfg.N, cfg.D, cfg.Cq, cfg.Ck, cfg.causal, cfg.block, 1,
                                             cfg.topk_clusters, cfg.topk_blocks, hierarchy=hier),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)

    def step():
        binding.attn_fwd(q, k, v, cfg.Cq, cfg.Ck, cfg.iters, causal=cfg.causal, block=cfg.block, out=out,
                         topk_clusters=cfg.topk_clusters, topk_blocks=cfg.topk_blocks, hierarchy=hier,
                         workspace=ws)

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        step()
    torch.cuda.synchronize()
    ref = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    torch.cuda.synchronize()
    for _ in range(3):
        out.zero_()  # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)


@pytest.mark.parametrize("name,over", [
    ("acausal_8k", {"B": 1, "H": 2, "N": 1536}),
    ("causal_16k", {"B": 1, "H": 2, "N": 2048, "block": 512}),
])
def test_backward_graph_replay_matches_eager(muse_lib, name, over):
    # the backward pass with a caller's workspace records no allocation, memset or
    # synchronisation, so it captures too; every replay reproduces the eager gradients
    from clustered_softmax_attention_amd import binding
    cfg = scaled_config(name, **over)
    q, k, v = (to_device(t, cfg.dtype) for t in make_inputs(cfg))
    _, ex = binding.attn_fwd(q, k, v, cfg.Cq, cfg.Ck, cfg.iters, causal=cfg.causal, block=cfg.block,
                             return_trace=True)
    lq = ex["labels_q_trace"][-1].contiguous()
    lk = ex["labels_k_trace"][-1].contiguous()
    gen = torch.Generator(device="cuda").manual_seed(5)
    dO = torch.randn(q.shape, generator=gen, device="cuda", dtype=torch.float32).to(q.dtype)
    ws = torch.empty(binding.bwd_workspace_bytes(cfg.B, cfg.H, cfg.N, cfg.D, cfg.Cq, cfg.Ck, cfg.causal, cfg.block,
                                                 1), dtype=torch.uint8, device="cuda")

    def step():
        return binding.attn_bwd(q, k, v, dO, lq, lk, cfg.Cq, cfg.Ck, causal=cfg.causal, block=cfg.block,
                                workspace=ws)

    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        ref = [t.clone() for t in step()]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        outs = step()
    torch.cuda.synchronize()
    for _ in range(3):
        for t in outs:
            t.zero_()  # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, r in zip(outs, ref):
            assert torch.equal(t, r)
