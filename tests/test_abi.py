"""The C-ABI library loads and exports every symbol include/muse.h declares; argument
validation runs on the host before any launch (CPU only: no GPU call is made)."""

import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "muse.h")
LIB = os.path.join(ROOT, "clustered_softmax_attention_amd", "libmuse.so")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(muse_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from clustered_softmax_attention_amd import build
        build.build(verbose=False)
    from clustered_softmax_attention_amd import binding
    return binding.load(LIB)


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("muse_attn_fwd", "muse_exact_attn_fwd", "muse_attn_fwd_ex", "muse_attn_fwd_workspace_bytes",
              "muse_fwd_params_init", "muse_last_error", "muse_version"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (muse_\w+)", out))
    for n in declared_functions():
        assert n in exported, n
        assert hasattr(lib, n)


def test_binding_covers_the_exports():
    from clustered_softmax_attention_amd import binding
    assert sorted(binding.EXPORTED) == declared_functions()


def test_params_struct_layout_matches(lib):
    from clustered_softmax_attention_amd.binding import FwdParams
    p = FwdParams()
    lib.muse_fwd_params_init(ctypes.byref(p))
    assert p.out_dtype == -1 and p.dipole == 1 and p.scale == 0.0 and p.topk_clusters == 0 and p.hierarchy == 0
    # 5 ints/floats, pad, 8 pointers, size_t, pointer, int, pad, 4 bucket-order pointers, int,
    # pad, double
    assert ctypes.sizeof(FwdParams) == 4 * 5 + 4 + 8 * 8 + 8 + 8 + 4 + 4 + 4 * 8 + 4 + 4 + 8
    assert FwdParams.cap_ratio.offset == ctypes.sizeof(FwdParams) - 8
    assert p.single_stream == 0 and p.cap_ratio == 0.0
    assert p.perm_q_out is None and p.offs_k_out is None


def _call(lib, **kw):
    args = dict(q=1, k=2, v=3, out=4, B=1, H=1, N=1024, D=64, Cq=8, Ck=32, iters=5, causal=0, block=0, dtype=0)
    args.update(kw)
    vp = ctypes.c_void_p
    return lib.muse_attn_fwd(vp(args["q"]), vp(args["k"]), vp(args["v"]), vp(args["out"]), args["B"], args["H"],
                             args["N"], args["D"], args["Cq"], args["Ck"], args["iters"], args["causal"],
                             args["block"], args["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), -1), (dict(D=96), -2), (dict(N=0), -1), (dict(Cq=0), -1), (dict(Ck=2000), -1),
    (dict(Cq=200, N=4096), -2), (dict(iters=0), -1), (dict(dtype=7), -1),
    (dict(causal=1, block=100), -1), (dict(causal=1, block=0), -1), (dict(causal=1, block=2048), -1),
    (dict(causal=2), -1), (dict(out=1), -1),
    # valid blocks (divisors of N) that the kernels do not implement: below 64 tokens or
    # not a multiple of 64
    (dict(causal=1, block=1), -2), (dict(causal=1, block=32), -2), (dict(causal=1, block=512, N=1536), 0),
    (dict(causal=1, block=192, N=1536), 0), (dict(causal=1, block=96, N=1536), -2),
])
def test_invalid_arguments_are_rejected_before_launch(lib, kw, code):
    if code == 0:
        # accepted shapes: checked through the workspace query, which launches nothing
        a = dict(B=1, H=1, N=1024, D=64, Cq=8, Ck=32, causal=0, block=0, dtype=0)
        a.update({k: v for k, v in kw.items() if k in a})
        assert lib.muse_attn_fwd_workspace_bytes(a["B"], a["H"], a["N"], a["D"], a["Cq"], a["Ck"], a["causal"],
                                                 a["block"], a["dtype"], None) > 0
        return
    assert _call(lib, **kw) == code
    assert lib.muse_last_error().decode() != ""


def test_workspace_query(lib):
    from clustered_softmax_attention_amd.binding import FwdParams
    n_ac = lib.muse_attn_fwd_workspace_bytes(4, 8, 8192, 64, 32, 128, 0, 0, 1, None)
    n_c = lib.muse_attn_fwd_workspace_bytes(8, 8, 16384, 64, 16, 64, 1, 1024, 1, None)
    assert n_ac > 0 and n_c > 0
    assert lib.muse_attn_fwd_workspace_bytes(1, 1, 1024, 65, 8, 32, 0, 0, 1, None) == 0
    p = FwdParams()
    lib.muse_fwd_params_init(ctypes.byref(p))
    p.topk_clusters = 2  # acausal retrieval is invalid
    assert lib.muse_attn_fwd_workspace_bytes(1, 1, 1024, 64, 8, 32, 0, 0, 1, ctypes.byref(p)) == 0


def test_exact_rejects_bad_shapes(lib):
    vp = ctypes.c_void_p
    assert lib.muse_exact_attn_fwd(vp(1), vp(2), vp(3), vp(4), 1, 1, 64, 80, 0, 1, None) == -2
    assert lib.muse_exact_attn_fwd(vp(1), vp(2), vp(3), None, 1, 1, 64, 64, 0, 1, None) == -1
    assert lib.muse_version() >= 100


def test_dipole_modes(lib):
    # the binding's mode names follow the header's MUSE_DIPOLE_* values
    from clustered_softmax_attention_amd import binding
    from clustered_softmax_attention_amd.binding import FwdParams
    text = open(HEADER).read()
    for name, code in binding.DIPOLE_MODES.items():
        assert re.search(rf"\bMUSE_DIPOLE_{name.upper()}\s*=\s*{code}\b", text), name
    assert binding.dipole_code(True) == 1 and binding.dipole_code(False) == 0
    assert binding.dipole_code("untilted") == 2
    with pytest.raises(ValueError):
        binding.dipole_code("sideways")
    p = FwdParams()
    lib.muse_fwd_params_init(ctypes.byref(p))
    tilted = lib.muse_attn_fwd_workspace_bytes(4, 8, 8192, 64, 32, 128, 0, 0, 1, ctypes.byref(p))
    p.dipole = 2
    # acausal: the untilted mode adds the per key cluster covariances [B*H, Ck, D, D] fp32
    untilted = lib.muse_attn_fwd_workspace_bytes(4, 8, 8192, 64, 32, 128, 0, 0, 1, ctypes.byref(p))
    assert untilted >= tilted + 32 * 128 * 64 * 64 * 4
    # causal: the bucket statistics [B*H, nb*Ck, D, D] fp32 and their prefix means
    causal = lib.muse_attn_fwd_workspace_bytes(8, 8, 16384, 64, 16, 64, 1, 1024, 1, ctypes.byref(p))
    p.dipole = 1
    causal_tilted = lib.muse_attn_fwd_workspace_bytes(8, 8, 16384, 64, 16, 64, 1, 1024, 1, ctypes.byref(p))
    assert causal >= causal_tilted + 64 * 16 * 64 * 64 * 64 * 4
    # not combined with retrieval: refused before any launch
    p.dipole = 2
    p.topk_clusters, p.topk_blocks = 4, 2
    assert lib.muse_attn_fwd_workspace_bytes(8, 8, 16384, 64, 16, 64, 1, 1024, 1, ctypes.byref(p)) == 0
    assert "retrieval" in lib.muse_last_error().decode()
    p.topk_clusters, p.topk_blocks = 0, 0
    p.dipole = 3
    assert lib.muse_attn_fwd_workspace_bytes(4, 8, 8192, 64, 32, 128, 0, 0, 1, ctypes.byref(p)) == 0


def test_ex_entry_rejects_before_launch(lib):
    # everything below fails in the host-side checks, before any device call
    from clustered_softmax_attention_amd.binding import FwdParams
    vp = ctypes.c_void_p
    p = FwdParams()
    lib.muse_fwd_params_init(ctypes.byref(p))
    need = lib.muse_attn_fwd_workspace_bytes(1, 1, 1024, 64, 8, 32, 0, 0, 1, ctypes.byref(p))
    p.workspace = 0x1000
    p.workspace_bytes = need - 1
    args = (vp(1), vp(2), vp(3), vp(4), 1, 1, 1024, 64, 8, 32, 5, 0, 0, 1, None)
    assert lib.muse_attn_fwd_ex(*args, ctypes.byref(p)) == -5  # MUSE_ERR_WORKSPACE
    assert "workspace" in lib.muse_last_error().decode()
    p.workspace_bytes = need
    p.dipole = 2
    p.hierarchy = 1
    causal = (vp(1), vp(2), vp(3), vp(4), 1, 1, 1024, 64, 8, 32, 5, 1, 256, 1, None)
    assert lib.muse_attn_fwd_ex(*causal, ctypes.byref(p)) == -2  # untilted dipole: not with the hierarchy
    p.hierarchy = 0
    p.dipole = 1
    p.hierarchy = 1
    acausal = (vp(1), vp(2), vp(3), vp(4), 1, 1, 1024, 64, 8, 32, 5, 0, 0, 1, None)
    assert lib.muse_attn_fwd_ex(*acausal, ctypes.byref(p)) == -1  # hierarchy needs causal
    p.topk_clusters, p.topk_blocks = 2, 1
    assert lib.muse_attn_fwd_ex(*causal, ctypes.byref(p)) == -2  # not combined with retrieval
    p.topk_clusters, p.topk_blocks = 0, 0
    p.hierarchy = 2
    assert lib.muse_attn_fwd_ex(*causal, ctypes.byref(p)) == -1  # 0 or 1
    p.hierarchy = 0
    aliased = (vp(1), vp(2), vp(3), vp(1), 1, 1, 1024, 64, 8, 32, 5, 0, 0, 1, None)
    assert lib.muse_attn_fwd_ex(*aliased, ctypes.byref(p)) == -1  # out aliases q


def test_noalloc_entry_rejects_before_launch(lib):
    # the allocation-free entry: host-side checks only (no device call is reached)
    from clustered_softmax_attention_amd import binding
    from clustered_softmax_attention_amd.binding import FwdParams
    text = open(HEADER).read()
    m = re.search(r"#define MUSE_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == binding.NOALLOC_SCRATCH_BYTES
    vp = ctypes.c_void_p
    # the 8k workload (all 32 heads) needs far more than the scratch: refused, nothing launched
    big = (vp(1), vp(2), vp(3), vp(4), 4, 8, 8192, 64, 32, 128, 5, 0, 0, 1, None)
    assert lib.muse_attn_fwd_workspace_bytes(4, 8, 8192, 64, 32, 128, 0, 0, 1, None) > binding.NOALLOC_SCRATCH_BYTES
    assert lib.muse_attn_fwd_noalloc(*big, None) == -5  # MUSE_ERR_WORKSPACE
    assert "scratch" in lib.muse_last_error().decode()
    # a caller workspace is refused: the entry only uses its own scratch
    p = FwdParams()
    lib.muse_fwd_params_init(ctypes.byref(p))
    p.workspace, p.workspace_bytes = 0x1000, 1 << 30
    small = (vp(1), vp(2), vp(3), vp(4), 1, 1, 1024, 64, 8, 32, 5, 0, 0, 0, None)
    assert lib.muse_attn_fwd_noalloc(*small, ctypes.byref(p)) == -1
    # the usual validation still runs first
    bad = (vp(1), vp(2), vp(3), vp(4), 1, 1, 1024, 96, 8, 32, 5, 0, 0, 0, None)
    assert lib.muse_attn_fwd_noalloc(*bad, None) == -2


def test_cluster_cap_arguments(lib):
    from clustered_softmax_attention_amd.binding import FwdParams
    p = FwdParams()
    lib.muse_fwd_params_init(ctypes.byref(p))
    base = lib.muse_attn_fwd_workspace_bytes(4, 8, 8192, 64, 32, 128, 0, 0, 1, ctypes.byref(p))
    p.cap_ratio = 1.5
    # kept lengths [B*H, nb*Ck] int32 and a flag byte per key, each region 256-byte aligned
    capped = lib.muse_attn_fwd_workspace_bytes(4, 8, 8192, 64, 32, 128, 0, 0, 1, ctypes.byref(p))
    assert capped == base + 32 * 128 * 4 + 32 * 8192
    causal = lib.muse_attn_fwd_workspace_bytes(1, 1, 4096, 64, 16, 64, 1, 1024, 1, ctypes.byref(p))
    p.hierarchy = 1  # with the hierarchical decomposition: accepted
    assert lib.muse_attn_fwd_workspace_bytes(1, 1, 4096, 64, 16, 64, 1, 1024, 1, ctypes.byref(p)) == causal > 0
    p.hierarchy = 0
    p.dipole = 2  # untilted dipole: accepted
    assert lib.muse_attn_fwd_workspace_bytes(1, 1, 4096, 64, 16, 64, 1, 1024, 0, ctypes.byref(p)) > 0
    p.dipole = 1
    vp = ctypes.c_void_p
    causal_args = (vp(1), vp(2), vp(3), vp(4), 1, 1, 4096, 64, 16, 64, 5, 1, 1024, 1, None)
    p.topk_clusters, p.topk_blocks = 2, 1  # not with retrieval
    assert lib.muse_attn_fwd_ex(*causal_args, ctypes.byref(p)) == -2
    assert "cap" in lib.muse_last_error().decode()
    p.topk_clusters, p.topk_blocks = 0, 0
    for bad in (-1.0, float("nan")):
        p.cap_ratio = bad
        assert lib.muse_attn_fwd_ex(*causal_args, ctypes.byref(p)) == -1
        assert "cap_ratio" in lib.muse_last_error().decode()


def test_backward_entry_rejects_before_launch(lib):
    # muse_attn_bwd: host-side checks only (no device call is reached)
    from clustered_softmax_attention_amd.binding import FwdParams
    vp = ctypes.c_void_p
    p = FwdParams()
    lib.muse_fwd_params_init(ctypes.byref(p))
    ins = (vp(1), vp(2), vp(3), vp(4), vp(5), vp(6))
    outs = (vp(7), vp(8), vp(9))

    def call(B=1, H=1, N=1024, D=64, Cq=8, Ck=32, causal=0, block=0, dtype=1, ins=ins, outs=outs, pp=None):
        return lib.muse_attn_bwd(*ins, *outs, B, H, N, D, Cq, Ck, causal, block, dtype, None,
                                 None if pp is None else ctypes.byref(pp))

    assert lib.muse_attn_bwd_workspace_bytes(4, 8, 8192, 64, 32, 128, 0, 0, 1, None) > 0
    # causal calls: the tilted dipole or none, with the forward's block rules
    causal_ws = lib.muse_attn_bwd_workspace_bytes(1, 1, 1024, 64, 8, 32, 1, 256, 1, None)
    assert causal_ws > lib.muse_attn_bwd_workspace_bytes(1, 1, 1024, 64, 8, 32, 0, 0, 1, None)
    assert call(causal=1, block=100) == -1                      # block must divide N
    assert call(causal=1, block=32) == -2                       # blocks below 64 keys
    p.dipole = 2
    assert call(causal=1, block=256, pp=p) == -2 and "causal" in lib.muse_last_error().decode()
    assert lib.muse_attn_bwd_workspace_bytes(1, 1, 1024, 64, 8, 32, 1, 256, 1, ctypes.byref(p)) == 0
    p.dipole = 1
    assert call(D=128) == -2
    assert call(ins=ins[:4] + (None, vp(6))) == -1  # labels are required
    assert call(outs=(vp(7), vp(7), vp(9))) == -1   # distinct outputs
    assert call(outs=(vp(1), vp(8), vp(9))) == -1   # no output aliases an input
    # the cap is accepted (its workspace holds the kept lengths and flags); retrieval and
    # the hierarchy are not
    p.cap_ratio = 1.5
    assert lib.muse_attn_bwd_workspace_bytes(1, 1, 1024, 64, 8, 32, 0, 0, 1, ctypes.byref(p)) > 0
    p.cap_ratio = 0.0
    p.hierarchy = 1
    assert call(causal=1, block=256, pp=p) == -2 and "hierarchy" in lib.muse_last_error().decode()
    p.hierarchy = 0
    p.topk_clusters, p.topk_blocks = 2, 1
    assert call(causal=1, block=256, pp=p) == -2
    p.topk_clusters, p.topk_blocks = 0, 0
    p.lse_out = 0x1000                              # no forward outputs
    assert call(pp=p) == -1
    p.lse_out = None
    p.workspace, p.workspace_bytes = 0x1000, 16
    assert call(pp=p) == -5                          # workspace too small
    # the untilted mode needs the covariance regions, the tilted one the per-key tables
    p.workspace, p.workspace_bytes = None, 0
    p.dipole = 0
    none = lib.muse_attn_bwd_workspace_bytes(4, 8, 8192, 64, 32, 128, 0, 0, 1, ctypes.byref(p))
    p.dipole = 1
    tilted = lib.muse_attn_bwd_workspace_bytes(4, 8, 8192, 64, 32, 128, 0, 0, 1, ctypes.byref(p))
    assert tilted >= none + 3 * 32 * 32 * 8192 * 4
