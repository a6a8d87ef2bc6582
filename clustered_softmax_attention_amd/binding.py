"""Python binding of the MuSe C-ABI library (libmuse.so): argument marshalling only.

Tensors are torch CUDA tensors of shape [B, H, N, D], contiguous, float32 or
bfloat16; the library receives their device pointers and the current HIP stream.
Every computation happens in the library's HIP kernels. Loading fails loudly when
the library has not been built (``python -m clustered_softmax_attention_amd.build``).
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmuse.so")
_lib = None

MUSE_F32, MUSE_BF16 = 0, 1
MUSE_OK = 0
NOALLOC_SCRATCH_BYTES = 64 << 20  # MUSE_NOALLOC_SCRATCH_BYTES of include/muse.h
STATUS = {0: "MUSE_OK", -1: "MUSE_ERR_INVALID_ARG", -2: "MUSE_ERR_UNSUPPORTED", -3: "MUSE_ERR_HIP",
          -4: "MUSE_ERR_NO_MEMORY", -5: "MUSE_ERR_WORKSPACE"}

# C entry points declared in include/muse.h
EXPORTED = ("muse_attn_fwd", "muse_exact_attn_fwd", "muse_attn_fwd_ex", "muse_fwd_params_init",
            "muse_attn_fwd_workspace_bytes", "muse_last_error", "muse_version", "muse_prof_enable",
            "muse_prof_collect", "muse_prof_name", "muse_prof_total_ms", "muse_prof_launches",
            "muse_prof_reset", "muse_attn_fwd_noalloc", "muse_attn_bwd", "muse_attn_bwd_workspace_bytes")


class MuseError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


class FwdParams(ctypes.Structure):
    _fields_ = [
        ("scale", ctypes.c_float),
        ("out_dtype", ctypes.c_int),
        ("dipole", ctypes.c_int),
        ("topk_clusters", ctypes.c_int),
        ("topk_blocks", ctypes.c_int),
        ("labels_q_in", ctypes.c_void_p),
        ("labels_k_in", ctypes.c_void_p),
        ("labels_q_trace", ctypes.c_void_p),
        ("labels_k_trace", ctypes.c_void_p),
        ("centroids_q_out", ctypes.c_void_p),
        ("centroids_k_out", ctypes.c_void_p),
        ("lse_out", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("retrieval_trace", ctypes.c_void_p),
        ("hierarchy", ctypes.c_int),
        ("perm_q_out", ctypes.c_void_p),
        ("offs_q_out", ctypes.c_void_p),
        ("perm_k_out", ctypes.c_void_p),
        ("offs_k_out", ctypes.c_void_p),
        ("single_stream", ctypes.c_int),
        ("cap_ratio", ctypes.c_double),
    ]


def load(path: str = _LIB_PATH) -> ctypes.CDLL:
    """Load libmuse.so (raises if it is missing: there is no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} not found: build it with `python -m clustered_softmax_attention_amd.build`")
    lib = ctypes.CDLL(path)
    i, vp, sz = ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
    lib.muse_attn_fwd.argtypes = [vp, vp, vp, vp] + [i] * 10 + [vp]
    lib.muse_attn_fwd.restype = i
    lib.muse_attn_fwd_ex.argtypes = [vp, vp, vp, vp] + [i] * 10 + [vp, ctypes.POINTER(FwdParams)]
    lib.muse_attn_fwd_ex.restype = i
    lib.muse_attn_fwd_noalloc.argtypes = [vp, vp, vp, vp] + [i] * 10 + [vp, ctypes.POINTER(FwdParams)]
    lib.muse_attn_fwd_noalloc.restype = i
    lib.muse_attn_bwd.argtypes = [vp] * 9 + [i] * 9 + [vp, ctypes.POINTER(FwdParams)]
    lib.muse_attn_bwd.restype = i
    lib.muse_attn_bwd_workspace_bytes.argtypes = [i] * 9 + [ctypes.POINTER(FwdParams)]
    lib.muse_attn_bwd_workspace_bytes.restype = sz
    lib.muse_exact_attn_fwd.argtypes = [vp, vp, vp, vp] + [i] * 6 + [vp]
    lib.muse_exact_attn_fwd.restype = i
    lib.muse_fwd_params_init.argtypes = [ctypes.POINTER(FwdParams)]
    lib.muse_fwd_params_init.restype = None
    lib.muse_attn_fwd_workspace_bytes.argtypes = [i] * 9 + [ctypes.POINTER(FwdParams)]
    lib.muse_attn_fwd_workspace_bytes.restype = sz
    lib.muse_last_error.argtypes = []
    lib.muse_last_error.restype = ctypes.c_char_p
    lib.muse_version.argtypes = []
    lib.muse_version.restype = i
    lib.muse_prof_enable.argtypes = [i]
    lib.muse_prof_enable.restype = None
    lib.muse_prof_collect.argtypes = []
    lib.muse_prof_collect.restype = i
    lib.muse_prof_name.argtypes = [i]
    lib.muse_prof_name.restype = ctypes.c_char_p
    lib.muse_prof_total_ms.argtypes = [i]
    lib.muse_prof_total_ms.restype = ctypes.c_double
    lib.muse_prof_launches.argtypes = [i]
    lib.muse_prof_launches.restype = ctypes.c_long
    lib.muse_prof_reset.argtypes = []
    lib.muse_prof_reset.restype = None
    _lib = lib
    return lib


def _check(code: int):
    if code != MUSE_OK:
        raise MuseError(code, _lib.muse_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MUSE_F32
    if t.dtype == torch.bfloat16:
        return MUSE_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check_qkv(q, k, v):
    for t in (q, k, v):
        if not (t.is_cuda and t.is_contiguous() and t.dim() == 4):
            raise ValueError("q, k, v must be contiguous 4-D [B, H, N, D] device tensors")
    if not (q.shape == k.shape == v.shape and q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share shape and dtype")


def _stream() -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def exact_attn_fwd(q, k, v, causal: bool = False, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """muse_exact_attn_fwd: exact softmax attention (scale 1/sqrt(D)); out dtype = input dtype."""
    lib = load()
    _check_qkv(q, k, v)
    B, H, N, D = q.shape
    if out is None:
        out = torch.empty_like(q)
    _check(lib.muse_exact_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, N, D, int(causal),
                                   _dtype_code(q), _stream()))
    return out


DIPOLE_MODES = {"none": 0, "tilted": 1, "untilted": 2}  # MUSE_DIPOLE_* of include/muse.h


def dipole_code(dipole) -> int:
    """MUSE_DIPOLE_* code of a dipole argument: True (tilted), False (none), a name of
    DIPOLE_MODES, or the code itself."""
    if isinstance(dipole, bool):
        return 1 if dipole else 0
    if isinstance(dipole, str):
        if dipole not in DIPOLE_MODES:
            raise ValueError(f"unknown dipole mode {dipole!r}")
        return DIPOLE_MODES[dipole]
    return int(dipole)


def attn_fwd(q, k, v, Cq: int, Ck: int, kmeans_iters: int, causal: bool = False, block: int = 0,
             out: Optional[torch.Tensor] = None, *, scale: float = 0.0, out_dtype=None, dipole=True,
             topk_clusters: int = 0, topk_blocks: int = 0, labels_q_in=None, labels_k_in=None,
             return_trace: bool = False, return_centroids: bool = False, return_lse: bool = False,
             return_buckets: bool = False, workspace: Optional[torch.Tensor] = None, hierarchy: bool = False,
             single_stream: bool = False, cap_ratio: float = 0.0, _entry: str = "muse_attn_fwd_ex"):
    """muse_attn_fwd_ex. Returns out, or (out, extras) when any return_* flag is set, where
    extras holds 'labels_q_trace', 'labels_k_trace' [iters,B,H,N] int32, 'centroids_q',
    'centroids_k' [B,H,C,D] float32, 'lse' [B,H,N] float32, 'perm_q', 'perm_k' [B,H,N] and
    'offs_q', 'offs_k' [B,H,nb*C+1] int32 (bucket order) and, with retrieval,
    'retrieval_trace' [B,H,N/block,Cq,k1,1+k2] int32 as requested. cap_ratio > 0 caps the
    key clusters of the stage-1 summaries at ceil(cap_ratio * N / Ck) members."""
    lib = load()
    _check_qkv(q, k, v)
    B, H, N, D = q.shape
    dev = q.device
    if out_dtype is None:
        out_dtype = q.dtype
    if out is None:
        out = torch.empty((B, H, N, D), dtype=out_dtype, device=dev)
    p = FwdParams()
    lib.muse_fwd_params_init(ctypes.byref(p))
    p.scale = float(scale)
    p.out_dtype = _dtype_code(out)
    p.dipole = dipole_code(dipole)
    p.topk_clusters = int(topk_clusters)
    p.topk_blocks = int(topk_blocks)
    p.hierarchy = int(hierarchy)
    p.single_stream = int(single_stream)
    p.cap_ratio = float(cap_ratio)
    extras = {}
    keep = []
    for name, lab in (("labels_q_in", labels_q_in), ("labels_k_in", labels_k_in)):
        if lab is not None:
            lab = lab.to(device=dev, dtype=torch.int32).contiguous()
            keep.append(lab)
            setattr(p, name, lab.data_ptr())
    if return_trace:
        for name in ("labels_q_trace", "labels_k_trace"):
            t = torch.full((kmeans_iters, B, H, N), -1, dtype=torch.int32, device=dev)
            extras[name] = t
            setattr(p, name, t.data_ptr())
        if topk_clusters > 0 and causal:
            t = torch.full((B, H, N // block, Cq, topk_clusters, 1 + topk_blocks), -1, dtype=torch.int32,
                           device=dev)
            extras["retrieval_trace"] = t
            p.retrieval_trace = t.data_ptr()
    if return_centroids:
        extras["centroids_q"] = torch.empty((B, H, Cq, D), dtype=torch.float32, device=dev)
        extras["centroids_k"] = torch.empty((B, H, Ck, D), dtype=torch.float32, device=dev)
        p.centroids_q_out = extras["centroids_q"].data_ptr()
        p.centroids_k_out = extras["centroids_k"].data_ptr()
    if return_lse:
        extras["lse"] = torch.empty((B, H, N), dtype=torch.float32, device=dev)
        p.lse_out = extras["lse"].data_ptr()
    if return_buckets:
        nb = N // block if causal else 1
        for name, C in (("q", Cq), ("k", Ck)):
            extras["perm_" + name] = torch.full((B, H, N), -1, dtype=torch.int32, device=dev)
            extras["offs_" + name] = torch.full((B, H, nb * C + 1), -1, dtype=torch.int32, device=dev)
            setattr(p, f"perm_{name}_out", extras["perm_" + name].data_ptr())
            setattr(p, f"offs_{name}_out", extras["offs_" + name].data_ptr())
    if workspace is not None:
        p.workspace = workspace.data_ptr()
        p.workspace_bytes = workspace.numel() * workspace.element_size()
    _check(getattr(lib, _entry)(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, N, D, Cq, Ck, kmeans_iters,
                                int(causal), int(block), _dtype_code(q), _stream(), ctypes.byref(p)))
    del keep
    return (out, extras) if extras else out


def attn_bwd(q, k, v, dout, labels_q, labels_k, Cq: int, Ck: int, causal: bool = False, block: int = 0, *,
             scale: float = 0.0, dipole=True, cap_ratio: float = 0.0, workspace: Optional[torch.Tensor] = None):
    """muse_attn_bwd: (dq, dk, dv) float32 [B,H,N,D] of the forward output for the upstream
    gradient dout (the inputs' dtype), with the forward's final labels [B,H,N] held fixed."""
    lib = load()
    _check_qkv(q, k, v)
    if not (dout.is_cuda and dout.is_contiguous() and dout.shape == q.shape and dout.dtype == q.dtype):
        raise ValueError("dout must be a contiguous device tensor of q's shape and dtype")
    B, H, N, D = q.shape
    lq = labels_q.to(device=q.device, dtype=torch.int32).contiguous()
    lk = labels_k.to(device=q.device, dtype=torch.int32).contiguous()
    if lq.shape != (B, H, N) or lk.shape != (B, H, N):
        raise ValueError("labels must be [B, H, N]")
    dq, dk, dv = (torch.empty((B, H, N, D), dtype=torch.float32, device=q.device) for _ in range(3))
    p = FwdParams()
    lib.muse_fwd_params_init(ctypes.byref(p))
    p.scale = float(scale)
    p.dipole = dipole_code(dipole)
    p.cap_ratio = float(cap_ratio)
    if workspace is not None:
        p.workspace = workspace.data_ptr()
        p.workspace_bytes = workspace.numel() * workspace.element_size()
    _check(lib.muse_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(lq), _ptr(lk), _ptr(dq), _ptr(dk),
                             _ptr(dv), B, H, N, D, Cq, Ck, int(causal), int(block), _dtype_code(q), _stream(),
                             ctypes.byref(p)))
    return dq, dk, dv


def bwd_workspace_bytes(B, H, N, D, Cq, Ck, causal=False, block=0, dtype=MUSE_BF16, dipole=True,
                        cap_ratio: float = 0.0) -> int:
    lib = load()
    p = FwdParams()
    lib.muse_fwd_params_init(ctypes.byref(p))
    p.dipole = dipole_code(dipole)
    p.cap_ratio = float(cap_ratio)
    n = lib.muse_attn_bwd_workspace_bytes(B, H, N, D, Cq, Ck, int(causal), int(block), dtype, ctypes.byref(p))
    if n == 0:
        raise MuseError(-1, lib.muse_last_error().decode())
    return n


def attn_fwd_noalloc(q, k, v, Cq: int, Ck: int, kmeans_iters: int, causal: bool = False, block: int = 0,
                     out: Optional[torch.Tensor] = None, **kw):
    """muse_attn_fwd_noalloc: attn_fwd on the library's fixed per-device scratch (no device
    allocation in the call; shapes whose workspace exceeds the scratch are refused). Takes
    attn_fwd's keyword arguments except `workspace`. Output tensors the caller does not
    pass (out, and those of return_* flags) are still created here by torch."""
    if kw.get("workspace") is not None:
        raise ValueError("the allocation-free entry takes no workspace")
    return attn_fwd(q, k, v, Cq, Ck, kmeans_iters, causal, block, out, _entry="muse_attn_fwd_noalloc", **kw)


def attn_fwd_plain(q, k, v, Cq: int, Ck: int, kmeans_iters: int, causal: bool = False, block: int = 0,
                   out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """muse_attn_fwd: defaults only (scale 1/sqrt(D), tilted dipole, out dtype = input dtype)."""
    lib = load()
    _check_qkv(q, k, v)
    B, H, N, D = q.shape
    if out is None:
        out = torch.empty_like(q)
    _check(lib.muse_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, N, D, Cq, Ck, kmeans_iters, int(causal),
                             int(block), _dtype_code(q), _stream()))
    return out


def prof_enable(on: bool = True):
    """Bracket every library kernel launch with HIP events (see muse_prof_* in muse.h)."""
    load().muse_prof_enable(int(on))


def prof_reset():
    load().muse_prof_reset()


def prof_collect() -> dict:
    """{kernel name: (total ms, launches)} accumulated since the last reset (blocks on events)."""
    lib = load()
    n = lib.muse_prof_collect()
    return {lib.muse_prof_name(i).decode(): (lib.muse_prof_total_ms(i), lib.muse_prof_launches(i)) for i in range(n)}


def workspace_bytes(B, H, N, D, Cq, Ck, causal=False, block=0, dtype=MUSE_BF16, topk_clusters=0,
                    topk_blocks=0, dipole=True, hierarchy=False, cap_ratio=0.0) -> int:
    lib = load()
    p = FwdParams()
    lib.muse_fwd_params_init(ctypes.byref(p))
    p.topk_clusters, p.topk_blocks = topk_clusters, topk_blocks
    p.dipole = dipole_code(dipole)
    p.hierarchy = int(hierarchy)
    p.cap_ratio = float(cap_ratio)
    n = lib.muse_attn_fwd_workspace_bytes(B, H, N, D, Cq, Ck, int(causal), int(block), dtype, ctypes.byref(p))
    if n == 0:
        raise MuseError(-1, lib.muse_last_error().decode())
    return n
