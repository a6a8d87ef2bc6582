"""MuSe (Multipole Semantic Attention) forward pass for AMD MI355X (gfx950).

The computation lives in hand-written HIP kernels behind the C ABI of
``libmuse.so`` (declared in ``include/muse.h``); ``binding`` marshals torch
tensors into those calls. See ``binding.attn_fwd`` and ``binding.exact_attn_fwd``.
"""

from .binding import MuseError, attn_fwd, exact_attn_fwd, load, workspace_bytes  # noqa: F401
