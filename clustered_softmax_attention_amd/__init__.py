"""MuSe (Multipole Semantic Attention) forward and backward passes for AMD MI355X (gfx950).

The computation lives in hand-written HIP kernels behind the C ABI of
``libmuse.so`` (declared in ``include/muse.h``); ``binding`` marshals torch
tensors into those calls. See ``binding.attn_fwd``, ``binding.attn_bwd`` and
``binding.exact_attn_fwd``.
"""

from .binding import (MuseError, attn_bwd, attn_fwd, attn_fwd_plain, bwd_workspace_bytes,  # noqa: F401
                      exact_attn_fwd, load, workspace_bytes)
