"""CPU oracle of the MuSe forward pass: TEST INFRASTRUCTURE, not part of the product.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or run anything in this package. The GPU library and its
Python binding never call it and share no code with it; the only module both
sides read is the seeded input generator in ``workloads/``.

Parity status of each function is listed in the header of ``muse_ref.py``.
"""

from .muse_ref import (  # noqa: F401
    KMeansResult,
    MuseResult,
    Summaries,
    bucket_order,
    cap_key_labels,
    default_scale,
    exact_attention,
    hierarchy_squares,
    lloyd_kmeans,
    lse_merge,
    muse_acausal,
    muse_causal,
    refine,
    retrieval_selection,
    squared_distances,
    tilted_summaries,
)
from .muse_bwd_ref import (  # noqa: F401
    exact_attention_bwd,
    muse_acausal_bwd,
    muse_causal_bwd,
)
