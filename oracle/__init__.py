"""Plain CPU oracle for LVSA frame-block-sparse attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it.  It shares no code with the
HIP/C++ library under ``block_sparse_attention_lvsa_amd/``: no kernels,
headers, helpers, tables or pre/post-processing.

Two parts, each written from the method's description on the pages:

* :mod:`oracle.mask` -- the per-step key-frame sets A_s(t) = G_s ∪ W(t)
  (rotating global anchors plus an expanded local window), emitted as CSR.
  Pure Python integer code.
* :mod:`oracle.attention` -- masked softmax attention in float64 over the
  frame-block mask, plus a brute-force token-level form for tiny inputs.

Sources (cited by page title and section throughout):

* gist.science explainer "LVSA: Training-Free Sparse Attention for Long Video
  Diffusion", Technical Summary §2 (Methodology: Core Mechanism, Complexity);
  the same text exists in German and Arabic on the same site.
* TechWalker article on LVSA ("华为巴黎研究院让AI视频'不再原地打转'…"),
  §二 (core design: budget C, anchor spacing Tper, window extension) and
  §三 (rotating anchors).

Parity status: every function here is pinned by tests under ``tests/``
(``-m "not gpu"``).  The mask's behaviour beyond the invariants the pages
state (exact Tper rounding, window growth order, tie-break) rests on stated
readings; those readings are pinned by hand-worked examples and by an
independent sort-based definition, not by values printed on the pages (the
pages print none).
"""

from .mask import (  # noqa: F401
    ROT_MOD_TPER,
    ROT_MOD_T,
    FIXED_GRID,
    WINDOW_ONLY,
    MaskInfo,
    validate,
    schedule,
    anchors,
    key_frames,
    build_mask,
)
from .attention import (  # noqa: F401
    default_scale,
    block_attention,
    block_attention_rows,
    token_mask_attention,
)
