"""Oracle for the fused attention forward-mode derivative (JVP).

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  This package is a plain, slow, float64
CPU statement of what the GPU library computes.  Only the test suite, the smoke
check and the benchmark's CPU-baseline leg may import it; the library and its
Python binding never do, and it imports nothing from them.

Sources (the page "带分数正则的一致性蒸馏", gitcode.csdn.net, section 注意力):

* ``attention_jvp``  -- the dense definition: the attention formula of the
  subsection 普通注意力的实现, the chain rule for the output tangent given in the
  prose that follows it, and the log-sum-exp the 前向 kernel stores.
* ``streaming``      -- the pages' streaming recurrence for the same quantities
  (online max m, sum s, extra state r, A, B), written from the prose.
* ``masks``          -- the chunked frame window with anchor frames of the page
  "VDN-Minimax-H3 ... Stage A1" (yfxerp.com), used by the long-video workload.
* ``trigflow``       -- the TrigFlow <-> rectified-flow coefficients of the
  section 时间步转换 of the first page.
* ``merge``          -- the combination of results over disjoint key sets
  (derived from the definition; not on the pages).
* ``backward``       -- the primal gradients dQ, dK, dV from the saved
  log-sum-exp (subsection 反向).

Every function is pinned by the ``-m "not gpu"`` tests in ``tests/``.
"""

from .attention_jvp import attention_jvp, attention_jvp_rows
from .backward import attention_backward
from .masks import FrameWindow, frame_window_visible
from .merge import merge_partials
from .streaming import attention_jvp_streaming
from . import trigflow

__all__ = [
    "attention_backward",
    "attention_jvp",
    "attention_jvp_rows",
    "attention_jvp_streaming",
    "FrameWindow",
    "frame_window_visible",
    "merge_partials",
    "trigflow",
]
