"""Test infrastructure: a plain CPU oracle for the centroid-masked sparse head.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may import this package.  The product path never does.
"""

from .masked_head import *  # noqa: F401,F403
from .draft import *  # noqa: F401,F403
from .fp8_slabs import *  # noqa: F401,F403
