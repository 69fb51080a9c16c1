"""CPU oracle for the hybrid global-attention path (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import this package. The HIP library and its Python
binding never import it and share no code with it.
"""

from .zebra_oracle import *  # noqa: F401,F403
from .zebra_oracle import __all__  # noqa: F401
