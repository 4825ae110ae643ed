"""CPU oracle of the RAWINT4 routed-expert LoRA layer.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the CPU-baseline leg of ``bench.py``, never by the product package.
"""

from .oracle import *  # noqa: F401,F403
