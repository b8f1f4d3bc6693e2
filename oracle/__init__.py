"""CPU oracle of the LaCT layer: test infrastructure, never part of the product path.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.
"""
from .lact_oracle import *  # noqa: F401,F403
from .lact_oracle import Hyper, MUON_COEFFS  # noqa: F401
from . import lact_backward  # noqa: F401,E402
from .lact_backward import lact_chunked_backward, chunked_backward_pair  # noqa: F401,E402
from . import lact_block  # noqa: F401,E402
from .lact_block import window_attention, block_forward  # noqa: F401,E402
