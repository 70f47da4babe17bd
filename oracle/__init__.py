"""CPU oracle of the QuantWM quantized KV-cache hot path.

TEST INFRASTRUCTURE ONLY: imported by the tests, by ``__graft_entry__.smoke``
and by the bench's CPU-baseline leg, never by the product path.
"""

from .qwm_oracle import *  # noqa: F401,F403
from . import qwm_oracle  # noqa: F401
