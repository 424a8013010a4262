"""CPU oracle of the DFlash2 draft -> select -> verify step.

TEST INFRASTRUCTURE: imported only by tests/, __graft_entry__.smoke() and
bench.py's CPU-baseline leg.  The GPU library and its Python binding never
import it, and it shares no code with them."""
from .dflash2_oracle import *  # noqa: F401,F403
