"""CPU oracle for the BaKron solver. TEST INFRASTRUCTURE ONLY: only tests/,
__graft_entry__.smoke() and bench.py's cpu_baseline leg may import it."""
from .bakron_oracle import *  # noqa: F401,F403
from .bakron_oracle import (SCALE_COL, SCALE_NONE, SCALE_ROW, Alphabet, Result,  # noqa: F401
                            ReplayReport)
