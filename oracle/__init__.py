"""CPU oracle (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It shares no code with the GPU library and imports
nothing from it; the GPU library never imports it.
"""
from .kvc_oracle import *  # noqa: F401,F403
from .kvc_oracle import __all__  # noqa: F401
