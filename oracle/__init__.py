"""CPU oracle for the OSCAR INT2 KV path.

Test infrastructure: only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import it.  It shares no code with the HIP
library and never imports it.
"""
from .oscar_oracle import *  # noqa: F401,F403
