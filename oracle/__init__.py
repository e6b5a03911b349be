"""fp64 CPU oracle of the gated delta rule -- test infrastructure only.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It shares no code with the HIP library.  See
``gdn_oracle.c`` for the definition it follows.
"""
from .gdn_oracle import (  # noqa: F401
    build,
    lib_path,
    num_threads,
    set_num_threads,
    gdn_seq,
    verify,
    commit,
    prefill_seq,
    prefill_chunked,
)
from . import accept_oracle  # noqa: F401,E402  (acceptance and rewind, numpy fp64)
from . import attn_oracle  # noqa: F401,E402  (full-attention verify, numpy fp64)
from . import mixer_oracle  # noqa: F401,E402  (GDN mixer prologue/epilogue, numpy fp64)
