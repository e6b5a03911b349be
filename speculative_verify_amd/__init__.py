"""libgdn for MI355X: Gated DeltaNet speculative verify, GPU-resident commit and
chunked prefill as hand-written HIP kernels behind a C ABI (include/gdn.h).

``speculative_verify_amd.gdn`` is the Python binding (it loads libgdn.so and
fails if it is missing); ``speculative_verify_amd.inputs`` is the seeded input
recipe; ``speculative_verify_amd.build`` compiles the library.
"""
__all__ = ["gdn", "inputs", "build"]
