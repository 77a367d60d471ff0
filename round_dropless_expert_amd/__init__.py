"""Multi-round dropless mixture-of-experts layer forward for AMD MI355X.

The layer routes each token to its top-k experts, then runs one or more
rounds of dispatch -> expert SwiGLU FFN -> collect, each with a fixed
per-expert token capacity C, and finally the weighted combine. Every step is
a HIP kernel for gfx950 in libmoe_rounds.so, reached through the C ABI of
include/moe_rounds.h; `binding` is its ctypes binding.

Importing the package loads nothing; `binding` loads the library (and raises
if it has not been built).
"""
__all__ = ["configs", "synth", "binding"]
