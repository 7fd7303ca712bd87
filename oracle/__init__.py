"""Plain, slow CPU oracle of the sparse MoE decode path, in fp64, written
twice: as plain C++ loops (cpp/*.cpp, loaded through cpp_oracle.py) and as
numpy (formats.py, moe.py, lmhead.py).

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the CPU
baseline leg of bench.py may import or call anything here; the product path
(the HIP library and its Python binding) never does, and this package never
imports the product path.  It shares no code with the GPU kernels: the number
formats, the router, softmax and top-k, the SwiGLU experts, the combine, the
RMSNorm stack and the LM head are each written out from their definitions,
once in each language.  The two implementations share no arithmetic either:
the C++ one has its own decoders and loops, and takes from Python only the
layer containers and the margin-conditioned input picking (inputs.py).

Each function cites the passage of the pages it follows; where the pages are
silent the reading taken is stated in the function's module docstring.
Every function is pinned by tests/test_oracle_*.py against closed forms,
brute force over tiny inputs, hand-worked examples (tests/golden/) and
invariants, so a slip in the oracle fails a test that does not use the oracle
to compute its expected value.
"""
from . import formats, lmhead, moe  # noqa: F401
