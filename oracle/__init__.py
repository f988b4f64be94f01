"""CPU oracle for the OCTOPUS KV-cache codec and the attention that reads it.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library, its
Python binding, the kernels) may import, call, link or execute anything under
this directory.  Only the tests, the smoke check and the bench's CPU-baseline
leg use it.

The oracle is plain, slow and written in float64 NumPy, one step of the method
at a time, in the order and notation of the OCTOPUS paper
("OCTOPUS: Optimized KV Cache for Transformers via Octahedral Parametrization
Under optimal Squared error quantization", arXiv 2605.21226), with the
attention step written as the textbook definition of softmax attention.  It
shares no code, tables or constants with the HIP path: the only things both
sides see are the seeded inputs, the codebook artifact (an input to the codec,
like a weight file) and the bytes of the packed cache.

Modules
  splitmix      SplitMix64 counter generator -> sign vectors s, s'
  rotation      normalized Sylvester Hadamard H, R = H D_s, R' = H D_s'
  octahedral    octahedral encode (Eq. 5) / decode (Eq. 6)
  codebook      Monte-Carlo Lloyd-Max codebook training (Sec. 3.4)
  encode        the full encoder (Sec. 3.1-3.6, App. A summary) with margins
  pack          bit packing of the index streams and the 64-token tile layout
  attention     decode attention and chunk attention on a packed cache
  densities     the analytic marginals printed in the paper (Eq. 3, 4, f_xi)

Parity status of each function is stated in its docstring; every function
here is pinned by a CPU test (tests/test_oracle_*.py).  The pins are listed in
each test module's header.
"""
