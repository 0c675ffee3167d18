"""CPU oracle of the tensor-autograd hot path -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The product path (the HIP library and its Python binding) never
calls it, and the two share no code: the oracle is written from the pages'
definitions in plain numpy, in float64 unless a pin asks for the pages' own
float32 arithmetic.

Sources, cited by short tag in every module:

  [Autograd-1]  arabroot.io, "Build a language model in C# from scratch (1):
                the Autograd engine"
  [GPT2-4]      arabroot.io, "Build a language model in C# from scratch (4):
                running the GPT-2 weights"
  [ChainRule]   nextadmin.net, "Chain rule and automatic differentiation:
                Autograd from scratch"

Modules:
  ops        forward and backward rule of every tensor op (plain definitions)
  engine     Tensor + tape: record on forward, reverse topological replay
  scalar     scalar reverse mode (Value) and forward mode (Dual)
  gradcheck  central-difference gradient check with the pages' error measure
  optim      SGD and AdamW
  models     the MLP, char-MLP and GPT compositions of the ops
  decode     KV-cached single-token step and top-k/temperature sampling

Parity status: every function here is pinned by a test in tests/test_oracle_*.py
(closed forms, printed values of the pages, brute force or finite differences);
none is "parity unpinned".
"""
