"""Plain, slow, fp64 CPU oracle for low-bit KV-cache append and decode attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
leg of the bench may import this package.  The HIP library never calls it and
shares no code, table or constant generator with it.

Modules:
  numerics    round-to-nearest-even into bf16 / fp16 / fp32 (fp64 arithmetic)
  e2m1        the E2M1 (FP4) value set, nearest-value encode, decode
  lloyd_max   Lloyd-Max scalar quantiser for a Gaussian source
  rotation    Haar rotation from a Gaussian matrix (sign-fixed QR), QJL matrix
  formats     encoders/decoders of every cache format into packed bytes
  attention   single-query decode attention over a packed cache (the definition)
  bytes       bytes stored per token for each format

Every function cites the page and section it follows.  Where the pages leave a
step open, the reading taken is stated next to the code.
"""
