"""CPU oracle for exact attention (float64, S and P materialised).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the library or its Python binding.
It shares no code with the HIP path.

  reference  the plain definition (the oracle proper)
  online     the pages' streaming (m, l, u) recurrence and block merge,
             an independent cross-check of the definition
  brute      pure-Python loops for tiny shapes, another cross-check
"""
from .reference import (attention, attention_block_sparse, attention_grad,  # noqa: F401
                        attention_rows, attention_varlen, decode, decode_paged, head_attention,
                        head_attention_grad, f32_scale)
from . import online, brute  # noqa: F401
