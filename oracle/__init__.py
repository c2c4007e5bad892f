"""CPU oracle for the OScaR INT2 KV-cache path -- TEST INFRASTRUCTURE ONLY.

A plain, slow, float64 numpy implementation of what the GPU path computes:
the key quantizer (Hadamard rotation, per-token L2 scaling with an fp16 norm,
per-channel asymmetric INT2 over 128-token groups), the per-token value
quantizer, 2-bit packing, and single-query attention over the packed cache,
plus plain attention over bf16 keys/values.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library never calls it and
shares no code with it; the only module both sides use is ``synthetic``,
which generates seeded inputs and holds none of the method's arithmetic.

Sources: the OScaR abstract (arXiv 2605.19660, fugumt.com record, "Abstract")
and the ai-papers.net OScaR summary (section "OScaRの提案手法", Fig. 4).
Points the pages leave open (Hadamard order and normalisation, the INT2
formula, rounding, degenerate cases, the packed layout) follow the readings
listed in each module's docstring.

Pins: every function here is checked in ``tests/test_oracle_*.py`` against
something other than itself (scipy's Hadamard routine, brute-force searches,
closed forms, invariants).  Nothing here is "parity unpinned".
"""
from .fp16 import fp16_rne, fp16_bits, FP16_MAX  # noqa: F401
from .hadamard import hadamard  # noqa: F401
from .quantize import (  # noqa: F401
    rotate_keys, token_norms, scale_tokens, key_group_params, key_codes,
    quantize_keys, value_params, value_codes, quantize_values,
)
from .pack import pack_k_codes, unpack_k_codes, pack_v_codes, unpack_v_codes  # noqa: F401
from .attention import (  # noqa: F401
    dequant_keys_rotated, dequant_values, decode_slice, decode_bf16_slice,
    softmax_state, merge_states,
)
from .cache import quantize_slice, OracleSlice  # noqa: F401
