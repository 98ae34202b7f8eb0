"""fp64 CPU oracle for the LongFlow decode step (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg use this
package; the library never imports it.
"""

from .longflow_oracle import (attend_pair, bf16_bits_to_f64, decode_step, decode_step_fill, evict_topk,
                              write_slot)

from . import stack_oracle  # noqa: E402  (multi-layer decode step around the operator)

__all__ = ["stack_oracle", "attend_pair", "bf16_bits_to_f64", "decode_step", "decode_step_fill", "evict_topk", "write_slot"]
