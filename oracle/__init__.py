"""CPU oracle for absorbed-MLA decode and the latent-cache append.

This package is TEST INFRASTRUCTURE. Only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import it.
The HIP library and its Python binding never import, call or link anything
here, and nothing here imports them.

Everything is plain float64 numpy written straight from the method's
definition (naive MLA: decompress per-head keys and values, then ordinary
softmax attention), so a reader can check it against the pages by eye.

Parity status of each public function (what pins it is listed in
``tests/test_oracle_pins.py``):

* ``decode_naive``           pinned (associativity, brute force, special cases)
* ``decode_absorbed``        pinned (equals ``decode_naive`` to 1e-12 relative,
                             and the pure-Python brute force)
* ``output_rows``            pinned (head-block selector, brute force, the
                             merged W_O W_UV form of the same product)
* ``round_to_bf16``          pinned (vs torch.bfloat16 on binary32 inputs, ties)
* ``append_rows``            pinned (brute force, RMSNorm / RoPE invariants)
* ``query_rows``             pinned (head-block layout, query/key relative
                             position, norm scale invariance, full rank)
* ``rmsnorm``, ``rope``      pinned (closed-form invariants, complex form)
* ``slot_index``, ``gather_sequence``  pinned (brute force, permutation)
* ``e4m3fn_decode`` / ``e4m3fn_encode`` / ``quantize_rows_fp8``
                             pinned (format definition vs torch.float8_e4m3fn)
* ``bf16_bits_to_f64``       pinned (vs torch.bfloat16)
* ``sizes.*``                pinned (figures printed on the pages)
"""

from .mla_ref import (  # noqa: F401
    bf16_bits_to_f64,
    rmsnorm,
    rope,
    append_rows,
    query_rows,
    slot_index,
    gather_sequence,
    decode_naive,
    decode_absorbed,
    output_rows,
    default_softmax_scale,
    round_to_bf16,
)
from .fp8 import (  # noqa: F401
    E4M3FN_MAX,
    e4m3fn_decode,
    e4m3fn_encode,
    quantize_rows_fp8,
    dequantize_rows_fp8,
)
from . import sizes  # noqa: F401
