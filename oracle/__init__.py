"""CPU oracle for the Hadamard rotate + quantize path (TEST INFRASTRUCTURE ONLY).

Plain, slow, obviously correct numpy code in float64 that computes what the
GPU library computes, from the definitions on the pages:

* the rotation is the explicit dense product y = x . R with R built as a
  matrix (Sylvester Hadamard, block-diagonal Hadamard, or a Kronecker product
  of a Paley base matrix and a Sylvester matrix), normalised to be orthogonal;
* the quantizers (round-to-nearest integer groups, MXFP4, NVFP4) are
  evaluated element by element with numpy's round-half-to-even.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  It shares no code with the HIP library and
never imports it; the product path must not route through it.

Parity status of each function is stated in its docstring.  Two choices
are readings where the pages leave the matter open, each pinned to what the
mathematics and the public formats fix.  The Paley base matrices used for
widths that are not a power of two are this project's own construction,
because the pages' table of known matrices is not available.  They are
pinned to H_K . H_K^T = K I with +-1 entries, and to the Paley closed form
(bordered circulant of the quadratic character for prime K - 1).  Another
Hadamard matrix of the same order would be an equally valid rotation with
different outputs.  NVFP4 is named on the pages without its encoding.  Its
reading (module text of ``quant``) is pinned to the public format through
PyTorch's float8_e4m3fn conversion, E4M3 closed forms and hand-derived
cases.
"""
from .hadamard import (  # noqa: F401
    kron_factor,
    mixing_matrices,
    paley_hadamard,
    rotate,
    rotate_mixed,
    rotate_out,
    rotation_matrix,
    sylvester,
)
from .quant import (  # noqa: F401
    E2M1_VALUES,
    QuantResult,
    bf16_round,
    dequant_int,
    dequant_mxfp4,
    dequant_nvfp4,
    e2m1_round,
    e4m3_decode,
    e4m3_encode,
    fp32_round,
    mxfp4_quant,
    nvfp4_quant,
    pack_nibbles,
    round_scale,
    rtn_codes,
    rtn_quant,
    unpack_nibbles,
)
