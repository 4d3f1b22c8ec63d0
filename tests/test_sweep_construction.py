"""Host checks of the exhaustive sweep construction used by the GPU quantizer tests."""
import numpy as np

import oracle
import synthetic_inputs as si
from sweep_inputs import mxfp8_sweep_matrix


def test_sweep_matrix_covers_every_value_and_scale():
    """The construction above (host-only): every scale byte 0..247 occurs as an oracle block
    scale, and every finite BF16 magnitude occurs."""
    X = mxfp8_sweep_matrix()
    s = oracle.quant_mxfp8(si.from_bits(X).float().numpy(), oracle.ROWWISE)[1]
    assert set(range(248)) <= set(np.unique(s).tolist())
    assert np.unique(X & 0x7FFF).size == 0x7F80
