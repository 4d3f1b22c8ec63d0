import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: full-size case")


def parse_golden(name):
    """Rows of a tests/golden/*.txt fixture: '#' starts a comment; columns are split on
    runs of whitespace for 2-column files or on '|' for block files."""
    rows = []
    with open(os.path.join(ROOT, "tests", "golden", name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append(line)
    return rows


@pytest.fixture(scope="session")
def gpu():
    """The built library on a visible GPU; GPU tests skip on machines without one."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import glu_activation_microscaling_amd as glu
    if not os.path.exists(glu.LIB_PATH):
        from glu_activation_microscaling_amd import build
        build.build()
    glu.lib()
    return glu


def bits(t):
    """torch bfloat16 tensor (any device) -> numpy uint16 bit patterns."""
    import numpy as np
    import torch
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def u8(t):
    return t.detach().cpu().contiguous().numpy()
