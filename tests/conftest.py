import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


@pytest.fixture
def kernel_override():
    """Setter for the library's kernel-choice override (testing hook);
    every knob set through it is reset to automatic when the test ends."""
    import tiled_attention_03_amd as ta
    used = []

    def set_(knob, value):
        ta.attn_set_kernel_override(knob, value)
        used.append(knob)

    yield set_
    for knob in used:
        ta.attn_set_kernel_override(knob, 0)
