import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def built_lib():
    """Path of the HIP library, compiling it in-tree only if it is absent."""
    import qwen3_gqa_attention_amd as q3
    if not os.path.exists(q3.LIB_PATH):
        from qwen3_gqa_attention_amd.build import build
        build()
    return q3.LIB_PATH
