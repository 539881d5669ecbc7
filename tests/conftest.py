import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library, loaded; the test session fails loudly if it is missing."""
    import torch
    from kv_cache_decode_quest_amd import quest
    if not torch.cuda.is_available():
        pytest.fail("gpu test selected but no GPU is visible")
    quest.load()
    return quest
