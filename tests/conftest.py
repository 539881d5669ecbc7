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


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """How many selection rows differed from the oracle's only by near-tied
    pages (each such request's output was checked against the oracle's
    attention over the GPU's own selection)."""
    parity = sys.modules.get("parity")
    if parity is None or not parity.FLAGGED["requests_checked"]:
        return
    f = parity.FLAGGED
    terminalreporter.write_line(
        f"quest parity: {f['requests_checked']} request outputs checked against the oracle; "
        f"{f['rows']} near-tie flagged selection rows in {f['requests']} requests, each "
        f"checked against the oracle's attention over the GPU's own selection")
