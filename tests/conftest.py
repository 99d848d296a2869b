import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    # The sanitizer check (test_host_sanitized.py) reruns the host ABI tests
    # in a child process against the ASan/UBSan build of the library.
    lib = os.environ.get("GPT_TEST_LIB")
    if lib:
        from decoder_only_gpt_amd import gpt
        gpt.LIB_PATH = lib


@pytest.fixture(scope="session")
def gpu_available():
    import torch
    return torch.cuda.is_available()
