import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload; minutes on the CPU oracle")


def pytest_sessionstart(session):
    # The tests load the in-tree library; compile it only when none has been built.
    lib = os.path.join(ROOT, "gpt_lm_step_amd", "libgpt.so")
    if not os.path.exists(lib):
        from gpt_lm_step_amd import build
        build.build()
