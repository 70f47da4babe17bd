import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_sessionstart(session):
    """Refuse to test a library built from sources other than this tree's."""
    import video_world_model_amd.qwm as Q
    if os.path.exists(Q.LIB_PATH):
        try:
            Q.check_build()
        except RuntimeError as e:
            pytest.exit(str(e), returncode=3)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")
