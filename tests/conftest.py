import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


# Tests run against the test build of the library (libsiglip_test.so: the
# product library plus the stage-capture and workspace-poisoning hooks of
# include/siglip_test_hooks.h); checks of the product build load
# libsiglip.so explicitly by path.
import vision_transformer_so400m_amd as _V  # noqa: E402

_V.use_test_hooks()


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs a real MI355X (gfx950) and the built HIP library")
    config.addinivalue_line(
        "markers", "slow: long CPU oracle runs (still part of the default suite)")
