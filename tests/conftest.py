import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
for p in (ROOT, ROOT / "tests"):
    if str(p) not in sys.path:
        sys.path.insert(0, str(p))


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def orc():
    import oracle
    return oracle.get()


@pytest.fixture
def option():
    """set(name, value) for the library's kernel-choice options, undone after the test."""
    import paged_gqa_attention_attn_amd as pa
    saved = {}

    def set_(name, value):
        prev = pa.set_option(name, int(value))
        saved.setdefault(name, prev)

    yield set_
    for name, prev in saved.items():
        pa.set_option(name, prev)
