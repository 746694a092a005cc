"""Host-only checks of the bench's probe library (no GPU needed): it loads,
exports the probes bench.py calls, and refuses malformed arguments before
any launch."""

import ctypes
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PATH = os.path.join(ROOT, "fp8_paged_kv_pa_amd", "libhbmprobe.so")

PROBES = ("hbm_read_probe", "hbm_block_probe", "launch_floor_probe", "start_spread_probe", "issue_rate_probe")

vp = ctypes.c_void_p


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(PATH):
        pytest.skip("probe library not built")
    lib = ctypes.CDLL(PATH)
    lib.hbm_read_probe.argtypes = [vp, ctypes.c_int64, vp, ctypes.c_int, vp, vp, vp]
    lib.hbm_block_probe.argtypes = [vp] * 5 + [ctypes.c_int, ctypes.c_int] + [vp] * 4
    lib.launch_floor_probe.argtypes = [vp, vp, ctypes.c_int, ctypes.c_int, vp, vp, vp]
    lib.start_spread_probe.argtypes = [vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp]
    lib.issue_rate_probe.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp, ctypes.c_int, vp]
    return lib


def test_exports(lib):
    for name in PROBES:
        assert ctypes.cast(getattr(lib, name), vp).value, name


FAKE = 0x1000  # never dereferenced: every call below is refused on the host


@pytest.mark.parametrize("call", [
    lambda l: l.hbm_read_probe(None, 1 << 20, FAKE, 256, None, None, None),
    lambda l: l.hbm_read_probe(FAKE, 1000, FAKE, 256, None, None, None),         # not a multiple of 16
    lambda l: l.hbm_read_probe(FAKE, 1 << 20, FAKE, 256, FAKE, None, None),      # one event of two
    lambda l: l.hbm_block_probe(FAKE, FAKE, FAKE, None, FAKE, 1, 1, FAKE, None, None, None),  # one scale array
    lambda l: l.hbm_block_probe(FAKE, FAKE, None, None, FAKE, 0, 1, FAKE, None, None, None),
    lambda l: l.launch_floor_probe(FAKE, FAKE, 1, 2048, None, None, None),
    lambda l: l.start_spread_probe(FAKE, 1, 256, 200 * 1024, None),              # LDS above 160 KiB
    lambda l: l.start_spread_probe(FAKE, 1, 32, 0, None),
    lambda l: l.issue_rate_probe(5, 16, 1, FAKE, FAKE, 1, None),                 # no kind 5
    lambda l: l.issue_rate_probe(4, 16, 1, FAKE, FAKE, 1, None),                 # kind 4 needs two waves per SIMD
    lambda l: l.issue_rate_probe(0, 16, 3, FAKE, FAKE, 1, None),
])
def test_refusals(lib, call):
    assert call(lib) == -1
