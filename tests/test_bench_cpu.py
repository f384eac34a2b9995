"""Host-side pieces of bench.py that need no GPU."""
import importlib.util
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_kernel_source_hash_covers_every_source_file():
    """The hash that ties committed counter runs to the kernel sources reads
    every file under csrc, subdirectories included, and is stable."""
    b = _bench()
    h1 = b.kernel_source_hash()
    assert len(h1) == 16 and h1 == b.kernel_source_hash()


def test_measured_traffic_unknown_key_is_none():
    assert _bench().measured_traffic("no such kernel") is None
