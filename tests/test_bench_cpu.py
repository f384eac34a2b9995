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


def test_goals_report_sets_each_goal_beside_the_measurement():
    """The goals object carries the prefill MFMA goal with each measured
    workload's fraction and its ceiling at the HBM roofline (useful flops
    over the time its algorithmic bytes take at 8 TB/s: about 0.16, 0.48 and
    0.18 for the three prefill workloads), and the decode HBM goal."""
    import sys
    sys.path.insert(0, ROOT)
    from state_space_sequence_exp_amd import inputs as I
    b = _bench()
    names = [I.WORKLOADS[i].name for i in (1, 2, 3, 4)]
    line = {"roofline": {"mfma_frac": 0.03},
            "secondary": {names[1]: {"mfma_frac": 0.1}, names[2]: {"mfma_frac": 0.05},
                          names[3]: {"roofline": {"frac": 0.8}}}}
    g = b.goals_report(line)
    pre = g["prefill_bf16_mfma_frac"]
    assert pre["goal"] == 0.5
    assert pre["measured"] == {names[0]: 0.03, names[1]: 0.1, names[2]: 0.05}
    ceil = pre["ceiling_at_hbm_roofline"]
    assert abs(ceil[names[0]] - 0.16) < 0.01
    assert abs(ceil[names[1]] - 0.48) < 0.01
    assert abs(ceil[names[2]] - 0.18) < 0.01
    assert g["decode_hbm_frac"] == {"goal": 0.7, "measured": 0.8}
    # without the secondary workloads only the headline is reported
    only = b.goals_report({"roofline": {"mfma_frac": 0.03}})
    assert list(only) == ["prefill_bf16_mfma_frac"]
    assert list(only["prefill_bf16_mfma_frac"]["measured"]) == [names[0]]
