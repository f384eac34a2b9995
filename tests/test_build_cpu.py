"""Host-side checks of the build script: every source file that the
per-file instruction-scheduling table names exists (a renamed file would
otherwise fall back to the default strategy without notice), and only those
files get the extra flags."""
import os

from state_space_sequence_exp_amd import build as b


def test_sched_table_names_existing_sources():
    srcs = set(os.listdir(b.CSRC))
    for name, strategy in b.SCHED.items():
        assert name in srcs, name
        assert name.endswith(".hip")
        assert b.file_flags(os.path.join(b.CSRC, name)) == [
            "-mllvm", "-amdgpu-sched-strategy=" + strategy]


def test_other_sources_take_default_flags():
    for name in os.listdir(b.CSRC):
        if name.endswith(".hip") and name not in b.SCHED:
            assert b.file_flags(os.path.join(b.CSRC, name)) == []
