"""The committed tile loop of the wide fp16 forward (csrc/fwd_wide_loop.inc) is
exactly what csrc/gen_wide_loop.py writes, so an edit to the generator cannot
reach the library without the loop being regenerated (CPU only)."""
import importlib.util
import os

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "tree_masked_decode_amd", "csrc")


def test_committed_loop_is_the_generators_output(monkeypatch):
    # the generator's look-ahead depths are tunable through the environment;
    # the committed loop uses the defaults
    monkeypatch.delenv("TA_AHEAD_A", raising=False)
    monkeypatch.delenv("TA_AHEAD_B", raising=False)
    spec = importlib.util.spec_from_file_location(
        "gen_wide_loop_under_test", os.path.join(CSRC, "gen_wide_loop.py"))
    gen = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(gen)
    with open(os.path.join(CSRC, "fwd_wide_loop.inc")) as f:
        committed = f.read()
    assert gen.render() == committed
