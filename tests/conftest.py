import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter):
    """One line per output comparison against the oracle: tokens compared, how many of
    them were near-ties (ids not compared, outputs checked on the GPU's routing), and
    the worst error as a fraction of the 1e-2 x RMS tolerance."""
    helpers = sys.modules.get("parity_helpers")
    records = getattr(helpers, "RECORDS", None)
    if not records:
        return
    tr = terminalreporter
    tr.section("parity against the FP64 oracle")
    for test, tokens, near, worst in records:
        tr.write_line(f"{test}: {tokens} tokens compared, {near} near-ties, worst error / tolerance {worst:.3f}")
    tokens = sum(r[1] for r in records)
    near = sum(r[2] for r in records)
    tr.write_line(f"total: {len(records)} comparisons, {tokens} tokens, {near} near-ties checked on outputs, "
                  f"worst {max(r[3] for r in records):.3f}")
