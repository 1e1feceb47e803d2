import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def pytest_terminal_summary(terminalreporter):
    """After GPU parity runs: the worst raw output error per output dtype and
    the worst state error of the session, with the test that produced each
    (every comparison also prints its own figures to stderr)."""
    try:
        from tests import parity
    except Exception:
        return
    recs = parity.RECORDS
    if not recs:
        return
    tr = terminalreporter
    tr.section("parity against the oracle (worst of the session)")
    kinds = sorted({(r["kind"], r["dtype"]) for r in recs if r["kind"] != "state"})
    for kind, dt in kinds:
        outs = [r for r in recs if r["kind"] == kind and r["dtype"] == dt]
        w = max(outs, key=lambda r: r["raw"])
        a = max(outs, key=lambda r: r["asserted"])
        tr.write_line(f"{kind}s, {dt}, {len(outs)} comparisons: raw max abs error {w['raw']:.3e} ({w['test']}); "
                      f"beyond the output format's rounding {max(r['beyond_rounding'] for r in outs):.3e}; "
                      f"asserted {a['asserted']:.3e} ({a['test']})")
    sts = [r for r in recs if r["kind"] == "state"]
    if sts:
        w = max(sts, key=lambda r: r["rel"])
        tr.write_line(f"states, {len(sts)} comparisons: max-norm relative error {w['rel']:.3e} ({w['test']})")
