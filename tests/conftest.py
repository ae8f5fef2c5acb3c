import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter):
    """Worst parity figures per tensor kind of the GPU checks that ran:
    rel-Frobenius against 1e-2 and max|gpu-ref|/rms against 3e-2 (the plain
    figure, also where a weight-gradient block's floor applied)."""
    mod = sys.modules.get("tests._gpu")
    recs = getattr(mod, "RECORDS", None)
    if not recs:
        return
    kinds = {}
    for kind, label, rel, mxr, floor in recs:
        k = kinds.setdefault(kind, [0, 0.0, "", 0.0, "", set()])
        k[0] += 1
        if rel >= k[1]:
            k[1], k[2] = rel, label
        if mxr >= k[3]:
            k[3], k[4] = mxr, label
        k[5].add(floor)
    tr = terminalreporter
    tr.write_sep("-", "parity figures (worst per kind; bar: rel <= 1e-2, max-abs/rms <= 3e-2)")
    for kind in sorted(kinds):
        n, rel, _, mxr, mxl, floors = kinds[kind]
        fl = ",".join(sorted(f for f in floors if f != "none")) or "none"
        tr.write_line(f"{kind:22s} n={n:4d} rel {rel:.2e} max/rms {mxr:.2e} floor={fl} [{mxl[:40]}]")
