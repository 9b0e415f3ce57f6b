import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Headroom of every GPU-vs-oracle comparison made through tests.gpu_path.errors():
    max-abs and relative Frobenius error against the 2e-3 / 1e-3 bars."""
    mod = sys.modules.get("tests.gpu_path")
    margins = getattr(mod, "MARGINS", None) if mod else None
    if not margins:
        return
    tr = terminalreporter
    tr.write_sep("-", "parity margins (bars: max_abs 2e-3, rel_fro 1e-3)")
    worst = {}
    for name, ma, rf in margins:
        w = worst.get(name)
        worst[name] = (max(ma, w[0]), max(rf, w[1])) if w else (ma, rf)
    for name, (ma, rf) in sorted(worst.items(), key=lambda kv: -kv[1][0] / 2e-3):
        tr.write_line(f"{ma:9.3e} ({100 * ma / 2e-3:5.1f}%)  {rf:9.3e} ({100 * rf / 1e-3:5.1f}%)  {name}")
    ma = max(v[0] for v in worst.values())
    rf = max(v[1] for v in worst.values())
    tr.write_line(f"worst: max_abs {ma:.3e} ({100 * ma / 2e-3:.1f}% of bar), rel_fro {rf:.3e} "
                  f"({100 * rf / 1e-3:.1f}% of bar) over {len(margins)} comparisons")
