import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter):
    """One line per parity comparison the GPU tests recorded (output error,
    tokens accepted under another valid L2-input decision, L2-input code
    flips at decision boundaries)."""
    try:
        from tests.helpers import PARITY
    except Exception:                                    # pragma: no cover
        return
    if not PARITY:
        return
    terminalreporter.section("parity figures")
    for case, st in PARITY:
        parts = []
        for k, v in st.items():
            parts.append(f"{k}={v:.3e}" if isinstance(v, float) else f"{k}={v}")
        terminalreporter.write_line(f"{case}: " + " ".join(parts))
