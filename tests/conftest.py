import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")


def pytest_terminal_summary(terminalreporter):
    """The measured lse errors of the GPU parity checks, against their bound."""
    gu = sys.modules.get("gpu_util")
    if gu is None or not gu.LSE_ERRORS:
        return
    errs = sorted(gu.LSE_ERRORS, key=lambda t: -t[1])
    tot = len(errs)
    terminalreporter.write_line(f"lse vs oracle: {tot} checks, max |err| {errs[0][1]:.3e} ({errs[0][0]}), "
                                f"median {errs[tot // 2][1]:.3e}, bound {gu.LSE_ABS:.3e}")
