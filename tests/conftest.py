import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle

    oracle.lib()  # fails loudly if the oracle is not built
    return oracle


def pytest_terminal_summary(terminalreporter):
    """Scale-mismatch and one-code rates of the fused casts against the
    oracle, per workload, direction and layout (also under -q)."""
    from helpers import PARITY_RATES

    if not PARITY_RATES:
        return
    tr = terminalreporter
    tr.write_sep("-", "fused-cast parity rates against the oracle")
    tr.write_line(f"{'workload':44s} {'dir':4s} {'layout':6s} {'blocks':>10s} {'scale mism.':>11s} "
                  f"{'rate':>9s} {'one-code rate':>13s}")
    rows = []
    for (cfg, direction, lay), st in sorted(PARITY_RATES.items()):
        tr.write_line(f"{cfg:44s} {direction:4s} {lay:6s} {st.blocks:10d} {st.scale_mismatch:11d} "
                      f"{st.scale_mismatch_rate:9.2e} {st.one_code_rate:13.2e}")
        rows.append({"workload": cfg, "direction": direction, "layout": lay, **st.record()})
    path = os.environ.get("MXFP8_PARITY_RATES")
    if path:
        with open(path, "w") as f:
            json.dump(rows, f, indent=1)
