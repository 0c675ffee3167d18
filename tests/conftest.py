import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
for _p in (ROOT, os.path.join(ROOT, "tests")):
    if _p not in sys.path:
        sys.path.insert(0, _p)


def gpu_available():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: oracle work of more than a few seconds")


@pytest.fixture(scope="session")
def golden():
    import json

    def load(name):
        with open(os.path.join(ROOT, "tests", "golden", name)) as f:
            return json.load(f)
    return load


@pytest.fixture(scope="module")
def ctx():
    """A library context with a 4 GiB arena on cuda:0 (fp32 contractions)."""
    if not gpu_available():
        pytest.skip("no GPU")
    import transformer_fwd_bwd_amd as T
    c = T.Context(arena_bytes=4 << 30, precision="fp32")
    yield c
    c.close()


@pytest.fixture
def own_ctx():
    """A context of its own for one test (4 GiB arena, closed after it): released
    leaves give back their gradient and bf16 buffers only when their context
    closes, so tests with operands of hundreds of MB do not share one."""
    if not gpu_available():
        pytest.skip("no GPU")
    import transformer_fwd_bwd_amd as T
    c = T.Context(arena_bytes=4 << 30, precision="fp32")
    yield c
    c.close()


def pytest_terminal_summary(terminalreporter):
    """Achieved parity errors of this session's GPU comparisons, as fractions of
    their tolerance (1.0 = at the gate): per test its worst L2 and worst
    element-wise figure, tightest last, then the overall worst."""
    try:
        from parity import RESULTS
    except Exception:
        return
    if not RESULTS:
        return
    per = {}
    for test, what, l2, el in RESULTS:
        w = per.setdefault(test, [0.0, "", 0.0, "", 0])
        w[4] += 1
        if l2 >= w[0]:
            w[0], w[1] = l2, what
        if el >= w[2]:
            w[2], w[3] = el, what
    tr = terminalreporter
    tr.write_line("")
    tr.write_line(f"parity headroom: {len(RESULTS)} checks in {len(per)} tests "
                  "(error / tolerance; L2 = relative L2 gate, elem = element-wise gate)")
    for test, (l2, w2, el, we, n) in sorted(per.items(), key=lambda kv: max(kv[1][0], kv[1][2])):
        name = test.split("::", 1)[-1]
        tr.write_line(f"  {max(l2, el):6.3f}  L2 {l2:6.3f} elem {el:6.3f}  n={n:<4d} {name}  [{we if el >= l2 else w2}]")
    worst_l2 = max(RESULTS, key=lambda r: r[2])
    worst_el = max(RESULTS, key=lambda r: r[3])
    tr.write_line(f"parity worst: L2 {worst_l2[2]:.3f} of tol ({worst_l2[0].split('::', 1)[-1]}: {worst_l2[1]}); "
                  f"elem {worst_el[3]:.3f} of tol ({worst_el[0].split('::', 1)[-1]}: {worst_el[1]})")
