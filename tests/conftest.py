import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU case")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def lib():
    """The built HIP library (fails loudly when it is missing)."""
    from query_aware_prefill_amd import binding
    return binding.load()


@pytest.fixture(autouse=True)
def _context_debug_counters(request, monkeypatch):
    """Every context a GPU test creates through DeviceModel.context is checked
    after the test: no KV-pool guard region overwritten and no token id
    outside the vocabulary met (quail_ctx_check)."""
    if request.node.get_closest_marker("gpu") is None:
        yield
        return
    from query_aware_prefill_amd import binding as B
    from query_aware_prefill_amd.device import DeviceModel
    made = []
    orig = DeviceModel.context

    def context(self, *a, **kw):
        ctx = orig(self, *a, **kw)
        made.append(ctx)
        return ctx

    monkeypatch.setattr(DeviceModel, "context", context)
    yield
    for ctx in made:
        chk = B.quail_ctx_check(ctx)
        # a test that plants a bad token id or a guard overwrite says so
        want = getattr(ctx, "expect_counts", {"guard_errors": 0, "bad_tokens": 0})
        assert chk == want, (chk, want)
