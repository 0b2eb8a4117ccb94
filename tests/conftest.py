import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long CPU test")


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle
    oracle.lib()
    return oracle


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session", autouse=True)
def device_checks_clean():
    """With MOE_FFN_DEBUG set the library is the debug build: after the
    session, no device bounds check may have failed."""
    yield
    if os.environ.get("MOE_FFN_DEBUG", "0") in ("", "0") or not gpu_available():
        return
    import routed_expert_ffn_topk_amd as moe
    if moe._lib is None:
        return
    enabled, where = moe.moe_ffn_device_check()
    assert enabled, "MOE_FFN_DEBUG is set but the loaded library is not the debug build"
    assert where == 0, f"a device bounds check failed: file {where // 100000}, line {where % 100000}"
