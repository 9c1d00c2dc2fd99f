import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU test")


def pytest_collection_modifyitems(config, items):
    # GPU tests need a device; without one they are skipped, never silently
    # rerouted to a CPU path.
    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        has_gpu = False
    if has_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)


@pytest.fixture(scope="session")
def model32():
    """The 32-block, hidden-4096 model shared by the 384^2, 1024^2 and 2048^2
    workloads (same widths, depth and seeds), uploaded once per session:
    {"dims", "model" (device), "blocks" (host bf16 bits per block), "shared"}."""
    import concurrent.futures as cf

    import block_causal_attention_qi_amd as qi
    import qi_synth as qs
    from tests.gpu_util import log
    wl = qs.workload(4)
    log("generating 32 blocks of bf16 weights")
    with cf.ThreadPoolExecutor(16) as ex:
        blocks = list(ex.map(lambda b: qs.block_weights(wl, b, as_bf16=True, threads=1), range(wl.n_blocks)))
    shared = qs.shared_weights(wl, as_bf16=True)
    dims = qi.make_dims(wl.hidden, wl.ffn, wl.n_blocks, wl.txt_dim)
    model = qi.DeviceModel(dims, shared, blocks)
    log("weights on device")
    return {"dims": dims, "model": model, "blocks": blocks, "shared": shared}
