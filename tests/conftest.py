import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def golden():
    import json

    def load(name):
        with open(os.path.join(GOLDEN, name)) as f:
            return json.load(f)

    return load


@pytest.fixture(scope="session", autouse=True)
def _every_batch_passes_the_metadata_check():
    """Every batch a test builds through the workload generators goes through
    pa_check_batch (the calls' device-side preconditions, on the host) before
    any kernel sees it."""
    from paged_kv_cache_103_amd import _lib as pa
    from paged_kv_cache_103_amd import workloads as W

    if not os.path.exists(pa.LIB_PATH):
        yield
        return
    finish, mla = W._finish_batch, W.make_mla_batch

    def checked_finish(*args, **kw):
        b = finish(*args, **kw)
        pa.check_batch(b.block_table, b.context_lens, b.num_blocks, b.max_context_len, b.cu_seqlens, b.max_q_len,
                       b.sliding_window, b.slot_mapping)
        return b

    def checked_mla(*args, **kw):
        b = mla(*args, **kw)
        pa.check_batch(b.block_table, b.context_lens, int(b.cache.shape[0]), b.max_context_len)
        return b

    W._finish_batch, W.make_mla_batch = checked_finish, checked_mla
    yield
    W._finish_batch, W.make_mla_batch = finish, mla
