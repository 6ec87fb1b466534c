import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


_POOL_STREAMS = []


@pytest.fixture(scope="session", autouse=True)
def _pool_streams_first(request):
    """The slot pool's compute stream waits in-stream for a word its copy stream writes, so the
    two must not share a hardware queue: the pool's streams are created together before any other
    stream of the session (the library's stated precondition; a framework's stream pool, created
    later by a graph capture for instance, would otherwise take queues round-robin beside them).
    Only when a GPU test is collected on a machine with a GPU."""
    if any(item.get_closest_marker("gpu") for item in request.session.items):
        import torch

        if torch.cuda.is_available():
            from mixture_experts_route_amd import native as N

            _POOL_STREAMS.extend([N.new_stream(), N.new_stream(), N.new_stream()])
    yield


@pytest.fixture(scope="session")
def pool_streams():
    """(compute, device->host copy, host->device copy) streams of the slot-pool tests."""
    if len(_POOL_STREAMS) != 3:
        pytest.skip("no GPU")
    return tuple(_POOL_STREAMS)
