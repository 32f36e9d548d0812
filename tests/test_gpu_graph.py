"""The decode step under HIP graph capture: every call of the step enqueues kernels
(and, with one split, a device-to-device copy) on the caller's stream and nothing
else -- no allocation, memset or synchronisation -- so a captured step replays.
Each replay, with eager work on the same buffers between replays, must reproduce
the eager step's output bit for bit (the step is idempotent: the append rewrites the
same decode row)."""
import dataclasses

import pytest

import mla_latent_kv_dkv_amd as M
from mla_latent_kv_dkv_amd import inputs as I
from mla_latent_kv_dkv_amd.harness import DeviceWorkload
from tests.gpu_util import note

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.mark.parametrize("name,splits", [("full", 4), ("full", 1), ("lite-fp8", 8)])
def test_decode_step_replays_from_a_hip_graph(name, splits):
    w = dataclasses.replace(I.WORKLOADS[name], batch=8, context=1000, num_splits=splits)
    note(f"graph replay {name} S={splits}")
    M.load()
    dw = DeviceWorkload(w)
    dw.step()
    torch.cuda.synchronize()
    ref = dw.u.clone()
    # warm-up on a side stream, then capture one step
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dw.step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dw.step()
    torch.cuda.synchronize()
    for i in range(3):
        dw.u.fill_(123.0)             # eager work on the output between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(dw.u, ref), f"replay {i} differs from the eager step"
    assert M.mla_device_error() == 0
