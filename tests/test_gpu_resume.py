"""Checkpoint and resume of a chain of calls.

The only state Echo carries between calls is each rank's error state (the
short and long memories, [JP] 'Echoの仕組み②').  Copying it to the host after
call k, restoring it into freshly allocated buffers and continuing must give
results bit-identical to an uninterrupted chain.

[JP] = 'テンソル並列の通信を4bitに圧縮する「Echo」——誤差補償で精度を保ちながら
分散LLMを高速化する仕組み'.
"""
import pytest
import torch

from error_compensated_bit_amd import binding as B
from error_compensated_bit_amd import sim
from error_compensated_bit_amd.inputs import WORKLOADS, make_x

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("state_dtype", [B.ECHO_STATE_F32, B.ECHO_STATE_BF16])
def test_resume_from_host_checkpoint_is_bit_identical(state_dtype):
    w = WORKLOADS["chain56_p4_512x1024"]
    P, n = w.P, w.n
    cfg = B.make_config(state_dtype=state_dtype)
    sites, cut = 12, 5
    inputs = [[make_x(w, s, p, device=DEV) for p in range(P)] for s in range(sites)]
    ref = sim.alloc_ranks(cfg, P, n, DEV)
    ref_out = []
    for s in range(sites):
        sim.allreduce(cfg, ref, inputs[s])
        ref_out.append(ref.out.clone())
    a = sim.alloc_ranks(cfg, P, n, DEV)
    for s in range(cut):
        sim.allreduce(cfg, a, inputs[s])
    checkpoint = [t.cpu() for t in a.state]           # host copy after call `cut`
    del a
    torch.cuda.synchronize()
    b = sim.alloc_ranks(cfg, P, n, DEV)                # fresh buffers, reset state
    for p in range(P):
        b.state[p].copy_(checkpoint[p])
    for s in range(cut, sites):
        sim.allreduce(cfg, b, inputs[s])
        assert torch.equal(b.out.view(torch.int16), ref_out[s].view(torch.int16)), f"call {s}"
    for p in range(P):
        assert torch.equal(b.state[p].view(torch.uint8), ref.state[p].view(torch.uint8))
