"""One rank's share captured in a HIP graph and replayed.

The three entry points only launch kernels (the state reset is a fill
kernel, not a memset node), so a caller can capture a share once and replay
it.  Every replay is checked bit for bit against the same share run eagerly
on twin buffers, with unrelated eager GPU work and synchronizations between
the replays.
"""
import pytest
import torch

from error_compensated_bit_amd import binding as B
from error_compensated_bit_amd import sim
from error_compensated_bit_amd.inputs import WORKLOADS, make_x

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def same(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.view(torch.uint8), b.view(torch.uint8))


@pytest.mark.parametrize("state_dtype", [B.ECHO_STATE_F32, B.ECHO_STATE_BF16])
def test_graph_replays_match_eager_calls(state_dtype):
    w = WORKLOADS["chain56_p4_512x1024"]
    P, n = w.P, w.n
    cfg = B.make_config(state_dtype=state_dtype)
    xs = [make_x(w, 0, p, device=DEV) for p in range(P)]
    rg = sim.alloc_ranks(cfg, P, n, DEV)
    re = sim.alloc_ranks(cfg, P, n, DEV)
    sim.allreduce(cfg, rg, xs)
    sim.allreduce(cfg, re, xs)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sim.share(cfg, rg, 1, xs[1], stream=torch.cuda.current_stream())
    for replay in range(4):
        g.replay()
        noise = torch.randn(1 << 20, device=DEV).sum()     # unrelated eager work in between
        sim.share(cfg, re, 1, xs[1])
        torch.cuda.synchronize()
        assert torch.isfinite(noise)
        assert same(rg.state[1], re.state[1]), f"state differs after replay {replay}"
        assert same(rg.out, re.out), f"output differs after replay {replay}"
        assert same(rg.owned[1].codes, re.owned[1].codes) and same(rg.owned[1].params, re.owned[1].params)
        for o in range(P):
            if o != 1:
                assert same(rg.sent[1][o].codes, re.sent[1][o].codes)
                assert same(rg.sent[1][o].params, re.sent[1][o].params)


def test_prepared_calls_match_plain_calls_eager_and_captured():
    """The pre-marshalled calls the benchmark times give the same bytes as
    the plain binding calls, run eagerly and replayed from a HIP graph."""
    w = WORKLOADS["single_p2_256k"]
    P, n = w.P, w.n
    cfg = B.make_config()
    xs = [make_x(w, 0, p, device=DEV) for p in range(P)]
    rs = [sim.alloc_ranks(cfg, P, n, DEV) for _ in range(3)]
    for r in rs:
        sim.allreduce(cfg, r, xs)
    torch.cuda.synchronize()

    def prepared(r, st):
        inp = [None if p == 0 else r.sent[p][0] for p in range(P)]
        return (B.prepare_quantize_feedback(cfg, P, 0, n, xs[0], r.state[0], r.sent[0], st),
                B.prepare_owner_reduce_requant(cfg, P, 0, n, xs[0], r.state[0], inp, r.owned[0], st),
                B.prepare_dequant_gather(cfg, P, n, r.owned, r.out, st))

    eager = prepared(rs[1], None)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for k in prepared(rs[2], torch.cuda.current_stream()):
            k()
    for call in range(3):
        sim.share(cfg, rs[0], 0, xs[0])
        for k in eager:
            k()
        g.replay()
        torch.cuda.synchronize()
        for r in rs[1:]:
            assert same(r.state[0], rs[0].state[0]), f"state differs, call {call}"
            assert same(r.out, rs[0].out), f"output differs, call {call}"
            assert same(r.owned[0].codes, rs[0].owned[0].codes)
            assert same(r.sent[0][1].codes, rs[0].sent[0][1].codes)
