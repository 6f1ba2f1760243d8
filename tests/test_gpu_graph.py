"""A layer forward recorded as a HIP graph (MoELayer.capture): every replay
gives the eager forward's output bit for bit, with eager forwards of another
batch (on the same buffers) and host synchronisations between the replays, and
a new batch written into the graph's input buffer is picked up."""
import pytest
import torch

from tests.gpu_common import bf16_dev, inputs, layer, say

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


@pytest.mark.parametrize("cfg_id", [1, 2, 5, 4])
def test_graph_replay_matches_eager(cfg_id):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    inp = inputs(cfg_id)
    L = layer(cfg_id)
    x = bf16_dev(inp["x"])
    x2 = torch.flip(x, [0]).contiguous()  # another batch of the same shape
    say(f"graph replay workload {cfg_id} ({inp['cfg']['name']}) T={x.shape[0]}")
    ref1 = L.forward(x).clone()
    ref2 = L.forward(x2).clone()
    torch.cuda.synchronize()
    assert not torch.equal(_bits(ref1), _bits(ref2))
    xs = x.clone()
    g = L.capture(xs)
    torch.cuda.synchronize()
    for i in range(3):
        out = g.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(out), _bits(ref1)), f"replay {i} differs from the eager forward"
        e = L.forward(x2)
        torch.cuda.synchronize()
        assert torch.equal(_bits(e), _bits(ref2)), f"eager forward after replay {i} differs"
    xs.copy_(x2)
    out = g.replay()
    torch.cuda.synchronize()
    assert torch.equal(_bits(out), _bits(ref2)), "replay on a new batch"
    xs.copy_(x)
    out = g.replay()
    torch.cuda.synchronize()
    assert torch.equal(_bits(out), _bits(ref1)), "replay on the first batch again"
