"""The Python binding rejects tensors whose shape, dtype, layout or device does
not match the call before any pointer reaches the C ABI (CPU tensors: no GPU is
touched). Status codes follow include/cpla.h: 1 invalid, 2 shape, 3 dtype."""
import pytest
import torch

import context_state_passing_amd as cpla
from context_state_passing_amd import api
from context_state_passing_amd._lib import CplaError

B, T, H, DK, DV = 1, 128, 2, 64, 128


def _la(**over):
    bf = torch.bfloat16
    t = dict(q=torch.zeros(B, T, H, DK, dtype=bf), k=torch.zeros(B, T, H, DK, dtype=bf),
             v=torch.zeros(B, T, H, DV, dtype=bf), g=torch.zeros(B, T, H, DK))
    t.update(over)
    return t


def _status(fn, *a, **kw):
    with pytest.raises(CplaError) as e:
        fn(*a, **kw)
    return e.value.status, e.value.message


@pytest.mark.parametrize("over,status", [
    (dict(k=torch.zeros(B, T + 1, H, DK, dtype=torch.bfloat16)), 2),     # k longer than q
    (dict(v=torch.zeros(B, T, H + 1, DV, dtype=torch.bfloat16)), 2),     # more heads in v
    (dict(k=torch.zeros(B, T, H, DK)), 3),                               # k fp32, q bf16
    (dict(g=torch.zeros(B, T, H, DK, dtype=torch.bfloat16)), 3),         # g must be fp32
    (dict(g=torch.zeros(B, T, H, DK + 1)), 2),                           # per-key-dim g of the wrong width
    (dict(q=torch.zeros(B, T, H, DK, dtype=torch.float16),
          k=torch.zeros(B, T, H, DK, dtype=torch.float16)), 3),          # fp16 unsupported
    (dict(v=torch.zeros(B, T, H, 2 * DV, dtype=torch.bfloat16)[..., ::2]), 1),   # strided v
])
def test_forward_rejects_mismatched_inputs(over, status):
    t = _la(**over)
    st, _ = _status(cpla.forward, t["q"], t["k"], t["v"], t["g"], num_shards=2)
    assert st == status


def test_forward_rejects_optional_tensors():
    t = _la()
    assert _status(cpla.forward, t["q"], t["k"], t["v"], t["g"], num_shards=2,
                   initial_state=torch.zeros(B, H, DV, DK))[0] == 2
    assert _status(cpla.forward, t["q"], t["k"], t["v"], None, num_shards=2,
                   w=torch.zeros(B, T, H, dtype=torch.float64))[0] == 3
    assert _status(cpla.forward, t["q"], t["k"], t["v"], t["g"], num_shards=2,
                   out=torch.zeros(B, T, H, DK, dtype=torch.bfloat16))[0] == 2


def test_forward_rejects_host_tensors():
    t = _la()
    st, msg = _status(cpla.forward, t["q"], t["k"], t["v"], t["g"], num_shards=2)
    assert st == 1 and "GPU" in msg


def test_backward_rejects_mismatched_dO():
    t = _la()
    ctx = api.Context(problem=None, decay=2, q=t["q"], k=t["k"], v=t["v"], g=t["g"], packed=None,
                      fwd_summary=None, shard_in_state=None, final_state=None,
                      chunk_states=torch.zeros(1), has_initial_state=False)
    assert _status(cpla.backward, torch.zeros(B, T, H, DK, dtype=torch.bfloat16), ctx)[0] == 2
    assert _status(cpla.backward, torch.zeros(B, T, H, DV), ctx)[0] == 3
    assert _status(cpla.backward, torch.zeros(B, T, H, DV, dtype=torch.bfloat16), ctx,
                   d_final_state=torch.zeros(B, H, DK, DK))[0] == 2


def test_ssd_and_delta_reject_mismatched_inputs():
    bf = torch.bfloat16
    x, dt, A = torch.zeros(1, 64, 4, 64, dtype=bf), torch.zeros(1, 64, 4), torch.zeros(4)
    Bm, Cm = torch.zeros(1, 64, 2, 128, dtype=bf), torch.zeros(1, 64, 2, 128, dtype=bf)
    assert _status(cpla.ssd_forward, x, dt, torch.zeros(3), Bm, Cm, num_shards=1)[0] == 2
    assert _status(cpla.ssd_forward, x, dt, A, Bm, Cm.float(), num_shards=1)[0] == 3
    assert _status(cpla.ssd_forward, x, dt, A, Bm, Cm, num_shards=1,
                   initial_state=torch.zeros(1, 4, 64, 128))[0] == 2
    st, msg = _status(cpla.ssd_forward, x, dt, A, Bm, Cm, num_shards=1)
    assert st == 1 and "GPU" in msg
    q = torch.zeros(1, 64, 2, 32)
    g, beta = torch.zeros(1, 64, 2), torch.zeros(1, 64, 2)
    assert _status(cpla.delta_forward, q, q, q, g, beta.double(), num_shards=1)[0] == 3
    assert _status(cpla.delta_forward, q, q, q, g, torch.zeros(1, 63, 2), num_shards=1)[0] == 2


def test_grouped_qk_heads_shapes():
    """q and k may have fewer heads than v (a divisor of H: groups of heads share
    them); the problem then carries qk_heads, and the shapes are checked as such."""
    bf = torch.bfloat16
    q1, k1 = torch.zeros(B, T, 1, DK, dtype=bf), torch.zeros(B, T, 1, DK, dtype=bf)
    v, g = torch.zeros(B, T, H, DV, dtype=bf), torch.zeros(B, T, H)
    p = api.make_problem(q1, v, 2, 1)
    assert (p.H, p.qk_heads, p.dk, p.dv) == (H, 1, DK, DV)
    assert api.make_problem(torch.zeros(B, T, H, DK, dtype=bf), v, 2, 1).qk_heads == 0   # one per head
    # accepted shapes reach the device check (host tensors)
    st, msg = _status(cpla.forward, q1, k1, v, g, num_shards=2)
    assert st == 1 and "GPU" in msg
    # k with other heads than q, q heads not dividing v's, g per q/k head
    assert _status(cpla.forward, q1, torch.zeros(B, T, H, DK, dtype=bf), v, g, num_shards=2)[0] == 2
    v3 = torch.zeros(B, T, 3, DV, dtype=bf)
    assert _status(cpla.forward, torch.zeros(B, T, 2, DK, dtype=bf), torch.zeros(B, T, 2, DK, dtype=bf), v3,
                   torch.zeros(B, T, 3), num_shards=2)[0] == 2
    assert _status(cpla.forward, q1, k1, v, torch.zeros(B, T, 1), num_shards=2)[0] == 2
    # the autograd adapter returns per-head gradients, so it takes q and k per head
    assert _status(cpla.chunkwise_linear_attention, q1, k1, v, g, None, num_shards=2)[0] == 2
