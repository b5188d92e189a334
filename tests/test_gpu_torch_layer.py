"""The autograd bridge (HEALayer): loss.backward() through the fused adjoint pass gives
the oracle's gradient; stale saved states are refused."""
import numpy as np
import pytest

import hqml_inputs
import oracle
from gpu_util import assert_e_close, assert_grad_close, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.mark.parametrize("n,L,B,compute,ent", [(5, 3, 4, "fp32", "cz"), (16, 3, 3, "fp32", "cz"),
                                               (16, 2, 2, "fp64", "cz"), (6, 3, 2, "fp32", "cnot"),
                                               (15, 3, 2, "fp32", "cnot")])
def test_layer_backward_matches_oracle(n, L, B, compute, ent):
    from qml_gradients_amd.torch_layer import HEALayer
    x, th, y = hqml_inputs.make_inputs(n, L, B, seed=1400 + n)
    say(f"[gpu] HEALayer n={n} L={L} {compute} {ent}")
    layer = HEALayer(n, L, B, compute=compute, theta=torch.from_numpy(th), entangler=ent)
    dt = layer.theta.dtype
    X = torch.from_numpy(x).cuda().to(dt)
    Y = torch.from_numpy(y).cuda().to(dt)
    e = layer(X)
    loss = torch.mean((e - Y) ** 2)
    loss.backward()
    e_ref, loss_ref, g_ref = oracle.train_step(x, th, y, entangler=1 if ent == "cnot" else 0)
    g = layer.theta.grad.cpu().numpy()
    if compute == "fp64":
        assert np.max(np.abs(e.detach().cpu().numpy() - e_ref)) <= 1e-10
        assert np.max(np.abs(g - g_ref)) <= 1e-10
    else:
        assert_e_close(e.detach().cpu().numpy(), e_ref, n, L)
        assert_grad_close(g, g_ref)


def test_layer_refuses_stale_saved_states():
    from qml_gradients_amd.torch_layer import HEALayer
    n, L, B = 14, 2, 2
    x, th, _ = hqml_inputs.make_inputs(n, L, B, seed=5)
    layer = HEALayer(n, L, B, theta=torch.from_numpy(th))
    X = torch.from_numpy(x).cuda()
    e1 = layer(X)
    layer(X)          # a second forward replaces the saved states
    with pytest.raises(RuntimeError):
        e1.sum().backward()
