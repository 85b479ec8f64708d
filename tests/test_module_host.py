"""Host-side pieces of the DilatedAttention module that run on the CPU: the
projection autograd function (split-K weight gradients, accumulated input
gradient) against torch's own autograd through nn.Linear, in float64."""
import pytest
import torch

from sparse_long_sequence_attn_amd.module import DilatedAttention, _project


@pytest.mark.parametrize("R", [65536, 1000, 2048 * 32])
@pytest.mark.parametrize("biases", [(True, False, True), (False,)])
def test_projection_gradients_match_torch(R, biases):
    torch.manual_seed(R)
    ls = [torch.nn.Linear(64, 48, bias=b).double() for b in biases]
    x = torch.randn(4, R // 4, 64, dtype=torch.float64)
    x1, x2 = x.clone().requires_grad_(), x.clone().requires_grad_()
    ys = _project(x1, ls)
    sum((y * (i + 1)).sum() for i, y in enumerate(ys)).backward()
    got = [l.weight.grad.clone() for l in ls] + [l.bias.grad.clone() for l in ls if l.bias is not None]
    for l in ls:
        l.zero_grad()
    sum((l(x2) * (i + 1)).sum() for i, l in enumerate(ls)).backward()
    ref = [l.weight.grad for l in ls] + [l.bias.grad for l in ls if l.bias is not None]
    for a, b in zip(got + [x1.grad], ref + [x2.grad]):
        assert float((a - b).abs().max() / b.abs().max()) < 1e-13


def test_module_config_validation():
    with pytest.raises(ValueError):
        DilatedAttention(500, 8, 2, 64)
    with pytest.raises(ValueError):
        DilatedAttention(512, 8, [2, 4], [64])
    m = DilatedAttention(512, 8, [1, 2], [2048, 4096], qk_norm=True)
    assert m.patterns == ((2048, 1), (4096, 2))
