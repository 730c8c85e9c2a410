"""The expert-FFN oracle against its pins (CPU only)."""
import pytest

from tests import pins


@pytest.mark.parametrize("pin", pins.FFN_PINS, ids=lambda f: f.__name__)
def test_ffn_pin(pin):
    pin()


def test_share_takes_torch_bf16_inputs():
    # the oracle is fed the same torch tensors as the GPU path
    import numpy as np
    import torch

    import oracle
    g = torch.Generator().manual_seed(0)
    x = torch.randn(7, 16, generator=g).to(torch.bfloat16)
    w13 = (torch.randn(3, 32, 16, generator=g) * 0.2).to(torch.bfloat16)
    w2 = (torch.randn(3, 16, 16, generator=g) * 0.2).to(torch.bfloat16)
    lg = torch.randn(7, 6, generator=g).to(torch.bfloat16)
    r = oracle.route(lg, 2, "bf16")
    a = oracle.moe_ffn_share(x, r.topk_idx, r.topk_w, w13, w2, "silu", 2)
    b = oracle.moe_ffn_share(x, r.topk_idx, r.topk_w, w13.double().numpy(), w2.double().numpy(),
                             "silu", 2)
    assert np.array_equal(a, b)
