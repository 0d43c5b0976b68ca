"""The fp64 oracle against its pins (CPU only).

See ``oracle_pins.py``: brute force on tiny inputs, hand-derived rational
examples, probability-row properties, constant V, key/value permutation,
the merge identity, the pages' tiled schedules (deferred vs per-step
division), closed forms (scale = 0, single visible key, N = 1), key-shift
invariance, the causal prefix property, huge separated scores, and
batch/head independence.  A cross-check against torch's float64 softmax is
the library special case.
"""

import numpy as np
import pytest
import torch

import oracle.exact_attention as ref
from oracle_pins import PINS


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_float64_softmax(causal):
    g = torch.Generator().manual_seed(5)
    B, H, N, d = 2, 2, 33, 16
    q, k, v = (torch.randn(B, H, N, d, generator=g, dtype=torch.float64) for _ in range(3))
    s = 0.25 * (q @ k.transpose(-1, -2))
    if causal:
        s = s.masked_fill(torch.triu(torch.ones(N, N, dtype=torch.bool), 1), float("-inf"))
    o_t = torch.softmax(s, dim=-1) @ v
    l_t = torch.logsumexp(s, dim=-1)
    o, lse = ref.attention_ref(q.numpy(), k.numpy(), v.numpy(), 0.25, causal)
    np.testing.assert_allclose(o, o_t.numpy(), atol=1e-13, rtol=0)
    np.testing.assert_allclose(lse, l_t.numpy(), atol=1e-13, rtol=0)


def test_bf16_inputs_upcast_exactly():
    g = torch.Generator().manual_seed(9)
    q, k, v = (torch.randn(1, 1, 20, 8, generator=g).to(torch.bfloat16) for _ in range(3))
    o1, l1 = ref.attention_ref(q.to(torch.float64).numpy(), k.to(torch.float64).numpy(),
                               v.to(torch.float64).numpy(), 0.5, True)
    o2, l2 = ref.attention_ref(q.float().numpy(), k.float().numpy(), v.float().numpy(), 0.5, True)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
