"""The bf16 rounding model of the LaCT kernels (tests/lact_rounding_model.py),
which sets the GPU tests' bar for the change a call makes, is checked here on
the CPU: with its roundings turned off it is the method itself (equal to the
oracle's chunk-matmul form, for every update rule and order), and with them on
it departs from the oracle by the bf16 floor (more than nothing, well under
the 2e-2 x RMS output bar)."""
import numpy as np
import pytest

import ttt_inputs as ti
from oracle import dense
from tests.lact_rounding_model import lact_head_bf16_model
from tests.parity import lact_change_errors

CASES = [
    dict(loss=0, order=0, rule=0), dict(loss=1, order=0, rule=0), dict(loss=0, order=1, rule=0),
    dict(loss=0, order=0, rule=1, beta=0.9), dict(loss=1, order=1, rule=2, beta=0.5, ns_steps=3,
                                                   lr=0.05),
    dict(loss=0, order=0, rule=2, beta=0.0, ns_steps=5, lr=0.02),
]


def _inputs(seed):
    inp = ti.gen_lact(1, 1, 96, 160, 32, 48, seed=seed, eta_scale=20.0)
    return [inp[n][0, 0] for n in ("q", "k", "v", "eta", "w1", "w2", "w3")]


@pytest.mark.parametrize("kw", CASES)
def test_model_without_rounding_is_the_method(kw):
    sub = _inputs(7)
    uses_m = kw["rule"] == 1 or (kw["rule"] == 2 and kw.get("beta", 0.0) != 0.0)
    m_a = [0.01 * np.ones_like(w, dtype=np.float64) for w in sub[4:]] if uses_m else None
    m_b = [a.copy() for a in m_a] if uses_m else None
    got = lact_head_bf16_model(*sub, chunk=64, m=m_a, exact=True, **kw)
    ref = dense.lact_head(*sub, chunk=64, m=m_b, **kw)
    for a, b in zip(got, ref):
        assert np.max(np.abs(a - b)) <= 1e-12 * max(1.0, np.max(np.abs(b)))
    if uses_m:
        for a, b in zip(m_a, m_b):
            assert np.max(np.abs(a - b)) <= 1e-12


@pytest.mark.parametrize("kw", CASES[:3])
def test_model_rounding_floor(kw):
    sub = _inputs(8)
    got = lact_head_bf16_model(*sub, chunk=64, **kw)
    ref = dense.lact_head(*sub, chunk=64, **kw)
    rms = np.sqrt(np.mean(ref[0] ** 2))
    err = np.max(np.abs(got[0] - ref[0])) / rms
    assert 1e-4 < err < 2e-2
    for i in (1, 2, 3):
        e = lact_change_errors(got[i], ref[i], sub[3 + i], output=False)
        assert 1e-4 < e < 0.1
