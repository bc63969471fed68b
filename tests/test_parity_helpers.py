"""CPU checks of the parity helpers: the output-rounding allowance is half a
unit in the last place of the storage type, computed from the type's
significand width (bf16: 8 bits, fp32: 24 bits)."""
import numpy as np
import torch

import parity as P


def test_half_ulp_values():
    assert P.half_ulp(np.array([1.0]), "bf16")[0] == 2.0 ** -8
    assert P.half_ulp(np.array([1.5]), "bf16")[0] == 2.0 ** -8
    assert P.half_ulp(np.array([10.0]), "bf16")[0] == 2.0 ** -5
    assert P.half_ulp(np.array([-0.3]), "bf16")[0] == 2.0 ** -10  # 0.3 in [1/4, 1/2)
    assert P.half_ulp(np.array([1.0]), "fp32")[0] == 2.0 ** -24


def test_half_ulp_bounds_actual_bf16_rounding():
    # fp32 values rounded to bf16 (as the kernels store their fp32 results)
    x = (torch.randn(100000, dtype=torch.float32) * 10).double()
    r = x.float().to(torch.bfloat16).double()
    err = (x - r).abs().numpy()
    lim = P.half_ulp(np.maximum(np.abs(x.numpy()), np.abs(r.numpy())), "bf16")
    assert np.all(err <= lim)
    # and it is tight: some values round by nearly the whole half ulp
    assert np.max(err / lim) > 0.99


def test_out_error_only_forgives_rounding():
    ref = np.array([12.3456, -0.5, 3.0])
    got = torch.tensor(ref).to(torch.bfloat16).double().numpy()
    assert P.out_error(got, ref, "bf16") <= 0.0
    assert abs(P.out_error(got + np.array([0.0, 0.05, 0.0]), ref, "bf16") - (0.05 - 2.0 ** -9)) < 1e-12
