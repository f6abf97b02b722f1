"""The torch wrappers without a GPU: host tensors are refused before any
pointer reaches the library (the library dereferences every pointer on the
GPU, so a host pointer would fault there; there is no CPU path)."""
import pytest
import torch

from mla_tree_verify_amd import _lib, api

Q, H, P = 9, 64, 40
N = P + Q


def host_case():
    bf = torch.bfloat16
    return (torch.zeros(Q, H, 512, dtype=bf), torch.zeros(Q, H, 64, dtype=bf), torch.zeros(N, 512, dtype=bf),
            torch.zeros(N, 64, dtype=bf), torch.full((Q,), -1, dtype=torch.int32))


def test_single_sequence_refuses_host_tensors():
    qn, qr, lat, rope, par = host_case()
    with pytest.raises(ValueError, match="GPU"):
        api.mla_verify(qn, qr, lat, rope, par, P, 0.07)


def test_batched_refuses_host_tensors():
    qn, qr, lat, rope, par = host_case()
    offs = torch.tensor([0, N], dtype=torch.int64)
    with pytest.raises(ValueError, match="GPU"):
        api.mla_verify_batched(qn[None], qr[None], lat, rope, par[None], offs, 0.07)


def test_paged_refuses_host_tensors():
    qn, qr, lat, rope, par = host_case()
    idx = torch.arange(N, dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU"):
        api.mla_verify_paged(qn, qr, lat, rope, idx, par, 0.07)


def test_partials_refuses_host_tensors():
    qn, qr, lat, rope, par = host_case()
    plan = _lib.Plan(2, 32, 32, 0, 0)
    with pytest.raises(ValueError, match="GPU"):
        api.mla_verify_partials(qn, qr, lat, rope, par, P, 0.07, plan)


def test_combine_refuses_host_tensors():
    with pytest.raises(ValueError, match="GPU"):
        api.combine(torch.zeros(2, 64, 512), torch.zeros(2, 64))


def test_non_tensor_inputs_are_type_errors():
    with pytest.raises(TypeError):
        api.mla_verify([0.0], None, None, None, None, P, 0.07)
