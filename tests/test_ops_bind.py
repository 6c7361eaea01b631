"""Host logic of the bound calls in ops (no GPU): a bound call keeps the tensors of its scope,
runs the library function with the arguments marshalled once, checks the status and returns
the unbound call's result."""
import pytest
import torch

from rwkv_wkv_mixing_amd import _lib as L
from rwkv_wkv_mixing_amd import ops


def test_bound_call_runs_with_marshalled_args_and_returns_result():
    seen = []

    def fn(*args):
        seen.append(args)
        return 0

    t = torch.zeros(3)
    call = ops._launch(True, "wkv_forward", fn, (1, 2, None), "result", {"t": t, "pair": (t, None), "n": 5})
    assert isinstance(call, ops.BoundCall) and seen == []  # binding launches nothing
    assert call() == "result" and call() == "result"
    assert seen == [(1, 2, None), (1, 2, None)]
    assert any(x is t for x in call._keep)  # the scope's tensors stay alive with the call


def test_unbound_launch_checks_status():
    assert ops._launch(False, "wkv_forward", lambda *a: 0, (), 7, {}) == 7
    with pytest.raises(L.WkvError) as e:
        ops._launch(False, "wkv_forward", lambda *a: 1, (), 7, {})
    assert e.value.status == 1


def test_bound_call_checks_status_each_time():
    codes = iter([0, 1])
    call = ops._launch(True, "wkv_backward", lambda *a: next(codes), (), None, {})
    call()
    with pytest.raises(L.WkvError):
        call()
