"""Host logic of the AdamWSR optimizer (CPU only; no kernel runs here):
global positions (base_index) as running numel in parameter order, rejected
options, and a state_dict round trip that keeps the f32 moment states f32
for bf16 parameters (torch's loader would cast them to the param dtype)."""

import pytest
import torch

from adamw_optimizer_stochastic_amd import AdamWSR


def test_base_index_is_running_numel_in_group_order():
    a = torch.nn.Parameter(torch.zeros(3, 5))
    b = torch.nn.Parameter(torch.zeros(7))
    c = torch.nn.Parameter(torch.zeros(2, 2))
    opt = AdamWSR([{"params": [a, b]}, {"params": [c], "lr": 1e-4}])
    assert [opt.base_index(p) for p in (a, b, c)] == [0, 15, 22]
    d = torch.nn.Parameter(torch.zeros(11))
    opt.add_param_group({"params": [d]})
    assert opt.base_index(d) == 26 and opt.base_index(a) == 0


@pytest.mark.parametrize("kw", [dict(amsgrad=True), dict(maximize=True), dict(foreach=True),
                                dict(fused=True), dict(capturable=True)])
def test_unsupported_options_raise(kw):
    with pytest.raises(NotImplementedError):
        AdamWSR([torch.nn.Parameter(torch.zeros(4))], **kw)


@pytest.mark.parametrize("kw", [dict(lr=-1.0), dict(eps=-1e-8), dict(betas=(1.0, 0.9)),
                                dict(weight_decay=-0.1), dict(seed=-1), dict(seed=1 << 32),
                                dict(rounding="rz")])
def test_bad_values_raise(kw):
    with pytest.raises(ValueError):
        AdamWSR([torch.nn.Parameter(torch.zeros(4))], **kw)


def test_unsupported_param_dtypes():
    for dt in (torch.float16, torch.float64, torch.complex64):
        with pytest.raises(NotImplementedError):
            AdamWSR([torch.nn.Parameter(torch.zeros(4, dtype=dt))])


def test_state_dict_round_trip_keeps_f32_states():
    m = torch.nn.Linear(4, 3).to(torch.bfloat16)
    opt = AdamWSR(m.parameters(), seed=9, weight_decay=0.05)
    torch.manual_seed(0)
    for p in m.parameters():
        opt.state[p] = {"step": torch.tensor(3.0), "exp_avg": torch.randn(p.shape),
                        "exp_avg_sq": torch.rand(p.shape)}
    sd = opt.state_dict()
    m2 = torch.nn.Linear(4, 3).to(torch.bfloat16)
    opt2 = AdamWSR(m2.parameters())
    opt2.load_state_dict(sd)
    assert opt2.seed == 9 and opt2.param_groups[0]["weight_decay"] == 0.05
    for p2, p in zip(m2.parameters(), m.parameters()):
        s2, s = opt2.state[p2], opt.state[p]
        assert s2["exp_avg"].dtype == torch.float32
        assert torch.equal(s2["exp_avg"], s["exp_avg"])
        assert torch.equal(s2["exp_avg_sq"], s["exp_avg_sq"])
        assert float(s2["step"]) == 3.0


def test_check_disjoint():
    from adamw_optimizer_stochastic_amd.ops import check_disjoint
    check_disjoint([(0, 16, "a"), (16, 16, "b"), (64, 0, "empty"), (40, 8, "c")])
    check_disjoint([(100, 0, "x"), (100, 4, "y")])          # empty ranges never overlap
    with pytest.raises(ValueError, match="b.*c|c.*b"):
        check_disjoint([(0, 16, "a"), (32, 16, "b"), (47, 4, "c")])   # one byte shared
    with pytest.raises(ValueError):
        check_disjoint([(8, 8, "inner"), (0, 32, "outer")])  # nested
    with pytest.raises(ValueError):
        check_disjoint([(0, 8, "p"), (0, 8, "p again")])     # identical


def test_step_count_passes_2pow24(monkeypatch):
    """The step count is an integer: past 2**24 (where a float32 count stops
    moving) each step still passes its own t, so the key (seed, t) changes
    from step to step ("adamw-sr" page, Method: keyed by (seed, step))."""
    from adamw_optimizer_stochastic_amd import optim as optim_mod
    seen = []
    monkeypatch.setattr(optim_mod.ops, "adamw_step",
                        lambda *a, **kw: seen.append(kw["step"]))
    p = torch.nn.Parameter(torch.zeros(6, dtype=torch.bfloat16))
    p.grad = torch.ones(6, dtype=torch.bfloat16)
    opt = AdamWSR([p])
    monkeypatch.setattr(opt, "_workspace", lambda device, numels: None)
    opt.state[p] = {"step": torch.tensor((1 << 24) - 1, dtype=torch.int64),
                    "exp_avg": torch.zeros(6), "exp_avg_sq": torch.zeros(6)}
    opt.step()
    opt.step()
    opt.step()
    assert seen == [1 << 24, (1 << 24) + 1, (1 << 24) + 2]
    # a state dict keeps the count exactly, above 2**24
    p2 = torch.nn.Parameter(torch.zeros(6, dtype=torch.bfloat16))
    opt2 = AdamWSR([p2])
    opt2.load_state_dict(opt.state_dict())
    assert int(opt2.state[p2]["step"]) == (1 << 24) + 2
    assert opt2.state[p2]["step"].dtype == torch.int64
    # and a count saved by torch's AdamW (a float32 tensor) loads as an int
    sd = opt.state_dict()
    sd["state"][0]["step"] = torch.tensor(5.0)
    opt2.load_state_dict(sd)
    assert int(opt2.state[p2]["step"]) == 5


def test_moment_states_are_views_of_flat_buffers():
    """AdamWSR's f32 moment states of the parameters that get their state
    together are views into one buffer per moment, 256-byte aligned, zero,
    in the parameters' shapes; a later parameter gets buffers of its own."""
    ps = [torch.nn.Parameter(torch.zeros(s, dtype=torch.bfloat16)) for s in ((3, 5), (7,), (64,))]
    late = torch.nn.Parameter(torch.zeros(9))
    opt = AdamWSR(ps + [late])
    opt._init_states(ps)
    for key in ("exp_avg", "exp_avg_sq"):
        ts = [opt.state[p][key] for p in ps]
        assert len({t.untyped_storage().data_ptr() for t in ts}) == 1
        assert [t.shape for t in ts] == [p.shape for p in ps]
        assert all(t.dtype == torch.float32 and not t.any() for t in ts)
        assert all(t.storage_offset() % 64 == 0 for t in ts)
        assert [t.storage_offset() for t in ts] == [0, 64, 128]
    assert opt.state[ps[0]]["exp_avg"].untyped_storage().data_ptr() != \
        opt.state[ps[0]]["exp_avg_sq"].untyped_storage().data_ptr()
    assert len(opt.state[late]) == 0
    opt._init_states([late] + ps)          # only the parameter without state gets one
    assert opt.state[late]["exp_avg"].untyped_storage().data_ptr() != \
        opt.state[ps[0]]["exp_avg"].untyped_storage().data_ptr()
    assert int(opt.state[late]["step"]) == 0
