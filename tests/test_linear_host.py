"""Host-side checks of the module-level helpers (no GPU): which layers the
8-bit replacement policy swaps, what the layer keeps before its first use,
that it refuses to run without a GPU instead of falling back, and the
threshold suggestion from given column statistics."""

import pytest
import torch

import int8_quantized_matmul_col_amd as mm


def _net():
    net = torch.nn.Sequential()
    net.add_module("small", torch.nn.Linear(64, 128))
    block = torch.nn.Sequential()
    block.add_module("q_proj", torch.nn.Linear(1024, 1024, bias=False))
    block.add_module("lm_head", torch.nn.Linear(1024, 32))
    net.add_module("block", block)
    net.add_module("f32", torch.nn.Linear(1024, 16))
    net.add_module("lm_head", torch.nn.Linear(16, 8))
    for name in ("small", "block", "lm_head"):
        getattr(net, name).half()
    return net


def test_replacement_policy_size_and_skip():
    net = mm.replace_linear_with_int8(_net(), threshold=5.0, min_in_features=600,
                                      skip_modules=("lm_head",))
    assert type(net.small) is torch.nn.Linear            # below the size threshold
    assert isinstance(net.block.q_proj, mm.Int8Linear)   # replaced
    assert type(net.block.lm_head) is torch.nn.Linear    # skipped by name at any depth
    assert type(net.f32) is torch.nn.Linear              # not float16: left alone
    assert type(net.lm_head) is torch.nn.Linear
    q = net.block.q_proj
    assert q.threshold == 5.0 and q.bias is None and not q.quantized
    assert q.in_features == 1024 and q.out_features == 1024


def test_replacement_skips_qualified_names():
    net = mm.replace_linear_with_int8(_net(), min_in_features=0, skip_modules=("block.q_proj",))
    assert type(net.block.q_proj) is torch.nn.Linear
    assert isinstance(net.block.lm_head, mm.Int8Linear)  # the default skip list is replaced
    assert isinstance(net.small, mm.Int8Linear)


def test_from_linear_copies_weight_and_bias():
    lin = torch.nn.Linear(32, 48).half()
    m = mm.Int8Linear.from_linear(lin, threshold=6.0)
    assert torch.equal(m.weight, lin.weight) and torch.equal(m.bias, lin.bias)
    assert m.Wq is None and m.w_scale is None
    with pytest.raises(TypeError):
        mm.Int8Linear.from_linear(torch.nn.Linear(4, 4))  # float32 layer
    with pytest.raises(ValueError):
        mm.Int8Linear(4, 4, threshold=-1.0)


def test_forward_refuses_to_run_on_the_host():
    m = mm.Int8Linear.from_linear(torch.nn.Linear(32, 48).half())
    with pytest.raises(RuntimeError, match="GPU"):
        m(torch.zeros(2, 32, dtype=torch.float16))
    with pytest.raises(TypeError):
        m(torch.zeros(2, 32))
    with pytest.raises(ValueError):
        m(torch.zeros(2, 31, dtype=torch.float16))


def test_suggest_threshold_from_stats():
    stats = {"K": 1000, "n_outliers": {4.0: 40, 5.0: 11, 6.0: 10, 7.0: 3, 8.0: 0, 10.0: 0,
                                       16.0: 0}}
    assert mm.suggest_threshold(stats=stats, max_fp16_fraction=0.01) == 6.0
    assert mm.suggest_threshold(stats=stats, max_fp16_fraction=0.05) == 4.0
    assert mm.suggest_threshold(stats=stats, max_fp16_fraction=0.0) == 8.0
    stats["n_outliers"] = {t: 999 for t in stats["n_outliers"]}
    assert mm.suggest_threshold(stats=stats, max_fp16_fraction=0.01) == float("inf")
    with pytest.raises(ValueError):
        mm.suggest_threshold(stats={"K": 10, "n_outliers": {}}, candidates=(6.0,))


def test_state_dict_of_a_prepared_layer_loads_without_requantizing():
    # a prepared layer's state (fabricated here: preparing needs a GPU)
    q = {"Wq": torch.arange(512 * 128, dtype=torch.int32).remainder(255).sub(127)
               .to(torch.int8).reshape(512, 128),
         "w_scale": torch.linspace(0.1, 1.0, 300),
         "bias": torch.full((300,), 0.5, dtype=torch.float16)}
    m = mm.Int8Linear(70, 300)
    assert sorted(m.state_dict()) == ["bias", "weight"]
    m.load_state_dict(q)
    assert m.quantized and m.weight is None
    assert torch.equal(m.Wq, q["Wq"]) and torch.equal(m.w_scale, q["w_scale"])
    assert sorted(m.state_dict()) == ["Wq", "bias", "w_scale"]
    m2 = mm.Int8Linear(70, 300)
    m2.load_state_dict(m.state_dict())
    assert m2.quantized and torch.equal(m2.Wq, m.Wq)
    # an fp16 state turns a prepared layer back into the fp16 form
    m2.load_state_dict(mm.Int8Linear(70, 300).state_dict())
    assert not m2.quantized and m2.weight.shape == (300, 70)
    # a prepared weight of the wrong shape is refused
    bad = dict(q, Wq=torch.zeros((256, 128), dtype=torch.int8))
    with pytest.raises(RuntimeError, match="Wq"):
        mm.Int8Linear(70, 300).load_state_dict(bad)
