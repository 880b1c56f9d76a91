"""Plans (recorded call sequences, vitattn_plan_*) on the GPU: every launch
of a plan gives bitwise the output of the same vitattn_fwd calls made one by
one, replay after replay, with other work and synchronisations between the
replays; and the recorded calls read their inputs as they are at launch."""
import numpy as np
import pytest

import oracle
from gpu_util import LAYOUT_PACKED, LAYOUT_SEPARATE, assert_parity, bits_of, logical, to_device
from workloads import WORKLOADS, Workload, make_layer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def va():
    import vit_self_attention_amd
    return vit_self_attention_amd


def _inputs(wl, layers, dev, **sizes):
    lis = [make_layer(wl, layer, **sizes) for layer in range(layers)]
    calls = []
    for li in lis:
        ts = [to_device(a, dev) for a in li.in_layout(wl.layout)]
        calls.append(ts[0] if wl.layout == LAYOUT_PACKED else tuple(ts))
    return lis, calls


def _eager(va, wl, calls):
    outs = []
    for c in calls:
        q, k, v = (c, None, None) if wl.layout == LAYOUT_PACKED else c
        outs.append(va.fwd(q, k, v, scale=wl.scale))
    return outs


def _replays_match_eager(va, dev, wl, calls, plan, stream=None, replays=3):
    import torch
    ref = [bits_of(o) for o in _eager(va, wl, calls)]
    torch.cuda.synchronize(dev)
    other = _eager(va, wl, calls[:1])  # unrelated eager work between replays
    for r in range(replays):
        for o in plan.outs:
            o.zero_()
        if stream is None:
            plan.launch()
        else:
            with torch.cuda.stream(stream):
                plan.launch(stream)
            stream.synchronize()
        torch.cuda.synchronize(dev)
        for layer, (o, want) in enumerate(zip(plan.outs, ref)):
            assert np.array_equal(bits_of(o), want), f"replay {r} layer {layer} differs from eager"
        other = _eager(va, wl, calls[:1])
        torch.cuda.synchronize(dev)
    del other


def test_plan_siglip224_all_layers_bitwise(dev, va):
    """The SigLIP 224 px sequence (27 layers) recorded once and replayed."""
    wl = WORKLOADS["c3"]
    print(f"[plan] {wl.name}", flush=True)
    lis, calls = _inputs(wl, wl.layers, dev)
    plan = va.Plan(calls, scale=wl.scale)
    try:
        _replays_match_eager(va, dev, wl, calls, plan)
        # and the replayed output meets the oracle (first and last layer)
        for layer in (0, wl.layers - 1):
            li = lis[layer]
            B, N, H, D = li.q.shape
            ref = oracle.attention(*li.in_layout(wl.layout), wl.layout, B, H, N, D, wl.scale)
            assert_parity(logical(plan.outs[layer], wl.layout), ref, f"plan c3 layer {layer}")
    finally:
        plan.close()


def test_plan_separate_layout_on_side_stream(dev, va):
    import torch
    wl = WORKLOADS["c1"]
    _, calls = _inputs(wl, 3, dev)
    plan = va.Plan(calls, scale=wl.scale)
    try:
        _replays_match_eager(va, dev, wl, calls, plan, stream=torch.cuda.Stream(dev))
    finally:
        plan.close()


def test_plan_siglip384_persistent_kernel(dev, va):
    """One call of the 384 px workload (the looping-workgroup kernel)."""
    wl = WORKLOADS["c5"]
    _, calls = _inputs(wl, 1, dev)
    plan = va.Plan(calls, scale=wl.scale)
    try:
        _replays_match_eager(va, dev, wl, calls, plan, replays=2)
    finally:
        plan.close()


def test_plan_reads_inputs_at_launch(dev, va):
    """Changing the recorded input buffers in place changes the next launch's
    output exactly as an eager call on the new contents would."""
    import torch
    wl = Workload("t", "plan inputs", B=2, N=150, H=3, D=72, layout=LAYOUT_PACKED, layers=2,
                  kind="iid", index=60)
    _, calls = _inputs(wl, 2, dev)
    plan = va.Plan(calls, scale=wl.scale)
    try:
        plan.launch()
        torch.cuda.synchronize(dev)
        first = [bits_of(o) for o in plan.outs]
        _, fresh = _inputs(Workload("t", "plan inputs", B=2, N=150, H=3, D=72,
                                    layout=LAYOUT_PACKED, layers=2, kind="iid", index=61), 2, dev)
        for dst, src in zip(calls, fresh):
            dst.copy_(src)
        plan.launch()
        torch.cuda.synchronize(dev)
        want = [bits_of(o) for o in _eager(va, wl, calls)]
        torch.cuda.synchronize(dev)
        for layer in range(2):
            assert np.array_equal(bits_of(plan.outs[layer]), want[layer])
            assert not np.array_equal(first[layer], want[layer])
    finally:
        plan.close()


def test_plan_argument_errors(dev, va):
    import torch
    wl = WORKLOADS["c1"]
    _, calls = _inputs(wl, 2, dev)
    with pytest.raises(ValueError):
        va.Plan([])
    q, k, v = calls[0]
    short = (q[:, :, :100].contiguous(), k[:, :, :100].contiguous(), v[:, :, :100].contiguous())
    with pytest.raises(ValueError):
        va.Plan([calls[1], short])  # every call must have the same shape
    with pytest.raises(ValueError):
        va.Plan(calls, outs=[torch.empty(1, device=dev, dtype=torch.bfloat16)] * 2)


def test_sublayer_captured_by_torch_graph(dev, va):
    """Every entry point is capturable: the attention sublayer (qkv
    projection, attention, output projection with residual) recorded with
    torch.cuda.CUDAGraph and replayed three times, with eager work and
    synchronisations in between, matches the eager calls bitwise each time."""
    import math
    import torch
    torch.manual_seed(3)
    B, N, H, D = 2, 256, 16, 72
    E = H * D
    x = torch.randn(B, N, E, device=dev).to(torch.bfloat16)
    wqkv = (torch.randn(3 * E, E, device=dev) / math.sqrt(E)).to(torch.bfloat16)
    bqkv = (torch.randn(3 * E, device=dev) * 0.1).to(torch.bfloat16)
    wo = (torch.randn(E, E, device=dev) / math.sqrt(E)).to(torch.bfloat16)
    bo = (torch.randn(E, device=dev) * 0.1).to(torch.bfloat16)
    qkv = torch.empty(B, N, 3 * E, device=dev, dtype=torch.bfloat16)
    o = torch.empty(B, N, H, D, device=dev, dtype=torch.bfloat16)
    y = torch.empty(B, N, E, device=dev, dtype=torch.bfloat16)

    def sublayer():
        va.linear(x, wqkv, bqkv, out=qkv)
        va.fwd(qkv.view(B, N, 3, H, D), out=o)
        va.linear(o.view(B, N, E), wo, bo, residual=x, out=y)

    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        sublayer()  # warm up on the capture stream
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize(dev)
    want = bits_of(y)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        sublayer()
    for _ in range(3):
        y.zero_()
        qkv.zero_()
        graph.replay()
        torch.cuda.synchronize(dev)
        assert np.array_equal(bits_of(y), want)
        sublayer()  # eager work between replays
        torch.cuda.synchronize(dev)
        assert np.array_equal(bits_of(y), want)
