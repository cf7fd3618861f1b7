"""The library's calls under HIP graph capture (torch.cuda.CUDAGraph).

Every entry point is asynchronous on the caller's stream, takes its
metadata through kernel arguments (a step of more than 48 tensors uploads
its tensor table with a small kernel whose argument holds it, and may fill
a slot table on the device; a shorter list passes the table in the step
kernels' own arguments), and calls no allocation or memset, so a sequence
of calls can be captured once and replayed. One iteration -- an AdamW-SR
step (a size class and a table launch; a two-tensor list, or 53 tensors
with a device-filled slot table), the SR conversion, the SR GEMM in its
persistent launch, and dropout -- is captured, then replayed three times
with eager work and synchronizations in between. After every replay the state and the outputs
must equal, bit for bit, those of the same iterations run eagerly (the
replayed step repeats its captured step number, as the eager runs do)."""

import numpy as np
import pytest
import torch

from adamw_optimizer_stochastic_amd import ops, random as arng, workloads as wl
from _gpu_util import gpu, require_gpu, announce, to_host, assert_bits_equal, bf16_tensor

pytestmark = gpu

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


@pytest.mark.parametrize("n_tiny", [0, 50], ids=["inline", "uploaded"])
def test_graph_replays_match_eager(n_tiny):
    dev = torch.device("cuda", 0)
    announce("graph capture: inputs", n_tiny)
    gen = wl.device_generator(dev, wl.CFG_SMALL, 41)
    # 2049 slots (a size class) and a table launch; with the tiny tensors,
    # 53 tensors and a table of 835 slots (filled on the device)
    sizes = [(1 << 21) + 77, 3000] + ([800_001] + [17 * k + 1 for k in range(n_tiny)]
                                      if n_tiny else [])
    p0 = [wl.device_normal(n, 0.02, gen, dev, torch.bfloat16) for n in sizes]
    grads = [wl.device_normal(n, 1e-3, gen, dev, torch.bfloat16) for n in sizes]
    bases = [int(x) for x in np.cumsum([0] + sizes[:-1])]
    x = wl.device_normal((1 << 20) + 5, 1.0, gen, dev, torch.float32)
    m, n, k = 4100, 4200, 256            # 17 x 17 big tiles: the persistent launch
    a_bits, b_bits = wl.gemm_operands_host(m, n, k, "int", seed=5)
    a, b = bf16_tensor(a_bits), bf16_tensor(b_bits)
    ws = ops.make_workspace(sizes, dev)

    def fresh():
        return dict(p=[t.clone() for t in p0],
                    m=[torch.zeros(t.numel(), dtype=torch.float32, device=dev) for t in p0],
                    v=[torch.zeros(t.numel(), dtype=torch.float32, device=dev) for t in p0],
                    cvt=torch.empty(x.shape, dtype=torch.bfloat16, device=dev),
                    c=torch.empty((m, n), dtype=torch.bfloat16, device=dev))

    def iteration(st):
        ops.adamw_step(st["p"], grads, st["m"], st["v"], bases, step=1, seed=3, workspace=ws,
                       **HP)
        ops.cvt_f32_bf16_sr(x, 5, 2, 11, out=st["cvt"])
        ops.gemm_bf16(a, b, rounding="sr", seed=7, step=1, base_index=3, out=st["c"])
        return arng.dropout(x, 0.3, seed=9, step=1, base_index=4)

    def snapshot(st, y):
        return ([to_host(t) for t in st["p"]], [to_host(t) for t in st["m"]],
                [to_host(t) for t in st["v"]], to_host(st["cvt"]), to_host(st["c"]), to_host(y))

    announce("graph capture: eager reference")
    eager = fresh()
    ref = []
    for _ in range(3):
        y = iteration(eager)
        torch.cuda.synchronize()
        ref.append(snapshot(eager, y))
    del eager

    announce("graph capture: capture")
    st = fresh()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        y_graph = iteration(st)
    torch.cuda.synchronize()
    for r in range(3):
        announce("graph capture: replay", r)
        graph.replay()
        # eager work of the program's own between replays
        z = torch.ones(1 << 16, device=dev)
        assert float(z.sum()) == float(1 << 16)
        torch.cuda.synchronize()
        got = snapshot(st, y_graph)
        want = ref[r]
        for i in range(len(sizes)):
            assert_bits_equal(got[0][i], want[0][i], f"replay {r} param {i}")
            assert_bits_equal(got[1][i], want[1][i], f"replay {r} m {i}")
            assert_bits_equal(got[2][i], want[2][i], f"replay {r} v {i}")
        assert_bits_equal(got[3], want[3], f"replay {r} conversion")
        assert_bits_equal(got[4].reshape(-1), want[4].reshape(-1), f"replay {r} gemm")
        assert_bits_equal(got[5], want[5], f"replay {r} dropout")
    # the replays really advanced the state: replay 3 differs from replay 1
    assert not np.array_equal(ref[0][0][0], ref[2][0][0])


def test_graph_noalloc_step_replays_match_eager():
    """asr_adamw_step_noalloc -- the step for callers that cannot allocate,
    e.g. under graph capture -- captured once (after one eager call, which
    finds the device's scratch) and replayed three times with eager work in
    between: each replay equals the same eager step bit for bit."""
    from adamw_optimizer_stochastic_amd import _abi
    dev = torch.device("cuda", 0)
    announce("graph capture noalloc: inputs")
    gen = wl.device_generator(dev, wl.CFG_SMALL, 43)
    # 53 tensors: more than travel in the kernel arguments, so the step's
    # metadata and slot table live in the scratch
    sizes = [(1 << 21) + 77, 3000, 65537] + [29 * k + 3 for k in range(50)]
    p0 = [wl.device_normal(n, 0.02, gen, dev, torch.bfloat16) for n in sizes]
    grads = [wl.device_normal(n, 1e-3, gen, dev, torch.bfloat16) for n in sizes]
    bases = [int(x) for x in np.cumsum([5] + sizes[:-1])]

    def fresh():
        return dict(p=[t.clone() for t in p0],
                    m=[torch.zeros(t.numel(), dtype=torch.float32, device=dev) for t in p0],
                    v=[torch.zeros(t.numel(), dtype=torch.float32, device=dev) for t in p0])

    def step(st, t):
        descs = [_abi.AsrTensor(p.data_ptr(), g.data_ptr(), m.data_ptr(), v.data_ptr(), p.numel(),
                                b, _abi.ASR_BF16, _abi.ASR_BF16)
                 for p, g, m, v, b in zip(st["p"], grads, st["m"], st["v"], bases)]
        _abi.asr_adamw_step_noalloc(descs, HP["lr"], HP["beta1"], HP["beta2"], HP["eps"],
                                    HP["weight_decay"], t, 3, _abi.ASR_ROUND_SR,
                                    torch.cuda.current_stream(dev).cuda_stream)

    def snapshot(st):
        return [to_host(x) for key in ("p", "m", "v") for x in st[key]]

    announce("graph capture noalloc: eager reference")
    eager = fresh()
    ref = []
    for _ in range(3):
        step(eager, 2)
        torch.cuda.synchronize()
        ref.append(snapshot(eager))
    del eager
    st = fresh()
    warm = fresh()
    step(warm, 2)                # the first call on the device looks up the scratch
    torch.cuda.synchronize()
    del warm
    announce("graph capture noalloc: capture")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(st, 2)
    torch.cuda.synchronize()
    for r in range(3):
        announce("graph capture noalloc: replay", r)
        graph.replay()
        z = torch.ones(1 << 16, device=dev)
        assert float(z.sum()) == float(1 << 16)
        torch.cuda.synchronize()
        for i, (g_, w_) in enumerate(zip(snapshot(st), ref[r])):
            assert_bits_equal(g_, w_, f"replay {r} array {i}")
    assert not np.array_equal(ref[0][0], ref[2][0])
