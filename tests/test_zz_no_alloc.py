"""asr_adamw_step_noalloc, the step for callers that cannot allocate (it
runs on the library's static scratch instead of a workspace), against
asr_adamw_step through the C ABI: calls in a row, the second with a smaller
list, bit for bit on params, m and v; and a list too large for the scratch
is rejected before anything is enqueued."""

import numpy as np
import pytest
import torch

from adamw_optimizer_stochastic_amd import _abi, ops
from adamw_optimizer_stochastic_amd import workloads as wl
from _gpu_util import gpu, require_gpu, announce, to_host, assert_bits_equal

pytestmark = gpu
HP = (1e-3, 0.9, 0.999, 1e-8, 0.01)
DT = {torch.float32: _abi.ASR_F32, torch.bfloat16: _abi.ASR_BF16}


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _make_list(specs, seed):
    """specs: (numel, param dtype, grad dtype, view offset). Returns tensors
    (device) and the AsrTensor descriptors."""
    dev = torch.device("cuda", 0)
    gen = wl.device_generator(dev, wl.CFG_SMALL, 900 + seed)
    ts, base = [], 3
    for n, pdt, gdt, off in specs:
        p = wl.device_normal(n + off, 0.02, gen, dev, pdt)[off:]
        g = wl.device_normal(n + off, 1e-3, gen, dev, gdt)[off:]
        m = wl.device_normal(n + off, 1e-4, gen, dev, torch.float32)[off:]
        v = wl.device_normal(n + off, 1e-7, gen, dev, torch.float32).abs()[off:]
        ts.append(dict(p=p, g=g, m=m, v=v, base=base, pdt=pdt, gdt=gdt))
        base += n
    return ts


def _descs(ts):
    return [_abi.AsrTensor(t["p"].data_ptr(), t["g"].data_ptr(), t["m"].data_ptr(),
                           t["v"].data_ptr(), t["p"].numel(), t["base"], DT[t["pdt"]],
                           DT[t["gdt"]]) for t in ts]


def _clone(ts):
    return [dict(t, p=t["p"].clone(), m=t["m"].clone(), v=t["v"].clone()) for t in ts]


def _run_both(ts, step, rounding):
    stream = torch.cuda.current_stream().cuda_stream
    ref = _clone(ts)
    ws = ops.make_workspace([t["p"].numel() for t in ref], ref[0]["p"].device)
    _abi.asr_adamw_step(_descs(ref), *HP, step, 17, rounding, ws.data_ptr(),
                        ws.numel(), stream)
    _abi.asr_adamw_step_noalloc(_descs(ts), *HP, step, 17, rounding, stream)
    torch.cuda.synchronize()
    for k, (a, b) in enumerate(zip(ts, ref)):
        for name in ("p", "m", "v"):
            assert_bits_equal(to_host(a[name]), to_host(b[name]), f"tensor {k} {name}")


def test_noalloc_matches_step_two_calls_second_smaller():
    # Lists of more than 48 tensors keep their metadata in the scratch (a
    # shorter list passes it in the kernel arguments and leaves the scratch
    # alone). Call 1: a size class (3 x 700,001 elements: 684 slots each,
    # 2,052 in all), shifted views, a mixed-size rest and 45 tiny tensors,
    # every dtype pair: 54 tensors; the bf16/bf16 slot table (about 1,030
    # entries) is filled on the device, the other pairs' tables come from
    # the host. Call 2: a smaller list of 50 tensors (host-built tables), so
    # stale entries of call 1 remain in the scratch past what call 2 writes.
    # Then call 1's list again, and a list short enough to travel in the
    # kernel arguments.
    tiny = [(1 + (37 * k) % 1000, torch.bfloat16, torch.bfloat16, k % 4) for k in range(45)]
    first = [(700_001, torch.bfloat16, torch.bfloat16, 0)] * 2 + \
            [(700_001, torch.bfloat16, torch.bfloat16, 3)] + \
            [(n, pdt, gdt, off) for n, pdt, gdt, off in (
                (1, torch.bfloat16, torch.bfloat16, 0), (4097, torch.float32, torch.float32, 1),
                (65_537, torch.bfloat16, torch.float32, 2), (300_007, torch.float32, torch.bfloat16, 0),
                (2_049, torch.bfloat16, torch.bfloat16, 5), (1_000_003, torch.bfloat16, torch.bfloat16, 0))] + tiny
    short = [(5, torch.bfloat16, torch.bfloat16, 0), (3_001, torch.float32, torch.float32, 0),
             (10_007, torch.bfloat16, torch.bfloat16, 1)]
    second = short + [(1 + (53 * k) % 900, torch.bfloat16, torch.bfloat16, k % 3) for k in range(47)]
    assert len(first) == 54 and len(second) == 50
    for k, (specs, step, rounding) in enumerate(((first, 3, _abi.ASR_ROUND_SR),
                                                 (second, 4, _abi.ASR_ROUND_RN),
                                                 (first, 5, _abi.ASR_ROUND_SR),
                                                 (short, 6, _abi.ASR_ROUND_SR))):
        announce("noalloc call", k + 1, len(specs), "tensors")
        _run_both(_make_list(specs, k), step, rounding)


def test_noalloc_rejects_a_list_beyond_the_scratch():
    """2,000 tensors of distinct sizes below a size class (all in the slot
    table: about 3 M slots, 12 MB of table) do not fit in 4 MiB: rejected
    on the host with ASR_EWORKSPACE, nothing enqueued (the buffer addresses
    are never touched)."""
    descs = [_abi.AsrTensor(0x10000000, 0x20000000, 0x30000000, 0x40000000,
                            (1000 + k) * 1024, 0, _abi.ASR_BF16, _abi.ASR_BF16)
             for k in range(2000)]
    with pytest.raises(_abi.AsrError) as e:
        _abi.asr_adamw_step_noalloc(descs, *HP, 1, 0, _abi.ASR_ROUND_SR, None)
    assert e.value.status == _abi.ASR_EWORKSPACE
    assert "scratch" in _abi.asr_last_error()
    # argument errors come back as for asr_adamw_step
    bad = [_abi.AsrTensor(0x1001, 0x2000, 0x3000, 0x4000, 8, 0, _abi.ASR_BF16, _abi.ASR_BF16)]
    with pytest.raises(_abi.AsrError) as e:
        _abi.asr_adamw_step_noalloc(bad, *HP, 1, 0, _abi.ASR_ROUND_SR, None)
    assert e.value.status == _abi.ASR_EALIGN
    _abi.asr_adamw_step_noalloc([], *HP, 1, 0, _abi.ASR_ROUND_SR, None)
