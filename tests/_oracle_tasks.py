"""Work items the CPU pool (tests/_cpu_pool.py) runs for the full-size GPU
parity tests: each runs the oracle on one piece of a large input, compares
it with the GPU's output for that piece, and returns what differs. Pieces
are independent: every element's result depends only on its own inputs and
its global position (the "adamw-sr" page, Correctness: a tensor updated in
pieces that carry their own base_index matches the one-piece update bit for
bit), so a piece is checked with the oracle called on that piece alone.

These functions only call the oracle and compare bit patterns; none of them
computes any part of the method itself."""

import numpy as np

import oracle
from oracle.adamw import F32, BF16


def _diff(got, want, what):
    """(count, first indices, got, want) of the positions whose bits differ."""
    g = np.ascontiguousarray(got)
    w = np.ascontiguousarray(want)
    if g.dtype == np.float32:
        g, w = g.view(np.uint32), w.view(np.uint32)
    bad = np.nonzero(g != w)[0]
    if bad.size == 0:
        return None
    i = bad[:6]
    return (what, int(bad.size), i.tolist(), [hex(int(x)) for x in g[i]],
            [hex(int(x)) for x in w[i]])


def convert_piece(args):
    """SR conversion of one piece: x (f32) at global positions base + i."""
    x, got, base, seed, step = args
    want = oracle.cvt_f32_bf16_sr(x, seed, step, base)
    return _diff(got, want, f"convert [{base}, {base + x.size})")


def f32_steps_piece(args):
    """One piece of the f32 workload run for len(grads) steps from m = v = 0:
    returns the differences of the state after step 1 and after the last
    step."""
    p, grads, got_first, got_last, base, hp = args
    n = p.size
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    out = []
    for t in range(1, len(grads) + 1):
        p, m, v = oracle.step_tensor(p, grads[t - 1], m, v, param_dtype=F32, grad_dtype=F32,
                                     base_index=base, step=t, seed=hp["seed"], lr=hp["lr"],
                                     beta1=hp["beta1"], beta2=hp["beta2"], eps=hp["eps"],
                                     weight_decay=hp["weight_decay"])
        if t == 1 or t == len(grads):
            got = got_first if t == 1 else got_last
            for name, g_, w_ in zip(("param", "m", "v"), got, (p, m, v)):
                d = _diff(g_, w_, f"step {t} {name} [{base}, {base + n})")
                if d:
                    out.append(d)
    return out


def bf16_steps_piece(args):
    """One piece of a bf16/bf16 SR tensor run for `steps` steps (same
    gradient each step) from m = v = 0; returns the differences of the
    final param, m and v."""
    p, g, got, base, steps, hp, what = args
    n = p.size
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    for t in range(1, steps + 1):
        p, m, v = oracle.step_tensor(p, g, m, v, param_dtype=BF16, grad_dtype=BF16,
                                     base_index=base, step=t, seed=hp["seed"], lr=hp["lr"],
                                     beta1=hp["beta1"], beta2=hp["beta2"], eps=hp["eps"],
                                     weight_decay=hp["weight_decay"])
    out = []
    for name, g_, w_ in zip(("param", "m", "v"), got, (p, m, v)):
        d = _diff(g_, w_, f"{what} {name}")
        if d:
            out.append(d)
    return out
