"""GPU parity at full size, in the launch configuration the benchmark times:
  * the SR conversion of 2**30 f32 values with 0.1% +-Inf/NaN/FLT_MAX,
    every output against the oracle;
  * the f32 workload, 16,777,216 elements x 100 steps, bit-exact;
  * a 268,435,456-element bf16 step run whole, as 8 shards with their own
    base_index, and split at an odd element (adamw-sr page, Correctness:
    sharded and one-piece updates must agree bit for bit);
  * one multi-tensor call over the whole Llama-3-8B-shaped list (layers 0
    and 31 in full), and over one data-parallel rank's share of it (pieces
    with global base_index).
Outputs are checked bit for bit against the oracle, in full where the
oracle can run over the whole output on the CPU pool (tests/_cpu_pool.py)
and otherwise on the pieces named in each test.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle.adamw import BF16
from adamw_optimizer_stochastic_amd import ops
from adamw_optimizer_stochastic_amd import workloads as wl
from _gpu_util import gpu, require_gpu, announce, to_host, assert_bits_equal
import _cpu_pool
import _oracle_tasks

pytestmark = gpu
HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_convert_2pow30_with_specials():
    """The conversion workload in the benchmark's launch configuration:
    2**30 f32 values with 0.1% +-Inf/NaN/FLT_MAX, seed 7, step 0. Every
    output is compared with the oracle, run in pieces on the CPU pool."""
    n, seed, step = 1 << 30, 7, 0
    announce("convert 2**30: inputs")
    dev = torch.device("cuda", 0)
    gen = wl.device_generator(dev, wl.CFG_CONVERT, 0)
    x = wl.device_normal(n, 1.0, gen, dev, torch.float32)
    rng = wl.host_rng(wl.CFG_CONVERT, 0, 1)
    k = int(round(0.001 * n))
    pos = np.sort(rng.choice(n, size=k, replace=False))
    specials = wl.SPECIAL_F32_BITS[np.arange(k) % wl.SPECIAL_F32_BITS.size]
    x.view(torch.int32)[torch.from_numpy(pos).to(dev)] = torch.from_numpy(
        specials.view(np.int32)).to(dev)
    announce("convert 2**30: kernel")
    out = ops.cvt_f32_bf16_sr(x, seed, step, 0)
    torch.cuda.synchronize()
    # Every special position first (names the failing kind of input).
    got_sp = to_host(out[torch.from_numpy(pos).to(dev)])
    want_sp = oracle.sr_bf16(specials, oracle.random16(pos.astype(np.uint64), seed, step))
    assert_bits_equal(got_sp, want_sp, "special positions")
    # Every output, against the oracle, in pieces of 2**24 on the CPU pool.
    piece = 1 << 24
    announce(f"convert 2**30: oracle on {n // piece} pieces, {_cpu_pool.workers()} workers")

    def pieces():
        for s in range(0, n, piece):
            yield (to_host(x[s:s + piece]), to_host(out[s:s + piece]), s, seed, step)

    with _cpu_pool.pool() as pool:
        bad = [d for d in pool.imap_unordered(_oracle_tasks.convert_piece, pieces()) if d]
    assert not bad, bad[:4]


def test_f32_workload_full_size_100_steps():
    """The f32 workload at its full size: 16,777,216 f32 params ~N(0, 0.02),
    f32 grads ~N(0, 1e-2) drawn afresh each step, m = v = 0, lr 1e-3, wd
    0.01, 100 steps, one size-class launch per step (16,384 slots). The
    state after step 1 and after step 100 must equal the oracle's bit for
    bit; the oracle runs the 100 steps in 16 pieces on the CPU pool."""
    n, steps = 1 << 24, 100
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, seed=0)
    dev = torch.device("cuda", 0)
    announce("f32 16M x 100: inputs")
    gen = wl.device_generator(dev, wl.CFG_F32, 0)
    p = wl.device_normal(n, 0.02, gen, dev, torch.float32)
    p0 = to_host(p)
    m = torch.zeros(n, dtype=torch.float32, device=dev)
    v = torch.zeros(n, dtype=torch.float32, device=dev)
    grads = np.empty((steps, n), np.float32)
    ws = ops.make_workspace([n], dev)
    for t in range(1, steps + 1):
        g = wl.device_normal(n, 1e-2, gen, dev, torch.float32)
        grads[t - 1] = to_host(g)
        ops.adamw_step([p], [g], [m], [v], [0], step=t, workspace=ws, **hp)
        if t == 1:
            first = (to_host(p), to_host(m), to_host(v))
        if t % 25 == 0:
            announce("f32 16M x 100: step", t)
    torch.cuda.synchronize()
    last = (to_host(p), to_host(m), to_host(v))
    piece = n // 16
    announce(f"f32 16M x 100: oracle on 16 pieces, {_cpu_pool.workers()} workers")

    def pieces():
        for s in range(0, n, piece):
            e = s + piece
            yield (p0[s:e], np.ascontiguousarray(grads[:, s:e]), [a[s:e] for a in first],
                   [a[s:e] for a in last], s, hp)

    with _cpu_pool.pool() as pool:
        bad = [d for r in pool.imap_unordered(_oracle_tasks.f32_steps_piece, pieces())
               for d in r]
    assert not bad, bad[:4]


def test_268M_whole_equals_8_shards_and_odd_split():
    n = 268435456
    dev = torch.device("cuda", 0)
    announce("268M: inputs")
    gen = wl.device_generator(dev, wl.CFG_SHARDS, 0)
    p0 = wl.device_normal(n, 0.02, gen, dev, torch.bfloat16)
    g = wl.device_normal(n, 1e-3, gen, dev, torch.bfloat16)
    rng = wl.host_rng(wl.CFG_SHARDS, 0, 1)
    windows = [0, n - (1 << 16)] + [int(rng.integers(0, n - (1 << 16))) for _ in range(14)]
    host_in = [(to_host(p0[s:s + (1 << 16)]), to_host(g[s:s + (1 << 16)])) for s in windows]

    def fresh():
        return (p0.clone(), torch.zeros(n, dtype=torch.float32, device=dev),
                torch.zeros(n, dtype=torch.float32, device=dev))

    announce("268M: whole")
    wp, wm, wv = fresh()
    ops.adamw_step([wp], [g], [wm], [wv], [0], step=1, seed=0, **HP)
    announce("268M: 8 shards")
    sp, sm, sv = fresh()
    shard = n // 8
    for k in range(8):
        a, b = k * shard, (k + 1) * shard
        ops.adamw_step([sp[a:b]], [g[a:b]], [sm[a:b]], [sv[a:b]], [a], step=1, seed=0, **HP)
    torch.cuda.synchronize()
    assert torch.equal(wp.view(torch.int16), sp.view(torch.int16))
    assert torch.equal(wm.view(torch.int32), sm.view(torch.int32))
    assert torch.equal(wv.view(torch.int32), sv.view(torch.int32))
    del sp, sm, sv
    announce("268M: odd split")
    op, om, ov = fresh()
    cut = 33554433
    ops.adamw_step([op[:cut], op[cut:]], [g[:cut], g[cut:]], [om[:cut], om[cut:]],
                   [ov[:cut], ov[cut:]], [0, cut], step=1, seed=0, **HP)
    torch.cuda.synchronize()
    assert torch.equal(wp.view(torch.int16), op.view(torch.int16))
    assert torch.equal(wm.view(torch.int32), om.view(torch.int32))
    del op, om, ov
    announce("268M: oracle windows")
    z = np.zeros(1 << 16, np.float32)
    for s, (hp_, hg) in zip(windows, host_in):
        want = oracle.step_tensor(hp_, hg, z, z, param_dtype=BF16, grad_dtype=BF16, base_index=s,
                                  step=1, seed=0, **HP)
        assert_bits_equal(to_host(wp[s:s + (1 << 16)]), want[0], f"param window {s}")
        assert_bits_equal(to_host(wm[s:s + (1 << 16)]), want[1], f"m window {s}")
        assert_bits_equal(to_host(wv[s:s + (1 << 16)]), want[2], f"v window {s}")


def test_llama3_8b_list_two_steps_sampled():
    """The benchmark's call: all 291 tensors in one multi-tensor call, two
    steps. Against the oracle (both steps):
      * every tensor of layers 0 and 31 in full, and 16 random windows of
        2**20 elements in each of embed_tokens and lm_head (each window run
        by the oracle with its own base_index), on the CPU pool;
      * windows at the start, middle and end of every other tensor, and
        every RMSNorm weight in full, in this process."""
    dev = torch.device("cuda", 0)
    announce("llama3-8b: inputs (96 GB)")
    state = wl.llama3_8b_state(dev, seed=0)
    assert len(state) == 291
    assert sum(t["param"].numel() for t in state) == 8030261248
    rng = wl.host_rng(wl.CFG_LLAMA, 0, 5)
    win, big_win, piece = 1 << 14, 1 << 20, 1 << 24
    samples = []       # checked here: (tensor, start, end, p0, g)
    pool_pieces = []   # checked on the pool: (tensor, start, end, p0, g)
    for t in state:
        n = t["param"].numel()
        name = t["name"]
        if name.startswith("layers.0.") or name.startswith("layers.31."):
            for s0 in range(0, n, piece):
                e = min(n, s0 + piece)
                pool_pieces.append((t, s0, e, to_host(t["param"][s0:e]), to_host(t["grad"][s0:e])))
            continue
        if name in ("embed_tokens", "lm_head"):
            for s0 in sorted(int(x) for x in rng.integers(0, n - big_win, size=16)):
                pool_pieces.append((t, s0, s0 + big_win, to_host(t["param"][s0:s0 + big_win]),
                                    to_host(t["grad"][s0:s0 + big_win])))
        starts = [0] if n <= 3 * win else [0, n // 2 - win // 2 + 3, n - win]
        for s0 in starts:
            e = min(n, s0 + (n if n <= 3 * win else win))
            samples.append((t, s0, e, to_host(t["param"][s0:e]), to_host(t["grad"][s0:e])))
    assert sum(e - s0 for _, s0, e, _, _ in pool_pieces) == 2 * 218112000 + 32 * big_win
    ws = ops.make_workspace([t["param"].numel() for t in state], dev)
    lists = ([t["param"] for t in state], [t["grad"] for t in state],
             [t["exp_avg"] for t in state], [t["exp_avg_sq"] for t in state],
             [t["base_index"] for t in state])
    for step in (1, 2):
        announce("llama3-8b: step", step)
        ops.adamw_step(*lists, step=step, seed=0, rounding="sr", workspace=ws, **HP)
    torch.cuda.synchronize()
    announce("llama3-8b: oracle on", len(samples), "windows")
    for t, s, e, hp_, hg in samples:
        m = np.zeros(e - s, np.float32)
        v = np.zeros(e - s, np.float32)
        p = hp_
        for step in (1, 2):
            p, m, v = oracle.step_tensor(p, hg, m, v, param_dtype=BF16, grad_dtype=BF16,
                                         base_index=t["base_index"] + s, step=step, seed=0, **HP)
        what = f"{t['name']}[{s}:{e}]"
        assert_bits_equal(to_host(t["param"][s:e]), p, what + " param")
        assert_bits_equal(to_host(t["exp_avg"][s:e]), m, what + " m")
        assert_bits_equal(to_host(t["exp_avg_sq"][s:e]), v, what + " v")
    announce(f"llama3-8b: oracle on {len(pool_pieces)} pieces (layers 0 and 31, "
             f"embed/lm_head windows), {_cpu_pool.workers()} workers")
    hp = dict(HP, seed=0)

    def tasks():
        for t, s, e, hp_, hg in pool_pieces:
            got = (to_host(t["param"][s:e]), to_host(t["exp_avg"][s:e]),
                   to_host(t["exp_avg_sq"][s:e]))
            yield (hp_, hg, got, t["base_index"] + s, 2, hp, f"{t['name']}[{s}:{e}]")

    with _cpu_pool.pool() as pool:
        bad = [d for r in pool.imap_unordered(_oracle_tasks.bf16_steps_piece, tasks()) for d in r]
    assert not bad, bad[:4]
    del state, lists


def test_llama3_8b_rank_share_two_steps_sampled():
    """One data-parallel rank's share of the Llama-3-8B list (rank 3 of 8 of
    the flattened list, ZeRO-1 layout: 42 pieces, cut inside a tensor at
    both ends), as the benchmark's rank workload launches it: one call, two
    steps, each piece with its global base_index. The oracle runs both steps
    on windows at the start, middle and end of every piece, so each piece's
    random bits must come from its global positions."""
    dev = torch.device("cuda", 0)
    announce("llama3-8b rank 3/8: inputs (12 GB)")
    state = wl.llama3_8b_rank_state(dev, 3, 8, seed=0)
    assert len(state) == 42 and state[0]["offset"] > 0
    assert sum(t["param"].numel() for t in state) == 8030261248 // 8
    win = 1 << 14
    samples = []
    for t in state:
        n = t["param"].numel()
        starts = [0] if n <= 3 * win else [0, n // 2 - win // 2 + 1, n - win]
        for s0 in starts:
            e = min(n, s0 + (n if n <= 3 * win else win))
            samples.append((t, s0, e, to_host(t["param"][s0:e]), to_host(t["grad"][s0:e])))
    lists = ([t["param"] for t in state], [t["grad"] for t in state],
             [t["exp_avg"] for t in state], [t["exp_avg_sq"] for t in state],
             [t["base_index"] for t in state])
    for step in (1, 2):
        announce("llama3-8b rank 3/8: step", step)
        ops.adamw_step(*lists, step=step, seed=0, rounding="sr", **HP)
    torch.cuda.synchronize()
    announce("llama3-8b rank 3/8: oracle on", len(samples), "windows")
    for t, s0, e, hp_, hg in samples:
        m = np.zeros(e - s0, np.float32)
        v = np.zeros(e - s0, np.float32)
        p = hp_
        for step in (1, 2):
            p, m, v = oracle.step_tensor(p, hg, m, v, param_dtype=BF16, grad_dtype=BF16,
                                         base_index=t["base_index"] + s0, step=step, seed=0,
                                         **HP)
        what = f"{t['name']}[{t['offset'] + s0}:{t['offset'] + e}]"
        assert_bits_equal(to_host(t["param"][s0:e]), p, what + " param")
        assert_bits_equal(to_host(t["exp_avg"][s0:e]), m, what + " m")
        assert_bits_equal(to_host(t["exp_avg_sq"][s0:e]), v, what + " v")
    del state, lists


def test_tensors_beyond_2pow32_elements_and_two_launches():
    """Two equal tensors of 4,400,000,037 bf16 elements each: element offsets
    past 2**32 inside one tensor, and more slots than one launch covers, so
    the size class is split over two launches. Windows around element 2**32,
    around the launch boundary, at both ends of each tensor, against the
    oracle; base indices with an odd phase."""
    n = 4_400_000_037
    dev = torch.device("cuda", 0)
    announce("beyond 2**32: inputs (106 GB)")
    gen = wl.device_generator(dev, wl.CFG_SHARDS, 77)
    ts = []
    for k in range(2):
        p = torch.empty(n, dtype=torch.bfloat16, device=dev)
        g = torch.empty(n, dtype=torch.bfloat16, device=dev)
        for s in range(0, n, 1 << 30):                     # bounded temporaries
            e = min(n, s + (1 << 30))
            p[s:e] = wl.device_normal(e - s, 0.02, gen, dev, torch.bfloat16)
            g[s:e] = wl.device_normal(e - s, 1e-3, gen, dev, torch.bfloat16)
        ts.append(dict(p=p, g=g, m=torch.zeros(n, dtype=torch.float32, device=dev),
                       v=torch.zeros(n, dtype=torch.float32, device=dev)))
    base0 = (1 << 40) + 3
    bases = [base0, base0 + n]
    slot = 1024                                             # elements per slot
    per = -(-n // slot)                                     # slots per tensor
    second = (1 << 23) - per                                # launch boundary in tensor 1
    w = 4096
    wins = [(0, 0), (0, (1 << 32) - w // 2), (0, n - w - 5), (1, 0),
            (1, second * slot - w // 2), (1, (1 << 32) - w // 2), (1, n - w)]
    host = [(k, s, to_host(ts[k]["p"][s:s + w]), to_host(ts[k]["g"][s:s + w])) for k, s in wins]
    announce("beyond 2**32: step")
    ops.adamw_step([t["p"] for t in ts], [t["g"] for t in ts], [t["m"] for t in ts],
                   [t["v"] for t in ts], bases, step=3, seed=21, **HP)
    torch.cuda.synchronize()
    z = np.zeros(w, np.float32)
    for k, s, hp_, hg in host:
        want = oracle.step_tensor(hp_, hg, z, z, param_dtype=BF16, grad_dtype=BF16,
                                  base_index=bases[k] + s, step=3, seed=21, **HP)
        what = f"tensor {k} [{s}:{s + w}]"
        assert_bits_equal(to_host(ts[k]["p"][s:s + w]), want[0], what + " param")
        assert_bits_equal(to_host(ts[k]["m"][s:s + w]), want[1], what + " m")
        assert_bits_equal(to_host(ts[k]["v"][s:s + w]), want[2], what + " v")
    del ts


def test_convert_beyond_2pow32_elements():
    n = (1 << 32) + 4099
    dev = torch.device("cuda", 0)
    announce("convert beyond 2**32: inputs")
    gen = wl.device_generator(dev, wl.CFG_CONVERT, 9)
    x = torch.empty(n, dtype=torch.float32, device=dev)
    for s in range(0, n, 1 << 30):
        e = min(n, s + (1 << 30))
        x[s:e] = wl.device_normal(e - s, 1.0, gen, dev, torch.float32)
    base = (1 << 33) + 1
    out = ops.cvt_f32_bf16_sr(x, 5, 11, base)
    torch.cuda.synchronize()
    for s in (0, (1 << 31) - 100, (1 << 32) - 3000, n - 5000):
        xs = to_host(x[s:s + 5000])
        assert_bits_equal(to_host(out[s:s + 5000]), oracle.cvt_f32_bf16_sr(xs, 5, 11, base + s),
                          f"window {s}")
