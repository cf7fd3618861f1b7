"""Seeded synthetic workloads (shapes and input generators only).

Nothing here computes any part of the method: these functions only draw
inputs, which the tests and the benchmark feed byte-identically to the GPU
path and to the oracle. Draws are N(0, std) (std = standard deviation);
bf16 inputs are f32 draws cast by torch's round-to-nearest-even cast.

Workloads (sizes as used by the tests and the benchmark):
  * small:   one bf16 tensor of 65,536 elements, params ~N(0, 0.02), grads
             ~N(0, 1e-3) drawn afresh each step, m = v = 0, 10 steps;
  * subulp:  1,048,576 bf16 params equal to 1.0, grad = w - 1.5 (f32),
             lr 1e-4, wd 0, 6,000 steps;
  * f32:     16,777,216 f32 params ~N(0, 0.02), f32 grads ~N(0, 1e-2) each
             step, 100 steps;
  * convert: 2**30 f32 values ~N(0, 1) with 0.1% of positions replaced by
             a cycle of +-Inf, NaNs with various payloads and +-FLT_MAX;
  * shards:  268,435,456 bf16 params ~N(0, 0.02), bf16 grads ~N(0, 1e-3);
  * llama3_8b: the parameter list of a Llama-3-8B-shaped model (291
             tensors, 8,030,261,248 elements), bf16 matrices ~N(0, 0.02),
             RMSNorm weights 1.0, bf16 grads ~N(0, 1e-3), f32 m = v = 0
             allocated after params and grads, in flat buffers as the
             optimizer allocates them (or per tensor, on request).
  * llama3_8b rank share: what one of R data-parallel ranks holds when the
             flattened list is split into R equal contiguous ranges (the
             ZeRO-1 layout): the pieces of the tensors inside its range,
             each with its global base_index; values drawn as above.
  * gemm:    bf16 operands of C = A B^T. "randn": A ~N(0, 1) (activations),
             B ~N(0, 0.02) (weights); "int": integers uniform in [-8, 8]
             (every f32 partial sum is then exact). The full-size case is
             the gate/up projection of one Llama-3-8B MLP over 8,192
             tokens: M = 8192, N = 14336, K = 4096.
"""

import numpy as np
import torch

# ---------------------------------------------------------------- shapes
LLAMA3_8B = dict(hidden=4096, ffn=14336, layers=32, q_heads=32, kv_heads=8, head_dim=128,
                 vocab=128256)


def llama3_8b_shapes(cfg=LLAMA3_8B):
    """(name, shape) of every parameter, in module registration order."""
    h, f, hd = cfg["hidden"], cfg["ffn"], cfg["head_dim"]
    q, kv = cfg["q_heads"] * hd, cfg["kv_heads"] * hd
    out = [("embed_tokens", (cfg["vocab"], h))]
    for i in range(cfg["layers"]):
        pre = f"layers.{i}."
        out += [(pre + "self_attn.q_proj", (q, h)), (pre + "self_attn.k_proj", (kv, h)),
                (pre + "self_attn.v_proj", (kv, h)), (pre + "self_attn.o_proj", (h, q)),
                (pre + "mlp.gate_proj", (f, h)), (pre + "mlp.up_proj", (f, h)),
                (pre + "mlp.down_proj", (h, f)),
                (pre + "input_layernorm", (h,)), (pre + "post_attention_layernorm", (h,))]
    out += [("norm", (h,)), ("lm_head", (cfg["vocab"], h))]
    return out


def numel(shape):
    n = 1
    for s in shape:
        n *= int(s)
    return n


# ------------------------------------------------------------ host draws
CFG_SMALL, CFG_SUBULP, CFG_F32, CFG_CONVERT, CFG_SHARDS, CFG_LLAMA = 1, 2, 3, 4, 5, 6
CFG_GEMM, CFG_RANK = 7, 8

GEMM_LLAMA3_8B_MLP_UP = dict(m=8192, n=LLAMA3_8B["ffn"], k=LLAMA3_8B["hidden"])


def host_rng(cfg_id, seed=0, step=0):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg_id, seed, step])))


def normal_f32(rng, n, std):
    return (rng.standard_normal(n) * std).astype(np.float32)


def f32_to_bf16_bits(x):
    """float32 numpy array -> uint16 bf16 patterns by torch's RNE cast."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_tensor(h, device):
    return torch.from_numpy(np.ascontiguousarray(h, dtype=np.uint16).view(np.int16)).view(
        torch.bfloat16).to(device)


def tensor_to_bf16_bits(t):
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


SPECIAL_F32_BITS = np.array([0x7F800000, 0xFF800000, 0x7FC00000, 0xFFC00000, 0x7F800001,
                             0x7FFFFFFF, 0xFFFFFFFF, 0xFF800001, 0x7F7FFFFF, 0xFF7FFFFF],
                            dtype=np.uint32)


def inject_specials(x, fraction, rng):
    """Replace round(fraction * n) distinct positions of float32 array x (in
    place) by a cycle over SPECIAL_F32_BITS. Returns the positions."""
    n = x.size
    k = int(round(fraction * n))
    pos = np.sort(rng.choice(n, size=k, replace=False))
    x.view(np.uint32)[pos] = SPECIAL_F32_BITS[np.arange(k) % SPECIAL_F32_BITS.size]
    return pos


# ---------------------------------------------------------- device draws
def device_generator(device, cfg_id, seed=0, step=0):
    g = torch.Generator(device=device)
    g.manual_seed((cfg_id << 40) ^ (seed << 20) ^ step)
    return g


def device_normal(n, std, gen, device, dtype):
    x = torch.randn(n, generator=gen, device=device, dtype=torch.float32)
    x.mul_(std)
    return x if dtype == torch.float32 else x.to(dtype)


STATE_ALIGN = 64  # elements of f32: flat-state views start on 256-byte boundaries


def zero_states(numels, device, layout="flat"):
    """f32 zero moment states (exp_avg, exp_avg_sq) for tensors of these
    sizes, allocated after the parameters and gradients as an optimizer
    does at its first step. "flat": two buffers, one per moment, each
    tensor's state a view starting on a 256-byte boundary (the layout
    AdamWSR allocates); "separate": one allocation per state, per tensor in
    turn (the layout of zeros_like per parameter)."""
    if layout == "separate":
        return [(torch.zeros(n, dtype=torch.float32, device=device),
                 torch.zeros(n, dtype=torch.float32, device=device)) for n in numels]
    if layout != "flat":
        raise ValueError(layout)
    offs, total = [], 0
    for n in numels:
        offs.append(total)
        total += (n + STATE_ALIGN - 1) // STATE_ALIGN * STATE_ALIGN
    m = torch.zeros(max(total, 1), dtype=torch.float32, device=device)
    v = torch.zeros(max(total, 1), dtype=torch.float32, device=device)
    return [(m[o:o + n], v[o:o + n]) for o, n in zip(offs, numels)]


def llama3_8b_state(device, seed=0, param_std=0.02, grad_std=1e-3, cfg=LLAMA3_8B,
                    states="flat"):
    """Allocates the full list on `device`: list of dicts with name, param,
    grad, exp_avg, exp_avg_sq, base_index (running total of numel). Params
    and grads first (the model), then the moment states (see zero_states)."""
    gen = device_generator(device, CFG_LLAMA, seed)
    out, base = [], 0
    for name, shape in llama3_8b_shapes(cfg):
        n = numel(shape)
        if len(shape) == 1:
            p = torch.ones(n, dtype=torch.bfloat16, device=device)
        else:
            p = device_normal(n, param_std, gen, device, torch.bfloat16)
        g = device_normal(n, grad_std, gen, device, torch.bfloat16)
        out.append(dict(name=name, param=p, grad=g, base_index=base))
        base += n
    for t, (m, v) in zip(out, zero_states([t["param"].numel() for t in out], device, states)):
        t["exp_avg"], t["exp_avg_sq"] = m, v
    return out


def llama3_8b_rank_pieces(rank, ranks, cfg=LLAMA3_8B):
    """(name, shape, offset, length, base_index) of every piece rank `rank`
    of `ranks` holds: the flattened list is split into `ranks` equal
    contiguous ranges, and a tensor crossing a range boundary is cut there.
    base_index is the piece's global position (its tensor's running total
    of numel plus the offset)."""
    shapes = llama3_8b_shapes(cfg)
    total = sum(numel(s) for _, s in shapes)
    lo, hi = total * rank // ranks, total * (rank + 1) // ranks
    out, base = [], 0
    for name, shape in shapes:
        n = numel(shape)
        a, b = max(base, lo), min(base + n, hi)
        if a < b:
            out.append((name, shape, a - base, b - a, a))
        base += n
    return out


def llama3_8b_rank_state(device, rank, ranks, seed=0, param_std=0.02, grad_std=1e-3,
                         cfg=LLAMA3_8B, states="flat"):
    """Allocates one rank's pieces on `device`: list of dicts with name,
    offset, param, grad, exp_avg, exp_avg_sq, base_index (states as in
    llama3_8b_state)."""
    gen = device_generator(device, CFG_RANK, seed, rank)
    out = []
    for name, shape, off, n, base in llama3_8b_rank_pieces(rank, ranks, cfg):
        if len(shape) == 1:
            p = torch.ones(n, dtype=torch.bfloat16, device=device)
        else:
            p = device_normal(n, param_std, gen, device, torch.bfloat16)
        g = device_normal(n, grad_std, gen, device, torch.bfloat16)
        out.append(dict(name=name, offset=off, param=p, grad=g, base_index=base))
    for t, (m, v) in zip(out, zero_states([t["param"].numel() for t in out], device, states)):
        t["exp_avg"], t["exp_avg_sq"] = m, v
    return out


def gemm_operands_host(m, n, k, kind, seed=0):
    """bf16 patterns of A (m x k) and B (n x k)."""
    rng = host_rng(CFG_GEMM, seed, (m * 1000003 + n) * 1000003 + k)
    if kind == "int":
        a = rng.integers(-8, 9, size=(m, k)).astype(np.float32)
        b = rng.integers(-8, 9, size=(n, k)).astype(np.float32)
    elif kind == "randn":
        a = rng.standard_normal((m, k)).astype(np.float32)
        b = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    else:
        raise ValueError(kind)
    return f32_to_bf16_bits(a).reshape(m, k), f32_to_bf16_bits(b).reshape(n, k)


def gemm_operands_device(m, n, k, device, seed=0):
    """The "randn" operands drawn on the device (for sizes too large to draw
    on the host): bf16 tensors A (m x k) and B (n x k)."""
    gen = device_generator(device, CFG_GEMM, seed)
    a = device_normal(m * k, 1.0, gen, device, torch.bfloat16).view(m, k)
    b = device_normal(n * k, 0.02, gen, device, torch.bfloat16).view(n, k)
    return a, b
