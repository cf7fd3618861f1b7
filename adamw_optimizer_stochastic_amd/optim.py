"""AdamWSR: a torch.optim.Optimizer over the fused AdamW-SR kernels.

From the "adamw-sr" page (Usage section): a drop-in for torch.optim.AdamW
taking lr, weight_decay and seed; optimizer states are float32; parameters
and gradients may be f32 or bf16; stochastic rounding is on by default for
bf16 parameters. The Method section derives the random bits from each
element's position in the whole parameter set; reading: the position of a
tensor's first element is the running total of numel over all parameters
of the optimizer, in param_groups order and then parameter order, fixed
when the parameter is added (later groups are appended after it).

Unsupported AdamW options raise NotImplementedError rather than silently
computing something else.

Moment states live in flat buffers: the f32 exp_avg of every parameter that
gets its state in one step is a view into one contiguous buffer per device,
and so is exp_avg_sq, each view starting on a 256-byte boundary (the layout
of flat-buffer optimizers and ZeRO partitions), allocated once the
parameters and gradients exist. On MI355X the step over a Llama-3-8B-shaped
list ran at 6.02-6.10 TB/s with states allocated that way (flat about 1%
ahead of one allocation per state), and at 5.61-5.62 TB/s when each
tensor's states were allocated between the parameters, gradients and their
temporaries, tensor by tensor.
"""

import torch

from . import ops


def _step_count(x):
    """A saved step count as a Python int: from an int, or from a tensor of
    any dtype (torch's own AdamW saves a float32 tensor)."""
    if isinstance(x, torch.Tensor):
        x = x.item()
    if float(x) != int(x) or int(x) < 0:
        raise ValueError(f"step count must be a non-negative integer (got {x})")
    return int(x)


class AdamWSR(torch.optim.Optimizer):
    def __init__(self, params, lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=1e-2,
                 *, seed=0, rounding="sr", amsgrad=False, maximize=False, foreach=None,
                 capturable=False, differentiable=False, fused=None):
        if amsgrad:
            raise NotImplementedError("AdamWSR: amsgrad is not supported")
        if maximize:
            raise NotImplementedError("AdamWSR: maximize is not supported")
        if capturable or differentiable:
            raise NotImplementedError("AdamWSR: capturable/differentiable are not supported")
        if foreach or fused:
            raise NotImplementedError("AdamWSR is always one fused multi-tensor kernel; "
                                      "foreach/fused flags are not accepted")
        if isinstance(lr, torch.Tensor):
            raise NotImplementedError("AdamWSR: tensor lr is not supported")
        if not 0.0 <= lr:
            raise ValueError(f"Invalid learning rate: {lr}")
        if not 0.0 <= eps:
            raise ValueError(f"Invalid epsilon value: {eps}")
        if not (0.0 <= betas[0] < 1.0 and 0.0 <= betas[1] < 1.0):
            raise ValueError(f"Invalid beta parameters: {betas}")
        if not 0.0 <= weight_decay:
            raise ValueError(f"Invalid weight_decay value: {weight_decay}")
        if rounding not in ("sr", "rn"):
            raise ValueError("rounding must be 'sr' or 'rn'")
        if not (isinstance(seed, int) and 0 <= seed < (1 << 32)):
            raise ValueError("seed must be an integer in [0, 2**32)")
        self.seed = seed
        self._base_index = {}
        self._next_index = 0
        self._workspaces = {}
        self._desc_cache = {}
        defaults = dict(lr=lr, betas=tuple(betas), eps=eps, weight_decay=weight_decay,
                        rounding=rounding)
        super().__init__(params, defaults)

    def add_param_group(self, param_group):
        super().add_param_group(param_group)
        for p in self.param_groups[-1]["params"]:
            if p in self._base_index:
                continue
            if p.is_sparse or p.is_complex() or p.dtype not in (torch.float32, torch.bfloat16):
                raise NotImplementedError(
                    f"AdamWSR supports dense float32/bfloat16 params (got {p.dtype})")
            self._base_index[p] = self._next_index
            self._next_index += p.numel()

    def base_index(self, p):
        """Global position of element 0 of parameter p."""
        return self._base_index[p]

    @staticmethod
    def _flat_states(params):
        """Zero f32 exp_avg / exp_avg_sq views for `params` (one device), in
        two flat buffers, each view 256-byte aligned."""
        align = 64
        offs, total = [], 0
        for p in params:
            offs.append(total)
            total += (p.numel() + align - 1) // align * align
        dev = params[0].device
        bufs = (torch.zeros(max(total, 1), dtype=torch.float32, device=dev),
                torch.zeros(max(total, 1), dtype=torch.float32, device=dev))
        return [(bufs[0][o:o + p.numel()].view(p.shape), bufs[1][o:o + p.numel()].view(p.shape))
                for o, p in zip(offs, params)]

    def _init_states(self, params):
        """Creates the state of every parameter in `params` that has none:
        step 0 and zero moments in flat buffers per device."""
        by_dev = {}
        for p in params:
            if len(self.state[p]) == 0:
                by_dev.setdefault(p.device, []).append(p)
        for ps in by_dev.values():
            for p, (m, v) in zip(ps, self._flat_states(ps)):
                # int64, not torch's float32: a float32 count stops at 2**24,
                # and from there every step would reuse one key (seed, step)
                self.state[p] = {"step": torch.tensor(0, dtype=torch.int64), "exp_avg": m,
                                 "exp_avg_sq": v}

    def _workspace(self, device, params):
        """A cached workspace for this device and its current stream, big
        enough for a step over `params`. The step kernels read their metadata
        from the workspace asynchronously, so a workspace is only reused on
        the stream that last used it (stream order then separates the
        steps); another stream gets its own. The size bound depends only on
        the number of tensors and their sizes."""
        sizes = tuple(p.numel() for p in params)
        key = (device, torch.cuda.current_stream(device).cuda_stream)
        ws, known = self._workspaces.get(key, (None, None))
        if ws is None or known != sizes:
            need = ops.workspace_bytes(sizes)
            if ws is None or ws.numel() < need:
                ws = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
            self._workspaces[key] = (ws, sizes)
        return ws

    @torch.no_grad()
    def step(self, closure=None):
        loss = None
        if closure is not None:
            with torch.enable_grad():
                loss = closure()
        live = [p for g in self.param_groups for p in g["params"] if p.grad is not None]
        for p in live:
            if p.grad.is_sparse:
                raise NotImplementedError("AdamWSR does not support sparse gradients")
            if not p.is_contiguous() or not p.grad.is_contiguous():
                raise NotImplementedError("AdamWSR needs contiguous params and grads")
        self._init_states(live)
        for gi, group in enumerate(self.param_groups):
            beta1, beta2 = group["betas"]
            ps_all = [p for p in group["params"] if p.grad is not None]
            if not ps_all:
                continue
            states = [self.state[p] for p in ps_all]
            counts = [st["step"] for st in states]
            # every count moves on together (one call, not one per tensor)
            torch._foreach_add_(counts, 1)
            ts = [int(t) for t in torch.stack(counts).tolist()]
            batches = {}  # (device, step) -> lists
            for p, st, t in zip(ps_all, states, ts):
                b = batches.setdefault((p.device, t), ([], [], [], [], []))
                b[0].append(p)
                b[1].append(p.grad)
                b[2].append(st["exp_avg"])
                b[3].append(st["exp_avg_sq"])
                b[4].append(self._base_index[p])
            for (device, t), (ps, gs, ms, vs, bases) in batches.items():
                # the checked descriptors are reused while the tensors stay put
                cache = self._desc_cache.setdefault((gi, device, tuple(map(id, ps))), {})
                ops.adamw_step(ps, gs, ms, vs, bases, lr=group["lr"], beta1=beta1, beta2=beta2,
                               eps=group["eps"], weight_decay=group["weight_decay"], step=t,
                               seed=self.seed, rounding=group["rounding"],
                               workspace=self._workspace(device, ps), _cache=cache)
        return loss

    def state_dict(self):
        sd = super().state_dict()
        sd["adamw_sr"] = {"seed": self.seed}
        return sd

    def load_state_dict(self, state_dict):
        """Like torch's, except that the moment states stay float32 whatever
        the parameter dtype (torch's loader would cast them to it)."""
        extra = state_dict.get("adamw_sr")
        saved_state = state_dict.get("state", {})
        plain = {k: v for k, v in state_dict.items() if k not in ("adamw_sr", "state")}
        plain["state"] = {}
        super().load_state_dict(plain)
        saved_ids = [i for g in state_dict["param_groups"] for i in g["params"]]
        params = [p for g in self.param_groups for p in g["params"]]
        loaded = [(p, saved_state[pid]) for pid, p in zip(saved_ids, params)
                  if saved_state.get(pid) is not None]
        for p, _ in loaded:
            self.state[p] = {}
        self._init_states([p for p, _ in loaded])   # flat buffers, then the saved values
        for p, st in loaded:
            state = self.state[p]
            state["step"].fill_(_step_count(st["step"]))
            state["exp_avg"].copy_(st["exp_avg"].detach().reshape(p.shape))
            state["exp_avg_sq"].copy_(st["exp_avg_sq"].detach().reshape(p.shape))
        if extra is not None:
            self.seed = int(extra["seed"])
