"""A pool of CPU worker processes that runs the oracle over large inputs in
pieces, beside the GPU tests (the full-size parity cases).

The workers are forked from a server process that the test session starts
before anything touches the GPU (tests/conftest.py), so none of them holds
the GPU or inherits its state; inputs and results travel through pipes.
The pool is sized to the CPUs this process may run on, at most 16 (the
host share of one GPU on the machines these tests target)."""

import multiprocessing
import os

_ctx = None


def start():
    """Start the fork server (call before the GPU is first used)."""
    global _ctx
    if _ctx is not None:
        return
    ctx = multiprocessing.get_context("forkserver")
    ctx.set_forkserver_preload(["numpy", "oracle", "_oracle_tasks"])
    from multiprocessing import forkserver
    forkserver.ensure_running()
    _ctx = ctx


def workers():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def pool():
    """A new multiprocessing pool (use it as a context manager)."""
    if _ctx is None:
        raise RuntimeError("the CPU pool's server was not started before the GPU was used "
                           "(tests/conftest.py starts it)")
    return _ctx.Pool(workers())
