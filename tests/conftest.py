import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU; parity tests through the C-ABI")
    # The full-size GPU parity tests run the oracle on a pool of CPU workers;
    # their fork server must start before this process first uses the GPU.
    if "not gpu" not in (config.option.markexpr or ""):
        tests_dir = os.path.dirname(os.path.abspath(__file__))
        if tests_dir not in sys.path:
            sys.path.insert(0, tests_dir)
        import _cpu_pool
        _cpu_pool.start()
