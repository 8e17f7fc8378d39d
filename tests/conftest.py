import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def _gpu_visible() -> bool:
    # counting devices does not initialise the HIP runtime
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


# The GPU modules load libq4.so when they are imported.  Without the built
# library and without a GPU (a fresh CPU-only checkout) only the CPU tier can
# run, so they are not collected; with a GPU visible they are collected and a
# missing library fails loudly at import.
_LIB = os.path.join(ROOT, "quantized_q4_block_amd", "libq4.so")
collect_ignore_glob = []
if not os.path.exists(_LIB) and not _gpu_visible():
    collect_ignore_glob = ["test_gpu_*.py", "test_zz_*.py"]


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")
