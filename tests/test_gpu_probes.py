"""GPU checks of the calibration kernels: the streaming read touches every 16-byte word of
its buffer (a sentinel placed in the first or last word is seen), writes nothing for a
buffer without one, and the matrix-instruction loop runs to completion."""
import os

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SENTINEL = 0x9E3779B9


@pytest.mark.parametrize("nbytes", [16, 4096, (24 << 20) + 48])
@pytest.mark.parametrize("where", ["first", "last", "none"])
def test_probe_read_covers_the_buffer(lib, nbytes, where):
    import torch
    import w4a16_mixed_precision_offline_amd as w4
    buf = torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda")
    if where != "none":
        idx = 0 if where == "first" else nbytes // 4 - 1
        buf[idx] = torch.tensor(SENTINEL, dtype=torch.int64).to(torch.int32)
    out = torch.zeros(4, dtype=torch.int32, device="cuda")
    w4.w4a16_probe_read(buf, nbytes, out)
    got = int(out[0].item()) & 0xFFFFFFFF
    assert got == (SENTINEL if where != "none" else 0)
    assert int(out[1:].abs().sum().item()) == 0


def test_probe_mfma_runs(lib):
    import torch
    import w4a16_mixed_precision_offline_amd as w4
    out = torch.zeros(4, dtype=torch.float32, device="cuda")
    w4.w4a16_probe_mfma(512, 64, out)
    torch.cuda.synchronize()
    assert float(out.abs().sum().item()) == 0.0
    assert w4.w4a16_probe_mfma_flops(512, 64) == 512 * 4 * 64 * 4 * 32768


def test_importing_the_binding_before_torch(lib):
    """The binding works whichever of it and torch a program imports first (torch ships
    its own HIP runtime with the system runtime's soname; the binding loads torch's before
    the library, so one runtime serves both).  Runs in a fresh interpreter."""
    import subprocess
    import sys
    code = (
        "import ctypes, sys\n"
        f"sys.path.insert(0, {ROOT!r})\n"
        "import w4a16_mixed_precision_offline_amd as w4\n"
        "import torch\n"
        "x = torch.zeros(16, dtype=torch.float32, device='cuda')\n"
        "rc = w4._lib.w4a16_probe_read(ctypes.c_void_p(x.data_ptr()), 64,\n"
        "                              ctypes.c_void_p(x.data_ptr()), None)\n"
        "torch.cuda.synchronize()\n"
        "print('rc', rc)\n"
        "sys.exit(0 if rc == 0 else 1)\n")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, (r.stdout, r.stderr[-2000:])
