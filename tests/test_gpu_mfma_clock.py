"""Matrix-core issue rate and clock under load (measurement support).

The probe library (csrc/probe_mfma_clock.hip, built next to the decode
library) makes every wave issue independent MFMAs back to back and records
shader-clock cycles and 100 MHz real time.  The issue rate per wave is a
property of the instruction (asserted); the clock is the part's response to
the load and to the operand data (printed: run with -s; the figures behind
the roofline discussion of the decode kernels, which divide by the published
2.5 PFLOP/s that the part reaches only with few matrix cores busy).
"""

import ctypes
import os

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROBE_LIB = os.path.join(ROOT, "mla_latent_cache_decode_amd", "libmla_probe.so")
ITERS = 4000
MFMA_PER_ITER = 8
CYCLES = {0: 32.0, 1: 64.0}        # f16 32x32x16: 8 passes; scaled fp8 32x32x64: 16 passes
NAMES = {0: "v_mfma_f32_32x32x16_f16", 1: "v_mfma_scale_f32_32x32x64_f8f6f4"}


def _lib():
    if not os.path.exists(PROBE_LIB):
        pytest.skip("libmla_probe.so is not built")
    lib = ctypes.CDLL(PROBE_LIB)
    lib.mla_probe_mfma_clock.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_void_p]
    lib.mla_probe_mfma_clock.restype = ctypes.c_int
    lib.mla_probe_mfma_valu.argtypes = lib.mla_probe_mfma_clock.argtypes
    lib.mla_probe_mfma_valu.restype = ctypes.c_int
    return lib


def test_probe_rejects_bad_arguments_without_a_gpu_call():
    lib = _lib()
    dummy = ctypes.c_void_p(16)
    for kind, grid, iters in ((2, 1, 1), (0, 0, 1), (0, 4097, 1), (1, 1, 0), (1, 1, 1000001)):
        assert lib.mla_probe_mfma_clock(kind, grid, iters, dummy, dummy, None) != 0
    for kind, n, iters in ((2, 0, 1), (0, 3, 1), (1, 20, 1), (0, 4, 0), (1, 8, 1000001)):
        assert lib.mla_probe_mfma_valu(kind, n, iters, dummy, dummy, None) != 0


@pytest.mark.gpu
def test_mfma_issue_rate_is_fixed_and_the_clock_falls_with_load():
    import torch
    lib = _lib()
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(1)
    data = {"random": torch.tensor(rng.uniform(-1.0, 1.0, 1024), dtype=torch.float32, device=dev),
            "zeros": torch.zeros(1024, dtype=torch.float32, device=dev)}
    stream = torch.cuda.current_stream()
    rows = []
    for kind in (0, 1):
        for grid, name in ((1, "random"), (256, "random"), (256, "zeros")):
            out = torch.zeros(grid * 4 * 2, dtype=torch.int64, device=dev)
            # twenty back-to-back launches (tens of ms under load); the last one is read
            for _ in range(20):
                st = lib.mla_probe_mfma_clock(kind, grid, ITERS, data[name].data_ptr(), out.data_ptr(),
                                              ctypes.c_void_p(stream.cuda_stream))
                assert st == 0, st
            torch.cuda.synchronize()
            v = out.cpu().numpy().reshape(grid * 4, 2).astype(np.float64)
            per_mfma = np.median(v[:, 0]) / (ITERS * MFMA_PER_ITER)
            clock = np.median(v[:, 0] / (v[:, 1] * 10.0))
            rows.append((NAMES[kind], grid, name, per_mfma, clock))
            # within 5 % of the instruction's passes (the loop's own control
            # instructions add about a cycle per MFMA)
            assert abs(per_mfma / CYCLES[kind] - 1.0) <= 0.05, (kind, grid, name, per_mfma)
    print()
    print(f"{'instruction':36s} {'CUs':>4s} {'operands':>8s} {'cycles/MFMA/wave':>17s} {'clock GHz':>10s}")
    for n, g, d, c, f in rows:
        print(f"{n:36s} {g:4d} {d:>8s} {c:17.2f} {f:10.3f}")


@pytest.mark.gpu
def test_valu_instructions_under_a_running_mfma():
    """One CU: a few conversions per MFMA issue free while the matrix core
    works, more stretch the MFMA step (the hooks of the decode's tile loop
    are priced by this)."""
    import torch
    lib = _lib()
    dev = torch.device("cuda:0")
    data = torch.tensor(np.random.default_rng(2).uniform(-1.0, 1.0, 1024), dtype=torch.float32, device=dev)
    out = torch.zeros(4, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream()
    cyc = {}
    for kind in (0, 1):
        for n in (0, 4, 8, 12, 16):
            for _ in range(3):
                assert lib.mla_probe_mfma_valu(kind, n, ITERS, data.data_ptr(), out.data_ptr(),
                                               ctypes.c_void_p(stream.cuda_stream)) == 0
            torch.cuda.synchronize()
            cyc[kind, n] = float(np.median(out.cpu().numpy())) / (ITERS * 2)
    print()
    print(f"{'instruction':36s} " + " ".join(f"{n:>7d}" for n in (0, 4, 8, 12, 16)) + "  conversions per MFMA")
    for kind in (0, 1):
        print(f"{NAMES[1 - kind]:36s} " + " ".join(f"{cyc[kind, n]:7.2f}" for n in (0, 4, 8, 12, 16)))
    assert abs(cyc[0, 0] / 64.0 - 1.0) <= 0.05 and abs(cyc[1, 0] / 32.0 - 1.0) <= 0.05
    assert cyc[0, 4] <= 1.1 * cyc[0, 0]          # four hide under a 64-cycle MFMA
    assert cyc[0, 16] >= 1.3 * cyc[0, 0]         # sixteen do not
    assert cyc[1, 8] >= 1.3 * cyc[1, 0]          # eight do not under a 32-cycle one
