"""The C ABI called from several host threads at once, each on its own HIP
stream (ctypes releases the GIL during the call): first calls of new
geometries race on the plan cache and the dynamic-LDS limit, and every
result must equal the one computed alone.  The geometries are used by no
other test, so their plans are made here, concurrently.  Offsets are small
(no sample leaves the tiles' halo), so grad_value has no device atomics.
The output and grad_offset_mask are deterministic and compared bit for bit;
grad_value sums each cell's records in the order the block's LDS counters
placed them, which depends on wave timing, so it is held to the fp32 parity
bound (1e-5 + 1e-5 |x|).
"""
import threading

import pytest
import torch

from dynamic_sparse_vision_amd import dcnv4
from dynamic_sparse_vision_amd import flash_deform_attn as fda
from dynamic_sparse_vision_amd.workloads import FdaWorkload, Workload
from tests.test_gpu_fdattn import to_dev
from tests.test_gpu_parity import device_inputs, say

pytestmark = pytest.mark.gpu

CASES = [
    Workload("conc_fp32_37x41", 2, 37, 41, 64, 4, "fp32", seed=501, sigma_value=1.0, sigma_off=1.0,
             sigma_m=0.7, direction="fwd"),
    Workload("conc_bf16_29x33_k5", 2, 29, 33, 32, 2, "bf16", seed=502, sigma_value=1.0, sigma_off=1.0,
             sigma_m=0.7, direction="fwd", kernel=(5, 5), pad=(2, 2)),
    Workload("conc_fp16_31x23_g8", 1, 31, 23, 128, 8, "fp16", seed=503, sigma_value=1.0, sigma_off=1.0,
             sigma_m=0.7, direction="fwd"),
]


def _run(w, d):
    out = dcnv4.forward(d["v"], d["om"], **w.kwargs())
    gv, gom = dcnv4.backward(d["v"], d["om"], d["g"], **w.kwargs())
    return out, gv, gom


def test_threads_on_separate_streams():
    inputs = [device_inputs(w, with_grad=True) for w in CASES]
    torch.cuda.synchronize()
    results = {}
    errors = []
    n_threads, rounds = 6, 8
    start = threading.Barrier(n_threads)

    def worker(t):
        try:
            s = torch.cuda.Stream()
            start.wait()
            with torch.cuda.stream(s):
                for r in range(rounds):
                    i = (t + r) % len(CASES)
                    got = _run(CASES[i], inputs[i])
                    s.synchronize()
                    results.setdefault((t, r), (i, [x.clone() for x in got]))
                    s.synchronize()
        except Exception as e:   # reported by the main thread
            errors.append((t, repr(e)))

    say(f"[concurrency] {n_threads} threads x {rounds} rounds over {[w.name for w in CASES]}")
    threads = [threading.Thread(target=worker, args=(t,)) for t in range(n_threads)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    alone = [[x.clone() for x in _run(w, d)] for w, d in zip(CASES, inputs)]
    torch.cuda.synchronize()
    for (t, r), (i, got) in sorted(results.items()):
        for name, a, b in zip(("output", "grad_value", "grad_offset_mask"), got, alone[i]):
            if name == "grad_value":
                ok = bool(((a - b).abs() <= 1e-5 + 1e-5 * b.abs()).all())
            else:
                ok = torch.equal(a, b)
            assert ok, f"thread {t} round {r} {CASES[i].name} {name} differs from the call alone"
    say(f"  {len(results)} threaded calls agree with the calls alone")


FDA_CASES = [
    FdaWorkload("conc_fda_fp32", 2, ((9, 11), (5, 6), (3, 3)), 3, 32, 4, "fp32", seed=511, Q=71),
    FdaWorkload("conc_fda_bf16", 1, ((13, 7), (7, 4)), 2, 16, 3, "bf16", seed=512, Q=0),
]


def test_flash_deform_attn_threads_on_separate_streams():
    """The same for flash deformable attention (each backward takes its own
    workspace); the output and grad_loc_attn bit for bit, grad_value within
    the fp32 bound."""
    inputs = []
    for w in FDA_CASES:
        (v, _), (la, _), (g, _) = to_dev(w.make_inputs(), w.dtype)
        inputs.append((v, la, g))
    torch.cuda.synchronize()

    def run(i):
        w = FDA_CASES[i]
        v, la, g = inputs[i]
        out = fda.forward(v, w.shapes, la, w.K)
        gv, gla = fda.backward(v, w.shapes, la, g, w.K)
        return out, gv, gla

    results, errors = {}, []
    n_threads, rounds = 4, 6
    start = threading.Barrier(n_threads)

    def worker(t):
        try:
            s = torch.cuda.Stream()
            start.wait()
            with torch.cuda.stream(s):
                for r in range(rounds):
                    i = (t + r) % len(FDA_CASES)
                    got = run(i)
                    s.synchronize()
                    results[(t, r)] = (i, [x.clone() for x in got])
                    s.synchronize()
        except Exception as e:
            errors.append((t, repr(e)))

    say(f"[concurrency] flash deformable attention, {n_threads} threads x {rounds} rounds")
    threads = [threading.Thread(target=worker, args=(t,)) for t in range(n_threads)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    alone = [[x.clone() for x in run(i)] for i in range(len(FDA_CASES))]
    torch.cuda.synchronize()
    for (t, r), (i, got) in sorted(results.items()):
        for name, a, b in zip(("output", "grad_value", "grad_loc_attn"), got, alone[i]):
            if name == "grad_value":
                ok = bool(((a - b).abs() <= 1e-5 + 1e-5 * b.abs()).all())
            else:
                ok = torch.equal(a, b)
            assert ok, f"thread {t} round {r} {FDA_CASES[i].name} {name} differs from the call alone"
    say(f"  {len(results)} threaded calls agree with the calls alone")
