"""Parity of the backward pass at full workload sizes, in the launch
configuration bench.py --backward times: for two seeded heads, 128 query rows
of dQ and 128 keys of dK and dV are checked against the oracle, each element
within twice the first-order bound of the library's bf16 roundings (the gate
of the test-size backward tests).  The backward of the sampled heads takes
the oracle's forward output and row statistic, so the comparison sees the
backward's arithmetic only; the other heads use the library's forward."""
import multiprocessing as mp
from multiprocessing import shared_memory

import numpy as np
import pytest
import torch

from tests import fullsize as FS
from workloads import CONFIGS, make_inputs

pytestmark = pytest.mark.gpu

SAMPLES = 128


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["llm_prefill_fp8_causal", "dense_fp8_16k"])
def test_full_size_backward_sampled(gpu_lib, name):
    cfg = CONFIGS[name]
    print("full-size backward", name, flush=True)
    x = make_inputs(cfg, as_torch=True)
    rng = np.random.default_rng(1000 * cfg.index + 8)
    heads = rng.choice(cfg.H, 2, replace=False)
    rows = np.sort(rng.choice(cfg.n_real, SAMPLES, replace=False))
    cols = np.sort(rng.choice(cfg.n_real, SAMPLES, replace=False))
    g = torch.Generator().manual_seed(1000 * cfg.index + 7)
    dout = torch.randn((cfg.B, cfg.H, cfg.n_real, cfg.d), generator=g).to(torch.bfloat16)
    mode = {"dense": 0, "causal": 1}[cfg.mode]
    _, bn = gpu_lib.attention_info("fp8_block", cfg.d, mode)
    arrays = {"q": x["q"], "k": x["k"], "v": x["v"], "do": dout.float().numpy()}
    shms = []
    try:
        for a in arrays.values():
            shm = shared_memory.SharedMemory(create=True, size=a.nbytes)
            shms.append(shm)
            np.ndarray(a.shape, np.float32, buffer=shm.buf)[:] = a
        jobs = [(name, [s.name for s in shms], arrays["q"].shape, int(h), rows, cols, bn) for h in heads]
        with mp.get_context("spawn").Pool(len(jobs)) as pool:
            pending = pool.imap_unordered(FS.head_backward_job, jobs, chunksize=1)
            dev = torch.device("cuda:0")
            qd, kd, vd = (x[n].to(dev) for n in ("q_t", "k_t", "v_t"))
            qq = gpu_lib.quantize(qd, "fp8_block", cfg.blk)
            kq = gpu_lib.quantize(kd, "fp8_block", cfg.blk)
            vq = gpu_lib.quantize(vd, "fp8_channel")
            del qd, kd, vd
            out, lse = gpu_lib.attention_dense(qq, kq, vq, causal=cfg.mode == "causal", lse=True)
            torch.cuda.synchronize()
            print("  gpu forward done", flush=True)
            results = list(pending)
    finally:
        for s in shms:
            s.close()
            s.unlink()
    print("  oracle done", flush=True)
    for head, o, l, _, _ in results:
        out[0, head] = torch.from_numpy(o).to(out.device)
        lse[0, head] = torch.from_numpy(l).to(lse.device)
    dq, dk, dv = gpu_lib.attention_backward(qq, kq, vq, out, dout.to(out.device), lse,
                                            causal=cfg.mode == "causal")
    torch.cuda.synchronize()
    for head, _, _, ref, bounds in results:
        got = (dq[0, head, rows].cpu().numpy(), dk[0, head, cols].cpu().numpy(),
               dv[0, head, cols].cpu().numpy())
        for nm, g_, r, b in zip("qkv", got, ref, bounds):
            assert np.all(np.isfinite(g_)), "head %d d%s: non-finite" % (head, nm)
            err = np.abs(g_.astype(np.float64) - r)
            scale = np.abs(r).max()
            lim = 2 * b + 1e-6 * scale
            print("  head %d d%s: max err/bound %.3f, max-abs %.3g of max|ref| %.3g" % (
                head, nm, (err / lim).max(), err.max(), scale), flush=True)
            assert np.all(err <= lim), "head %d d%s" % (head, nm)
            assert err.mean() <= 1e-3 * scale
