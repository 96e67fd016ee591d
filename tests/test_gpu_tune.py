"""The geometry tuner on the GPU: every candidate it reports was timed, the
choice is the fastest, and encoding with the chosen geometry gives a blob
whose fused GEMV matches the oracle."""
import numpy as np
import pytest

import oracle
import workloads
from decode_gemv_byte_amd import tune


def _tol_ok(y, w, x):
    # FP32 output: within 2^-10 of sum |w x| per row of the FP64 oracle
    yr, a = oracle.gemv(w, x)
    return bool(np.all(np.abs(np.asarray(y, np.float64) - yr) <= 2.0 ** -10 * a))


@pytest.mark.gpu
@pytest.mark.parametrize("batch", [1, 4])
def test_tune_two_matrices_and_parity(batch):
    import torch

    import decode_gemv_byte_amd as nwc
    mats = [workloads.gaussian_bits((1000, 2560), 0.02, seed=s) for s in (11, 12)]
    r = tune.tune_geometry(mats, batch=batch, reps=20)
    assert len(r.candidates) == len(tune.DEFAULT_CANDIDATES)
    timed = [c for c in r.candidates if c.us != float("inf")]
    assert timed and all(c.us > 0 for c in timed)
    assert r.best.us == min(c.us for c in timed)
    d = r.as_dict()
    assert d["best"] == r.params() and d["batch"] == batch
    # the chosen geometry, end to end: parity of the fused product
    dev = torch.device("cuda", 0)
    rng = np.random.default_rng(3)
    for w in mats:
        blob = nwc.nwc_encode(w, r.params())
        info = nwc.nwc_inspect(blob)
        assert info.tile_rows == r.best.tile_rows and info.max_code_len == r.best.max_code_len
        x = workloads.f32_to_bf16_bits(rng.standard_normal((batch, w.shape[1])).astype(np.float32))
        bd = torch.from_numpy(blob).to(dev)
        xd = torch.from_numpy(x.view(np.int16)).to(dev)
        y = torch.empty((batch, w.shape[0]), dtype=torch.float32, device=dev)
        ws = torch.zeros(max(1, nwc.nwc_workspace_size(info, batch)), dtype=torch.uint8, device=dev)
        if batch == 1:
            nwc.nwc_gemv(info, bd, xd[0], y[0], ws)
        else:
            nwc.nwc_gemm_skinny(info, bd, xd, y, ws)
        yh = y.cpu().numpy()
        for b in range(batch):
            assert _tol_ok(yh[b], w, x[b])
