"""The pages' statistical law on the oracle (CPU only).

"ssm-state-quantization" README, Findings: the relative state error of a rounded Mamba-2 state
grows with the decay, like 1/sqrt(1 - lambda^2) (the error recurrence Delta_t = A_t Delta_(t-1)
+ R_t of "Mamba state quantization for inference", *Quantization error returns on the next
token*, summed over the state's memory).  The law is qualitative here (the pages measured it with
a per-head scale and model activations); this checks its direction on the synthetic inputs:
after 400 rounded steps the slow-decay band's relative error exceeds the medium band's, which
exceeds the fast band's.  A state that did not carry its rounding error into the next token
would show the same per-step error in every band.
"""
import numpy as np
import pytest

import oracle
import synth


@pytest.mark.parametrize("fmt", ["int8_asym", "int8_sym", "int4_asym"])
def test_relative_state_error_grows_with_the_decay(fmt):
    B, H, G, P, T = 2, 6, 1, 16, 400
    x, dt, Bm, Cm, A, D = synth.mamba2_scan_inputs(7, 0, B, T, H, G, P, 128)
    rows = B * H * P
    lam = np.exp(dt.astype(np.float64) * A.astype(np.float64)[None, None, :])
    med = np.median(lam, axis=(0, 1))
    # head h is in band h mod 3: median decay <= 0.9, in (0.9, 0.99], above 0.99
    assert np.all(med[0::3] <= 0.9) and np.all((med[1::3] > 0.9) & (med[1::3] <= 0.99)) and np.all(med[2::3] > 0.99)
    sq = oracle.make_state(fmt, rows, 128)
    sf = oracle.make_state("fp32", rows, 128)
    oracle.mamba2_scan(sq, x, dt, A, Bm, Cm, D)
    oracle.mamba2_scan(sf, x, dt, A, Bm, Cm, D)
    hq = sq.dequant().astype(np.float64).reshape(B, H, P, 128)
    hf = sf.h.astype(np.float64).reshape(B, H, P, 128)
    err = np.linalg.norm(hq - hf, axis=3) / np.linalg.norm(hf, axis=3)
    band = [np.median(err[:, b::3]) for b in range(3)]
    assert band[1] > 1.3 * band[0] and band[2] > 1.5 * band[1], band
    # direction of the law: the ratio of slowest to fastest band follows 1/sqrt(1 - lambda^2)
    pred = [np.median(1 / np.sqrt(1 - med[b::3] ** 2)) for b in range(3)]
    assert band[2] / band[0] > 0.3 * pred[2] / pred[0], (band, pred)
