"""Pins of the progressive residual quantization oracle (QVG summary Sec. 2B)."""
import numpy as np

import datagen
from oracle import lloyd, prq
from oracle import quantize as Qz


def _tokens(T=400):
    w = datagen.make_workload("480p", heads=[0], n_chunks=1, chunk=T)
    return w.K[:, 0].astype(np.float64)


def test_one_stage_is_the_value_codec():
    X = _tokens()
    first, C, last, e = prq.prq_quantize(X, 1, 3, seed=5)
    assert first == []
    C2 = lloyd.lloyd(X, 256, 3, seed=5)
    ref = Qz.quantize_values(X, C2)
    assert np.array_equal(C, C2)
    for k in ("idx", "q", "zero"):
        assert np.array_equal(last[k], ref[k])
    assert np.array_equal(last["scale"], ref["scale"])


def test_reconstruction_error_is_the_last_stage_codec_error():
    """X - reconstruction = (e^{S-1} - its INT2 reconstruction) + the fp32
    roundings of the stage residuals; per channel |.| <= s_g / 2 (1 + 2^-22) plus
    that rounding (each residual exact to 2^-24 relative)."""
    X = _tokens()
    for S in (2, 3):
        first, C, last, e = prq.prq_quantize(X, S, 3, seed=7)
        Xh = prq.prq_reconstruct(first, C, last)
        s = np.repeat(np.asarray(last["scale"], np.float64), 64, axis=1)
        slack = 2.0 ** -23 * (np.abs(X) + S * np.max(np.abs(X)))
        assert np.all(np.abs(X - Xh) <= s / 2 * (1 + 2.0 ** -22) + slack)
        # the bound catches a dropped stage term
        Xbad = Xh - np.asarray(first[-1][0], np.float64)[np.asarray(first[-1][1], np.int64)]
        assert not np.all(np.abs(X - Xbad) <= s / 2 * (1 + 2.0 ** -22) + slack)


def test_more_stages_lower_the_error():
    """Coarse to fine: the second stage only adds information."""
    X = _tokens(600)
    mse = []
    for S in (1, 2):
        first, C, last, e = prq.prq_quantize(X, S, 4, seed=3)
        mse.append(np.mean((X - prq.prq_reconstruct(first, C, last)) ** 2))
    assert mse[1] < mse[0]
