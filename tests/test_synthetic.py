"""Checks on the seeded input generators (CPU only): determinism, exact byte
counts of every workload, field uniformity, activation recipes."""
import json
import os

import numpy as np
import pytest

import oracle
import synthetic

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_deterministic_and_seed_sensitive():
    a = synthetic.q4k_matrix(16, 512, seed=3)
    b = synthetic.q4k_matrix(16, 512, seed=3)
    c = synthetic.q4k_matrix(16, 512, seed=4)
    assert a.shape == (16, 2 * 144) and a.dtype == np.uint8
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    x = synthetic.activations(4, 512, seed=3)
    assert x.dtype == np.float32 and np.array_equal(x, synthetic.activations(4, 512, seed=3))


def test_workload_byte_counts():
    gold = json.load(open(os.path.join(GOLDEN, "shapes_ch8_s8_2.json")))
    assert synthetic.FC_IN == gold["fc_in"] == gold["hidden_states_concatenated"] * gold["target_hidden"]
    assert synthetic.HIDDEN == gold["fc_out"]
    assert synthetic.LAYERS == gold["target_layers"]
    assert synthetic.LM_HEAD["m"] == gold["block_size"] == synthetic.LM_HEAD["k_draft"] + 1
    b = lambda n, k: n * synthetic.q4k_bytes_per_row(k)
    assert b(512, 1024) == 294_912
    assert b(6656, 6656) == 24_920_064
    assert b(6656, 33280) == 124_600_320
    assert b(131072, 6656) == 490_733_568
    mats = synthetic.stack_matrices()
    assert len(mats) == 52 * 7
    assert sum(g.weight_bytes for g in mats) == 15_649_800_192
    assert synthetic.stack_weight_bytes() == 16_140_533_760
    assert len({g.seed for g in mats}) == len(mats)


def test_header_fields_in_range_and_finite():
    w = synthetic.q4k_matrix(64, 2048, seed=8).reshape(-1, 144)
    dd = w[:, :4].copy().view(np.float16).astype(np.float64)
    assert np.all(np.isfinite(dd))
    # fp16 rounding of U(0.001, 0.05) stays within half an ulp of the range
    assert dd.min() >= 0.001 * (1 - 2 ** -11) and dd.max() <= 0.05 * (1 + 2 ** -11)


def test_fields_uniform():
    w = synthetic.q4k_matrix(256, 4096, seed=9).reshape(-1, 144)
    sc_all, mn_all = [], []
    for blk in w[:4000]:
        sc, mn = oracle.scales_mins(bytes(blk[4:16]))
        sc_all.extend(sc); mn_all.extend(mn)
    for vals, bins in ((np.array(sc_all), 64), (np.array(mn_all), 64)):
        h = np.bincount(vals, minlength=bins)
        e = len(vals) / bins
        chi2 = float(np.sum((h - e) ** 2 / e))
        assert chi2 < bins + 6 * np.sqrt(2 * bins)
    q = w[:, 16:].reshape(-1)
    nib = np.concatenate([q & 15, q >> 4])
    h = np.bincount(nib, minlength=16)
    e = len(nib) / 16
    assert float(np.sum((h - e) ** 2 / e)) < 16 + 6 * np.sqrt(32)


def test_fc_rows_are_unit_rms_slices():
    x = synthetic.fc_activations(3, seed=2)
    assert x.shape == (3, 33280) and x.dtype == np.float32
    for r in range(3):
        for v in range(5):
            s = x[r, v * 6656:(v + 1) * 6656].astype(np.float64)
            assert np.sqrt(np.mean(s * s)) == pytest.approx(1.0, abs=1e-6)
    # 16 rows of fc input are the capture block the pages move: 2,129,920 B
    assert synthetic.fc_activations(16, seed=2).nbytes == 2_129_920


def test_injection_and_forced_draft():
    t = np.arange(15) * 7 % 100
    d = synthetic.inject_mismatches(t, 100, seed=1, probs=[0.0] * 15)
    assert np.array_equal(d, t)
    d = synthetic.inject_mismatches(t, 100, seed=1, probs=[1.0] * 15)
    assert np.all(d != t) and np.all((d >= 0) & (d < 100))
    for acc in range(16):
        f = synthetic.forced_draft(t, acc, 100)
        am = list(t) + [5]
        assert oracle.accept(f, am)[0] == acc


def test_centred_matrix_fields():
    """q4k_matrix_centred: every sub-block's min equals its scale, dmin is
    7.5 d rounded to fp16, d and the quants are q4k_matrix's; the decoded
    weights are centred on zero."""
    base = synthetic.q4k_matrix(12, 1024, 31).reshape(-1, 144)
    w = synthetic.q4k_matrix_centred(12, 1024, 31).reshape(-1, 144)
    assert np.array_equal(w[:, 0:2], base[:, 0:2]) and np.array_equal(w[:, 16:], base[:, 16:])
    d = w[:, 0:2].copy().view(np.float16)[:, 0].astype(np.float64)
    dmin = w[:, 2:4].copy().view(np.float16)[:, 0]
    assert np.array_equal(dmin, (7.5 * d).astype(np.float16))
    for b in range(w.shape[0]):
        sc, mn = oracle.scales_mins(bytes(w[b, 4:16]))
        sc0, _ = oracle.scales_mins(bytes(base[b, 4:16]))
        assert np.array_equal(sc, mn) and np.array_equal(sc, sc0)
    W = oracle.decode_matrix(synthetic.q4k_matrix_centred(64, 2048, 32), 2048)
    assert abs(W.mean()) < 0.02 * np.abs(W).mean()
