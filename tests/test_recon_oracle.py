"""CPU pins of the oracle's compact bf16 forms (the inputs of the
reconstructive GEMM of "Unweight", "Four approaches to using compressed
weights"): every weight is rebuilt exactly from each form, the sign+mantissa
stream and the verbatim store; a few words are recomputed by explicit loops
from the weights and the palette; the verbatim ranks follow the store."""
import numpy as np
import pytest

import oracle as O
import synth


@pytest.fixture(scope="module")
def case():
    w, _ = synth.gen_bf16_custom(192, 768, 11, outlier_frac=0.004)
    b = O.build_bundle_bf16(w)
    return w, b, O.transcode_forms(b, w)


@pytest.mark.parametrize("form", ["palette", "exponent"])
def test_forms_rebuild_every_weight(case, form):
    w, b, f = case
    assert b["n_verbatim"] > 0
    assert np.array_equal(O.rebuild_from_form(b, f, form, 192, 768), w)


def test_form_words_by_hand(case):
    w, b, f = case
    pal = [int(v) for v in b["palette"][:b["n_pal"]]]
    ncb = 768 // 256
    verb = set()
    for t in range(b["vb_start"].size - 1):
        for bit in range(256):
            if (int(b["vb_bits"][t * 8 + bit // 32]) >> (bit % 32)) & 1:
                verb.add((64 * (t // ncb) + bit // 4, 256 * (t % ncb) + 64 * (bit % 4)))

    def index(r, c):
        if (r, c - c % 64) in verb:
            return 0
        return pal.index((int(w[r, c]) >> 7) & 0xFF)

    for (rb, cb, g, i) in [(0, 0, 0, 0), (1, 2, 31, 63), (2, 1, 7, 5), (0, 2, 16, 33)]:
        t = rb * ncb + cb
        r = 64 * rb + i
        word = 0
        for j in range(8):
            word |= index(r, 256 * cb + 8 * g + j) << (4 * j)
        assert int(f["palette"][t * 2048 + g * 64 + i]) == word
        g4 = 2 * g + 1
        word = 0
        for j in range(4):
            word |= pal[index(r, 256 * cb + 4 * g4 + j)] << (8 * j)
        assert int(f["exponent"][t * 4096 + g4 * 64 + i]) == word


def test_vrank_follows_the_store(case):
    w, b, f = case
    vr = f["vrank"]
    got = np.sort(vr[vr >= 0])
    assert np.array_equal(got, np.arange(b["n_verbatim"]))              # each stored segment named once
    nrb, ncb = 192 // 64, 768 // 256
    v4 = vr.reshape(nrb * ncb, 4, 64)
    for t in range(nrb * ncb):
        for s in range(4):
            for i in range(64):
                v = int(v4[t, s, i])
                if v >= 0:
                    r, c0 = 64 * (t // ncb) + i, 256 * (t % ncb) + 64 * s
                    assert np.array_equal(b["verbatim"][64 * v:64 * v + 64], w[r, c0:c0 + 64])


def test_no_outliers_no_ranks():
    w, _ = synth.gen_bf16_custom(64, 256, 12)
    b = O.build_bundle_bf16(w)
    f = O.transcode_forms(b, w)
    if b["n_verbatim"] == 0:
        assert np.all(f["vrank"] == -1)
    assert np.array_equal(O.rebuild_from_form(b, f, "palette", 64, 256), w)
