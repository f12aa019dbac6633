"""The owner rank of an expert as the kernels compute it: e / epr by one
float multiply, (int)((float(e) + 0.5f) * (1.0f / epr)), in IEEE single
precision with a correctly rounded reciprocal.  Checked here against the
integer quotient for every expert of every shape the library accepts
(E <= 4096, R <= 64, R dividing E), with numpy's float32 arithmetic, which
rounds each operation as the GPU's does."""

import numpy as np


def test_float_owner_rank_is_exact_for_every_accepted_shape():
    e_all = np.arange(4096, dtype=np.int64)
    checked = 0
    for E in range(1, 4097):
        e = e_all[:E]
        ef = e.astype(np.float32) + np.float32(0.5)
        for R in range(1, min(E, 64) + 1):
            if E % R:
                continue
            epr = E // R
            inv = np.float32(1.0) / np.float32(epr)
            got = (ef * inv).astype(np.float32).astype(np.int64)   # truncation toward zero
            assert np.array_equal(got, e // epr), (E, R)
            checked += E
    assert checked > 1_000_000
