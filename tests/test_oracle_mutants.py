"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins
catch every one of them: a dropped term, a wrong sign or index, a transposed
operand, a missing factor."""
import numpy as np
import pytest

import oracle.flp_oracle as O
from oracle_pins import ALL_PINS

_orig = {k: getattr(O, k) for k in ("logits", "row_lse", "valid_mask", "select_logp", "dlogits",
                                     "selected_rows")}


def _logits_no_bias(H, W, bias=None, temperature=None):
    return _orig["logits"](H, W, None, temperature)


def _logits_temp_mul(H, W, bias=None, temperature=None):
    Z = _orig["logits"](H, W, bias, None)
    return Z if temperature is None else Z * temperature[:, None]


def _logits_no_temp(H, W, bias=None, temperature=None):
    return _orig["logits"](H, W, bias, None)


def _logits_transposed(H, W, bias=None, temperature=None):
    Z = H @ W
    if bias is not None:
        Z = Z + bias[None, :]
    return Z if temperature is None else Z / temperature[:, None]


def _logits_bias_after_temp(H, W, bias=None, temperature=None):
    Z = H @ W.T
    if temperature is not None:
        Z = Z / temperature[:, None]
    return Z if bias is None else Z + bias[None, :]


def _lse_no_log(Z):
    m = Z.max(axis=1)
    return m + np.exp(Z - m[:, None]).sum(axis=1) - 1.0


def _lse_drop_max(Z):
    m = Z.max(axis=1)
    return np.log(np.exp(Z - m[:, None]).sum(axis=1))


def _valid_wraps(t, V):
    t = np.asarray(t, dtype=np.int64)
    return (t >= -V) & (t < V)


def _valid_off_by_one(t, V):
    t = np.asarray(t, dtype=np.int64)
    return (t >= 0) & (t <= V)


def _select_sign(Z, lse, t):
    return -_orig["select_logp"](Z, lse, t)


def _select_shift(Z, lse, t):
    t = np.asarray(t, dtype=np.int64)
    ok = (t >= 0) & (t < Z.shape[1])
    tt = np.where(ok, (t + 1) % Z.shape[1], 0)
    return np.where(ok, Z[np.arange(Z.shape[0]), tt] - lse, 0.0)


def _select_no_mask(Z, lse, t):
    t = np.asarray(t, dtype=np.int64)
    return Z[np.arange(Z.shape[0]), t % Z.shape[1]] - lse


def _dlogits_sign(Z, lse, t, g, temperature=None):
    return -_orig["dlogits"](Z, lse, t, g, temperature)


def _dlogits_no_temp(Z, lse, t, g, temperature=None):
    return _orig["dlogits"](Z, lse, t, g, None)


def _dlogits_no_onehot(Z, lse, t, g, temperature=None):
    G = np.asarray(g, dtype=np.float64)
    ok = (np.asarray(t) >= 0) & (np.asarray(t) < Z.shape[1])
    G = np.where(ok, G, 0.0)
    if temperature is not None:
        G = G / temperature
    return -G[:, None] * np.exp(Z - lse[:, None])


def _dlogits_no_rowmask(Z, lse, t, g, temperature=None):
    t = np.asarray(t, dtype=np.int64)
    G = np.asarray(g, dtype=np.float64)
    if temperature is not None:
        G = G / temperature
    dZ = -G[:, None] * np.exp(Z - lse[:, None])
    ok = (t >= 0) & (t < Z.shape[1])
    r = np.nonzero(ok)[0]
    dZ[r, t[r]] += G[r]
    return dZ


def _dlogits_temp_squared(Z, lse, t, g, temperature=None):
    d = _orig["dlogits"](Z, lse, t, g, temperature)
    return d if temperature is None else d / temperature[:, None]


def _sel_keeps_duplicates(n, ids):
    r = np.asarray(ids, dtype=np.int64).reshape(-1)
    return np.sort(r[(r >= 0) & (r < n)])


def _sel_wraps_negative(n, ids):
    r = np.asarray(ids, dtype=np.int64).reshape(-1)
    return np.unique(r[(r >= -n) & (r < n)] % n)


def _sel_off_by_one(n, ids):
    r = np.asarray(ids, dtype=np.int64).reshape(-1)
    return np.unique(r[(r >= 0) & (r <= n)] % n)


def _emb_bwd_drops_repeats(grad, ids, num_embeddings):
    G = np.asarray(grad, dtype=np.float64)
    i = np.asarray(ids, dtype=np.int64)
    ok = (i >= 0) & (i < num_embeddings)
    out = np.zeros((num_embeddings, G.shape[1]))
    out[i[ok]] += G[ok]            # fancy-index += keeps one of the repeated ids
    return out


def _emb_fwd_wraps(weight, ids):
    E = np.asarray(weight, dtype=np.float64)
    return E[np.asarray(ids, dtype=np.int64) % E.shape[0]]


MUTANTS = {
    "logits_no_bias": ("logits", _logits_no_bias),
    "logits_temp_multiplies": ("logits", _logits_temp_mul),
    "logits_no_temperature": ("logits", _logits_no_temp),
    "logits_transposed_W": ("logits", _logits_transposed),
    "logits_bias_after_temperature": ("logits", _logits_bias_after_temp),
    "lse_missing_log": ("row_lse", _lse_no_log),
    "lse_drops_row_max": ("row_lse", _lse_drop_max),
    "valid_wraps_negative": ("valid_mask", _valid_wraps),
    "valid_off_by_one": ("valid_mask", _valid_off_by_one),
    "logp_sign": ("select_logp", _select_sign),
    "logp_target_index_shift": ("select_logp", _select_shift),
    "logp_no_ignore_mask": ("select_logp", _select_no_mask),
    "dlogits_sign": ("dlogits", _dlogits_sign),
    "dlogits_missing_1_over_T": ("dlogits", _dlogits_no_temp),
    "dlogits_missing_onehot": ("dlogits", _dlogits_no_onehot),
    "dlogits_ignored_rows_not_zeroed": ("dlogits", _dlogits_no_rowmask),
    "dlogits_T_twice": ("dlogits", _dlogits_temp_squared),
    "selection_keeps_duplicate_ids": ("selected_rows", _sel_keeps_duplicates),
    "selection_wraps_negative_ids": ("selected_rows", _sel_wraps_negative),
    "selection_accepts_id_N": ("selected_rows", _sel_off_by_one),
    "embedding_grad_drops_repeated_ids": ("embedding_backward", _emb_bwd_drops_repeats),
    "embedding_lookup_wraps_ids": ("embedding_forward", _emb_fwd_wraps),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(O, attr, fn)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(O)
        except Exception:  # noqa: BLE001 - any failure of a pin counts
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name}"
