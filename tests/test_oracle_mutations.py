"""Planted mistakes in the oracle must be caught by its pins.

Each case swaps one step of the oracle for a plausible wrong variant (on the
CPU, inside this test only) and checks that at least one pin fails.
"""
import numpy as np
import pytest

import oracle.conv as oconv
import oracle.gdn as ogdn
from tests import test_oracle_pins as pins


def _step_output_before_write(S, a, b, kt, vt, qt, scale):
    S = S * a[:, None, None]
    o = np.einsum("hkv,hk->hv", S, scale * qt)
    u = b[:, None] * (vt - np.einsum("hkv,hk->hv", S, kt))
    return S + kt[:, :, None] * u[:, None, :], o


def _step_erase_before_decay(S, a, b, kt, vt, qt, scale):
    u = b[:, None] * (vt - np.einsum("hkv,hk->hv", S, kt))
    S = S * a[:, None, None] + kt[:, :, None] * u[:, None, :]
    return S, np.einsum("hkv,hk->hv", S, scale * qt)


def _step_no_beta_on_erase(S, a, b, kt, vt, qt, scale):
    S = S * a[:, None, None]
    u = b[:, None] * vt - np.einsum("hkv,hk->hv", S, kt)
    S = S + kt[:, :, None] * u[:, None, :]
    return S, np.einsum("hkv,hk->hv", S, scale * qt)


def _step_decay_sign(S, a, b, kt, vt, qt, scale):
    return ogdn.__dict__["_orig_step"](S, 1.0 / a, b, kt, vt, qt, scale)


GDN_PINS = [
    lambda: pins.test_gdn_tree_matches_matrix_form_brute_force(2, 4, 4, 6),
    pins.test_gdn_closed_form_orthonormal_keys,
    pins.test_gdn_single_token,
    pins.test_gdn_no_decay_full_erase_copies_values,
    pins.test_gdn_scalar_closed_form,
    pins.test_gdn_oracle_matches_chunked_form_of_the_method,
]


def _fails(fns):
    for fn in fns:
        try:
            fn()
        except (AssertionError, ValueError):
            return True
    return False


@pytest.mark.parametrize("bad", [_step_output_before_write, _step_erase_before_decay,
                                 _step_no_beta_on_erase, _step_decay_sign])
def test_planted_gdn_mistake_is_caught(monkeypatch, bad):
    monkeypatch.setitem(ogdn.__dict__, "_orig_step", ogdn._token_step)
    monkeypatch.setattr(ogdn, "_token_step", bad)
    assert _fails(GDN_PINS)


def _conv_taps_reversed(xp, w, bias=None, act=None, dtype=np.float64, ctx=None):
    return ORIG_CONV(xp, np.asarray(w)[:, ::-1], bias, act, dtype, ctx=ctx)


def _conv_no_padding_history(xp, w, bias=None, act=None, dtype=np.float64, ctx=None):
    y = ORIG_CONV(xp, w, bias, act, dtype, ctx=ctx)
    y[: w.shape[1] - 1] = 0.0
    return y


def _conv_context_ignored(xp, w, bias=None, act=None, dtype=np.float64, ctx=None):
    return ORIG_CONV(xp, w, bias, act, dtype)


def _conv_context_reversed(xp, w, bias=None, act=None, dtype=np.float64, ctx=None):
    return ORIG_CONV(xp, w, bias, act, dtype, ctx=None if ctx is None else np.asarray(ctx)[::-1])


ORIG_CONV = oconv.conv_on_path
CONV_PINS = [
    lambda: pins.test_conv_chain_matches_torch_conv1d(None, 4),
    pins.test_conv_onehot_reads_path_history_bitwise,
    lambda: pins.test_conv_tree_matches_brute_force(None),
    pins.test_conv_root_context_is_the_eq11_concatenation,
    pins.test_conv_context_out_is_the_path_walk,
]


@pytest.mark.parametrize("bad", [_conv_taps_reversed, _conv_no_padding_history, _conv_context_ignored,
                                 _conv_context_reversed])
def test_planted_conv_mistake_is_caught(monkeypatch, bad):
    monkeypatch.setattr(oconv, "conv_on_path", bad)
    assert _fails(CONV_PINS)


def _gdn_init_ignored(q, k, v, g, beta, scale=1.0, snap_at=(), heads=None, init=None, dtype=np.float64):
    return ORIG_GDN(q, k, v, g, beta, scale, snap_at, heads, None, dtype)


ORIG_GDN = ogdn.gdn_on_path


def test_planted_initial_state_mistake_is_caught(monkeypatch):
    monkeypatch.setattr(ogdn, "gdn_on_path", _gdn_init_ignored)
    assert _fails([pins.test_partition_gateway_reproduces_the_uncut_trie])
