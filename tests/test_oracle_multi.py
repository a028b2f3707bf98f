"""Pins of the multi-token oracle (CPU), and planted mistakes they must catch."""

import numpy as np
import pytest

from oracle import multi_token
import pins_multi


@pytest.mark.parametrize("pin", pins_multi.ALL, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(multi_token)


def _mutations():
    orig_lens = multi_token.token_lengths

    def sees_own_successor(seq_lens, T):          # causal limit one position late
        return np.minimum(orig_lens(seq_lens, T) + 1, np.asarray(seq_lens)[:, None])

    def tokens_reversed(seq_lens, T):             # token t placed at L-1-t
        return orig_lens(seq_lens, T)[:, ::-1]

    def all_see_everything(seq_lens, T):          # no causal mask inside the tile
        L = np.asarray(seq_lens, dtype=np.int64)
        return np.repeat(L[:, None], T, axis=1)

    return [("token_lengths", sees_own_successor), ("token_lengths", tokens_reversed),
            ("token_lengths", all_see_everything)]


@pytest.mark.parametrize("name,fn", _mutations(), ids=lambda x: getattr(x, "__name__", str(x)))
def test_planted_mistake_is_caught(monkeypatch, name, fn):
    monkeypatch.setattr(multi_token, name, fn)
    failed = []
    for pin in pins_multi.ALL:
        try:
            pin(multi_token)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"no pin caught the planted mistake in {name}"
