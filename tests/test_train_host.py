"""Host logic of the multi-step trainer: its learning-rate schedule against the oracle's."""

import pytest

import oracle
from decoder_only_gpt_amd import train


@pytest.mark.parametrize("warmup,decay", [(0, 10), (4, 12), (3, 3), (2, 100)])
def test_cosine_lr_matches_oracle(warmup, decay):
    for t in range(1, decay + 5):
        a = train.cosine_lr(t, 6e-4, 6e-5, warmup, decay)
        b = oracle.cosine_lr(t, 6e-4, 6e-5, warmup, decay)
        assert a == pytest.approx(b, rel=1e-14, abs=0.0), t


def test_empty_step_rejected():
    with pytest.raises(ValueError):
        train.train_step(object(), [], 1e-3, 0.0)
