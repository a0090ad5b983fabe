"""The fp64 oracle against its independent pins (CPU)."""
import pytest

import oracle
import pins


@pytest.mark.parametrize("pin", pins.ATTN_PINS, ids=lambda f: f.__name__)
def test_attention_pin(pin):
    pin(oracle.block_attention)


@pytest.mark.parametrize("pin", pins.CONF_PINS, ids=lambda f: f.__name__)
def test_confidence_pin(pin):
    pin(oracle.row_confidence)


@pytest.mark.parametrize("pin", pins.COMMIT_PINS, ids=lambda f: f.__name__)
def test_commit_pin(pin):
    pin(oracle.confidence_commit)


@pytest.mark.parametrize("pin", pins.LOOP_PINS, ids=lambda f: f.__name__)
def test_loop_pin(pin):
    pin(oracle.denoise_loop)


@pytest.mark.parametrize("pin", pins.STEP_PINS, ids=lambda f: f.__name__)
def test_step_pin(pin):
    pin(oracle.denoise_step)


@pytest.mark.parametrize("pin", pins.APPEND_PINS, ids=lambda f: f.__name__)
def test_append_pin(pin):
    pin(oracle.cache_append)


@pytest.mark.parametrize("pin", pins.LMHEAD_LOGIT_PINS, ids=lambda f: f.__name__)
def test_lmhead_logits_pin(pin):
    pin(oracle.lmhead_logits)


@pytest.mark.parametrize("pin", pins.LMHEAD_PINS, ids=lambda f: f.__name__)
def test_lmhead_commit_pin(pin):
    pin(oracle.lmhead_commit)


@pytest.mark.parametrize("pin", pins.MAMBA_PINS, ids=lambda f: f.__name__)
def test_mamba_pin(pin):
    pin(oracle.mamba_block_scan)


@pytest.mark.parametrize("pin", pins.ADALN_PINS, ids=lambda f: f.__name__)
def test_adaln_pin(pin):
    pin(oracle.adaln_modulate)
