"""Pins of the storage rate and of the pages' memory arithmetic, computed from
the byte counts of buffers the oracle really produces. The expected figures are
the pages' printed numbers (tests/golden/pages_figures.json, each cited)."""
import json
import os

import pytest

from oracle import storage

HERE = os.path.dirname(os.path.abspath(__file__))
GOLD = json.load(open(os.path.join(HERE, "golden", "pages_figures.json")))


def test_exact_rates():
    assert storage.bits_per_param(double_quant=False) == 4.5
    assert storage.bits_per_param(double_quant=True) == 4.126953125
    assert storage.code_bits() == 4.0


def test_summary_page_rate_reading():
    """The summary page's 0.125 bits is the 8-bit codes alone (8/64); the
    figure-4 page's 0.127 adds one fp32 step per 256 blocks."""
    bufs = storage.format_buffers(1 << 16)
    assert 8 * bufs["qscale"].nbytes / (1 << 16) == 0.125
    assert abs(storage.scale_overhead_bits() - 0.125) < 0.002


@pytest.mark.parametrize("fig", GOLD["figures"], ids=lambda f: f["id"])
def test_printed_memory_figures(fig):
    got = storage.breakdown_gb(fig["params"])[fig["what"]]
    assert abs(got - fig["value"]) <= fig["tol"], (fig["source"], got)


def _rate(name):
    return next(r for r in GOLD["rates"] if r["id"] == name)


def test_printed_rates():
    r = _rate("overhead_before_dq_bits")
    assert abs(storage.scale_overhead_bits(double_quant=False) - r["value"]) <= r["tol"]
    r = _rate("overhead_after_dq_bits")
    assert abs(storage.scale_overhead_bits() - r["value"]) <= r["tol"]
    r = _rate("dq_saving_bits")
    saving = storage.scale_overhead_bits(double_quant=False) - storage.scale_overhead_bits()
    assert abs(saving - r["value"]) <= r["tol"]
    r = _rate("dq_saving_65b_gb")
    b = storage.breakdown_gb(65e9)
    assert abs(b["fp32_constants"] - b["dq_constants"] - r["value"]) <= r["tol"]
    r = _rate("full_finetune_65b_gb")
    assert abs(storage.full_finetune_gb(65e9) - r["value"]) <= r["tol"]
    r = _rate("fits_48gb")
    assert storage.frozen_base_gb(65e9) < r["value"]
