"""The bench's accounting reproduces numbers printed on the pages."""
import pytest

from sparse_long_context_csa_amd import accounting as acc
from golden_util import load


def test_hierarchical_indexer_macs_printed():
    g = load("pages_printed_values.json")["hier_indexer_macs"]
    full = acc.indexer_macs(g["heads"], g["head_dim"], g["positions"])
    pool = acc.indexer_macs(g["heads"], g["head_dim"], g["pool_blocks"] * g["block_size"])
    assert full == g["full_macs"]
    assert pool == g["pool_macs"]
    assert round(100 * pool / full, 2) == g["pool_percent_printed"]
    assert round(full / pool, 1) == g["cheaper_factor_printed"]


def test_selector_share_printed():
    g = load("pages_printed_values.json")
    d = g["v4_flash_dims"]
    kw = dict(n_csa=d["n_csa"], n_hca=d["n_hca"], n_swa=d["n_swa"], heads=d["n_heads"],
              head_dim=d["head_dim"], idx_heads=d["idx_heads"], idx_dim=d["idx_dim"], m=d["m"],
              m_hca=d["m_hca"], top_k=d["top_k"], window=d["window"])
    s1m = acc.selector_share(1_048_576, **kw)
    s32k = acc.selector_share(32_768, **kw)
    assert round(100 * s1m) == g["selector_share"]["share_1m_percent_printed"]
    assert s32k == pytest.approx(g["selector_share"]["share_32k_fraction_printed"], abs=0.01)
    assert s1m == pytest.approx(g["selector_share"]["share_1m_fraction_printed"], abs=0.01)


def test_decode_bytes_dominated_by_key_scan_at_1m():
    b = acc.decode_step_bytes(B=4, n_vis=262144, m=4, D=512, H=64, H_I=64, d_I=128, K=512, W=128)
    assert b.keys == 4 * 262144 * 256
    assert b.gather == 4 * 640 * 1024
    assert 270e6 < b.total < 273e6
    assert acc.scan_bytes(4, 262144, 64, 128) == 268_435_456 + 4 * (16384 + 256)


def test_prefill_flops():
    s = acc.sum_visible(126976, 131072, 4, 32768)
    assert s == 132_119_552
    assert acc.prefill_indexer_flops(s, 64, 128) == pytest.approx(2.1646e12, rel=1e-4)
