"""Pins of the storage accounting against the memory figures printed on the pages."""
import json
import os

from oracle import accounting as Ac

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_bits_per_token_head():
    assert Ac.key_bits() == 380
    assert Ac.value_bits() == 300
    assert Ac.bits_per_token_head() == 680
    assert abs(Ac.ratio_per_token() - 4096 / 680) < 1e-12


def test_pages_memory_figures():
    g = json.load(open(os.path.join(GOLD, "pages_numbers.json")))
    lc = g["kv_memory_longcat_gib"]
    bits = 4096 * lc["quantwm"] / lc["bf16"]          # bits per token-head implied by the pages
    assert abs(bits - 684.0) < 0.05
    assert abs(bits / Ac.bits_per_token_head() - 1) < 0.006
    hy = g["kv_memory_hyworld_gib"]
    assert abs(hy["bf16"] / hy["quantwm"] - g["max_compression"]["value"]) < 0.005
    # per-token ratio sits between LongCat's 5.99x and the 6.20x ceiling
    assert lc["bf16"] / lc["quantwm"] < Ac.ratio_per_token() < g["max_compression"]["value"]


def test_rank_overhead_order_of_magnitude():
    """Rank 8 -> 16 adds r*8 bits to each Key token-head: 64 bits over 256
    K+V elements = 0.25 bit per element, the same size as the pages' 0.2569
    (Causal-Forcing) and above HY-World's 0.1341 (sparse coefficient layout)."""
    g = json.load(open(os.path.join(GOLD, "pages_numbers.json")))["rank8_to_16_extra_bits"]
    extra = (Ac.key_bits(r=16) - Ac.key_bits(r=8)) / 256
    assert extra == 0.25
    assert abs(extra / g["causal_forcing"] - 1) < 0.03
    assert g["hyworld"] < extra


def test_tables_and_resident_ratios():
    assert Ac.table_bytes() == 133120
    assert abs(Ac.resident_ratio(4096, 1) - 4.36) < 0.01
    assert abs(Ac.resident_ratio(1560, 25) - 3.01) < 0.01
    assert abs(Ac.resident_ratio(3600, 25) - 4.20) < 0.01
    assert abs(Ac.resident_ratio(28000, 1) - 5.70) < 0.01


def test_coefficient_layout_bytes_of_the_library():
    """The library's host-side layout sizes (qwm_coefficient_bytes) equal the
    oracle's dense and sparse layout sizes (oracle.storage, QuantWM App. D.1)."""
    from oracle import storage as St
    from bit_kv_cache_head_amd._abi import lib, QWM_LAYOUT_DENSE, QWM_LAYOUT_SPARSE
    for r in (8, 16, 32):
        for T in (1, 63, 64, 65, 1560, 28000, 70000):
            for kept in sorted({0, 1, T // 3, T // 2, T - 1, T} - {-1}):
                assert lib.qwm_coefficient_bytes(QWM_LAYOUT_DENSE, T, kept, r) == St.dense_bytes(T, r)
                assert lib.qwm_coefficient_bytes(QWM_LAYOUT_SPARSE, T, kept, r) == St.sparse_bytes(T, kept, r)
    assert lib.qwm_coefficient_bytes(QWM_LAYOUT_SPARSE, 10, 11, 8) == -1
    assert lib.qwm_coefficient_bytes(7, 10, 1, 8) == -1
