"""Pool-sizing helpers of the C ABI (host arithmetic) against the figures the
Day 38 page prints (tests/golden/pool_sizing.json)."""

import json
import os

import pytest

import paged_kv_cache_scatter_amd as pkv

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pool_sizing.json")))
GIB = 1 << 30
KIB = 1 << 10
MIB = 1 << 20


def test_block_bytes_llama_1b():
    g = GOLD["block_bytes_llama_3_2_1b"]
    assert pkv.block_bytes(g["layers"], g["block_size"], g["kv_heads"], g["head_dim"],
                           g["itemsize"]) == g["bytes"]
    # the attention-head mistake gives four times the bytes
    assert pkv.block_bytes(16, 16, 32, 64, 2) == 4 * g["bytes"]
    assert pkv.block_bytes(0, 16, 8, 64, 2) == 0


def test_gib_is_2048_blocks():
    g = GOLD["gib"]
    bb = GOLD["block_bytes_llama_3_2_1b"]["bytes"]
    nb, nr = pkv.plan_pool(g["bytes"], g["bytes"], 1.0, 0, bb, 16, 16)
    assert nb == g["blocks"] and nb * 16 == g["tokens"]
    assert nr == g["blocks"]


@pytest.mark.parametrize("row", GOLD["card_24gib"]["rows"], ids=lambda r: f"{r['slots']}x{r['max_len']}")
def test_card_table_blocks_and_requests(row):
    bb = GOLD["block_bytes_llama_3_2_1b"]["bytes"]
    # exact block count: any budget in [blocks, blocks + 1) blocks
    nb, nr = pkv.plan_pool(row["blocks"] * bb + 100 * KIB, 24 * GIB, 1.0, 0, bb, 16,
                           row["max_len"])
    assert (nb, nr) == (row["blocks"], row["requests"])
    # the budget formula: what is free before the reserve (18.70 GiB on the page),
    # minus the activation reserve, gives the printed pool to its 0.01 GiB rounding
    util = 0.9
    before = GOLD["card_24gib"]["kv_budget_before_reserve_gib"]
    free = int((before + (1 - util) * 24) * GIB)
    nb2, _ = pkv.plan_pool(free, 24 * GIB, util, int(row["reserve_gib"] * GIB), bb, 16,
                           row["max_len"])
    assert abs(nb2 - row["blocks"]) <= 0.011 * 2048, (nb2, row["blocks"])


def test_refuses_a_pool_under_one_request():
    g = GOLD["one_request_floor"]
    bb = GOLD["block_bytes_llama_3_2_1b"]["bytes"]
    assert g["blocks"] * bb == g["gib"] * GIB
    nb, nr = pkv.plan_pool(g["blocks"] * bb, 80 * GIB, 1.0, 0, bb, 16, g["max_len"])
    assert (nb, nr) == (g["blocks"], 1)
    with pytest.raises(pkv.PkvError) as e:
        pkv.plan_pool(g["blocks"] * bb - 1, 80 * GIB, 1.0, 0, bb, 16, g["max_len"])
    assert e.value.status_name == "PKV_ERR_CAPACITY"
    assert str((g["blocks"] - 1) * 16) in str(e.value)   # names the longest servable length


def test_tied_copy_bytes_to_blocks():
    g = GOLD["tied_copy"]
    bb = GOLD["block_bytes_llama_3_2_1b"]["bytes"]
    nb, _ = pkv.plan_pool(g["mib"] * MIB, g["mib"] * MIB, 1.0, 0, bb, 16, 16)
    assert nb == g["blocks"] and nb * 16 == g["tokens"]


def test_bad_arguments():
    for args in ((-1, 1, 1.0, 0, 1, 16, 16), (1, 1, 0.0, 0, 1, 16, 16), (1, 1, 1.5, 0, 1, 16, 16),
                 (1, 1, 1.0, 0, 0, 16, 16), (1, 1, 1.0, 0, 1, 0, 16)):
        with pytest.raises(pkv.PkvError) as e:
            pkv.plan_pool(*args)
        assert e.value.status_name == "PKV_ERR_SHAPE"
    # a budget that goes negative is an empty pool, refused for any request
    with pytest.raises(pkv.PkvError):
        pkv.plan_pool(GIB, 24 * GIB, 0.5, 0, 512 * KIB, 16, 16)


def test_block_bytes_past_int64_is_an_error():
    # 2 * (2^31 - 1)^3 * 8 bytes does not fit in int64: refused, not wrapped
    big = 2**31 - 1
    with pytest.raises(pkv.PkvError) as e:
        pkv.block_bytes(big, big, big, 128, 8)
    assert e.value.status_name == "PKV_ERR_SHAPE" and "exceed int64" in str(e.value)
    # the largest sizes that fit still give the exact product
    assert pkv.block_bytes(2**15, 256, 2**10, 2**10, 4) == 2 * 2**15 * 256 * 2**10 * 2**10 * 4
    assert pkv.block_bytes(0, 16, 8, 128, 2) == 0
