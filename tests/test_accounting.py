"""Accounting helpers against the numbers the pages print (tests/golden/printed_values.json)."""

import json
import math

import numpy as np
import os

import pytest

from kv_cache_decode_split_amd import accounting as A

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "printed_values.json")


def _golden():
    with open(GOLDEN) as f:
        return {e["name"]: e for e in json.load(f)["entries"]}


def _agrees(value, printed, digits):
    """``value`` rounds to ``printed`` at the number of significant digits the page printed."""
    if printed == 0:
        return value == 0
    scale = 10 ** (math.floor(math.log10(abs(printed))) - digits + 1)
    return round(value / scale) == round(printed / scale)


def test_golden_fixture_cites_every_entry():
    for e in _golden().values():
        assert e["source"] and ("Ch." in e["source"] or "Appendix" in e["source"])


def test_eq3_gpt3_kv_per_request():
    e = _golden()["gpt3_kv_bytes_per_request"]
    got = A.kv_cache_bytes_eq3(**e["inputs"])
    assert got == 2 * 96 * 12288 * 2048 * 2
    assert _agrees(got, e["printed"], e["printed_digits"])
    e2 = _golden()["gpt3_max_concurrent_requests"]
    assert _agrees(e2["inputs"]["free_bytes"] / e2["inputs"]["per_request_bytes_printed"],
                   e2["printed"], e2["printed_digits"])


def test_decode_throughput_definitions():
    g = _golden()
    agg = g["aggregate_tokens_per_s"]
    assert A.aggregate_tokens_per_s(**agg["inputs"]) == pytest.approx(agg["printed"])
    per = g["per_sequence_tokens_per_s"]
    assert A.per_sequence_tokens_per_s(**per["inputs"]) == pytest.approx(per["printed"])


def test_ridge_point():
    e = _golden()["a100_ridge_point"]
    assert _agrees(A.ridge_point(**e["inputs"]), e["printed"], e["printed_digits"])


def test_llama7b_decode_step_bound():
    e = _golden()["llama7b_decode_step_bound"]
    t = A.decode_step_bandwidth_bound(**e["inputs"])
    assert _agrees(t, e["printed"], e["printed_digits"])
    assert 0.0085 < t < 0.0095


def test_kv_bytes_per_token_and_sequence():
    g = _golden()
    e = g["kv_bytes_per_token_7b"]
    per_tok = A.kv_bytes_per_token(**e["inputs"])
    assert per_tok == e["printed"]
    for name in ("kv_bytes_per_sequence_4k", "kv_bytes_per_sequence_32k"):
        e = g[name]
        i = e["inputs"]
        assert A.kv_bytes_per_token(i["num_layers"], i["hidden"], i["elem_bytes"]) * i["seq_len"] == e["printed"]


def test_selftest_q1_is_compute_bound():
    g = _golden()
    mem, comp = g["selftest_q1_memory_time"], g["selftest_q1_compute_time"]
    t_mem = mem["inputs"]["bytes"] / mem["inputs"]["bandwidth"]
    t_comp = comp["inputs"]["flops"] / comp["inputs"]["peak_flops"]
    assert _agrees(t_mem, mem["printed"], mem["printed_digits"])
    assert _agrees(t_comp, comp["printed"], comp["printed_digits"])
    t = A.roofline_time(comp["inputs"]["flops"], mem["inputs"]["bytes"],
                        comp["inputs"]["peak_flops"], mem["inputs"]["bandwidth"])
    assert t == pytest.approx(t_comp)


def test_intensity_is_flops_over_unique_kv_bytes():
    """Ch. 10 §5: the FLOP/byte ratio of decode attention reduces to 2 h_q / (h_kv b_kv)."""
    for hq, hkv, d, b, lens in [(8, 8, 64, 4, [256]), (32, 32, 128, 2, [4096] * 8),
                                (32, 8, 128, 2, [8192] * 64), (64, 8, 128, 2, [131072] * 4),
                                (32, 8, 128, 2, [128, 32768, 999])]:
        flops = A.decode_attention_flops(lens, hq, d)
        nbytes = A.unique_kv_read_bytes(lens, hkv, d, b)
        assert flops / nbytes == pytest.approx(A.decode_attention_intensity(hq, hkv, b))
    assert A.decode_attention_intensity(8, 8, 4) == 0.5
    assert A.decode_attention_intensity(32, 32, 2) == 1.0
    assert A.decode_attention_intensity(32, 8, 2) == 4.0
    assert A.decode_attention_intensity(64, 8, 2) == 8.0


def test_workload_byte_counts():
    assert A.unique_kv_read_bytes(256, 8, 64, 4, batch=1) == 1 << 20
    assert A.unique_kv_read_bytes(4096, 32, 128, 2, batch=8) == 512 << 20
    assert A.unique_kv_read_bytes(4096, 32, 128, 2, batch=8, num_layers=32) == 16 << 30
    assert A.unique_kv_read_bytes(8192, 8, 128, 2, batch=64) == 2 << 30
    assert A.unique_kv_read_bytes(131072, 8, 128, 2, batch=4) == 2 << 30
    assert A.unique_kv_bytes_per_position(8, 128, 2) == 4096


def test_roofline_sum():
    ks = [(0.0, 8e9, 1.0, 8e12), (1e9, 0.0, 1e12, 1.0)]
    assert A.roofline_time_sum(ks, exposed_other=1e-6) == pytest.approx(1e-3 + 1e-3 + 1e-6)


def test_attended_length_counts_the_oracle_positions():
    """The bench's byte count under a window equals the number of positions the oracle attends."""
    from oracle import attended_positions
    for length in (0, 1, 5, 16, 17, 100, 4096):
        assert A.attended_length(length) == length
        for window in (1, 3, 16, 64, 5000):
            for sinks in (0, 1, 4, 50, 10000):
                want = len(attended_positions(length, window, sinks))
                assert A.attended_length(length, window, sinks) == want, (length, window, sinks)


def test_attended_length_of_several_tokens_counts_the_union_of_their_positions():
    """With γ query tokens the byte count is the size of the union of the positions the oracle's
    γ tokens attend (token j: the attended positions of the first T - γ + 1 + j)."""
    from oracle import attended_positions
    for length in (0, 1, 3, 16, 17, 100, 700):
        for gamma in (1, 2, 4, 16):
            for window in (None, 1, 3, 16, 64, 5000):
                for sinks in (0, 4, 50):
                    union = set()
                    for j in range(gamma):
                        visible = length - gamma + 1 + j
                        if visible > 0:
                            union |= set(np.asarray(attended_positions(visible, window, sinks)).tolist())
                    got = A.attended_length(length, window, sinks, num_queries=gamma)
                    assert got == len(union), (length, gamma, window, sinks)


def test_verify_flops_sum_the_tokens_visible_positions():
    from oracle import attended_positions
    for length, gamma, window, sinks in [(100, 4, None, 0), (3, 8, None, 0), (700, 4, 64, 4)]:
        want = 0
        for j in range(gamma):
            visible = length - gamma + 1 + j
            if visible > 0:
                want += len(attended_positions(visible, window, sinks))
        assert A.verify_attention_flops(length, 32, 128, gamma, window, sinks) == 4 * 32 * 128 * want
    # one token is the single-token count
    assert A.verify_attention_flops(4096, 32, 128, 1) == A.decode_attention_flops([4096], 32, 128)
