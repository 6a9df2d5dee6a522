"""The library's cost accounting against the pages' analytic figures."""
import os

from linear_attention_05_amd import accounting as acc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "decode_cost.txt")


def test_decode_cost_matches_pages():
    rows = [l.split() for l in open(GOLDEN) if l.strip() and not l.startswith("#")]
    assert rows
    for D, flops, state_bytes in rows:
        D = int(D)
        assert acc.decode_flops_per_head_token(D, D) == int(flops)
        assert acc.decode_state_bytes_per_head_token(D, D) == int(state_bytes)


def test_prefill_flop_convention():
    # six D x D products per token (W S, Qd S, Kc^T U, each 2*Dk*Dv per token)
    # plus the C x C and C x D chunk products
    assert acc.prefill_flops_per_token_head(128, 128) == 180224
    assert acc.io_bytes_per_token_head(128, 128, 2) == 1796
    assert acc.io_bytes_per_token_head(64, 64, 4) == 1284
    assert acc.handoff_bytes_per_chunk_head(128, 2) == 61952
