"""The seeded generator: determinism, packing rules, bf16 rounding."""
import numpy as np
import pytest

from synthetic import CONFIGS, bf16_bits_to_f32, f32_to_bf16_bits, make_microbatch
from synthetic.microbatch import pack_cu_seqlens


def test_same_seed_same_bytes():
    a = make_microbatch("tiny_ctx512_w512", 3)
    b = make_microbatch("tiny_ctx512_w512", 3)
    for name in ("cu_seqlens", "q_bits", "k_bits", "v_bits", "dout_bits"):
        assert np.array_equal(getattr(a, name), getattr(b, name))
    c = make_microbatch("tiny_ctx512_w512", 4)
    assert not np.array_equal(a.q_bits, c.q_bits)


@pytest.mark.parametrize("name", ["tiny_ctx512_w512", "ctx512_w512", "ctx4096_global"])
def test_cu_seqlens_rules(name):
    cfg = CONFIGS[name]
    for seed in range(3):
        mb = make_microbatch(name, seed)
        cu = mb.cu_seqlens
        assert cu.dtype == np.int32 and cu[0] == 0 and cu[-1] == cfg.total_tokens
        assert np.all(np.diff(cu) > 0)
        # every row end is a cut, no segment crosses a row end
        assert set(range(0, cfg.total_tokens + 1, cfg.ctx)) <= set(cu.tolist())
        assert mb.max_seqlen <= cfg.ctx
        assert mb.q_bits.shape == (cfg.total_tokens, cfg.num_q_heads, cfg.head_dim)
        assert mb.k_bits.shape == (cfg.total_tokens, cfg.num_kv_heads, cfg.head_dim)


def test_pack_cuts_documents_and_rows():
    # stream: docs of 5, 7, 20 tokens; burn-in 3; microbatch of 16 with rows of 8
    cu = pack_cu_seqlens(np.array([5, 7, 20]), 16, 8, burn_in=3)
    # doc ends at stream 5 and 12 -> local 2 and 9; rows cut at 8, 16
    assert cu.tolist() == [0, 2, 8, 9, 16]


def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, -2.5, 1.0 + 2**-9, 3.0e38], dtype=np.float32)
    got = bf16_bits_to_f32(f32_to_bf16_bits(x))
    # 1+2^-8 is a tie between 1 and 1+2^-7: ties go to the even mantissa (1.0)
    want = np.array([1.0, 1.0, 1.0 + 2**-6, -2.5, 1.0, 2.9969e38], dtype=np.float32)
    assert np.allclose(got[:5], want[:5], rtol=0, atol=0)
    assert abs(got[5] - 3.0e38) / 3.0e38 < 2**-8
    # exactly representable values survive the round trip
    b = np.arange(0, 65536, 97, dtype=np.uint16)
    b = b[(b & 0x7F80) != 0x7F80]            # skip inf/nan patterns
    assert np.array_equal(f32_to_bf16_bits(bf16_bits_to_f32(b)), b)


def test_lognormal_median_and_tail():
    from synthetic.microbatch import draw_document_lengths
    lens = draw_document_lengths(np.random.default_rng(0), 20_000_000)
    assert abs(np.median(lens) - 457) < 15
    assert lens.min() >= 8 and lens.max() <= 65536
