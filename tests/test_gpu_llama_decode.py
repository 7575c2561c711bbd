"""The decoder stack around the Adamas step: every attention call inside a
multi-layer decode loop matches the CPU oracle on the inputs that call saw
(codes bit for bit, including the key appended by the step, selections exactly,
outputs within 2e-3 of the row norm), dense layers match the oracle's dense
attention, and a HIP graph of the loop replays bit-identically to eager steps.

Shapes are small (3 layers, 2 query / 1 KV heads of 128, ragged lengths 1200
and 517); the 32-layer Llama-3.1-8B shape runs in bench.py.
"""
import numpy as np
import pytest

from helpers import assert_out_close, from_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import sparse_attention_long_fwht_amd as A
    from sparse_attention_long_fwht_amd.llama_decode import DecoderShape, LlamaShapedDecoder
    import oracle
    return torch, DecoderShape, LlamaShapedDecoder, oracle


TINY = dict(layers=3, hidden=256, q_heads=2, kv_heads=1, ffn=512, vocab=1000)


def u16(t):
    return from_dev(t.contiguous().view(__import__("torch").int16), np.uint16)


def check_trace(trace, oracle, budget, scale, **forced):
    n_sparse = 0
    for call in trace:
        q, k, v = u16(call["q"]), u16(call["k"]), u16(call["v"])
        kv_len = from_dev(call["kv_len"])
        if call["dense"]:
            ref = oracle.dense_attention(q, k, v, kv_len, scale, threads=8)
            assert_out_close(from_dev(call["out"]), ref)
            continue
        n_sparse += 1
        codes_ref = oracle.encode_keys(k, kv_len)
        codes = from_dev(call["codes"])
        for b in range(q.shape[0]):
            L = int(kv_len[b])
            assert np.array_equal(codes[b, :, :L], codes_ref[b, :, :L]), "codes differ"
        out_r, sel_r, _, _ = oracle.decode_step(q, k, v, codes_ref, kv_len, budget, scale, threads=8,
                                                want_dist=False, **forced)
        assert np.array_equal(from_dev(call["sel"]), sel_r), "selected indices differ"
        assert_out_close(from_dev(call["out"]), out_r)
    return n_sparse


@pytest.mark.parametrize("forced", [{}, dict(sink=4, recent=16)])
def test_decode_loop_attention_matches_oracle(env, forced):
    torch, DecoderShape, LlamaShapedDecoder, oracle = env
    m = LlamaShapedDecoder(DecoderShape(**TINY), batch=2, capacity=1500, attention="adamas", budget=64,
                           dense_last=1, seed=3, **forced)
    m.fill_cache([1200, 517], seed=4)
    m.trace = []
    for _ in range(3):
        m.step()
    torch.cuda.synchronize()
    assert len(m.trace) == 9
    assert check_trace(m.trace, oracle, 64, m.scale, **forced) == 6
    assert np.array_equal(from_dev(m.kv_len), [1203, 520])


def test_decode_loop_dense_matches_oracle(env):
    torch, DecoderShape, LlamaShapedDecoder, oracle = env
    m = LlamaShapedDecoder(DecoderShape(**TINY), batch=2, capacity=1500, attention="dense", seed=5)
    m.fill_cache([900, 1400], seed=6)
    m.trace = []
    m.step()
    torch.cuda.synchronize()
    assert check_trace(m.trace, oracle, 64, m.scale) == 0


def test_decode_loop_graph_replays_match_eager(env):
    """Four eager steps, then four replays of a one-step graph from the same
    state, with eager work between replays: tokens, lengths and the caches'
    new rows agree bit for bit after every step."""
    torch, DecoderShape, LlamaShapedDecoder, oracle = env
    m = LlamaShapedDecoder(DecoderShape(**TINY), batch=2, capacity=1500, attention="adamas", budget=64,
                           dense_last=1, seed=7)
    m.fill_cache([1000, 333], seed=8)
    compared = lambda: (m.layers[0].k, m.layers[0].codes, m.layers[1].v)
    start = m.state()
    start_caches = [t.clone() for t in compared()]
    eager = []
    for _ in range(4):
        m.step()
        eager.append((m.tokens.clone(), m.kv_len.clone()) + tuple(t.clone() for t in compared()))

    def reset():  # (rows past the lengths are never read; the compared caches are restored whole)
        m.restore(start)
        for t, t0 in zip(compared(), start_caches):
            t.copy_(t0)

    reset()
    g = m.capture(1)
    reset()
    torch.cuda.synchronize()
    for i in range(4):
        g.replay()
        torch.cuda.synchronize()
        got = (m.tokens, m.kv_len) + compared()
        for a, b in zip(got, eager[i]):
            assert torch.equal(a, b), "replay %d differs from the eager step" % i
        torch.zeros(1 << 20, device="cuda").add_(1.0)  # unrelated eager work between replays
        torch.cuda.synchronize()


def test_decode_loop_switch_attention(env):
    """use(): the same model timed dense and with dense_last, as the bench does;
    layer flags follow the switch."""
    torch, DecoderShape, LlamaShapedDecoder, oracle = env
    m = LlamaShapedDecoder(DecoderShape(**TINY), batch=1, capacity=600, attention="adamas", budget=32, seed=9)
    m.fill_cache([500], seed=10)
    m.use("dense")
    assert all(L.dense for L in m.layers)
    m.use("adamas", dense_last=2)
    assert [L.dense for L in m.layers] == [False, True, True]
    m.trace = []
    m.step()
    torch.cuda.synchronize()
    assert check_trace(m.trace, oracle, 32, m.scale) == 1
