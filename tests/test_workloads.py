"""The seeded input generators (no GPU): encoding, determinism and structure."""
import numpy as np
import torch

from grouped_query_attention_gqa_amd import workloads as W


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1.0, 1.00390625, 1.01171875, -2.5, 0.0, -0.0, 3.4e38, 1e-40],
                                 np.float32)])
    ours = W.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert W.f32_to_bf16_bits(np.array([np.nan], np.float32))[0] == 0x7FC0
    back = W.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_decode_generation_is_deterministic_and_structured():
    wl = W.WORKLOADS["llama3_8b_decode"].replace(B=4, ctx=("uniform", 20, 90))
    a = W.make_decode(wl)
    b = W.make_decode(wl)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.k, b.k) and np.array_equal(a.ctx, b.ctx)
    assert a.k.shape == (4, 8, 90, 128) and a.q.shape == (4, 1, 32, 128)
    assert ((a.ctx >= 20) & (a.ctx <= 90)).all()
    for i in range(4):
        n = int(a.ctx[i])
        assert (a.k[i, :, n:] == 0x7FC0).all() and (a.v[i, :, n:] == 0x7FC0).all()
        assert not (a.k[i, :, :n] == 0x7FC0).any()
    z = W.make_decode(wl, fill="zero")
    assert np.array_equal(z.q, a.q)
    assert (z.k[0, :, int(z.ctx[0]):] == 0).all()


def test_paged_generation_block_table_is_a_permutation():
    wl = W.WORKLOADS["paged_long_decode"].replace(B=6, ctx=("loguniform", 17, 300))
    inp = W.make_decode(wl)
    bs = wl.block_size
    need = (inp.ctx + bs - 1) // bs
    ids = np.concatenate([inp.block_table[b, :need[b]] for b in range(wl.B)])
    assert sorted(ids.tolist()) == list(range(inp.n_blocks))
    for b in range(wl.B):
        assert (inp.block_table[b, need[b]:] == -1).all()
        last = int(inp.block_table[b, need[b] - 1])
        used = int(inp.ctx[b]) - (need[b] - 1) * bs
        assert (inp.k[last, :, used:] == 0x7FC0).all()
        assert not (inp.k[last, :, :used] == 0x7FC0).any()
    kn, vn = inp.new_token_rows()
    b = 2
    t = int(inp.ctx[b]) - 1
    assert np.array_equal(kn[b, 0], inp.k[inp.block_table[b, t // bs], :, t % bs])


def test_named_workload_shapes():
    w = W.WORKLOADS
    assert (w["llama2_70b_decode"].H, w["llama2_70b_decode"].K, w["llama2_70b_decode"].G) == (64, 8, 8)
    assert w["llama3_8b_decode"].G == 4 and w["causal_prefill_4k"].G == 4
    assert w["llama2_70b_decode_mha"].G == 1 and w["llama2_70b_decode_mqa"].G == 64
    assert w["tiny_prefill_f32"].scale == 1 / 8
    p = W.make_prefill(w["tiny_prefill_f32"])
    assert p.q.shape == (1, 128, 8, 64) and p.q.dtype == np.float32
    assert p.k_new.shape == (1, 128, 2, 64)
