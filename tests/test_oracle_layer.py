"""Pins of the oracle's decoder-layer arithmetic against independent library code:
the Hugging Face Llama implementation (RMSNorm, half-split RoPE, GQA attention,
SwiGLU MLP) and torch's scaled_dot_product_attention, both on the CPU."""
import numpy as np
import pytest
import torch

import fixtures as F
import oracle as O


def _hf_model(sh, weights, emb):
    from transformers import LlamaConfig, LlamaModel
    cfg = LlamaConfig(vocab_size=sh.vocab, hidden_size=sh.d_model, intermediate_size=sh.ffn_dim,
                      num_hidden_layers=len(weights), num_attention_heads=sh.n_q_heads,
                      num_key_value_heads=sh.n_kv_heads, head_dim=sh.head_dim, rms_norm_eps=sh.rms_eps,
                      rope_theta=sh.rope_base, attention_bias=False, mlp_bias=False,
                      max_position_embeddings=4096, tie_word_embeddings=False)
    cfg._attn_implementation = "eager"
    m = LlamaModel(cfg).eval()
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    with torch.no_grad():
        m.embed_tokens.weight.copy_(t(emb))
        for layer, w in zip(m.layers, weights):
            a, f = layer.self_attn, layer.mlp
            a.q_proj.weight.copy_(t(w["w_q"]))
            a.k_proj.weight.copy_(t(w["w_k"]))
            a.v_proj.weight.copy_(t(w["w_v"]))
            a.o_proj.weight.copy_(t(w["w_o"]))
            f.gate_proj.weight.copy_(t(w["w_gate"]))
            f.up_proj.weight.copy_(t(w["w_up"]))
            f.down_proj.weight.copy_(t(w["w_down"]))
            layer.input_layernorm.weight.copy_(t(w["g_attn"]))
            layer.post_attention_layernorm.weight.copy_(t(w["g_ffn"]))
    return m


@pytest.mark.parametrize("cfg", ["tiny", "tiny_gqa"])
def test_full_prefill_matches_hf_llama(cfg):
    wl = F.get_config(cfg)
    sh = wl.shape
    W = [F.layer_weights(sh, l) for l in range(1, sh.n_layers + 1)]
    E = F.embedding(sh)
    toks = F.all_tokens(wl)
    ref = O.full_prefill(sh, W, E, toks)
    m = _hf_model(sh, W, E)
    with torch.no_grad():
        out = m(torch.from_numpy(toks.astype(np.int64))[None], use_cache=True, output_hidden_states=True)
    for l in range(sh.n_layers):
        hk = out.past_key_values.layers[l].keys[0].transpose(0, 1).double().numpy()
        hv = out.past_key_values.layers[l].values[0].transpose(0, 1).double().numpy()
        np.testing.assert_allclose(ref["k"][l], hk, atol=2e-5, rtol=1e-4)
        np.testing.assert_allclose(ref["v"][l], hv, atol=2e-5, rtol=1e-4)
    for l in range(sh.n_layers):  # residual streams before the final norm
        np.testing.assert_allclose(ref["hidden"][l], out.hidden_states[l][0].double().numpy(),
                                   atol=2e-5, rtol=1e-4)
    last = O.rmsnorm(ref["hidden"][-1], np.ones(sh.d_model), sh.rms_eps)
    np.testing.assert_allclose(last, out.last_hidden_state[0].double().numpy(), atol=2e-4, rtol=1e-4)


def test_sparse_query_attention_matches_sdpa():
    """Attention for a sorted subset of query rows equals torch SDPA with an explicit causal mask
    on those rows (GQA via repeated KV heads)."""
    rng = np.random.default_rng(7)
    n_tok, hq, hkv, dh = 97, 6, 2, 32
    q_rows = np.sort(rng.choice(n_tok, 23, replace=False))
    q = rng.standard_normal((23, hq, dh))
    k = rng.standard_normal((n_tok, hkv, dh))
    v = rng.standard_normal((n_tok, hkv, dh))
    got = O.causal_attention(q, k, v, q_rows)
    tq = torch.from_numpy(q).permute(1, 0, 2)
    tk = torch.from_numpy(k).repeat_interleave(hq // hkv, dim=1).permute(1, 0, 2)
    tv = torch.from_numpy(v).repeat_interleave(hq // hkv, dim=1).permute(1, 0, 2)
    mask = torch.from_numpy(np.arange(n_tok)[None, :] <= q_rows[:, None])
    want = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask)
    np.testing.assert_allclose(got, want.permute(1, 0, 2).numpy(), atol=1e-12)


def test_attention_special_cases():
    rng = np.random.default_rng(8)
    k = rng.standard_normal((10, 1, 8))
    v = rng.standard_normal((10, 1, 8))
    q = rng.standard_normal((3, 1, 8))
    # a query at position 0 sees only key 0: output is V[0]
    out = O.causal_attention(q[:1], k, v, [0])
    np.testing.assert_allclose(out[0, 0], v[0, 0], atol=1e-15)
    # zero query: uniform weights over the visible keys -> mean of V
    out = O.causal_attention(np.zeros((1, 1, 8)), k, v, [6])
    np.testing.assert_allclose(out[0, 0], v[:7, 0].mean(0), atol=1e-14)
    # shift invariance: RoPE'd q.k depends only on p - p', so shifting all positions is a no-op
    q0 = rng.standard_normal((4, 2, 16))
    k0 = rng.standard_normal((12, 2, 16))
    v0 = rng.standard_normal((12, 2, 16))
    rows = np.array([2, 5, 9, 11])
    a = O.causal_attention(O.rope_rotate(q0, rows, 1e4), O.rope_rotate(k0, np.arange(12), 1e4), v0, rows)
    s = 333
    kk = np.concatenate([np.zeros((s, 2, 16)), O.rope_rotate(k0, np.arange(12) + s, 1e4)])
    vv = np.concatenate([np.zeros((s, 2, 16)), v0])
    qq = O.rope_rotate(q0, rows + s, 1e4)
    # keys below s are masked out by giving them -inf via position gating: use explicit subset
    b = O.causal_attention(qq, kk, vv, rows + s)
    # rows + s also see the s zero-padded keys; compare against an attention that excludes them
    b2 = O.causal_attention(qq, kk[s:], vv[s:], rows)  # same keys, positions relabelled
    np.testing.assert_allclose(a, b2, atol=1e-12)
    assert np.abs(a - b).max() > 1e-6  # sanity: the padding really was visible in b


def test_rmsnorm_closed_form():
    x = np.array([[3.0, 4.0, 0.0, 0.0]])
    # mean square = 25/4 -> rms = 2.5
    np.testing.assert_allclose(O.rmsnorm(x, np.ones(4), 0.0), [[1.2, 1.6, 0.0, 0.0]], atol=1e-15)
    np.testing.assert_allclose(O.rmsnorm(x, np.array([2, 1, 1, 1.0]), 0.0), [[2.4, 1.6, 0, 0]], atol=1e-15)
