"""Host-side logic of the layer block (no GPU): the weight stacking and the views
of the projection output must hand each launch the columns the oracle's layer
composition uses for it."""
import numpy as np
import pytest
import torch

import oracle
from hybrid_linear_attention_amd.layer import GdnLayer, stack_weights
from hybrid_linear_attention_amd.workloads import TINY_DIMS


def test_projection_views_match_oracle_split():
    d = TINY_DIMS
    hidden, T = 24, 5
    rng = np.random.default_rng(7)
    cq = 2 * d.num_k_heads * d.head_dim_k + d.num_v_heads * d.head_dim_v
    cz = d.num_v_heads * d.head_dim_v
    W_qkvz = torch.from_numpy(rng.standard_normal((hidden, cq + cz)))
    W_ba = torch.from_numpy(rng.standard_normal((hidden, 2 * d.num_v_heads)))
    W_o = torch.from_numpy(rng.standard_normal((cz, hidden)))
    conv_w = torch.from_numpy(rng.standard_normal((cq, 4)))
    g_in = torch.ones(hidden, dtype=torch.float64)
    g_out = torch.ones(d.head_dim_v, dtype=torch.float64)
    w = stack_weights(d, W_qkvz, W_ba, W_o, conv_w, g_in, g_out, device="cpu")
    assert tuple(w.W_in.shape) == (cq + cz + 2 * d.num_v_heads, hidden)
    assert tuple(w.W_out.shape) == (hidden, cz)
    layer = GdnLayer(d, w, T, 1, T - 2, 2, device="cpu")
    X = rng.standard_normal((T, hidden))
    qsl = np.array([0, T - 2, T - 1, T], np.int32)
    _, _, _, inter = oracle.gdn_layer(
        X, np.ones(hidden), W_qkvz.numpy(), W_ba.numpy(), conv_w.numpy(), np.ones(d.head_dim_v),
        W_o.numpy(), np.zeros((3, cq, 3)), np.zeros((3, d.num_v_heads, d.head_dim_v,
                                                     d.head_dim_k)),
        qsl, np.arange(3, dtype=np.int32), np.zeros(3, np.uint8), d.num_k_heads, d.num_v_heads,
        d.head_dim_k, d.head_dim_v, 1e-6, 1e-6)
    Uo = inter["U"]
    # project the oracle's own U through the stacked weight
    layer.P = torch.from_numpy(Uo) @ w.W_in.t()
    np.testing.assert_allclose(layer.x_qkv().numpy(), inter["x_qkv"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(layer.z().numpy().reshape(T, d.num_v_heads, d.head_dim_v),
                               inter["Z"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(layer.a().numpy(), inter["a"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(layer.b().numpy(), inter["b"], rtol=1e-12, atol=1e-12)


def test_layer_rejects_inconsistent_batch():
    d = TINY_DIMS
    cq = 2 * d.num_k_heads * d.head_dim_k + d.num_v_heads * d.head_dim_v
    cz = d.num_v_heads * d.head_dim_v
    w = stack_weights(d, torch.zeros(8, cq + cz), torch.zeros(8, 2 * d.num_v_heads),
                      torch.zeros(cz, 8), torch.zeros(cq, 4), torch.ones(8),
                      torch.ones(d.head_dim_v), device="cpu")
    with pytest.raises(ValueError):
        GdnLayer(d, w, 10, 1, 8, 3, device="cpu")
    bad = stack_weights(d, torch.zeros(8, cq), torch.zeros(8, 2 * d.num_v_heads),
                        torch.zeros(cz, 8), torch.zeros(cq, 4), torch.ones(8),
                        torch.ones(d.head_dim_v), device="cpu")
    with pytest.raises(ValueError):
        GdnLayer(d, bad, 10, 1, 8, 2, device="cpu")


@pytest.mark.parametrize("fused", [True, False], ids=["fused", "separate"])
def test_every_stage_gets_the_stream(monkeypatch, fused):
    """Each launch of GdnLayer.stages binds the stream it is given to the entry
    point's `stream` parameter (an argument passed by position into the wrong
    slot would go unnoticed with the default stream)."""
    import inspect

    from hybrid_linear_attention_amd import gdn

    d = TINY_DIMS
    hidden, T = 24, 5
    cq = 2 * d.num_k_heads * d.head_dim_k + d.num_v_heads * d.head_dim_v
    cz = d.num_v_heads * d.head_dim_v
    w = stack_weights(d, torch.zeros(hidden, cq + cz), torch.zeros(hidden, 2 * d.num_v_heads),
                      torch.zeros(cz, hidden), torch.zeros(cq, 4), torch.ones(hidden),
                      torch.ones(d.head_dim_v), device="cpu")
    layer = GdnLayer(d, w, T, 1, T - 2, 2, device="cpu", fused=fused)
    seen = []
    for name in ("gdn_rmsnorm", "gdn_gemm_bf16", "gdn_prefill_fused", "gdn_decode_fused",
                 "gdn_conv1d_update", "gdn_prefill_varlen", "gdn_decode_step", "gdn_gated_norm"):
        orig = getattr(gdn, name)

        def rec(*args, _orig=orig, _name=name, **kw):
            bound = inspect.signature(_orig).bind(*args, **kw)
            seen.append((_name, bound.arguments.get("stream")))
        monkeypatch.setattr(gdn, name, rec)
    sentinel = object()
    meta = torch.zeros(4, dtype=torch.int32)
    for _, fn in layer.stages(torch.zeros(T, hidden), None, None, meta, meta, meta, sentinel):
        fn()
    assert len(seen) == (5 if fused else 7)
    assert all(s is sentinel for _, s in seen), seen
