"""Pins of the oracle's expert FFN, combine and stacked layers against
brute force (every expert evaluated densely with torch's fp64 ops, then the
router's mask applied) and closed-form special cases."""
import numpy as np
import pytest
import torch

import synth
from oracle import moe as om


def _tiny(gate_up="q2k", shared=0, E=8, k=2, zipf=None, L=1, shared_format="bf16", tail=0):
    return synth.Workload("pin", 99, 256, E, k, 256, shared, gate_up, "q2k", L, (1,), zipf_s=zipf,
                          shared_format=shared_format, tail_layers=tail)


def _dense_reference(wl, lw, cb, x):
    """All E experts evaluated densely with torch fp64, combined through a
    one-hot selection mask built from torch.topk on the logits."""
    xt = torch.from_numpy(x.astype(np.float64))
    lg = xt @ torch.from_numpy(lw.router.astype(np.float64)).T
    if lw.router_bias is not None:
        lg = lg + torch.from_numpy(lw.router_bias.astype(np.float64))
    vals, idx = torch.topk(lg, wl.top_k, dim=1)
    wts = torch.softmax(vals, dim=1)
    mask = torch.zeros(lg.shape, dtype=torch.float64)
    mask.scatter_(1, idx, wts)
    y = torch.zeros((x.shape[0], wl.hidden), dtype=torch.float64)
    gf, df = lw.gate_up_format, lw.down_format
    for e in range(wl.n_experts):
        wg = torch.from_numpy(om.dequant_matrix(lw.gate[e], gf, cb).astype(np.float64))
        wu = torch.from_numpy(om.dequant_matrix(lw.up[e], gf, cb).astype(np.float64))
        wd = torch.from_numpy(om.dequant_matrix(lw.down[e], df, cb).astype(np.float64))
        o = (torch.nn.functional.silu(xt @ wg.T) * (xt @ wu.T)) @ wd.T
        y += mask[:, e:e + 1] * o
    if wl.shared_ffn and wl.shared_format == "q8":
        sg, su, sd = (torch.from_numpy(om.dequant_matrix(m, "q8").astype(np.float64)) for m in
                      (lw.shared_gate, lw.shared_up, lw.shared_down))
        y += (torch.nn.functional.silu(xt @ sg.T) * (xt @ su.T)) @ sd.T
    elif wl.shared_ffn:
        sg, su, sd = (torch.from_numpy(om.bf16_bits_to_f64(m)) for m in
                      (lw.shared_gate, lw.shared_up, lw.shared_down))
        y += (torch.nn.functional.silu(xt @ sg.T) * (xt @ su.T)) @ sd.T
    return y.numpy(), idx.numpy()


@pytest.mark.parametrize("gate_up,shared,zipf,sfmt,tail", [("q2k", 0, None, "bf16", 0), ("cb2", 0, None, "bf16", 0),
                                                           ("cb2", 256, 1.1, "bf16", 0), ("q2k", 256, None, "bf16", 0),
                                                           ("cb2", 256, 1.1, "q8", 0), ("cb2", 256, 1.1, "bf16", 1)])
def test_routed_layer_equals_dense_masked_brute_force(gate_up, shared, zipf, sfmt, tail):
    """(tail = 1: the layer's experts in the Q4_K-style type.)"""
    wl = _tiny(gate_up, shared, zipf=zipf, shared_format=sfmt, tail=tail)
    lw = synth.layer_weights(wl, 0)
    cb = synth.codebook()
    x = synth.tokens(wl, 6)
    r = om.moe_layer(om.Layer(wl, lw, cb), x)
    y, idx = _dense_reference(wl, lw, cb, x)
    assert np.all(r["gap"] > 1e-9)                 # no near-ties in the set
    assert np.array_equal(r["ids"], idx)
    assert np.max(om.rel_l2(r["y"], y)) < 1e-6      # fp32 rounding of the output only


def test_silu_matches_torch():
    v = np.linspace(-30, 30, 2001)
    assert np.allclose(om.silu(v), torch.nn.functional.silu(torch.from_numpy(v)).numpy(),
                       rtol=1e-14, atol=1e-300)
    assert om.silu(np.array([0.0]))[0] == 0.0


def test_identical_experts_make_routing_irrelevant():
    """All experts equal and no shared expert: y = FFN(x) for any routing."""
    wl = _tiny("cb2", 0, E=6, k=3)
    lw = synth.layer_weights(wl, 0)
    for m in (lw.gate, lw.up, lw.down):
        m[:] = m[0]
    cb = synth.codebook()
    x = synth.tokens(wl, 3)
    r = om.moe_layer(om.Layer(wl, lw, cb), x)
    xt = torch.from_numpy(x.astype(np.float64))
    wg = torch.from_numpy(om.dequant_matrix(lw.gate[0], "cb2", cb).astype(np.float64))
    wu = torch.from_numpy(om.dequant_matrix(lw.up[0], "cb2", cb).astype(np.float64))
    wd = torch.from_numpy(om.dequant_matrix(lw.down[0], "q2k", cb).astype(np.float64))
    ref = ((torch.nn.functional.silu(xt @ wg.T) * (xt @ wu.T)) @ wd.T).numpy()
    assert np.max(om.rel_l2(r["y"], ref)) < 1e-6


def test_zero_input_gives_zero_output():
    wl = _tiny("cb2", 256)
    lw = synth.layer_weights(wl, 0)
    r = om.moe_layer(om.Layer(wl, lw, synth.codebook()), np.zeros((2, wl.hidden), np.float32))
    assert np.all(r["y"] == 0.0)


def test_k1_output_is_the_argmax_expert_plus_shared():
    wl = _tiny("q2k", 256, E=5, k=1)
    lw = synth.layer_weights(wl, 0)
    cb = synth.codebook()
    L = om.Layer(wl, lw, cb)
    x = synth.tokens(wl, 2)
    r = om.moe_layer(L, x)
    lg = om.router_logits(x, lw.router)
    for t in range(2):
        e = int(np.argmax(lg[t]))
        _, o = om.swiglu_ffn(x[t], *L.expert(e))
        _, s = om.swiglu_ffn(x[t], *L.shared())
        assert np.max(om.rel_l2(r["y"][t], o + s)) < 1e-6


def _scale_fields(down, fn):
    for field in (80, 82):
        bits = down[..., field].astype(np.uint16) | (down[..., field + 1].astype(np.uint16) << 8)
        bits = fn(bits)
        down[..., field] = bits & 0xFF
        down[..., field + 1] = bits >> 8


def test_combine_is_linear_in_expert_outputs():
    """Scaling every down matrix by 2 (exactly: d and dmin exponents +1)
    doubles the routed part of the output."""
    wl = _tiny("cb2", 0)
    cb = synth.codebook()
    x = synth.tokens(wl, 2)
    lw = synth.layer_weights(wl, 0)
    _scale_fields(lw.down, lambda b: np.where((b >> 10) & 0x1F == 0, b | 0x0400, b))  # all normal
    lw2 = synth.layer_weights(wl, 0)
    lw2.down[:] = lw.down
    _scale_fields(lw2.down, lambda b: b + 0x0400)                                    # exactly 2x
    y1 = om.moe_layer(om.Layer(wl, lw, cb), x)["y"]
    y2 = om.moe_layer(om.Layer(wl, lw2, cb), x)["y"]
    assert np.max(om.rel_l2(y2, 2 * y1.astype(np.float64))) < 1e-6


def test_residual_and_stack_chain():
    wl = _tiny("cb2", 256, L=3)
    cb = synth.codebook()
    layers = [om.Layer(wl, synth.layer_weights(wl, l), cb) for l in range(3)]
    x = synth.tokens(wl, 2)
    for prenorm in (False, True):
        out, per = om.moe_stack(layers, x, prenorm=prenorm)
        cur = x
        for l in range(3):
            r = om.moe_layer(layers[l], cur, prenorm=prenorm)
            cur = (cur.astype(np.float64) + r["y"].astype(np.float64))
            assert np.max(om.rel_l2(per[l]["y"], cur)) < 1e-6
            cur = per[l]["y"]
        assert np.array_equal(out, per[-1]["y"])


def test_rms_inv_matches_torch_rms_norm():
    x = np.random.default_rng(5).standard_normal((7, 512)).astype(np.float32) * 3
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x.astype(np.float64)), (512,), eps=om.RMS_EPS)
    got = x.astype(np.float64) * om.rms_inv(x)[:, None]
    assert np.allclose(got, ref.numpy(), rtol=1e-14, atol=0)
    c = 0.5
    assert om.rms_inv(np.full((1, 64), c))[0] == 1.0 / np.sqrt(c * c + om.RMS_EPS)


def test_prenorm_layer_is_scale_invariant():
    """With the pre-norm, MoE(RMSNorm(a*x)) = MoE(RMSNorm(x)) for a > 0 (up to
    the eps term), so y(a*x) - a*x equals y(x) - x."""
    wl = _tiny("cb2", 256, zipf=1.1)
    L = om.Layer(wl, synth.layer_weights(wl, 0), synth.codebook())
    x = synth.tokens(wl, 3)
    r1 = om.moe_layer(L, x, residual=False, prenorm=True)
    r2 = om.moe_layer(L, 8 * x, residual=False, prenorm=True)
    assert np.array_equal(r1["ids"], r2["ids"])
    assert np.max(om.rel_l2(r2["y"], r1["y"])) < 1e-5
    # and the routing equals routing the explicitly normalised input
    xn = (x.astype(np.float64) * om.rms_inv(x)[:, None]).astype(np.float32)
    r3 = om.moe_layer(L, xn, prenorm=False)
    assert np.array_equal(r1["ids"], r3["ids"])


def test_prenorm_chain_stays_bounded():
    wl = _tiny("cb2", 256, L=12, zipf=1.1)
    cb = synth.codebook()
    layers = [om.Layer(wl, synth.layer_weights(wl, l), cb) for l in range(12)]
    out, _ = om.moe_stack(layers, synth.tokens(wl, 2), prenorm=True)
    assert np.all(np.isfinite(out)) and np.sqrt(np.mean(out.astype(np.float64) ** 2)) < 10


def test_generator_is_deterministic_and_keyed():
    wl = synth.WORKLOADS["tiny_q2k"]
    a = synth.layer_weights(wl, 0)
    b = synth.layer_weights(wl, 0, experts=[3, 1])
    assert np.array_equal(a.gate[3], b.gate[0]) and np.array_equal(a.down[1], b.down[1])
    c = synth.layer_weights(wl, 1)
    assert not np.array_equal(a.gate, c.gate)
    assert np.array_equal(synth.tokens(wl, 4, 2), synth.tokens(wl, 4, 2))


def test_rel_l2_hand_worked():
    """Per row ||got - ref|| / ||ref||, worked by hand: (3,4)->(3,9) differs by
    (0,5), |ref| = 5 -> 1.0; (1,0,0)->(3,2,1) differs by (2,2,1), |.| = 3,
    |ref| = 1 -> 3.0; a zero reference row divides by 1 (|got| = 1 -> 1.0);
    an exact match gives 0."""
    got = om.rel_l2(np.array([[3.0, 9.0, 0.0], [3.0, 2.0, 1.0], [0.6, 0.8, 0.0], [1.5, -2.0, 0.25]]),
                    np.array([[3.0, 4.0, 0.0], [1.0, 0.0, 0.0], [0.0, 0.0, 0.0], [1.5, -2.0, 0.25]]))
    assert got.tolist() == [1.0, 3.0, 1.0, 0.0]
    assert om.rel_l2(np.array([2.0, 0.0]), np.array([1.0, 0.0])) == 1.0    # one row


def test_prenorm_logits_are_the_router_on_the_normalised_input():
    """With the pre-norm the router sees RMSNorm(x): torch's rms_norm (no
    weight) followed by a torch fp64 matmul and the bias gives the logits."""
    wl = _tiny("cb2", 0, zipf=1.1)
    lw = synth.layer_weights(wl, 0)
    x = synth.tokens(wl, 4) * 3
    r = om.moe_layer(om.Layer(wl, lw, synth.codebook()), x, prenorm=True)
    u = torch.nn.functional.rms_norm(torch.from_numpy(x.astype(np.float64)), (wl.hidden,), eps=om.RMS_EPS)
    ref = u @ torch.from_numpy(lw.router.astype(np.float64)).T + torch.from_numpy(
        lw.router_bias.astype(np.float64))
    assert np.allclose(r["logits"], ref.numpy(), rtol=1e-13, atol=1e-13)
