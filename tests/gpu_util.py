"""Helpers shared by the GPU tests: build a library handle for a synthetic
workload and compare it with the oracle."""
import sys

import numpy as np

import synth
from oracle import moe as om

TOL_REL_L2 = 1e-3          # max relative L2 error of the fp32 outputs


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def workload(key, **over):
    wl = synth.WORKLOADS[key]
    if over:
        d = dict(wl.__dict__)
        d.update(over)
        wl = synth.Workload(**d)
    return wl


def make_handle(qm, wl, n_layers=None, max_tokens=64, layers=None, **kw):
    """Create a handle and upload layers; returns (moe, [LayerWeights])."""
    cb = synth.codebook()
    n = n_layers or wl.n_layers
    moe = qm.MoE.for_workload(wl, cb, n_layers=n, max_tokens=max_tokens, **kw)
    lws = []
    for l in range(n) if layers is None else layers:
        lw = synth.layer_weights(wl, l)
        moe.upload(l, lw)
        lws.append(lw)
    return moe, lws


def oracle_layer(wl, lw):
    return om.Layer(wl, lw, synth.codebook())


def check_layer(wl, lw, x_np, y_gpu, ids_gpu=None, w_gpu=None, residual=False, prenorm=False,
                label="", tokens=None, steering=None):
    """Compare one layer's GPU outputs with the oracle (optionally only the
    token rows in ``tokens``); returns max rel-L2."""
    if tokens is not None:
        x_np, y_gpu = x_np[tokens], y_gpu[tokens]
        ids_gpu = None if ids_gpu is None else ids_gpu[tokens]
        w_gpu = None if w_gpu is None else w_gpu[tokens]
    ref = om.moe_layer(oracle_layer(wl, lw), x_np, residual=residual, prenorm=prenorm, steering=steering)
    assert np.all(ref["gap"] > 1e-9), f"{label}: near-tie in the routing set"
    if ids_gpu is not None:
        assert np.array_equal(ids_gpu, ref["ids"]), f"{label}: expert ids differ"
    if w_gpu is not None:
        assert np.max(np.abs(w_gpu - ref["w"])) < 1e-6, f"{label}: router weights differ"
    if residual:   # compare the MoE output itself, not the residual sum
        x64 = np.asarray(x_np, dtype=np.float64)
        err = float(np.max(om.rel_l2(y_gpu - x64, ref["y"] - x64)))
    else:
        err = float(np.max(om.rel_l2(y_gpu, ref["y"])))
    say(f"  {label}: max rel-L2 {err:.3e}")
    assert err <= TOL_REL_L2, f"{label}: rel-L2 {err} > {TOL_REL_L2}"
    return err
