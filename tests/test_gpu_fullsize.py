"""GPU parity at the full sizes of the stacked workloads, in the launch
configuration bench.py times (all layers resident, one decode call through
every layer with the pre-norm residual stream).

The oracle is teacher-forced: it gets the GPU's own input x_l of every layer
(from single-layer calls that chain bitwise-identically to the full call).
For every layer and every token the expert ids must equal the oracle's
routing exactly and the router weights must agree within 1e-6; for sampled
layers and tokens the whole layer output is compared as well."""
from types import SimpleNamespace

import numpy as np
import pytest
import torch

import synth
from oracle import moe as om
from tests.gpu_util import TOL_REL_L2, say, workload

pytestmark = pytest.mark.gpu

# workload -> (token counts, layers whose full output is checked, tokens checked per such layer)
CASES = {
    "a3b_stack40_zipf": ((1, 4, 16, 64), (0, 21, 39), 3),
    "a3b_routed40": ((1, 4), (0, 39), 2),
    "a3b_routed40_q2k": ((1,), (0, 39), 1),
    "a3b_stack40_zipf_q8": ((1, 4, 16), (0, 39), 2),
    "a3b_stack40_q4tail": ((1, 4, 16), (0, 33, 34, 39), 2),
    "flash_stack8_zipf": ((1, 8, 32), (0, 7), 2),
}
PARAMS = [(n, T) for n, c in CASES.items() for T in c[0]]


class Stack:
    def __init__(self, lib, name):
        self.name = name
        self.wl = wl = workload(name)
        check = CASES[name][1]
        cb = synth.codebook()
        say(f"generating and uploading {name}: {wl.n_layers} layers")
        self.moe = lib.MoE.for_workload(wl, cb, max_tokens=max(CASES[name][0]))
        self.oracle = {}
        self.routers = []
        for l in range(wl.n_layers):
            lw = synth.layer_weights(wl, l)
            self.moe.upload(l, lw)
            self.routers.append(SimpleNamespace(router=lw.router, router_bias=lw.router_bias))
            if l in check:
                self.oracle[l] = om.Layer(wl, lw, cb)   # dequantised experts cached across T


_stacks = {}


@pytest.fixture(scope="module")
def stacks(lib):
    yield _stacks
    for s in _stacks.values():
        s.moe.close()
    _stacks.clear()


@pytest.mark.parametrize("name,T", PARAMS, ids=[f"{n}-T{T}" for n, T in PARAMS])
def test_full_stack_parity(lib, stacks, name, T):
    if name not in stacks:
        for other in list(stacks):                 # one stack resident at a time
            stacks.pop(other).moe.close()
        stacks[name] = Stack(lib, name)
    st = stacks[name]
    wl, moe = st.wl, st.moe
    L = wl.n_layers
    n_tok = CASES[name][2]
    rng = np.random.default_rng(11 + T)
    say(f"{name} T={T}: full {L}-layer call")
    x = torch.from_numpy(synth.tokens(wl, T, 7)).cuda()
    ids = torch.empty((L, T, wl.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((L, T, wl.top_k), dtype=torch.float32, device="cuda")
    y_full = moe.decode(x, n_layers=L, residual=True, prenorm=True, ids_out=ids, w_out=w)
    moe.sync_status()
    assert torch.isfinite(y_full).all()
    idn, wn = ids.cpu().numpy(), w.cpu().numpy()
    cur = x
    for l in range(L):
        nxt = moe.decode(cur, layer0=l, n_layers=1, residual=True, prenorm=True)
        moe.sync_status()
        xin_all = cur.cpu().numpy()
        # routing of every token of this layer against the oracle's
        _, _, ids_ref, w_ref, gap = om.route(st.routers[l], xin_all, wl.top_k, prenorm=True)
        assert np.all(gap > 1e-9), f"layer {l}: near-tie in the routing set"
        assert np.array_equal(idn[l], ids_ref), f"layer {l}: expert ids differ"
        assert np.max(np.abs(wn[l] - w_ref)) < 1e-6, f"layer {l}: router weights differ"
        if l in st.oracle:
            toks = np.sort(rng.choice(T, size=min(n_tok, T), replace=False))
            xin = xin_all[toks]
            ref = om.moe_layer(st.oracle[l], xin, residual=True, prenorm=True)
            assert np.array_equal(idn[l][toks], ref["ids"])
            # the MoE output itself: subtract the residual input on both sides
            x64 = xin.astype(np.float64)
            err = float(np.max(om.rel_l2(nxt.cpu().numpy()[toks] - x64, ref["y"] - x64)))
            say(f"  {name} T={T} layer {l} tokens {toks.tolist()}: max rel-L2 {err:.3e}")
            assert err <= TOL_REL_L2
        cur = nxt
    say(f"  {name} T={T}: ids and weights of all {L} layers x {T} tokens match the oracle")
    assert torch.equal(cur, y_full), "full call differs from chained single-layer calls"
