"""GPU parity at the full sizes of the stacked workloads, in the launch
configuration bench.py times (all layers resident, one decode call through
every layer with the pre-norm residual stream).

The oracle is teacher-forced: for sampled layers it gets the GPU's own input
x_l (from single-layer calls that chain bitwise-identically to the full call)
and checks that layer's ids, weights and output for sampled tokens."""
import numpy as np
import pytest
import torch

import synth
from oracle import moe as om
from tests.gpu_util import TOL_REL_L2, say, workload

pytestmark = pytest.mark.gpu

# workload -> (token counts, layers checked against the oracle, tokens checked per layer)
CASES = {
    "a3b_stack40_zipf": ((1, 4, 16, 64), (0, 21, 39), 3),
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
        for l in range(wl.n_layers):
            lw = synth.layer_weights(wl, l)
            self.moe.upload(l, lw)
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
    y_full = moe.decode(x, n_layers=L, residual=True, prenorm=True, ids_out=ids, w_out=w,
                        path="persistent")
    torch.cuda.synchronize()
    assert torch.isfinite(y_full).all()
    cur = x
    for l in range(L):
        nxt = moe.decode(cur, layer0=l, n_layers=1, residual=True, prenorm=True, path="persistent")
        if l in st.oracle:
            torch.cuda.synchronize()
            toks = np.sort(rng.choice(T, size=min(n_tok, T), replace=False))
            xin = cur.cpu().numpy()[toks]
            ref = om.moe_layer(st.oracle[l], xin, residual=True, prenorm=True)
            assert np.all(ref["gap"] > 1e-9)
            assert np.array_equal(ids[l].cpu().numpy()[toks], ref["ids"])
            assert np.max(np.abs(w[l].cpu().numpy()[toks] - ref["w"])) < 1e-6
            # the MoE output itself: subtract the residual input on both sides
            x64 = xin.astype(np.float64)
            err = float(np.max(om.rel_l2(nxt.cpu().numpy()[toks] - x64, ref["y"] - x64)))
            say(f"  {name} T={T} layer {l} tokens {toks.tolist()}: max rel-L2 {err:.3e}")
            assert err <= TOL_REL_L2
        cur = nxt
    torch.cuda.synchronize()
    assert torch.equal(cur, y_full), "full call differs from chained single-layer calls"
    idn = ids.cpu().numpy()
    assert idn.min() >= 0 and idn.max() < wl.n_experts
    for l in range(L):
        for t in range(T):
            assert len(set(idn[l, t].tolist())) == wl.top_k
