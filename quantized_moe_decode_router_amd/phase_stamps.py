"""Per-phase timing of the small-batch persistent kernel (profiling only).

Runs decode calls through the profiling build of the library
(``libqsmoe_stamps.so``: ``python -m quantized_moe_decode_router_amd.build
--stamps``), in which thread 0 of each workgroup records the GPU's 100 MHz
wall clock (``s_memrealtime``) at the phase boundaries of every layer, and
prints where a layer's time goes: mean over workgroups and over the middle
layers of the stack, plus finer points within the last layer of the call.

    QSMOE_LIB_VARIANT=stamps python -m quantized_moe_decode_router_amd.phase_stamps a3b_stack40_zipf 1

(the variable must be set before the package is imported: it selects the
library that the binding loads).

Every input is the seeded synthetic workload of ``synth``.  A stamp costs
about 0.1 us (reading the clock waits for the wave's outstanding LDS and
scalar loads), so the layer period here is above the one ``bench.py``
implies by about 2 us at one token.
"""
from __future__ import annotations

import ctypes
import sys

import numpy as np

N_LAYERS, N_WGS, N_PTS = 64, 256, 24   # the stamp buffer's shape (qs_persist.h)

# main points of layer l (row l): name, from, to
MAIN = [
    ("x exchange: last store of the previous layer -> seen", "last14", 1),
    ("x seen -> this layer's staged rows landed", 1, 2),
    ("router (a1)", 2, 3),
    ("shared gate/up (a7)", 3, 4),
    ("logits exchange wait", 4, 5),
    ("top-k + grouping (a2, a3)", 5, 6),
    ("gate/up tile issue + x quantisation", 6, 7),
    ("barrier", 7, 8),
    ("gate/up GEMV + SwiGLU + stores (a4)", 8, 9),
    ("down-row copy issue", 9, 10),
    ("SwiGLU exchange wait", 10, 11),
    ("down rows landed", 11, 12),
    ("down GEMVs, routed + shared (a6, a7)", 12, 13),
    ("combine (a6)", 13, 14),
]
# finer points of the last layer (row N_LAYERS - 1), relative to its main points
FINE = [
    ("router: partial sums", ("m", 2), ("f", 20)),
    ("router: barrier", ("f", 20), ("f", 21)),
    ("router: final sums, RMS scale, stores", ("f", 21), ("m", 3)),
    ("top-k: keys and threshold", ("m", 5), ("f", 22)),
    ("top-k: candidates and rank", ("f", 22), ("f", 23)),
    ("top-k: weights, grouping, barrier", ("f", 23), ("m", 6)),
    ("gate/up tile loads issued", ("m", 6), ("f", 0)),
    ("x quantisation", ("f", 0), ("m", 7)),
    ("down tile 0: routed experts", ("f", 13), ("f", 14)),
    ("down tile 0: shared rows", ("f", 14), ("f", 15)),
]


def main(argv):
    name = argv[0] if argv else "a3b_stack40_zipf"
    T = int(argv[1]) if len(argv) > 1 else 1
    import torch
    import quantized_moe_decode_router_amd as qm
    import synth
    if not qm.LIB_PATH.endswith("libqsmoe_stamps.so"):
        raise SystemExit("the profiling build is not the one loaded: set QSMOE_LIB_VARIANT=stamps")
    read = qm.LIB.qs_debug_read_stamps
    read.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    wl = synth.WORKLOADS[name]
    L = wl.n_layers
    moe = qm.MoE.for_workload(wl, synth.codebook(), n_layers=L, max_tokens=T)
    for l in range(L):
        moe.upload(l, synth.layer_weights(wl, l))
    xs = [torch.from_numpy(synth.tokens(wl, T, b)).cuda() for b in range(3)]
    y = torch.empty_like(xs[0])
    main_v = {k[0]: [] for k in MAIN}
    fine_v = {k[0]: [] for k in FINE}
    periods = []
    for it in range(5):
        for x in xs:
            moe.decode(x, y, n_layers=L, residual=True, prenorm=True, exclusive=True)
        torch.cuda.synchronize()
        st = np.zeros(N_LAYERS * N_WGS * N_PTS, dtype=np.uint64)
        if read(st.ctypes.data, st.nbytes) != 0:
            raise SystemExit("qs_debug_read_stamps failed")
        S = st.reshape(N_LAYERS, N_WGS, N_PTS).astype(np.int64) * 10   # ns
        S = S[:, :min(N_WGS, wl.hidden // 8)]   # the small-batch grid: at most hidden / 8 workgroups
        mid = range(2, L - 1)
        periods += [(S[l + 1, :, 14].max() - S[l, :, 14].max()) / 1000 for l in mid]
        for lab, a, b in MAIN:
            for l in mid:
                va = S[l - 1, :, 14].max() if a == "last14" else S[l, :, a]
                main_v[lab].append(np.mean(S[l, :, b] - va) / 1000)
        M, R = S[L - 1], S[N_LAYERS - 1]
        for lab, (ka, ia), (kb, ib) in FINE:
            va = (M if ka == "m" else R)[:, ia]
            vb = (M if kb == "m" else R)[:, ib]
            d = (vb - va) / 1000
            ok = (d >= 0) & (d < 200)
            if ok.any():
                fine_v[lab].append(float(np.mean(d[ok])))
    print(f"== {name} T={T}: layer period {np.mean(periods):.2f} us (layers 2..{L - 2}, "
          f"5 x {len(xs)} calls; mean over workgroups)")
    for lab, _, _ in MAIN:
        print(f"  {lab:52s} {np.mean(main_v[lab]):6.2f} us")
    print("  last layer of the call:")
    for lab, _, _ in FINE:
        v = fine_v[lab]
        print(f"    {lab:50s} {np.mean(v):6.2f} us" if v else f"    {lab:50s}    -")


if __name__ == "__main__":
    main(sys.argv[1:])
