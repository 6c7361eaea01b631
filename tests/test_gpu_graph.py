"""The library's calls captured in a HIP graph (torch.cuda.CUDAGraph) and
replayed: every replay, on fresh inputs copied into the captured buffers, with
eager work and synchronisations between replays, equals bit for bit the same
calls run eagerly.  Covers the carry-slot clearing of the chained forward (a
kernel, not a memset node), the caller-owned workspaces and the in-place decode
state, so a serving or training loop may capture these calls."""
import numpy as np
import pytest
import torch

from _helpers import to_dev
from rwkv_wkv_mixing_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
REPLAYS = 3


def ops():
    from rwkv_wkv_mixing_amd import ops as O

    return O


def capture(fn):
    """Warm up on a side stream, then capture fn() into a graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def bf16_dev(bits):
    return to_dev(None, DEV, bits)


def test_forward_backward_graph_replays_equal_eager():
    """wkv_forward (saving states) then wkv_backward from them, bf16 with key
    spikes, T spanning several chained time blocks."""
    O = ops()
    B, T, C = 2, 700, 256
    probs = [W.make_problem(B, T, C, dtype="bf16", seed=60 + i, spike_frac=0.01, name=f"graph {i}")
             for i in range(REPLAYS + 1)]
    p0 = probs[0]
    w, u = to_dev(p0.w, DEV), to_dev(p0.u, DEV)
    k, v, gy = bf16_dev(p0.k_bits), bf16_dev(p0.v_bits), bf16_dev(p0.gy_bits)
    y = torch.empty((B, T, C), device=DEV)
    ck = O.new_ckpt(B, T, C, DEV)
    grads = (torch.empty((B, T, C), device=DEV), torch.empty((B, T, C), device=DEV), torch.empty(C, device=DEV),
             torch.empty(C, device=DEV))
    wsf = O.new_workspace(0, B, T, C, torch.bfloat16, DEV)
    wsb = O.new_workspace(1, B, T, C, torch.bfloat16, DEV)

    def step():
        O.wkv_forward(w, u, k, v, y=y, ckpt=ck, workspace=wsf)
        O.wkv_backward(w, u, k, v, gy, ckpt=ck, out=grads, workspace=wsb)

    g = capture(step)
    for i in range(1, REPLAYS + 1):
        p = probs[i]
        print(f"replay {i}", flush=True)
        for dst, src in ((k, p.k_bits), (v, p.v_bits), (gy, p.gy_bits)):
            dst.copy_(bf16_dev(src))
        g.replay()
        torch.cuda.synchronize()
        got = [y.clone()] + [x.clone() for x in grads]
        ref_y = O.wkv_forward(w, u, k, v)  # eager, on the same inputs, fresh buffers
        ref = [ref_y] + list(O.wkv_backward(w, u, k, v, gy))
        torch.cuda.synchronize()
        for n, a, b in zip(("y", "dk", "dv", "dw", "du"), got, ref):
            assert torch.equal(a, b), f"replay {i}: {n} differs from the eager call"


def test_gated_graph_replays_equal_eager():
    O = ops()
    B, T, C = 2, 300, 128
    probs = [W.make_problem(B, T, C, dtype="bf16", seed=70 + i, name=f"gated graph {i}") for i in range(3)]
    rng = np.random.default_rng(71)
    rbits = [W.bf16_round(rng.standard_normal((B, T, C)).astype(np.float32))[0] for _ in range(3)]
    p0 = probs[0]
    w, u = to_dev(p0.w, DEV), to_dev(p0.u, DEV)
    k, v, gy, r = bf16_dev(p0.k_bits), bf16_dev(p0.v_bits), bf16_dev(p0.gy_bits), bf16_dev(rbits[0])
    out = torch.empty((B, T, C), device=DEV)
    ck = O.new_ckpt(B, T, C, DEV)
    wsf = O.new_workspace(0, B, T, C, torch.bfloat16, DEV)
    wsb = O.new_workspace(1, B, T, C, torch.bfloat16, DEV)
    res = {}

    def step():
        O.wkv_forward_gated(w, u, k, v, r, out=out, ckpt=ck, workspace=wsf)
        res["g"] = O.wkv_backward_gated(w, u, k, v, r, gy, ckpt=ck, workspace=wsb)

    g = capture(step)
    for i in (1, 2):
        p = probs[i]
        for dst, src in ((k, p.k_bits), (v, p.v_bits), (gy, p.gy_bits), (r, rbits[i])):
            dst.copy_(bf16_dev(src))
        g.replay()
        torch.cuda.synchronize()
        got = [out.clone()] + [x.clone() for x in res["g"]]
        ref = [O.wkv_forward_gated(w, u, k, v, r)] + list(O.wkv_backward_gated(w, u, k, v, r, gy))
        torch.cuda.synchronize()
        for n, a, b in zip(("out", "dk", "dv", "dr", "dw", "du"), got, ref):
            assert torch.equal(a, b), f"replay {i}: {n} differs from the eager call"


def test_decode_step_graph_replays_equal_eager():
    """One captured wkv_step replayed token after token, its state updated in
    place, against the same steps run eagerly on a copy of the state."""
    O = ops()
    Ln, B, C = 2, 8, 192
    rng = np.random.default_rng(80)
    w = to_dev(np.exp(rng.uniform(-6, 1.5, (Ln, C))).astype(np.float32), DEV)
    u = to_dev(rng.standard_normal((Ln, C)).astype(np.float32), DEV)
    kb = [W.bf16_round(rng.standard_normal((Ln, B, C)).astype(np.float32))[0] for _ in range(6)]
    vb = [W.bf16_round(rng.standard_normal((Ln, B, C)).astype(np.float32))[0] for _ in range(6)]
    k, v = bf16_dev(kb[0]), bf16_dev(vb[0])
    a, b, p = O.empty_state(Ln, B, C, DEV)
    y = torch.empty((Ln, B, C), device=DEV)
    ea, eb, ep = O.empty_state(Ln, B, C, DEV)
    O.wkv_step(w, u, k, v, ea, eb, ep)  # the warm-up step inside capture() also advances the captured state
    g = capture(lambda: O.wkv_step(w, u, k, v, a, b, p, y=y))
    a.copy_(ea), b.copy_(eb), p.copy_(ep)  # both now one step in
    for t in range(1, 6):
        k.copy_(bf16_dev(kb[t]))
        v.copy_(bf16_dev(vb[t]))
        g.replay()
        torch.cuda.synchronize()
        ey = O.wkv_step(w, u, k, v, ea, eb, ep)
        torch.cuda.synchronize()
        for n, x1, x2 in (("y", y, ey), ("a", a, ea), ("b", b, eb), ("p", p, ep)):
            assert torch.equal(x1, x2), f"step {t}: {n} differs from the eager step"


@pytest.mark.parametrize("T", [150, 300])
@pytest.mark.parametrize("gen", [5, 6])
def test_matrix_state_graph_replays_equal_eager(gen, T):
    """RWKV-5 / RWKV-6: the forward saving its chunk-start states, then the
    backward from them, with a given initial state and final-state gradient
    (at 300 tokens the forward splits the sequence into segments)."""
    O = ops()
    B, H = 2, 2
    mk = W.make_wkv5 if gen == 5 else W.make_wkv6
    probs = [mk(B, T, H, seed=90 + i, with_state=True) for i in range(3)]
    gos = [W.wkv5_go(q, seed=95 + i)[0] for i, q in enumerate(probs)]
    p0 = probs[0]
    w, u = to_dev(p0.w, DEV), to_dev(p0.u, DEV)
    r, k, v, go = (bf16_dev(x) for x in (p0.r_bits, p0.k_bits, p0.v_bits, gos[0]))
    S0 = to_dev(p0.S0, DEV)
    dST = to_dev(np.random.default_rng(99).standard_normal((B, H, 64, 64)).astype(np.float32), DEV)
    fwd = O.wkv5_forward if gen == 5 else O.wkv6_forward
    bwd = O.wkv5_backward if gen == 5 else O.wkv6_backward
    o = torch.empty((B, T, 64 * H), device=DEV)
    ST = torch.empty((B, H, 64, 64), device=DEV)
    ck = O.new_wkv5_ckpt(B, T, H, DEV)
    nws = int((O.L.lib().wkv5_backward_workspace_bytes if gen == 5 else O.L.lib().wkv6_backward_workspace_bytes)(
        B, T, H, 64, 1))
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=DEV)
    res = {}

    def step():
        fwd(w, u, r, k, v, state_in=S0, state_out=ST, out=o, ckpt=ck)
        res["g"] = bwd(w, u, r, k, v, go, state_in=S0, grad_state_out=dST, need_state_grad=True, ckpt=ck,
                       workspace=ws)

    g = capture(step)
    for i in (1, 2):
        q = probs[i]
        for dst, src in ((r, q.r_bits), (k, q.k_bits), (v, q.v_bits), (go, gos[i])):
            dst.copy_(bf16_dev(src))
        g.replay()
        torch.cuda.synchronize()
        got = [o.clone(), ST.clone(), ck.clone()] + [x.clone() for x in res["g"]]
        # the eager pair also goes through saved states: a backward without them
        # recomputes the chunk-start states unsplit, which may round differently
        eck = O.new_wkv5_ckpt(B, T, H, DEV)
        eo, eS = fwd(w, u, r, k, v, state_in=S0, return_state=True, ckpt=eck)
        ref = [eo, eS, eck] + list(bwd(w, u, r, k, v, go, state_in=S0, grad_state_out=dST, need_state_grad=True,
                                       ckpt=eck))
        torch.cuda.synchronize()
        for n, a, b in zip(("o", "S_T", "ckpt", "dr", "dk", "dv", "dw", "du", "dS0"), got, ref):
            assert torch.equal(a, b), f"RWKV-{gen} replay {i}: {n} differs from the eager call"
