"""The attention path under HIP graph capture: SLA forward + backward, and the
STU layer forward, recorded once (caller-owned outputs and workspaces) and
replayed.  The kernels read the layout on the device and pick their work from
it, so one recording serves any input values; their sums run in a fixed
order, so each replay is bitwise equal to an eager call on the same inputs.
Every replay is checked against an eager result, with eager work and
synchronisations between the replays, and the inputs rewritten in place
between some of them."""
import numpy as np
import pytest
import torch

import sparse_sequence_attention_amd as sla
from synthetic import make_sla_workload, make_stack_workload

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _eager_work():
    a = torch.randn(512, 512, device=DEV)
    (a @ a).sum().item()
    torch.cuda.synchronize()


def test_sla_fwd_bwd_graph_replays_match_eager():
    w = make_sla_workload("jagged_2k", seed=3, with_dout=True,
                          lengths=[1910, 1533, 809, 923, 122, 225, 64, 1])
    t = lambda a: torch.from_numpy(a).to(DEV).to(torch.bfloat16)  # noqa: E731
    q, k, v, do = t(w.q), t(w.k), t(w.v), t(w.dout)
    offs = torch.from_numpy(w.offsets).to(DEV)
    kw = dict(k1=w.k1, k2=w.k2, contextual_len=w.contextual_len, max_seq_len=w.max_seq_len,
              alpha=w.alpha)
    T, H, d = q.shape
    print(f"[case] graph sla fwd+bwd T={T} H={H} d={d}", flush=True)
    o = torch.empty((T, H, d), dtype=torch.float32, device=DEV)
    dq, dk, dv = (torch.empty((T, H, d), dtype=torch.float32, device=DEV) for _ in range(3))
    pf = sla.make_problem(torch.bfloat16, offs, None, T, H, d, d, w.k1, w.k2, w.contextual_len,
                          w.max_seq_len, w.alpha, True)
    wsf = torch.empty(sla.workspace_size(pf, sla.SLA_OP_FWD), dtype=torch.uint8, device=DEV)
    wsb = torch.empty(sla.workspace_size(pf, sla.SLA_OP_BWD), dtype=torch.uint8, device=DEV)

    def run():
        sla.sla_fwd(q, k, v, offs, None, out=o, workspace=wsf, **kw)
        sla.sla_bwd(q, k, v, do, offs, None, dq=dq, dk=dk, dv=dv, workspace=wsb, **kw)

    def eager():
        run()
        torch.cuda.synchronize()
        return [x.clone() for x in (o, dq, dk, dv)]

    ref = eager()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()   # warm-up on the capture stream's side, as torch asks
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    rng = np.random.default_rng(4)
    for rep in range(4):
        if rep == 2:   # new input values, same layout: the recording still applies
            for x in (q, k, v, do):
                x.copy_(x.float().mul_(torch.from_numpy(
                    rng.uniform(0.5, 1.5, size=tuple(x.shape)).astype(np.float32)).to(DEV))
                    .bfloat16())
            ref = eager()
        for x in (o, dq, dk, dv):
            x.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, exp in zip(("O", "dQ", "dK", "dV"), (o, dq, dk, dv), ref):
            assert torch.equal(got, exp), f"replay {rep}: {name} differs from eager"
        _eager_work()


def test_stu_layer_fwd_graph_replays_match_eager():
    sw = make_stack_workload(seed=5, batch=3, min_len=300, max_len=700, layers=1, hidden=256,
                             heads=2, num_targets=16, contextual_len=8, k1=96, k2=16)
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(DEV)  # noqa: E731
    x = f32(sw.x).bfloat16()
    offs = torch.from_numpy(sw.offsets).to(DEV)
    tg = torch.from_numpy(sw.num_targets).to(DEV)
    ln1_w, ln2_w = f32(sw.ln1_w[0]), f32(sw.ln2_w[0])
    w_uvqk, w_out = f32(sw.w_uvqk[0]).bfloat16(), f32(sw.w_out[0]).bfloat16()
    T, D = x.shape
    kw = dict(heads=sw.heads, d_qk=sw.d, d_v=sw.d, k1=sw.k1, k2=sw.k2,
              contextual_len=sw.contextual_len, max_seq_len=sw.max_seq_len)
    print(f"[case] graph stu layer fwd T={T} D={D}", flush=True)
    ws = torch.empty(max(sla.stu_layer_workspace_bytes(T, D, offs, tg, **kw), 256),
                     dtype=torch.uint8, device=DEV)
    out = torch.empty_like(x)

    def run():
        sla.stu_layer_fwd(x, offs, tg, ln1_w, w_uvqk, ln2_w, w_out, out=out, workspace=ws, **kw)

    run()
    torch.cuda.synchronize()
    ref = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for rep in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {rep} differs from eager"
        _eager_work()
