"""sla_bwd_noalloc (the SLA backward whose workspace is the library's static
per-device array, for callers that cannot allocate device memory) against
sla_bwd with a caller-owned workspace.

sla_bwd_noalloc equals sla_bwd given a workspace of the array's size (dS is
stored for the dQ kernel where it fits, recomputed otherwise), so the
reference call gets a workspace of that size: both then run the same kernels
on the same inputs, and the backward is bitwise reproducible, so the
gradients must agree bit for bit.  Two calls in a row:
the second on a smaller problem, so it runs on the array as the first call
left it.  The outputs start as NaN, so an element either call fails to write
shows up."""
import pytest
import torch

import sparse_sequence_attention_amd as sla
from synthetic import make_sla_workload

pytestmark = pytest.mark.gpu

DEV = "cuda"

# lengths, targets, k1, k2, contextual_len, heads, d, gradient dtype.  The
# first case has global-prefix key tiles split into several row chunks (fp32
# partials in the array, then the reduce); the second is smaller.
CASES = [
    ([3000, 1500, 700], [64, 0, 30], 256, 200, 8, 2, 128, torch.float32),
    ([1300, 90], None, 128, 64, 4, 2, 128, torch.bfloat16),
]


def _run(i, case):
    lens, tg, k1, k2, ctx, heads, d, gdt = case
    w = make_sla_workload("jagged_2k", seed=90 + i, lengths=lens, num_targets=tg, heads=heads,
                          d=d, k1=k1, k2=k2, contextual_len=ctx, max_seq_len=max(lens),
                          dtype="bf16", with_dout=True)
    print(f"[case] noalloc call {i}: lengths={lens} targets={tg} k1={k1} k2={k2} ctx={ctx} "
          f"H={heads} d={d} grads={gdt}", flush=True)
    t = lambda a: torch.from_numpy(a).to(DEV).to(torch.bfloat16)  # noqa: E731  (exact)
    q, k, v, do = t(w.q), t(w.k), t(w.v), t(w.dout)
    offs = torch.from_numpy(w.offsets).to(DEV)
    tgd = None if w.num_targets is None else torch.from_numpy(w.num_targets).to(DEV)
    kw = dict(k1=w.k1, k2=w.k2, contextual_len=w.contextual_len, max_seq_len=w.max_seq_len,
              alpha=w.alpha)
    ws = torch.empty(sla.SLA_NOALLOC_SCRATCH_BYTES, dtype=torch.uint8, device=DEV)
    ref = sla.sla_bwd(q, k, v, do, offs, tgd, grad_dtype=gdt, workspace=ws, **kw)
    got = tuple(torch.full_like(r, float("nan")) for r in ref)
    sla.sla_bwd_noalloc(q, k, v, do, offs, tgd, dq=got[0], dk=got[1], dv=got[2], **kw)
    torch.cuda.synchronize()
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        assert torch.isfinite(g.float()).all(), f"call {i} {name}: unwritten or non-finite"
        assert torch.equal(g, r), f"call {i} {name}: differs from sla_bwd"


def test_noalloc_backward_matches_workspace_backward_twice():
    assert sum(CASES[1][0]) < sum(CASES[0][0])
    for i, case in enumerate(CASES):
        _run(i, case)
