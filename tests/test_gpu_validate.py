"""The optional layout check (environment SLA_VALIDATE): with it, bad device-resident
jagged layouts are rejected with SLA_ERR_INVALID before any attention kernel runs;
valid layouts give bitwise the same results as without it.  The bad inputs only ever
reach the check kernel, which reads offsets[0..B] and num_targets[0..B-1] and nothing
else."""
import pytest
import torch

import sparse_sequence_attention_amd as sla
from sparse_sequence_attention_amd import _capi as C

pytestmark = pytest.mark.gpu

DEV = "cuda"
KW = dict(k1=64, k2=8, contextual_len=4, max_seq_len=256)


def _qkv(T, H=2, d=64, seed=0):
    g = torch.Generator().manual_seed(seed)
    mk = lambda: (torch.randn(T, H, d, generator=g) * 0.5).to(DEV, torch.bfloat16)  # noqa: E731
    return mk(), mk(), mk(), mk()


def _offs(v):
    return torch.tensor(v, dtype=torch.int64, device=DEV)


def _expect_invalid(fn, text):
    with pytest.raises(C.SLAError) as ei:
        fn()
    assert ei.value.status == C.SLA_ERR_INVALID, str(ei.value)
    assert text in str(ei.value), str(ei.value)
    torch.cuda.synchronize()


def test_valid_layout_is_unchanged(monkeypatch):
    q, k, v, do = _qkv(150)
    offs = _offs([0, 100, 150])
    tg = torch.tensor([3, 7], dtype=torch.int32, device=DEV)
    monkeypatch.delenv("SLA_VALIDATE", raising=False)
    o_ref = sla.sla_fwd(q, k, v, offs, tg, **KW)
    g_ref = sla.sla_bwd(q, k, v, do, offs, tg, **KW)
    monkeypatch.setenv("SLA_VALIDATE", "1")
    o = sla.sla_fwd(q, k, v, offs, tg, **KW)
    g = sla.sla_bwd(q, k, v, do, offs, tg, **KW)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref)
    for a, b in zip(g, g_ref):
        assert torch.equal(a, b)
    monkeypatch.setenv("SLA_VALIDATE", "0")  # "0" turns it off again
    assert torch.equal(sla.sla_fwd(q, k, v, offs, tg, **KW), o_ref)


@pytest.mark.parametrize("offsets, targets, text", [
    ([5, 100, 150], None, "offsets[0] != 0"),
    ([0, 100, 50, 150], None, "offsets decrease at sequence 1"),
    ([0, 100, 140], None, "offsets[B] != total_tokens"),
    ([0, 100, 150], [10, 60], "num_targets[1] outside"),
    ([0, 100, 150], [-1, 0], "num_targets[0] outside"),
])
def test_bad_layouts_are_rejected(monkeypatch, offsets, targets, text):
    monkeypatch.setenv("SLA_VALIDATE", "1")
    q, k, v, do = _qkv(150)
    offs = _offs(offsets)
    tg = None if targets is None else torch.tensor(targets, dtype=torch.int32, device=DEV)
    print(f"validate case {offsets} {targets}", flush=True)
    _expect_invalid(lambda: sla.sla_fwd(q, k, v, offs, tg, **KW), text)
    _expect_invalid(lambda: sla.sla_bwd(q, k, v, do, offs, tg, **KW), text)
    _expect_invalid(lambda: sla.sla_schedule(offs, tg, op=sla.SLA_OP_FWD, heads=2, d=64,
                                             k1=KW["k1"], k2=KW["k2"],
                                             contextual_len=KW["contextual_len"],
                                             total_tokens=150),
                    text)


def test_truncation_needs_room_for_the_context(monkeypatch):
    monkeypatch.setenv("SLA_VALIDATE", "1")
    x = torch.randn(150, 128, device=DEV).to(torch.bfloat16)
    offs = _offs([0, 20, 150])
    # sequence 0 keeps history (10 targets of 20 tokens) but 16 + 10 > 20
    tg = torch.tensor([10, 5], dtype=torch.int32, device=DEV)
    _expect_invalid(lambda: sla.stu_truncate(x, offs, tg, contextual_len=16, tail_len=32),
                    "contextual_len + num_targets[0] > L_b")
    # a sequence of targets only keeps no history and is fine
    tg_ok = torch.tensor([20, 5], dtype=torch.int32, device=DEV)
    out = sla.stu_truncate(x, offs, tg_ok, contextual_len=16, tail_len=32)
    torch.cuda.synchronize()
    assert out[1].tolist()[0] == 0


def test_mfma_probe_reports_a_plausible_rate_and_clock():
    """The MFMA-only probe the bench reports next to the data-sheet peak: a
    rate between a fifth of and just above the 2516.6 TFLOP/s bf16 figure,
    and a shader clock between 1 and 3 GHz."""
    pm = sla.probe_mfma_peak(iters=1024)
    print(f"[case] mfma probe {pm}", flush=True)
    assert 500.0 < pm["tflops"] < 2600.0
    assert 1.0 < pm["sclk_ghz"] < 3.0


def test_issue_probe_reports_every_arrangement():
    """The issue-rate probe: every arrangement takes time; MFMA and FMA work
    issued together take at least as long as the slower of the two alone and
    at most as long as both added (with 5% for launch noise); a
    transcendental takes at least as long as an FMA."""
    r = sla.probe_issue_rates(iters=1024)
    print(f"[case] issue probe {r}", flush=True)
    tm, tv = r["mfma_only"], r["fma_only"]
    assert all(r[k] > 0.0 for k in sla.ops.ISSUE_PROBE_MODES)
    for k in ("split_waves", "mixed_waves", "split_waves_agpr"):
        assert 0.95 * max(tm, tv) <= r[k] <= 1.05 * (tm + tv), k
    assert r["exp_per_fma"] >= 0.95 and r["rcp_per_fma"] >= 0.95
