"""lvsa_attention_ws_static: the workspace path on the library's static
device scratch (for callers that cannot allocate), through the C ABI.

Its output is checked against lvsa_attention_ws on the same inputs (and,
on sampled rows, against the float64 oracle) on two calls in a row, the
second with a smaller input, so that the scratch's leftovers from the first
call (work counters, key norms, partial records) cannot leak into the
second.  An input whose key-norm table does not fit the scratch is refused
before anything is launched.
"""

import random

import pytest
import torch

import block_sparse_attention_lvsa_amd as L
import oracle.attention as oa
import oracle.mask as om
from block_sparse_attention_lvsa_amd.synth import WORKLOADS, make_qkv, make_random

pytestmark = pytest.mark.gpu

MAX_ABS = 1e-2
MEAN_ABS = 1e-3
REL_RMS = 1e-2


def close(out, ref, what):
    d = (out.double().cpu() - ref.double().cpu()).abs()
    rel = (d.pow(2).mean().sqrt() / ref.double().cpu().pow(2).mean().sqrt().clamp_min(1e-30)).item()
    print(f"  {what}: max|Δ| {d.max().item():.3e}  mean|Δ| {d.mean().item():.3e}  relRMS {rel:.3e}", flush=True)
    assert d.max().item() <= MAX_ABS and d.mean().item() <= MEAN_ABS and rel <= REL_RMS, what


def one_call(gpu, q, k, v, T, C, W, step, what):
    m = L.lvsa_build_mask(T, C, W, step).to(gpu)
    B, H, N, D = q.shape
    ws = torch.empty(L.lvsa_attention_workspace_bytes(B, H, N, D, T), dtype=torch.uint8, device=gpu)
    out_ws = torch.full_like(q, float("nan"))
    out_static = torch.full_like(q, float("nan"))
    L.lvsa_attention(q, k, v, m, out=out_ws, workspace=ws)
    L.lvsa_attention_ws_static(q, k, v, m, out=out_static)
    torch.cuda.synchronize()
    assert torch.isfinite(out_static).all(), "a row was not written"
    close(out_static, out_ws, f"{what}: static scratch vs caller workspace")
    rows = om.key_frames(T, C, W, step)
    P = N // T
    rnd = random.Random(step)
    toks = sorted({rnd.randrange(N) for _ in range(24)} | {0, P - 1, N - 1})
    for h in (0, H - 1):
        ref = oa.block_attention_rows(q[:, h:h + 1].cpu(), k[:, h:h + 1].cpu(), v[:, h:h + 1].cpu(), rows, 0, 0, toks)
        close(out_static[0, h, toks], ref, f"{what}: static scratch vs oracle, head {h}")


def test_static_scratch_two_calls_then_smaller(gpu):
    w = WORKLOADS["wan13b_6x"]
    print("[case] static scratch, call 1:", w, flush=True)
    q, k, v = make_qkv(w, device=gpu)
    one_call(gpu, q, k, v, w.T, w.C, w.W, 4, "wan13b_6x")
    del q, k, v
    B, H, T, P, d, C, W = 1, 3, 12, 200, 128, 5, 2
    print("[case] static scratch, call 2 (smaller):", (B, H, T, P, d, C, W), flush=True)
    q = make_random((B, H, T * P, d), 801).to(gpu)
    k = make_random((B, H, T * P, d), 802).to(gpu)
    v = make_random((B, H, T * P, d), 803).to(gpu)
    one_call(gpu, q, k, v, T, C, W, 1, "mid-size")


def test_static_scratch_refuses_an_oversized_norm_table(gpu):
    # 4,200 heads x 1,024 frames of one token: the key-norm table alone needs
    # more than the static scratch; the tensors are stride-0 views of one
    # small buffer, and the call must fail on the host before any launch.
    B, H, T, d = 1, 4200, 1024, 64
    print("[case] static scratch, oversized:", (B, H, T, d), flush=True)
    base = torch.zeros(1, 1, T, d, dtype=torch.bfloat16, device=gpu)
    x = base.expand(B, H, T, d)
    out = torch.zeros(1, 1, T, d, dtype=torch.bfloat16, device=gpu).expand(B, H, T, d)
    m = L.lvsa_build_mask(T, 4, 2, 0).to(gpu)
    assert B * H * T * 4 > L.LVSA_STATIC_SCRATCH_BYTES
    with pytest.raises(L.LvsaValueError) as ei:
        L.lvsa_attention_ws_static(x, x, x, m, out=out)
    assert ei.value.code == L.LVSA_ERR_CAPACITY
    print("  refused:", ei.value, flush=True)
