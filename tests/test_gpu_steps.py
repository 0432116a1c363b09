"""GPU: a whole run of denoising steps with no per-step host work.

The masks of every step are built once (lvsa_build_mask_steps) and copied to
the device in one transfer; each step's launch then points into that buffer,
and the step sequence can be captured in a HIP graph and replayed.  Outputs
must be bit-identical to per-step masks (same kernel, same mask contents),
and the eager path is checked against the oracle.
"""

import pytest
import torch

import block_sparse_attention_lvsa_amd as L
import oracle.attention as oa
import oracle.mask as om
from block_sparse_attention_lvsa_amd.synth import make_random

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)


def _inputs(gpu, B, H, T, P, d, seed):
    q = make_random((B, H, T * P, d), seed)
    k = make_random((B, H, T * P, d), seed + 1000)
    v = make_random((B, H, T * P, d), seed + 2000)
    return (q, k, v), tuple(x.to(gpu) for x in (q, k, v))


def test_prebuilt_masks_match_per_step_masks(gpu):
    B, H, T, P, d, C, W = 1, 2, 12, 200, 128, 5, 2
    say("prebuilt masks", (B, H, T, P, d, C, W))
    (q, k, v), (qd, kd, vd) = _inputs(gpu, B, H, T, P, d, 701)
    n = 9
    ms = L.lvsa_build_mask_steps(T, C, W, 0, n).to(gpu)
    for i in range(n):
        a = L.lvsa_attention(qd, kd, vd, ms.mask(i))
        b = L.lvsa_attention(qd, kd, vd, L.lvsa_build_mask(T, C, W, i).to(gpu))
        torch.cuda.synchronize()
        assert torch.equal(a, b), i
        if i in (0, 3, 4):  # first step, the period wrap (Tper = 4), its successor
            ref = oa.block_attention(q, k, v, om.key_frames(T, C, W, i))
            err = (a.double().cpu() - ref).abs().max().item()
            print(f"  step {i}: max|Δ| vs oracle {err:.3e}", flush=True)
            assert err <= 1e-2


@pytest.mark.parametrize("with_workspace", [False, True], ids=["running-max", "workspace"])
def test_graph_replay_of_the_step_sequence(gpu, with_workspace):
    # With a workspace each step is three kernels (key norms, attention, merge), all
    # captured.
    B, H, T, P, d, C, W = 1, 3, 11, 150, 128, 4, 2
    say("graph replay", (B, H, T, P, d, C, W), "workspace" if with_workspace else "")
    _, (qd, kd, vd) = _inputs(gpu, B, H, T, P, d, 801)
    n = 8
    ms = L.lvsa_build_mask_steps(T, C, W, 0, n).to(gpu)
    ws = (torch.empty(L.lvsa_attention_workspace_bytes(B, H, T * P, d, T), dtype=torch.uint8, device=gpu)
          if with_workspace else None)
    outs = [torch.empty_like(qd) for _ in range(n)]
    for i in range(n):
        L.lvsa_attention(qd, kd, vd, ms.mask(i), out=outs[i], workspace=ws)
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    assert not all(torch.equal(eager[0], e) for e in eager[1:])  # the steps differ

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            L.lvsa_attention(qd, kd, vd, ms.mask(i), out=outs[i], workspace=ws)
    other = torch.empty_like(qd)
    m_other = L.lvsa_build_mask(T, C, W, 17).to(gpu)
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        L.lvsa_attention(qd, kd, vd, m_other, out=other)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i in range(n):
            assert torch.equal(outs[i], eager[i]), (rep, i)
        print(f"  replay {rep}: {n} steps bit-identical to eager", flush=True)
