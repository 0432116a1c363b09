"""Oracle attention: masked softmax attention over a frame-block mask, float64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What is computed.  The token sequence is T latent frames of P tokens each,
token index = t·P + p (frame-major).  Query frame t attends exactly to the
tokens of the frames in A(t) ([gist] "Core Mechanism": the attended frame set
replaces {0..T−1}; [gist] "Complexity": per query O(C·P·d), so the block is
the frame).  For every query token i of frame t

    out[i] = Σ_j softmax_j( scale · q_i · k_j ) · v_j ,  j over tokens of A(t)

with scale = 1/sqrt(d) unless given.  Non-causal, no bias, no dropout; any
positional encoding is applied by the model before this call.  This is exact
masked attention, so the oracle is that definition written out: gather the
key/value tokens of A(t) in ascending frame order, scores, row softmax with
the row maximum subtracted, weighted sum.  The library matmul is used as the
dot-product step; nothing is blocked, fused or reordered beyond that.

[gist] = gist.science explainer "LVSA: Training-Free Sparse Attention for Long
Video Diffusion", Technical Summary §2.

Precision: inputs are the bf16 tensors the GPU receives, up-cast exactly to
float64; all arithmetic is float64.
"""

from __future__ import annotations

import math
from typing import Iterable, List, Optional, Sequence

import torch


def default_scale(d: int) -> float:
    """Softmax temperature 1/sqrt(d) (standard scaled dot-product attention)."""
    return 1.0 / math.sqrt(d)


def _as_f64(x: torch.Tensor) -> torch.Tensor:
    return x.detach().to(device="cpu", dtype=torch.float64)


def _frame_tokens(frames: Sequence[int], P: int) -> torch.Tensor:
    """Token indices of the given frames, in the given (ascending) order."""
    if len(frames) == 0:
        return torch.empty(0, dtype=torch.long)
    return torch.cat([torch.arange(f * P, (f + 1) * P, dtype=torch.long) for f in frames])


def _softmax_weighted_sum(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor,
                          scale: float) -> torch.Tensor:
    """softmax(scale · Q Kᵀ) V, row-wise, with the row maximum subtracted."""
    S = (Q @ K.transpose(0, 1)) * scale
    S = S - S.max(dim=1, keepdim=True).values
    E = torch.exp(S)
    return (E @ V) / E.sum(dim=1, keepdim=True)


def block_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                    rows: List[List[int]], scale: Optional[float] = None,
                    q_chunk: int = 256, frames: Optional[Sequence[int]] = None) -> torch.Tensor:
    """Full output [B, H, N, d] float64 of frame-block-sparse attention.

    q, k, v: [B, H, N, d] (any float dtype; bf16 is up-cast exactly).
    rows:    rows[t] = A(t), the key frames of query frame t (len T).
    frames:  if given, only these query frames are computed (the other
             output rows are left NaN) -- for bounded samples of large cases.
    """
    q64, k64, v64 = _as_f64(q), _as_f64(k), _as_f64(v)
    B, H, N, d = q64.shape
    T = len(rows)
    if N % T != 0:
        raise ValueError("N must be a multiple of T")
    P = N // T
    sc = default_scale(d) if scale is None else float(scale)
    out = torch.full_like(q64, float("nan"))
    tok = [_frame_tokens(r, P) for r in rows]
    todo = range(T) if frames is None else list(frames)
    for b in range(B):
        for h in range(H):
            for t in todo:
                K_A = k64[b, h, tok[t]]
                V_A = v64[b, h, tok[t]]
                for c0 in range(0, P, q_chunk):
                    c1 = min(P, c0 + q_chunk)
                    Qt = q64[b, h, t * P + c0: t * P + c1]
                    out[b, h, t * P + c0: t * P + c1] = _softmax_weighted_sum(Qt, K_A, V_A, sc)
    return out


def block_attention_rows(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                         rows: List[List[int]], b: int, h: int,
                         tokens: Iterable[int], scale: Optional[float] = None) -> torch.Tensor:
    """Output rows [len(tokens), d] float64 for selected query tokens of (b, h).

    Same definition as :func:`block_attention`, evaluated one query token at
    a time, so that single outputs of full-size problems can be checked.
    """
    d = q.shape[-1]
    N = q.shape[2]
    T = len(rows)
    P = N // T
    sc = default_scale(d) if scale is None else float(scale)
    kb = k[b, h]
    vb = v[b, h]
    res = []
    cache = {}
    for i in tokens:
        t = i // P
        if t not in cache:
            idx = _frame_tokens(rows[t], P)
            cache[t] = (_as_f64(kb[idx]), _as_f64(vb[idx]))
        K_A, V_A = cache[t]
        Qi = _as_f64(q[b, h, i:i + 1])
        res.append(_softmax_weighted_sum(Qi, K_A, V_A, sc)[0])
    return torch.stack(res) if res else torch.empty(0, d, dtype=torch.float64)


def token_mask_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                         rows: List[List[int]], scale: Optional[float] = None) -> torch.Tensor:
    """Brute force: dense N×N scores with an explicit token-level mask.

    Score (i, j) is kept iff frame(j) ∈ A(frame(i)), else −∞; then a dense
    row softmax.  Independent of the frame gathering in
    :func:`block_attention`; meant for tiny inputs only (O(N²) memory).
    """
    q64, k64, v64 = _as_f64(q), _as_f64(k), _as_f64(v)
    B, H, N, d = q64.shape
    T = len(rows)
    P = N // T
    sc = default_scale(d) if scale is None else float(scale)
    allowed = torch.zeros(N, N, dtype=torch.bool)
    for i in range(N):
        for f in rows[i // P]:
            allowed[i, f * P:(f + 1) * P] = True
    S = torch.einsum("bhid,bhjd->bhij", q64, k64) * sc
    S = S.masked_fill(~allowed, float("-inf"))
    S = S - S.max(dim=-1, keepdim=True).values
    E = torch.exp(S)
    return torch.einsum("bhij,bhjd->bhid", E, v64) / E.sum(dim=-1, keepdim=True)
