"""Oracle mask builder: the key-frame set A_s(t) of every query frame t.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Pure Python integers;
written from the method's description, step by step, in the pages' notation:

  T     number of latent frames in the sequence
  C     per-query-frame budget of key frames (the model's training horizon in
        latent frames)
  W     pre-tuned local window size
  s     denoising step index (``step``)
  Tper  spacing of the global anchors
  G_s   the global anchor frames at step s
  W(t)  the (expanded) local window of query frame t
  A(t)  = G_s ∪ W(t), the frames query frame t attends to

Sources:
  [gist] gist.science explainer "LVSA: Training-Free Sparse Attention for Long
         Video Diffusion", Technical Summary §2, "Core Mechanism".
  [tw2]  TechWalker article on LVSA ("华为巴黎研究院让AI视频'不再原地打转'…"),
         §二 (budget C = training horizon; Tper ≈ T/(C−W); window extension
         until the effective count is back at the target).
  [tw3]  same article, §三 (anchors move one slot per step, cyclically over
         the frame count; each frame an anchor once per period, a very few
         frames twice when T is not a multiple of the spacing; constant
         anchor count).

Readings where the pages leave a step open (each is a stated choice, pinned
by the tests, not by values the pages print):

  R1  Tper = ceil(T / (C − W)).  [tw2] gives only "Tper ≈ T/(C−W)"; the
      ceiling is the rounding that keeps the anchor count at most C − W, so
      the window keeps at least W frames and is only ever *extended* as
      [gist]/[tw2] describe, never shrunk.
  R2  n_g = ceil(T / Tper) anchors, positions taken modulo T, so that every
      frame is reached once per Tper steps ([gist]) and a few frames twice
      when Tper does not divide T ([tw3]).
  R3  Rotation.  Default: the offset is s mod Tper, the formula [gist]
      prints ("G_s shifts by s (mod Tper)").  Flag ROT_MOD_T: the offset is
      s itself, anchors stepping by one frame per step modulo T, as [tw3]
      words it.  The two coincide whenever Tper divides T.
  R4  Window: the C − n_g non-anchor frames nearest to t, nearest first,
      ties to the lower frame index, clipped to [0, T−1] so that near the
      ends it slides inward.  Anchors that fall inside the window do not
      count against it, which is the "extension" of [gist]/[tw2].
  R5  |A(t)| = min(C, T) exactly ([tw2]: extended "until the effective
      count reaches the target again").
  R6  T ≤ C: dense, A(t) = {0..T−1} for every t (C is the training horizon:
      at the 1× horizon the method is the dense model).
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import List, Tuple

# Flags, same meaning as the library's (values restated here, not shared).
ROT_MOD_TPER = 0  # default rotation: offset = s mod Tper   (R3, [gist])
ROT_MOD_T = 1     # rotation variant: offset = s mod T      (R3, [tw3])
FIXED_GRID = 2    # ablation: anchors never move (offset 0; the grid the
                  # pages name as the source of fixed-grid bias)
WINDOW_ONLY = 3   # ablation: no anchors, the C frames nearest to t (plain
                  # sliding-window attention, the prior-art pattern the pages
                  # contrast LVSA with)


class OracleArgError(ValueError):
    """Invalid (T, C, W, step, flags)."""


@dataclass(frozen=True)
class MaskInfo:
    c_eff: int      # min(C, T): key frames per query frame
    t_per: int      # anchor spacing (0 in the dense case)
    n_anchor: int   # anchor count n_g (0 in the dense case)
    offset: int     # anchor offset o_s used at this step (0 when dense)
    nnz: int        # T * c_eff


def validate(T: int, C: int, W: int, step: int, flags: int = ROT_MOD_TPER) -> None:
    """Argument domain: T ≥ 1, C ≥ 2, 1 ≤ W ≤ C − 1, step ≥ 0, known flag.

    The window W must leave room for at least one anchor slot (C − W ≥ 1),
    otherwise Tper = T/(C−W) of [tw2] is undefined.
    """
    for name, v in (("T", T), ("C", C), ("W", W), ("step", step), ("flags", flags)):
        if not isinstance(v, int):
            raise OracleArgError(f"{name} must be an int, got {type(v).__name__}")
    if T < 1:
        raise OracleArgError("T must be >= 1")
    if C < 2:
        raise OracleArgError("C must be >= 2")
    if W < 1 or W > C - 1:
        raise OracleArgError("W must satisfy 1 <= W <= C-1")
    if step < 0:
        raise OracleArgError("step must be >= 0")
    if flags not in (ROT_MOD_TPER, ROT_MOD_T, FIXED_GRID, WINDOW_ONLY):
        raise OracleArgError("unknown flags value")


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def schedule(T: int, C: int, W: int) -> Tuple[int, int]:
    """(Tper, n_g) for a sparse sequence (T > C), readings R1 and R2.

    Tper = ceil(T / (C − W))   [tw2: Tper ≈ T/(C−W)]
    n_g  = ceil(T / Tper)      enough anchors, Tper apart, to span T frames.
    """
    t_per = _ceil_div(T, C - W)
    n_g = _ceil_div(T, t_per)
    return t_per, n_g


def anchor_offset(T: int, t_per: int, step: int, flags: int) -> int:
    """Offset o_s of the first anchor at step s (reading R3)."""
    if flags == FIXED_GRID:
        return 0
    if flags == ROT_MOD_T:
        return step % T
    return step % t_per


def anchors(T: int, C: int, W: int, step: int, flags: int = ROT_MOD_TPER) -> List[int]:
    """G_s as a sorted list: {(o_s + k·Tper) mod T : 0 ≤ k < n_g}.

    [gist] "Rotating Global Anchors": periodic global frames whose set shifts
    with the denoising step; [tw3]: constant count, every frame in turn.
    Empty in the dense case T ≤ C (every frame is attended anyway).
    """
    validate(T, C, W, step, flags)
    if T <= C or flags == WINDOW_ONLY:
        return []
    t_per, n_g = schedule(T, C, W)
    o = anchor_offset(T, t_per, step, flags)
    g = set()
    for k in range(n_g):
        g.add((o + k * t_per) % T)
    assert len(g) == n_g  # (n_g − 1)·Tper < T keeps the positions distinct
    return sorted(g)


def _window(T: int, t: int, budget: int, anchor_set: set) -> List[int]:
    """Expanded local window of query frame t (reading R4).

    Visit frames in order of distance from t -- t, t−1, t+1, t−2, t+2, ... --
    skipping frames outside [0, T−1] and frames already anchors, until
    ``budget`` frames are collected.  Skipping anchors is what extends the
    window when it overlaps them ([gist] "Expanded Adaptive Windows"; [tw2]).
    """
    taken: List[int] = []
    dist = 0
    while len(taken) < budget:
        if dist > T:  # cannot happen for budget ≤ T − |anchors|
            raise AssertionError("window budget exceeds available frames")
        cands = [t] if dist == 0 else [t - dist, t + dist]
        for f in cands:  # lower index first on ties
            if 0 <= f < T and f not in anchor_set and len(taken) < budget:
                taken.append(f)
        dist += 1
    return taken


def key_frames(T: int, C: int, W: int, step: int, flags: int = ROT_MOD_TPER) -> List[List[int]]:
    """A_s(t) for t = 0..T−1, each sorted ascending.

    A(t) = G_s ∪ W(t) ([gist] "Core Mechanism"); |A(t)| = min(C, T)
    (reading R5); dense when T ≤ C (reading R6).
    """
    validate(T, C, W, step, flags)
    if T <= C:
        return [list(range(T)) for _ in range(T)]
    g = anchors(T, C, W, step, flags)
    gs = set(g)
    budget = C - len(g)
    rows = []
    for t in range(T):
        w = _window(T, t, budget, gs)
        rows.append(sorted(gs.union(w)))
    return rows


def build_mask(T: int, C: int, W: int, step: int, flags: int = ROT_MOD_TPER):
    """CSR form of the step's mask: (row_ptr [T+1], col_idx [T·c_eff], info).

    row_ptr[t] = t·c_eff, col_idx[row_ptr[t]:row_ptr[t+1]] = A_s(t) ascending.
    """
    rows = key_frames(T, C, W, step, flags)
    c_eff = min(C, T)
    row_ptr = [0]
    col_idx: List[int] = []
    for r in rows:
        col_idx.extend(r)
        row_ptr.append(len(col_idx))
    if T <= C or flags == WINDOW_ONLY:
        info = MaskInfo(c_eff=c_eff, t_per=0, n_anchor=0, offset=0, nnz=len(col_idx))
    else:
        t_per, n_g = schedule(T, C, W)
        info = MaskInfo(c_eff=c_eff, t_per=t_per, n_anchor=n_g,
                        offset=anchor_offset(T, t_per, step, flags), nnz=len(col_idx))
    return row_ptr, col_idx, info
