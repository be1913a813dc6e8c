"""View and split expansion (kimi-k3 "build_parameter_groups" page).

A registered view describes how the optimizer treats the rows of a stored
2-D weight as independent matrices ("Recording independent matrix geometry"):
every entry of the view shape is a positive integer, flattening the leading
axes gives back the stored (R, C) shape, and nothing new is allocated.  The
optional split sizes cut each view matrix's row axis again (MLA's K versus V
rows within a head, "The layout declarations are literal").  The Qwen3.8 notes
(section 4, fused matrices) state the same rule: each true sub-matrix is
orthogonalised on its own.  The same section sends the gate/vector sub-blocks
that do not suit Muon to AdamW instead; ``exclude`` names those pieces by
their position in the split list, the same in every view matrix (this
library's reading: the notes give no encoding).
"""

from typing import List, Optional, Sequence, Tuple


class ViewError(ValueError):
    pass


def validate_view(stored: Sequence[int], view: Optional[Sequence[int]],
                  split: Optional[Sequence[int]]) -> None:
    if len(stored) != 2:
        raise ViewError("views apply to 2-D weights only")
    if view is None:
        if split is not None:
            raise ViewError("split sizes need a view")
        return
    if len(view) < 2:
        raise ViewError("a view needs at least (rows, cols)")
    for s in view:
        if not isinstance(s, int) or isinstance(s, bool) or s <= 0:
            raise ViewError(f"view entry {s!r} is not a positive int")
    lead = 1
    for s in view[:-2]:
        lead *= s
    r, c = view[-2], view[-1]
    if lead * r != stored[0] or c != stored[1]:
        raise ViewError(f"view {tuple(view)} does not flatten to {tuple(stored)}")
    if split is not None:
        for q in split:
            if not isinstance(q, int) or isinstance(q, bool) or q <= 0:
                raise ViewError(f"split entry {q!r} is not a positive int")
        if sum(split) != r:
            raise ViewError(f"split {tuple(split)} does not sum to {r}")


def validate_exclude(split: Optional[Sequence[int]], exclude) -> None:
    """Excluded pieces are split positions; at least one piece stays Muon."""
    if not exclude:
        return
    if split is None:
        raise ViewError("excluded pieces need split sizes")
    for j in exclude:
        if not isinstance(j, int) or isinstance(j, bool) or not 0 <= j < len(split):
            raise ViewError(f"excluded piece {j!r} is not a split position")
    if len(set(exclude)) >= len(split):
        raise ViewError("every piece excluded: route the weight to AdamW instead")


def expand(stored: Sequence[int], view: Optional[Sequence[int]] = None,
           split: Optional[Sequence[int]] = None) -> List[Tuple[int, int, int]]:
    """Independent sub-matrices of a stored (R, C) weight as row slabs.

    Returns [(row_offset, rows, cols), ...] in row-major order of the view's
    leading index, then split order.  Leading index b of a view
    (s_0, ..., s_{k-1}, r, c) owns stored rows [b*r, (b+1)*r); split sizes
    (q_1, ..., q_j) cut that slab into consecutive pieces of height q_i.
    """
    validate_view(stored, view, split)
    R, C = stored
    if view is None:
        return [(0, R, C)]
    r = view[-2]
    nlead = R // r
    pieces = list(split) if split is not None else [r]
    out = []
    for b in range(nlead):
        off = b * r
        for q in pieces:
            out.append((off, q, C))
            off += q
    return out


def expand_pieces(stored: Sequence[int], view: Optional[Sequence[int]] = None,
                  split: Optional[Sequence[int]] = None, exclude=None):
    """``expand`` cut in two: (Muon slices, excluded slices).  A slice is
    excluded when its split position is listed in ``exclude``."""
    validate_exclude(split, exclude)
    muon, rest = [], []
    ex = set(exclude or ())
    npiece = len(split) if split is not None else 1
    for k, sl in enumerate(expand(stored, view, split)):
        (rest if k % npiece in ex else muon).append(sl)
    return muon, rest
