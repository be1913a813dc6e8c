"""View and split expansion (kimi-k3 "build_parameter_groups" page).

A registered view describes how the optimizer treats the rows of a stored
2-D weight as independent matrices ("Recording independent matrix geometry"):
every entry of the view shape is a positive integer, flattening the leading
axes gives back the stored (R, C) shape, and nothing new is allocated.  The
optional split sizes cut each view matrix's row axis again (MLA's K versus V
rows within a head, "The layout declarations are literal").  The Qwen3.8 notes
(section 4, fused matrices) state the same rule: each true sub-matrix is
orthogonalised on its own.
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
