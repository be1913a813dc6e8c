"""Role routing predicate and parameter grouping.

Follows the kimi-k3 "build_parameter_groups" page ("Exclusion and decay
rules"; "Classification happens once per original parameter identity") with
the OMN "Dual-Manifold Optimization" page's reading for the embedding (routing
paragraph: embeddings, head and norms travel AdamW at zero decay):

* frozen parameters are skipped;
* a parameter seen before (same identity, e.g. a tied head) is skipped;
* ndim < 2, or membership of the no-decay set -> ("adamw", None, None, False);
* ndim == 2 and not auxiliary (embedding / head) -> ("muon", view, split, True),
  or ("muon", view, split, True, exclude) when some split pieces are excluded
  (Qwen3.8 notes, section 4: those sub-blocks are stepped by AdamW);
* anything else -> ("adamw", None, None, True).

Groups are formed by key in order of first appearance; params keep the
caller's order inside a group.  No trainable parameter -> ValueError.
"""

from typing import Dict, List, Optional, Sequence, Tuple

from .views import validate_exclude, validate_view

AUXILIARY_ROLES = ("embedding", "head")


def route_one(ndim: int, role: str, no_decay: bool, view, split, exclude=None) -> Tuple:
    if ndim < 2 or no_decay:
        return ("adamw", None, None, False)
    if ndim == 2 and role not in AUXILIARY_ROLES:
        key = ("muon", None if view is None else tuple(view),
               None if split is None else tuple(split), True)
        return key + (tuple(sorted(set(exclude))),) if exclude else key
    return ("adamw", None, None, True)


def build_groups(descs: Sequence[dict]) -> List[dict]:
    """descs: dicts with name, shape, role, no_decay, requires_grad, ident,
    and optional view / split.  Returns groups: dicts with key, algorithm,
    decay, view, split, names, indices (positions in ``descs``)."""
    seen = set()
    views: Dict[object, Tuple] = {}
    groups: List[dict] = []
    by_key: Dict[Tuple, dict] = {}
    for i, d in enumerate(descs):
        ident = d.get("ident", d["name"])
        v, s, ex = d.get("view"), d.get("split"), d.get("exclude")
        if v is not None:
            validate_view(d["shape"], v, s)
            validate_exclude(s, ex)
            rec = (tuple(v), None if s is None else tuple(s),
                   tuple(sorted(set(ex))) if ex else None)
            prev = views.get(ident)
            if prev is not None and prev != rec:
                raise ValueError(f"conflicting views for {d['name']}")
            views[ident] = rec
        elif ex:
            raise ValueError(f"excluded pieces need a view and split sizes ({d['name']})")
        if not d.get("requires_grad", True):
            continue
        if ident in seen:
            continue
        seen.add(ident)
        key = route_one(len(d["shape"]), d.get("role", "matrix"),
                        bool(d.get("no_decay", False)), v, s, ex)
        g = by_key.get(key)
        if g is None:
            g = {"key": key, "algorithm": key[0], "view": key[1], "split": key[2],
                 "decay": key[3], "exclude": key[4] if len(key) > 4 else None,
                 "names": [], "indices": []}
            by_key[key] = g
            groups.append(g)
        g["names"].append(d["name"])
        g["indices"].append(i)
    if not groups:
        raise ValueError("no trainable parameters")
    return groups


def descs_from_specs(specs) -> List[dict]:
    """Turn workloads.ParamSpec-like objects into routing descriptors."""
    out = []
    for p in specs:
        out.append({"name": p.name, "shape": tuple(p.shape), "role": p.role,
                    "no_decay": p.no_decay, "requires_grad": p.requires_grad,
                    "ident": p.name, "view": p.view, "split": p.split,
                    "exclude": getattr(p, "exclude", None)})
    return out
