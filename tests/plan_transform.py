"""The library's fused fold, as a transform of the appendix-D cascade plan (test helper).

The FlashInfer paper summary's appendix D lets a tile write the final output only when it is
its rows' only state; the oracle's ``cascade_plan`` follows that rule.  The library goes one
step further: a request whose merge list is its level states plus exactly one own chunk is
finished by that chunk's decode item, which folds the level states into its own state and
writes the final output, so the request needs no merge pass.  That moves no work and changes
no state; it only hands the last merge of such a request to the item that produces the last
state.  ``fused_fold`` applies that rule to an oracle plan, so the host tests can check the C++
plan against the oracle plan transformed, and the oracle itself stays on the pages' rule.
"""

from __future__ import annotations

import copy


def fused_fold(cp):
    """Returns a copy of the oracle's CascadePlan ``cp`` with the fused fold applied:
    every request that is not write-through and whose own KV is exactly one suffix item
    becomes write-through through that item (slot -1, its entry dropped from the merge list,
    the level entries kept: they are what the item folds in); the remaining partial suffix
    items are renumbered densely in ascending w."""
    f = copy.deepcopy(cp)
    own = {}
    for it in f.suffix.items:
        own.setdefault(it.req, []).append(it.w)
    folded = set()
    for b, ws in own.items():
        if len(ws) == 1 and not f.write_through[b]:
            folded.add(ws[0])
            f.write_through[b] = True
    remap, n = {}, 0
    new_slots = []
    for it in f.suffix.items:
        old = f.suffix.slots[it.w]
        if it.w in folded or old < 0:
            new_slots.append(-1)
        else:
            remap[old] = n
            new_slots.append(n)
            n += 1
    for b in range(len(f.merge)):
        f.merge[b] = [(st, remap[s], r) if st == "suffix" else (st, s, r)
                      for (st, s, r) in f.merge[b] if not (st == "suffix" and s not in remap)]
    f.suffix.slots = new_slots
    return f
