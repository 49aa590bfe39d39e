"""Oracle of the Router tournament -- test infrastructure.

Only tests/ may use it.  Plain Python, written from "Julia-1: one score per
mask token, and a benchmark that turns on how the labels are worded" (More
than 20 options: the Router): the candidate list is cut, in order, into
consecutive groups of at most 20; each group is scored as one choice
question; a group keeps its winner alone when the winner's probability is
above 0.95 and every other option's is below 0.045, else its two best; this
repeats until at most 20 candidates remain, and one final call scores them.

Readings where the page is silent (also listed in the design doc): a group holding
a single candidate passes it on unscored (the head needs 2 options);
survivors keep their original order; the first of equal probabilities wins.
"""

GROUP = 20
WIN_ALONE = 0.95
OTHERS_BELOW = 0.045


def _first_max(p):
    w = 0
    for i in range(1, len(p)):
        if p[i] > p[w]:
            w = i
    return w


def group_survivors(cands, p):
    """Survivors of one scored group, in candidate order."""
    w = _first_max(p)
    if p[w] > WIN_ALONE and all(p[i] < OTHERS_BELOW for i in range(len(p)) if i != w):
        return [cands[w]]
    rest = [i for i in range(len(p)) if i != w]
    s = rest[_first_max([p[i] for i in rest])]
    return sorted([cands[w], cands[s]])


def route(score_group, n_options):
    """score_group(list of candidate indices) -> their probabilities (one
    choice question over exactly those options, in that order).

    Returns pick, pick_prob, final candidates, final probabilities, the
    number of scored groups (calls, final call included) and of rounds."""
    if n_options < 2:
        raise ValueError("a question needs at least 2 options")
    alive = list(range(n_options))
    calls = rounds = 0
    while len(alive) > GROUP:
        survivors = []
        for i in range(0, len(alive), GROUP):
            group = alive[i:i + GROUP]
            if len(group) == 1:
                survivors += group
                continue
            p = score_group(group)
            calls += 1
            survivors += group_survivors(group, p)
        alive = sorted(survivors)
        rounds += 1
    p = score_group(alive)
    calls += 1
    w = _first_max(p)
    return {"pick": alive[w], "pick_prob": p[w], "final": alive, "final_prob": list(p), "calls": calls,
            "rounds": rounds}


def group_sequence(prefix, suffix, options, cands, mask_id):
    """Token ids and marker positions of one scored group."""
    ids = list(prefix)
    marks = []
    for c in cands:
        marks.append(len(ids))
        ids.append(mask_id)
        ids += list(options[c])
    ids += list(suffix)
    return ids, marks
