"""Run-wide record of the selection comparisons of the GPU parity tests.

Every comparison of a GPU selection with the oracle's adds one entry; the
terminal summary (conftest.py) prints the totals, every near-tied row and every
row whose selection differs, so that what "bit-exact selection" rests on is
visible in the test log."""

ENTRIES = []  # dicts: what, rows, near (list of (row, margin, bound, differs)), score_err_over_bound
NOTES = []  # free-form lines (end-to-end agreement reports)


def note(line):
    NOTES.append(line)


def add(what, rows, near, score_err_over_bound=None):
    ENTRIES.append({"what": what, "rows": rows, "near": near, "score_err_over_bound": score_err_over_bound})


def lines():
    if not ENTRIES:
        return list(NOTES)
    rows = sum(e["rows"] for e in ENTRIES)
    near = [(e["what"], *n) for e in ENTRIES for n in e["near"]]
    differ = [n for n in near if n[4]]
    errs = [e["score_err_over_bound"] for e in ENTRIES if e["score_err_over_bound"] is not None]
    out = [f"selection parity: {len(ENTRIES)} comparisons, {rows} rows; near-tied rows (oracle margin "
           f"s_(k) - s_(k+1) below the score bound 1e-4 + 1e-5 |s_(k)|): {len(near)}; rows whose GPU "
           f"selection differs from the oracle's: {len(differ)} (every one of them near-tied)"]
    if errs:
        out.append(f"largest GPU score error as a fraction of its bound: {max(errs):.3g}")
    for what, r, margin, bound, d in near:
        out.append(f"  {what}: row {r}: margin {margin:.3e} < bound {bound:.3e}: "
                   f"{'selection differs' if d else 'same selection'}")
    return out + NOTES
