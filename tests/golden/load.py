"""Readers for the text fixtures in this folder (values printed on the pages)."""
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def worked_pq_example():
    """Returns (tokens, columns dict, scalars dict) of worked_pq_example.txt."""
    toks, cols, scal = [], {k: [] for k in ("p", "q", "min", "res_raw", "res")}, {}
    with open(os.path.join(HERE, "worked_pq_example.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            parts = line.split()
            if len(parts) == 6:
                toks.append(parts[0])
                for k, v in zip(("p", "q", "min", "res_raw", "res"), parts[1:]):
                    cols[k].append(float(v))
            elif len(parts) == 2:
                scal[parts[0]] = float(parts[1])
    return toks, cols, scal


def block_causal_mask():
    """The 9 x 9 visibility matrix of block_causal_3x3.txt as a list of rows
    of 0/1 ints (row = query position, column = key position)."""
    rows = []
    with open(os.path.join(HERE, "block_causal_3x3.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append([int(v) for v in line.split()])
    return rows
