"""Oracle of the token-file loader: batches cut from a raw int32 token
stream by plain array slicing.

TEST INFRASTRUCTURE ONLY (like the rest of this package): only the tests,
the smoke check and the CPU-baseline leg of the benchmark use it.

The data files of the pages are raw byte streams of int32 token ids with
no header (ujoy.net article "徒手用 1000 行 C 语言实现", section "训练过程").
Reading: a batch of B x T is the window ids[p : p + B*T + 1], tokens its
first B*T ids and targets its last B*T (the same tokens shifted by one);
p starts at 0, advances by B*T per batch and returns to 0 when the window
would run past the end; a pass is floor(len / (B*T)) batches (which is what
the page prints: 1192 batches of 256 from 305,260 ids, 128 from 32,768).
"""
import numpy as np


def read_ids(path):
    raw = np.fromfile(path, dtype="<i4")
    return raw.astype(np.int32)


def num_batches(n_ids, B, T):
    return n_ids // (B * T)


def batches(ids, B, T, count):
    """The first `count` batches as a list of (tokens, targets), each (B, T)."""
    ids = np.asarray(ids, dtype=np.int32)
    bt = B * T
    out = []
    p = 0
    for _ in range(count):
        if p + bt + 1 > ids.size:
            p = 0
        win = ids[p:p + bt + 1]
        out.append((win[:bt].reshape(B, T).copy(), win[1:].reshape(B, T).copy()))
        p += bt
    return out
