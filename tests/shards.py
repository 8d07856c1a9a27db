"""Reference for one GPU's share of an expert-parallel layer, built from the oracle: a shard holding
experts [first, first + n) outputs the layer's sum over the slots routed to those experts only, which
is the oracle's layer with every other slot weighted 0 (a zero-weighted slot adds exactly nothing)."""
import numpy as np

from oracle import moe_forward


def shard_ref(dims, x, ids, w, store, first, n, rows=None):
    local = (ids >= first) & (ids < first + n)
    return moe_forward(dims, x, ids, np.where(local, w, 0).astype(np.float32), store, rows=rows)
