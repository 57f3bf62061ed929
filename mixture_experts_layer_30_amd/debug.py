"""Debug checks of an alignment read back from the device.

The grouped FFN trusts the alignment (moe_align) blindly: a wrong count,
offset or row sends tokens to the wrong expert or reads past a bucket.  With
MOE_DEBUG=1 in the environment (or MoELayer(..., debug=True)) the layer copies
the five plan arrays to the host after every alignment and checks the
invariants that define them (Serving-tax notes, padding model, Section 5.1:
each pair lands in exactly one bucket, every bucket padded to a multiple of the
GEMM M-tile and at least its count); a violation raises PlanError naming it.
This is a host-side check for debugging, not part of the timed path; it costs
a device-to-host copy and a synchronisation per call.
"""
import os

import numpy as np


class PlanError(RuntimeError):
    """An alignment that breaks one of its invariants."""


def debug_enabled(flag=None):
    """flag if given, else whether MOE_DEBUG is set to a non-zero value."""
    if flag is not None:
        return bool(flag)
    return os.environ.get("MOE_DEBUG", "0") not in ("", "0")


def _host(a):
    if hasattr(a, "detach"):
        a = a.detach().cpu().numpy()
    return np.asarray(a, dtype=np.int64)


def check_plan(arrays, topk_ids, E, block_m, cap, pad="block"):
    """Check the alignment `arrays` (expert_counts [E], expert_offsets [E+1],
    sorted_ids [cap], block_expert [cap/B], inv_pos [T*K]; device tensors or
    arrays) of the routing `topk_ids` [T][K] (negative = unused slot) against:

      1. counts[e] = the pairs routed to e;
      2. offsets: 0 first, each bucket padded to ceil(count/B)*B rows ("block"), or
         every bucket the busiest one's ceil(max/B)*B ("max"); the total <= cap;
      3. bucket e = its pairs in ascending pair index, then the sentinel T*K up
         to the next bucket; every row past the total the sentinel;
      4. block_expert[b] = the expert whose bucket holds rows b*B.., -1 past the total;
      5. inv_pos[p] = the row holding pair p (-1 for an unused slot).

    Raises PlanError listing every violated invariant; returns None."""
    ids = _host(topk_ids)
    T, K = ids.shape
    B = int(block_m)
    n_pairs = T * K
    counts = _host(arrays["expert_counts"])
    offsets = _host(arrays["expert_offsets"])
    rows = _host(arrays["sorted_ids"])
    blocks = _host(arrays["block_expert"])
    inv = _host(arrays["inv_pos"])
    bad = []
    if cap % B:
        bad.append(f"cap {cap} is not a multiple of block_m {B}")
    if counts.shape != (E,) or offsets.shape != (E + 1,) or rows.shape != (cap,) or \
            blocks.shape != (cap // B,) or inv.shape != (n_pairs,):
        raise PlanError("plan array shapes: counts %s offsets %s sorted_ids %s block_expert %s "
                        "inv_pos %s" % (counts.shape, offsets.shape, rows.shape, blocks.shape,
                                        inv.shape))
    flat = ids.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    if ((flat >= E)).any():
        bad.append("topk_ids holds experts >= E")
    want_counts = np.bincount(flat[valid], minlength=E)[:E]
    diff = np.nonzero(counts != want_counts)[0]
    if diff.size:
        e = int(diff[0])
        bad.append(f"expert_counts differ at {diff.size} experts (e={e}: {counts[e]} != {want_counts[e]})")
    if pad == "block":
        size = -(-want_counts // B) * B
    elif pad == "max":
        size = np.full(E, -(-int(want_counts.max(initial=0)) // B) * B)
    else:
        raise ValueError(f"pad {pad!r}")
    want_off = np.concatenate([[0], np.cumsum(size)])
    diff = np.nonzero(offsets != want_off)[0]
    if diff.size:
        i = int(diff[0])
        bad.append(f"expert_offsets differ at {diff.size} entries (i={i}: {offsets[i]} != {want_off[i]})")
    total = int(want_off[-1])
    if total > cap:
        bad.append(f"padded total {total} exceeds cap {cap}")
    if bad:   # the rest is read through the offsets
        raise PlanError("; ".join(bad))
    want_rows = np.full(cap, n_pairs, np.int64)
    order = np.argsort(flat, kind="stable")
    order = order[valid[order]]
    pos = 0
    for e in range(E):
        n = int(want_counts[e])
        want_rows[want_off[e]:want_off[e] + n] = order[pos:pos + n]
        pos += n
    diff = np.nonzero(rows != want_rows)[0]
    if diff.size:
        r = int(diff[0])
        bad.append(f"sorted_ids differ at {diff.size} rows (row {r}: {rows[r]} != {want_rows[r]})")
    want_blocks = np.full(cap // B, -1, np.int64)
    for e in range(E):
        want_blocks[want_off[e] // B:want_off[e + 1] // B] = e
    diff = np.nonzero(blocks != want_blocks)[0]
    if diff.size:
        b = int(diff[0])
        bad.append(f"block_expert differs at {diff.size} blocks (block {b}: {blocks[b]} != {want_blocks[b]})")
    want_inv = np.full(n_pairs, -1, np.int64)
    held = want_rows < n_pairs
    want_inv[want_rows[held]] = np.nonzero(held)[0]
    diff = np.nonzero(inv != want_inv)[0]
    if diff.size:
        p = int(diff[0])
        bad.append(f"inv_pos differs at {diff.size} pairs (pair {p}: {inv[p]} != {want_inv[p]})")
    if bad:
        raise PlanError("; ".join(bad))
