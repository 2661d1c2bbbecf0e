"""Host-side model of the wavefront schedule of ssd_chunk_scan_segmented (no GPU): the
steps (segment s, layer l) of one anti-diagonal d = s + l run in one launch, layer l reads
the activation buffer act[(l - 1) & 1][s % depth] that step (s, l - 1) wrote one diagonal
earlier and writes act[l & 1][s % depth], and every step uses workspace slot s % depth.
This restates the slot arithmetic of step_problem() (csrc/ssd_common.h) and checks, for
many (segments, layers) pairs, that
  - every step's input is the output of (s, l - 1), not overwritten in between;
  - no two steps of one launch write the same buffer or use the same workspace slot;
  - every (s, l) runs exactly once, after (s, l - 1) and (s - 1, l)."""
import itertools

import pytest


def schedule(S, L):
    depth = min(S, L)
    diags = []
    for d in range(S + L - 1):
        lo, hi = max(0, d - (L - 1)), min(S - 1, d)
        diags.append([(s, d - s) for s in range(lo, hi + 1)])
    return depth, diags


@pytest.mark.parametrize("S,L", [(S, L) for S, L in itertools.product(range(1, 13), range(1, 13))] +
                         [(16, 24), (128, 24), (3, 40)])
def test_wavefront_buffers_and_order(S, L):
    depth, diags = schedule(S, L)
    done = {}
    content = {}                    # buffer -> the (s, l) whose output it holds
    for t, steps in enumerate(diags):
        assert len(steps) <= depth
        writes, slots = set(), set()
        for s, l in steps:
            assert l == 0 or done.get((s, l - 1), t) < t, "input step has not run"
            assert s == 0 or done.get((s - 1, l), t) < t, "layer state not ready"
            if 0 < l:
                src = ((l - 1) & 1, s % depth)
                assert content.get(src) == (s, l - 1), "input buffer overwritten or wrong"
            if l < L - 1:
                dst = (l & 1, s % depth)
                assert dst not in writes, "two steps of one launch write one buffer"
                writes.add(dst)
            slot = s % depth
            assert slot not in slots, "two steps of one launch share a workspace slot"
            slots.add(slot)
        # the steps of one launch run concurrently: none may write another's input buffer
        for s, l in steps:
            if 0 < l:
                assert ((l - 1) & 1, s % depth) not in writes
        for s, l in steps:
            if l < L - 1:
                content[(l & 1, s % depth)] = (s, l)
            done[(s, l)] = t
    assert len(done) == S * L
