"""Host-side launch planning of ops.GroupedStep (no GPU needed): which GEMMs
share a launch, in which order, and that a launch never mixes A-operand
code formats (the launch's E5M2 flag applies to every problem in it)."""
from types import SimpleNamespace

import pytest

from float8_mixed_precision_amd import ops


def _ffn(e5m2, rowwise=False, M=8192, D=4096, H=14336):
    mk = lambda n, k: SimpleNamespace(M=M, N=n, K=k, rowwise=rowwise, e5m2_grad=e5m2)
    return [mk(H, D), mk(H, D), mk(D, H)]


def test_plan_groups_w1_grad_w_with_w3():
    g = ops.GroupedStep(_ffn(False))
    assert g.plan == [[("grad_x", 0), ("fwd", 0)],
                      [("grad_x", 1), ("grad_w", 0), ("grad_w", 1), ("fwd", 1)],
                      [("fwd", 2), ("grad_w", 2), ("grad_x", 2)]]
    # E4M3 gradients: one launch per linear
    assert [len(g.launches(p)) for p in g.plan] == [1, 1, 1]
    assert all(not e5 for p in g.plan for e5, _ in g.launches(p))


@pytest.mark.parametrize("rowwise", [False, True])
def test_e5m2_forward_gets_its_own_launch(rowwise):
    g = ops.GroupedStep(_ffn(True, rowwise))
    for probs in g.plan:
        launches = g.launches(probs)
        # every problem launched exactly once, in plan order within a format
        flat = [p for _, chunk in launches for p in chunk]
        assert sorted(flat) == sorted(probs)
        for e5, chunk in launches:
            assert 1 <= len(chunk) <= ops.FP8L_MAX_GROUP
            for kind, i in chunk:
                # X's copies are E4M3; dY's (grad_x, grad_w) are E5M2
                assert e5 == (kind != "fwd")
            order = [probs.index(p) for p in chunk]
            assert order == sorted(order)
    assert g.launches(g.plan[0]) == [(True, [("grad_x", 0)]), (False, [("fwd", 0)])]
    assert g.launches(g.plan[1]) == [(True, [("grad_x", 1), ("grad_w", 0), ("grad_w", 1)]),
                                     (False, [("fwd", 1)])]


def test_chunks_of_at_most_max_group():
    g = ops.GroupedStep(_ffn(False))
    probs = [("grad_x", 0), ("grad_w", 0), ("fwd", 0), ("grad_x", 1), ("grad_w", 1)]
    launches = g.launches(probs)
    assert [len(c) for _, c in launches] == [4, 1]
