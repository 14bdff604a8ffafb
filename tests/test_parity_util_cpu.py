"""The stack drift rule of the GPU parity tests, on hand-made logits (CPU)."""
import numpy as np
import pytest

from parity_util import StackDrift, near_mask


def _logits():
    # 2 requests x 3 tokens, 4 experts, top-2; token 1 has a near tie between
    # experts 1 and 2 (gap 1e-4), every other token a clear boundary
    lg = np.array([[3.0, 2.0, 0.0, -1.0],
                   [3.0, 1.0, 0.9999, -1.0],
                   [0.0, 1.0, 2.0, 3.0],
                   [3.0, 2.0, 0.0, -1.0],
                   [3.0, 2.0, 0.0, -1.0],
                   [0.0, 1.0, 2.0, 3.0]])
    idx = np.argsort(-lg, axis=1, kind="stable")[:, :2]
    return lg, idx


def test_near_mask_marks_only_the_tie():
    lg, _ = _logits()
    assert near_mask(lg, 2, 1e-3).tolist() == [False, True, False, False, False, False]


def test_layer0_flip_inside_margin0_fails():
    lg, idx = _logits()
    d = StackDrift(2, 3, margin0=1e-5, drift=1e-3)
    gpu = idx.copy()
    gpu[1] = [0, 2]
    with pytest.raises(AssertionError):
        d.routing(0, gpu, lg, idx, 2)     # gap 1e-4 exceeds the layer-0 margin


def test_later_layer_flip_drops_the_request_tail():
    lg, idx = _logits()
    d = StackDrift(2, 3, margin0=1e-5, drift=1e-3, max_moved=1)
    here = d.routing(0, idx, lg, idx, 2)
    assert here.all()
    gpu = idx.copy()
    gpu[1] = [0, 2]
    here = d.routing(1, gpu, lg, idx, 2)
    assert here.tolist() == [True, False, True, True, True, True]
    assert d.alive.tolist() == [True, False, False, True, True, True]
    # a second token routed differently, near or far, exceeds max_moved
    gpu = idx.copy()
    gpu[3] = [1, 0]
    with pytest.raises(AssertionError):
        d.routing(2, gpu, lg, idx, 2)


def test_a_second_moved_token_fails():
    lg, idx = _logits()
    lg = lg.copy()
    lg[4] = [3.0, 1.0, 0.9999, -1.0]       # a second near tie, in request 1
    idx = np.argsort(-lg, axis=1, kind="stable")[:, :2]
    d = StackDrift(2, 3, margin0=1e-5, drift=1e-3)
    gpu = idx.copy()
    gpu[1] = [0, 2]
    d.routing(1, gpu, lg, idx, 2)          # one genuine near-tie is allowed
    gpu = idx.copy()
    gpu[4] = [0, 2]
    with pytest.raises(AssertionError):
        d.routing(2, gpu, lg, idx, 2)      # a second one is not


def test_layer0_far_flip_fails_and_input_error_is_relative():
    lg, idx = _logits()
    gpu = idx.copy()
    gpu[3] = [1, 0]                        # a clear boundary: never excused at layer 0
    d = StackDrift(2, 3, margin0=1e-5, drift=1e-3)
    with pytest.raises(AssertionError):
        d.routing(0, gpu, lg, idx, 2)
    x = np.ones((6, 4))
    assert d.input_error(x * (1 + 1e-3), x) == pytest.approx(1e-3)
