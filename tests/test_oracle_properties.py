"""Property-based pins of the oracle (hypothesis): on random small inputs,
including masked, out-of-range and duplicate ids, the oracle's layout equals
brute force and the stable-argsort route, dispatch then an identity combine
returns every received token's row, and combine stays inside the binary32
error bound around the exact float64 sum.

Sources: DeepEP overall-architecture page (EPHandle fields; dispatch and
combine data-flow figures). These tests share no arithmetic with the oracle:
brute force walks the entries one by one, the argsort route uses numpy, and
the combine bound is computed in float64.
"""
import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from combine_ep_layout_amd import inputs as I
from tests import pins

SETTINGS = settings(max_examples=60, deadline=None,
                    suppress_health_check=[HealthCheck.function_scoped_fixture])


@st.composite
def routings(draw):
    T = draw(st.integers(0, 40))
    K = draw(st.integers(1, 6))
    E = draw(st.integers(1, 12))
    A = draw(st.sampled_from([1, 2, 3, 4, 8, 16]))
    # ids in [-2, E + 1]: negatives and ids >= E are masked entries
    ids = draw(st.lists(st.integers(-2, E + 1), min_size=T * K, max_size=T * K))
    return np.array(ids, np.int32).reshape(T, K), E, A


@SETTINGS
@given(routings())
def test_layout_equals_bruteforce_and_argsort(oracle_mod, r):
    idx, E, A = r
    K = idx.shape[1]
    res = oracle_mod.layout(idx, E, A)
    counts, offsets, dst, rows = pins.layout_bruteforce(idx, E, A)
    pins.check_layout_matches(res, counts, offsets, dst,
                              np.array(rows, np.int64).reshape(-1, K + 2))
    pins.check_layout_matches(res, *pins.layout_by_argsort(idx, E, A))
    pins.check_layout_invariants(idx, E, A, res)


@SETTINGS
@given(routings(), st.integers(0, 2**31 - 1))
def test_dispatch_then_identity_combine_returns_x(oracle_mod, r, seed):
    idx, E, A = r
    T, K = idx.shape
    H = 16
    lay = oracle_mod.layout(idx, E, A)
    cap = max(int(lay["offsets"][-1]), 1)
    x = I.normal_bf16(seed, 2, T, H) if T else np.zeros((0, H), np.uint16)
    X, _, _ = oracle_mod.dispatch(x, lay["dst_slot"], cap)
    got = X.view(np.uint16).reshape(cap, H)
    dst = lay["dst_slot"]
    for t, k in zip(*np.nonzero(dst >= 0)):
        assert np.array_equal(got[dst[t, k]], x[t])
    # identity experts with one unit weight per token on its first unmasked entry:
    # the sum of one product 1.0 * x is exact, so combine returns x bit for bit
    w = np.zeros((T, K), np.float32)
    recv = (dst >= 0).any(axis=1)
    first = np.argmax(dst >= 0, axis=1)
    w[np.nonzero(recv)[0], first[recv]] = 1.0
    out = oracle_mod.combine(got, dst, w)
    assert np.array_equal(out[recv], x[recv])
    assert np.all(out[~recv] == 0)


@SETTINGS
@given(routings(), st.integers(0, 2**31 - 1), st.booleans())
def test_combine_inside_error_bound(oracle_mod, r, seed, with_bias):
    idx, E, A = r
    T, K = idx.shape
    H = 8
    lay = oracle_mod.layout(idx, E, A)
    cap = max(int(lay["offsets"][-1]), 1)
    y = I.normal_bf16(seed, 4, cap, H)
    w = I.router_weights(seed, T, K) if T else np.zeros((0, K), np.float32)
    bias = I.normal_bf16(seed, 9, T, H) if (with_bias and T) else None
    out = oracle_mod.combine(y, lay["dst_slot"], w, bias)
    pins.check_combine_bound(y, lay["dst_slot"], w, out, bias)
