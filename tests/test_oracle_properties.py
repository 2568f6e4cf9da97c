"""Property-based checks of the oracle (Hypothesis; CPU only).

Where the pins (tests/test_oracle_pins.py) fix values on chosen cases, these draw
many random cases and check what must hold for every one of them: the two routing
formulations agree and produce a stable grouping by key; sequence routing equals
token routing of the expanded ids; the LoRA branch is linear in x, commutes with a
permutation of the tokens, leaves no-LoRA rows alone and equals the grouped
formulation; the rounding helpers are idempotent and monotone.
"""
import numpy as np
import pytest

hypothesis = pytest.importorskip("hypothesis")
from hypothesis import given, settings, strategies as st  # noqa: E402

import oracle.lora_oracle as O  # noqa: E402

SETTINGS = settings(max_examples=150, deadline=None, derandomize=True)


@st.composite
def batches(draw, max_tokens=40, max_slots=12):
    S = draw(st.integers(1, max_slots))
    ids = draw(st.lists(st.integers(-3, S + 3), min_size=0, max_size=max_tokens))
    return ids, S


@SETTINGS
@given(batches())
def test_routing_formulations_agree_and_group_stably(case):
    ids, S = case
    a, b = O.route_by_sort(ids, S), O.route_by_counting(ids, S)
    for f in ("keys", "counts", "seg_offsets", "sorted_ids", "active_slots"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f
    assert a.num_active == b.num_active and a.n_invalid == b.n_invalid
    T = len(ids)
    assert sorted(a.sorted_ids.tolist()) == list(range(T))            # a permutation of the tokens
    assert int(a.counts.sum()) == T and a.seg_offsets[-1] == T
    for k in range(S + 1):                                              # each segment: its key, ascending
        seg = a.sorted_ids[a.seg_offsets[k]:a.seg_offsets[k + 1]]
        assert all(a.keys[t] == k for t in seg)
        assert np.all(np.diff(seg) > 0)
    valid = [(i >= 0 and i < S) for i in ids]
    assert a.n_invalid == sum(1 for i, v in zip(ids, valid) if not v and i != -1)
    assert a.active_slots.tolist() == sorted({i for i in ids if 0 <= i < S})


@SETTINGS
@given(batches(max_tokens=16), st.integers(1, 5))
def test_sequence_routing_is_token_routing_of_expanded_ids(case, p):
    seq_ids, S = case
    r = O.route_tokens_per_seq(seq_ids, S, p)
    tok = O.route_by_counting([i for i in seq_ids for _ in range(p)], S)
    for f in ("keys", "counts", "seg_offsets", "sorted_ids", "active_slots"):
        assert np.array_equal(getattr(r, f), getattr(tok, f)), f
    assert r.n_invalid == tok.n_invalid


def _adapters(rng, S, k, slices, Rmax, with_empty=True):
    ads = {}
    for s in range(S):
        if with_empty and s == S - 1 and S > 1:
            continue                                                   # one slot left empty
        r = int(rng.integers(1, Rmax + 1))
        A = [rng.standard_normal((r, k)) / np.sqrt(k) for _ in slices]
        B = [rng.standard_normal((d, r)) / np.sqrt(r) for d in slices]
        if len(slices) > 1 and rng.random() < 0.3:
            A[1] = None; B[1] = None                                   # a missing slice
        ads[s] = O.Adapter(rank=r, A=A, B=B, alpha=float(rng.integers(1, 65)), rslora=bool(rng.random() < 0.5))
    return ads


@st.composite
def lora_cases(draw):
    seed = draw(st.integers(0, 2 ** 31 - 1))
    S = draw(st.integers(1, 6))
    T = draw(st.integers(1, 12))
    k = draw(st.integers(1, 24))
    slices = draw(st.lists(st.integers(1, 10), min_size=1, max_size=3))
    Rmax = draw(st.integers(1, 8))
    return seed, S, T, k, slices, Rmax


@SETTINGS
@given(lora_cases())
def test_branch_is_linear_permutation_equivariant_and_grouped_equal(case):
    seed, S, T, k, slices, Rmax = case
    rng = np.random.default_rng(seed)
    ads = _adapters(rng, S, k, slices, Rmax)
    ids = rng.integers(-2, S + 2, size=T).tolist()
    D = sum(slices)
    x1, x2 = rng.standard_normal((T, k)), rng.standard_normal((T, k))
    y0 = rng.standard_normal((T, D))
    zero = np.zeros((T, D))
    f = lambda x: O.lora_apply(x, zero, ads, slices, ids, S, "f32", max_rank=Rmax)
    a, b = 1.75, -0.5
    lhs, rhs = f(a * x1 + b * x2), a * f(x1) + b * f(x2)
    assert np.allclose(lhs, rhs, rtol=1e-10, atol=1e-10)
    # on a base: the base plus the branch
    assert np.allclose(O.lora_apply(x1, y0, ads, slices, ids, S, "f32", max_rank=Rmax), y0 + f(x1),
                       rtol=1e-12, atol=1e-12)
    # no-LoRA tokens (invalid ids, -1, the empty slot) keep their base rows exactly
    y = O.lora_apply(x1, y0, ads, slices, ids, S, "f32", max_rank=Rmax)
    for t, i in enumerate(ids):
        if not (0 <= i < S) or i not in ads:
            assert np.array_equal(y[t], y0[t])
    # a permutation of the tokens permutes the rows
    perm = rng.permutation(T)
    yp = O.lora_apply(x1[perm], y0[perm], ads, slices, [ids[p] for p in perm], S, "f32", max_rank=Rmax)
    assert np.allclose(yp, y[perm], rtol=1e-12, atol=1e-12)
    # the grouped formulation (per slot: gather, two products, scatter)
    g = O.lora_apply_grouped(x1, y0, ads, slices, ids, S, "f32")
    assert np.allclose(g, y, rtol=1e-12, atol=1e-12)


@SETTINGS
@given(st.lists(st.floats(-2.0 ** 100, 2.0 ** 100, allow_nan=False, width=32), min_size=1, max_size=64))
def test_bf16_rounding_idempotent_and_monotone(vals):
    x = np.asarray(vals, dtype=np.float32)
    b = O.bf16_bits_to_f64(O.f32_to_bf16_bits(x))
    again = O.bf16_bits_to_f64(O.f32_to_bf16_bits(b.astype(np.float32)))
    assert np.array_equal(b, again)
    order = np.argsort(x, kind="stable")
    assert np.all(np.diff(b[order]) >= 0)
    # within half a bf16 unit in the last place: 2^-8 relative for normal values, half
    # the smallest bf16 subnormal (2^-134) below
    assert np.all(np.abs(b - x.astype(np.float64)) <= np.abs(x.astype(np.float64)) * 2.0 ** -8 + 2.0 ** -134)


@SETTINGS
@given(st.lists(st.floats(-1e4, 1e4, allow_nan=False), min_size=1, max_size=64))
def test_fp8_quantize_idempotent_monotone_and_clamped(vals):
    x = np.asarray(vals, dtype=np.float64)
    q = O.fp8_quantize(x)
    assert np.all(np.abs(q) <= 448.0)
    assert np.array_equal(O.fp8_quantize(q), q)
    order = np.argsort(x, kind="stable")
    assert np.all(np.diff(q[order]) >= 0)
    assert np.array_equal(O.fp8_e4m3_decode(O.fp8_e4m3_encode(q)), q)
