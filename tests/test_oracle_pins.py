"""Pins for the CPU oracle: what the pages and the mathematics fix, independent of the oracle.

Each pin is chosen so that a plausible mistake (a dropped term, a wrong sign or
index, a transposed operand, a wrong tie-break) fails at least one of them;
``test_planted_mistakes_are_caught`` plants such mistakes in the oracle and checks
that the pins notice.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle.lora_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------- pin checks
# Each check returns None when it holds and a message when it fails, so the same
# checks can be run against planted mistakes.

def check_scale_golden():
    for c in _load("scale_cases.json")["cases"]:
        got = O.lora_scale(c["alpha"], c["rank"], c["rslora"], c["adapter_scale"])
        want = np.uint32(int(c["expect_f32_hex"], 16)).view(np.float32)
        if np.float32(got).view(np.uint32) != want.view(np.uint32):
            return f"scale {c}: got {got!r}"
    return None


def _check_routing(R, c):
    for key in ("counts", "seg_offsets", "sorted_ids", "active_slots"):
        if list(map(int, getattr(R, key))) != c[key]:
            return f"{key}: got {list(getattr(R, key))} want {c[key]}"
    if R.num_active != len(c["active_slots"]) or R.n_invalid != c["n_invalid"]:
        return "num_active / n_invalid"
    return None


def check_routing_golden():
    for c in _load("routing_cases.json")["cases"]:
        for f in (O.route_by_sort, O.route_by_counting):
            msg = _check_routing(f(c["ids"], c["S"]), c)
            if msg:
                return f"{f.__name__} {c['ids']}: {msg}"
    return None


def _integer_case(premultiply=False):
    g = _load("integer_case.json")
    ads = {}
    for s, a in g["adapters"].items():
        A = [None if m is None else np.array(m, dtype=np.float64) for m in a["A"]]
        B = [None if m is None else np.array(m, dtype=np.float64) for m in a["B"]]
        ads[int(s)] = O.Adapter(rank=a["rank"], A=A, B=B, alpha=a["alpha"],
                                adapter_scale=a["adapter_scale"], premultiply=premultiply)
    return g, ads


def check_integer_golden():
    for pre in (False, True):
        g, ads = _integer_case(pre)
        x = np.array(g["x"], dtype=np.float64)
        yb = np.array(g["y_base"], dtype=np.float64)
        for f in (O.lora_apply, O.lora_apply_grouped):
            y = f(x, yb, ads, g["slices"], g["ids"], g["S"], "f32")
            if not np.array_equal(y, np.array(g["y"], dtype=np.float64)):
                return f"{f.__name__} premultiply={pre}: {y.tolist()}"
        u, mask = O.shrink_per_token(x, ads, g["slices"], g["ids"], g["S"], g["max_rank"])
        for key, vals in g["u_defined"].items():
            n, t = map(int, key.split(","))
            if not (mask[n, t, :len(vals)].all() and np.array_equal(u[n, t, :len(vals)], vals)):
                return f"u[{key}] = {u[n, t]}"
        if mask[:, 1].any():
            return "u defined on a no-LoRA row"
    return None


def _random_case(seed, T=9, S=3, k=13, slices=(5, 11), ranks=None, nolora=True):
    rng = np.random.default_rng(seed)
    ranks = ranks or {0: 3, 1: 6, 2: 1}
    ads = {}
    for s, r in ranks.items():
        ads[s] = O.Adapter(rank=r, A=[rng.standard_normal((r, k)) for _ in slices],
                           B=[rng.standard_normal((d, r)) for d in slices],
                           alpha=float(rng.integers(1, 40)), rslora=bool(s % 2))
    ids = rng.integers(-1 if nolora else 0, S, size=T)
    x = rng.standard_normal((T, k))
    W0 = rng.standard_normal((sum(slices), k))
    return ads, ids, x, W0


def check_linearity():
    """Unmerged branch == merged weight (W0 + s B A) x; per-token == grouped loop."""
    for seed in range(3):
        ads, ids, x, W0 = _random_case(seed)
        slices = (5, 11)
        yb = x @ W0.T
        y1 = O.lora_apply(x, yb, ads, slices, ids, 3, "f32")
        y2 = O.lora_apply_grouped(x, yb, ads, slices, ids, 3, "f32")
        y3 = O.merged_apply(x, W0, ads, slices, ids, 3, "f32")
        scale = np.abs(y3).max()
        if np.abs(y1 - y3).max() > 1e-10 * scale:
            return f"unmerged vs merged {np.abs(y1 - y3).max()}"
        if np.abs(y1 - y2).max() > 1e-12 * scale:
            return f"per-token vs grouped {np.abs(y1 - y2).max()}"
    return None


def check_identity_closed_form():
    """A = [I_r | 0], B = [I_r ; 0], s = 1  =>  delta_t = (x_t[0:r], 0, ...)."""
    r, k, d, T = 3, 7, 5, 4
    A = np.zeros((r, k)); A[:, :r] = np.eye(r)
    B = np.zeros((d, r)); B[:r, :] = np.eye(r)
    ads = {0: O.Adapter(rank=r, A=[A], B=[B], alpha=float(r))}
    x = np.arange(T * k, dtype=np.float64).reshape(T, k) - 9
    y = O.lora_apply(x, np.zeros((T, d)), ads, [d], [0] * T, 1, "f32")
    want = np.zeros((T, d)); want[:, :r] = x[:, :r]
    return None if np.array_equal(y, want) else f"identity: {y}"


def check_single_entry():
    """A = e_j e_c^T, B = e_i e_j^T  =>  delta[t, i] = s * x[t, c], nothing else.

    Fixes which index of A is the rank and which the input column, and which index
    of B is the output column: a transposed operand moves or loses the entry."""
    k, d, r = 6, 4, 3
    j, c, i = 2, 5, 1
    A = np.zeros((r, k)); A[j, c] = 1.0
    B = np.zeros((d, r)); B[i, j] = 1.0
    ads = {1: O.Adapter(rank=r, A=[A], B=[B], alpha=6.0)}   # s = 2
    x = np.arange(1, 3 * k + 1, dtype=np.float64).reshape(3, k)
    y = O.lora_apply(x, np.zeros((3, d)), ads, [d], [1, -1, 1], 2, "f32")
    want = np.zeros((3, d)); want[0, i] = 2 * x[0, c]; want[2, i] = 2 * x[2, c]
    return None if np.array_equal(y, want) else f"single entry: {y}"


def check_zero_branches():
    ads, ids, x, W0 = _random_case(7)
    yb = x @ W0.T
    for mut in ("B", "A", "scale"):
        z = {}
        for s, a in ads.items():
            A = [np.zeros_like(m) for m in a.A] if mut == "A" else a.A
            B = [np.zeros_like(m) for m in a.B] if mut == "B" else a.B
            z[s] = O.Adapter(rank=a.rank, A=A, B=B, alpha=a.alpha, rslora=a.rslora,
                             adapter_scale=0.0 if mut == "scale" else 1.0)
        y = O.lora_apply(x, yb, z, (5, 11), ids, 3, "f32")
        if not np.array_equal(y, yb):
            return f"zero {mut} changed y"
    y = O.lora_apply(x, yb, ads, (5, 11), ids, 3, "f32")
    rows = np.asarray(ids) < 0
    if not np.array_equal(y[rows], yb[rows]):
        return "no-LoRA rows changed"
    return None


def check_packed_equals_separate():
    ads, ids, x, W0 = _random_case(11)
    yb = np.zeros((x.shape[0], 16))
    y = O.lora_apply(x, yb, ads, (5, 11), ids, 3, "f32")
    parts = []
    for n, d in enumerate((5, 11)):
        sub = {s: O.Adapter(rank=a.rank, A=[a.A[n]], B=[a.B[n]], alpha=a.alpha, rslora=a.rslora)
               for s, a in ads.items()}
        parts.append(O.lora_apply(x, np.zeros((x.shape[0], d)), sub, (d,), ids, 3, "f32"))
    return None if np.array_equal(y, np.concatenate(parts, axis=1)) else "packed != separate"


def check_rank_padding():
    ads, ids, x, _ = _random_case(5)
    u1, m1 = O.shrink_per_token(x, ads, (5, 11), ids, 3, 6)
    u2, m2 = O.shrink_per_token(x, ads, (5, 11), ids, 3, 64)
    if not (np.array_equal(u1[m1], u2[:, :, :6][m1]) and not m2[:, :, 6:].any()):
        return "rank padding changed u"
    return None


PINS = [check_scale_golden, check_routing_golden, check_integer_golden, check_linearity,
        check_identity_closed_form, check_single_entry, check_zero_branches,
        check_packed_equals_separate, check_rank_padding, lambda: check_fp8_golden()]


@pytest.mark.parametrize("check", PINS, ids=lambda f: getattr(f, "__name__", "pin"))
def test_pin(check):
    msg = check()
    assert msg is None, msg


# -------------------------------------------------------- number-format pins
def test_bf16_rounding_known_values():
    cases = {
        1.0: 0x3F80, -2.5: 0xC020, 0.0: 0x0000,
        1.0 + 2.0 ** -8: 0x3F80,                   # exact tie, kept lsb even -> down
        1.0 + 3 * 2.0 ** -8: 0x3F82,               # exact tie, kept lsb odd -> up
        1.0 + 2.0 ** -8 + 2.0 ** -20: 0x3F81,      # just above the tie -> up
        float(np.finfo(np.float32).max): 0x7F80,   # rounds to +inf
        float("inf"): 0x7F80, float("-inf"): 0xFF80,
        1e-45: 0x0000,                             # smallest subnormal -> +0
    }
    for v, bits in cases.items():
        got = int(O.f32_to_bf16_bits(np.float32(v))[0])
        assert got == bits, (v, hex(got), hex(bits))
    assert int(O.f32_to_bf16_bits(np.float32(-0.0))[0]) == 0x8000
    assert np.isnan(O.bf16_bits_to_f64(O.f32_to_bf16_bits(np.float32("nan"))))


def test_bf16_rounding_matches_library_routine():
    """Round-to-nearest-even float32 -> bfloat16 is also what torch's dtype cast does."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(3)
    wide = rng.standard_normal(200000) * 10.0 ** rng.integers(-30, 30, 200000)
    bits = rng.integers(0, 2 ** 32, 50000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    a = np.concatenate([wide[np.abs(wide) < 3e38].astype(np.float32), bits[np.isfinite(bits)]])
    lib = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.f32_to_bf16_bits(a), lib)


def test_bf16_decode_is_exact():
    bits = np.arange(0, 2 ** 16, dtype=np.uint32).astype(np.uint16)
    v = O.bf16_bits_to_f64(bits)
    fin = np.isfinite(v)
    assert np.array_equal(O.f32_to_bf16_bits(v[fin].astype(np.float32)), bits[fin])


# ---------------------------------------------------------- routing brute force
def _independent_invariants(ids, S, R):
    T = len(ids)
    keys = [i if 0 <= i < S else S for i in ids]
    assert sorted(R.sorted_ids.tolist()) == list(range(T))
    assert len(R.counts) == S + 1 and len(R.seg_offsets) == S + 2
    assert R.seg_offsets[0] == 0 and R.seg_offsets[S + 1] == T
    for k in range(S + 1):
        seg = R.sorted_ids[R.seg_offsets[k]:R.seg_offsets[k + 1]].tolist()
        assert seg == [t for t in range(T) if keys[t] == k]
        assert R.counts[k] == len(seg)
    assert R.active_slots.tolist() == [k for k in range(S) if keys.count(k) > 0]
    assert R.n_invalid == sum(1 for i in ids if not (i == -1 or 0 <= i < S))


@pytest.mark.parametrize("S", [1, 2, 3])
def test_routing_brute_force(S):
    vals = list(range(-2, S + 1))
    for T in range(0, 7):
        for ids in itertools.product(vals, repeat=T):
            a = O.route_by_sort(list(ids), S)
            b = O.route_by_counting(list(ids), S)
            _independent_invariants(list(ids), S, a)
            for f in ("counts", "seg_offsets", "sorted_ids", "active_slots"):
                assert np.array_equal(getattr(a, f), getattr(b, f))


# --------------------------------------------------------------- page numbers
def test_page_numbers():
    g = _load("page_numbers.json")
    e = g["extra_macs"]
    ratio = O.extra_macs_per_token(e["k"], [e["d"]], e["r"]) / (e["d"] * e["k"])
    assert ratio == 2 * 16 / 4096
    assert round(100 * ratio, e["printed_digits"]) == e["printed_percent"]
    p = g["param_ratio"]
    assert round(100 * O.adapter_params(p["d"], [p["d"]], p["r"]) / p["d"] ** 2, p["printed_digits"]) == p["printed_percent"]
    a = g["adapter_7b"]
    d, f, r = a["d"], a["ffn"], a["r"]
    layer = [(d, [d])] * 4 + [(d, [f])] * 2 + [(f, [d])]
    per_layer = sum(O.adapter_params(k, sl, r) for k, sl in layer)
    assert round(per_layer / 1e6, 2) == a["printed_per_layer_M"]
    assert round(per_layer * a["layers"] / 1e6, 1) == a["printed_total_M"]
    assert round(per_layer * a["layers"] * 2 / 1e6) == a["printed_f16_MB"]
    base = sum(k * sl[0] for k, sl in layer)
    assert abs(base / 1e6 - a["printed_base_per_layer_M"]) < 0.1
    v = g["vllm_buffer"]
    total = v["layers"] * O.adapter_params(v["in"], [v["out"]], v["r"]) * v["bytes"] * v["max_loras"]
    assert total == v["expression_bytes"] == 128 * 2 ** 20
    assert v["printed_MB"] == 2 * total // 2 ** 20     # the page's figure is twice its own expression


# -------------------------------------------------------------- planted mistakes
def _mut_scale_ignores_rslora(alpha, rank, rslora, adapter_scale=1.0):
    return np.float32(adapter_scale * alpha / rank) if alpha else np.float32(adapter_scale)


def _mut_scale_alpha_missing_zero(alpha, rank, rslora, adapter_scale=1.0):
    if alpha == 0:
        return np.float32(0.0)
    return np.float32(adapter_scale * alpha / (math.sqrt(rank) if rslora else rank))


def _mut_scale_uses_rank_plus_one(alpha, rank, rslora, adapter_scale=1.0):
    if alpha == 0:
        return np.float32(adapter_scale)
    return np.float32(adapter_scale * alpha / (math.sqrt(rank) if rslora else rank + 1))


def _mut_keys_sentinel_first(ids, S):
    ids = np.asarray(ids, dtype=np.int64)
    valid = (ids >= 0) & (ids < S)
    # no-LoRA tokens under key 0 and every slot shifted up: the no-LoRA group sorts first
    return np.where(valid, ids, -1).astype(np.int64), int(np.count_nonzero(~valid & (ids != -1)))


def _mut_effective_b_double_scale(adapter, n, wdtype):
    B = adapter.B[n]
    s = adapter.scale()
    if B is None:
        return None, float(s)
    if adapter.premultiply:
        return np.float32(s) * np.asarray(B, dtype=np.float64), float(s)   # scale applied twice
    return np.asarray(B, dtype=np.float64), float(s)


def _mut_effective_b_drop_scale(adapter, n, wdtype):
    B = adapter.B[n]
    return (None if B is None else np.asarray(B, dtype=np.float64)), 1.0


_orig_shrink = O.shrink_per_token


def _mut_shrink_transposed_tokens(x, adapters, slices, ids, S, max_rank):
    return _orig_shrink(np.asarray(x)[::-1], adapters, slices, ids, S, max_rank)


def _mut_bf16_truncate(a):
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    return (f.view(np.uint32) >> 16).astype(np.uint16)


MUTANTS = [
    ("lora_scale", _mut_scale_ignores_rslora),
    ("lora_scale", _mut_scale_alpha_missing_zero),
    ("lora_scale", _mut_scale_uses_rank_plus_one),
    ("_keys", _mut_keys_sentinel_first),
    ("effective_b", _mut_effective_b_double_scale),
    ("effective_b", _mut_effective_b_drop_scale),
    ("shrink_per_token", _mut_shrink_transposed_tokens),
]


@pytest.mark.parametrize("name,mutant", MUTANTS, ids=lambda v: getattr(v, "__name__", v))
def test_planted_mistakes_are_caught(monkeypatch, name, mutant):
    monkeypatch.setattr(O, name, mutant)
    failures = []
    for check in PINS:
        try:
            msg = check()
        except Exception as e:  # a crash is also a caught mistake
            msg = repr(e)
        if msg:
            failures.append(check.__name__)
    assert failures, f"planted mistake {mutant.__name__} passed every pin"


def test_planted_rounding_mistake_is_caught(monkeypatch):
    monkeypatch.setattr(O, "f32_to_bf16_bits", _mut_bf16_truncate)
    with pytest.raises(AssertionError):
        test_bf16_rounding_known_values()


def test_planted_unstable_sort_is_caught(monkeypatch):
    original = O.route_by_counting

    def unstable(ids, S):
        R = original(ids, S)
        out = R.sorted_ids.copy()
        for k in range(S + 1):
            a, b = R.seg_offsets[k], R.seg_offsets[k + 1]
            out[a:b] = out[a:b][::-1]
        R.sorted_ids = out
        return R
    monkeypatch.setattr(O, "route_by_counting", unstable)
    assert check_routing_golden() is not None


# ---------------------------------------------------- several tokens per sequence
def test_routing_seq_golden():
    """Hand-worked cases of the sequence-to-token expansion (tests/golden/routing_seq_cases.json)."""
    for c in _load("routing_seq_cases.json")["cases"]:
        R = O.route_tokens_per_seq(c["seq_ids"], c["S"], c["tokens_per_seq"])
        assert _check_routing(R, c) is None, (c["seq_ids"], _check_routing(R, c))


def test_routing_seq_planted_interleave_fails_golden():
    """A plausible slip, expanding sequence-major as j*Q + q instead of q*p + j, does
    not match the hand-worked case."""
    c = _load("routing_seq_cases.json")["cases"][0]
    p, Q = c["tokens_per_seq"], len(c["seq_ids"])
    good = O.route_tokens_per_seq(c["seq_ids"], c["S"], p)
    q_order = [t // p for t in good.sorted_ids[::p]]
    wrong = [j * Q + q for q in q_order for j in range(p)]
    assert wrong != c["sorted_ids"]


@pytest.mark.parametrize("p", [1, 2, 3])
@pytest.mark.parametrize("S", [1, 2])
def test_routing_seq_brute_force(S, p):
    """Every sequence-id vector of up to 4 sequences: the page's sequence sort plus
    expansion equals a stable token-level sort of the ids repeated p times, and each
    sequence's tokens stay contiguous and in order."""
    vals = list(range(-2, S + 1))
    for Q in range(0, 5):
        for seq in itertools.product(vals, repeat=Q):
            a = O.route_tokens_per_seq(list(seq), S, p)
            b = O.route_by_sort([i for i in seq for _ in range(p)], S)
            for f in ("counts", "seg_offsets", "sorted_ids", "active_slots"):
                assert np.array_equal(getattr(a, f), getattr(b, f)), (seq, p, f)
            assert a.n_invalid == b.n_invalid
            srt = list(a.sorted_ids)
            for i in range(0, len(srt), p):
                assert srt[i] % p == 0 and srt[i:i + p] == list(range(srt[i], srt[i] + p))


# ---------------------------------------------------------------- embedding LoRA
def test_embedding_golden():
    """Hand-worked embedding case (tests/golden/embedding_case.json)."""
    g = _load("embedding_case.json")
    ad = O.Adapter(rank=g["rank"], A=[np.array(g["A"], dtype=np.float64)], B=[np.array(g["B"], dtype=np.float64)],
                   alpha=g["alpha"])
    y = O.embedding_apply(g["vocab_ids"], np.array(g["y_base"], dtype=np.float64), {0: ad}, g["vocab"],
                          g["slot_ids"], g["S"], "f32")
    assert np.array_equal(y, np.array(g["y"], dtype=np.float64))


@pytest.mark.parametrize("premultiply", [False, True])
def test_embedding_is_linear_lora_on_one_hot_inputs(premultiply):
    """get_rows of A by vocabulary id is A times a one-hot input: the embedding branch
    equals the linear branch (the per-token definition) on one-hot rows, exactly; a
    vocabulary id outside the table is an all-zero row."""
    rng = np.random.default_rng(7)
    S, V, d, T = 5, 40, 24, 60
    ranks = {0: 3, 1: 8, 2: 1, 4: 5}
    ads = {s: O.Adapter(rank=r, A=[rng.standard_normal((r, V))], B=[rng.standard_normal((d, r))],
                        alpha=float(2 * r + s), premultiply=premultiply) for s, r in ranks.items()}
    ids = rng.integers(-1, S + 1, size=T)
    vocab = rng.integers(-2, V + 2, size=T)
    yb = rng.standard_normal((T, d))
    onehot = np.zeros((T, V))
    for t, v in enumerate(vocab):
        if 0 <= v < V:
            onehot[t, v] = 1.0
    got = O.embedding_apply(vocab, yb, ads, V, ids, S, "f32")
    ref = O.lora_apply(onehot, yb, ads, [d], ids, S, "f32", max_rank=8)
    assert np.array_equal(got, ref)


# ------------------------------------------------------------------ FP8 (e4m3)
def _torch_fp8():
    torch = pytest.importorskip("torch")
    if not hasattr(torch, "float8_e4m3fn"):
        pytest.skip("torch without float8_e4m3fn")
    return torch


def test_fp8_decode_matches_torch_all_bytes():
    """Every e4m3 bit pattern decodes to torch's float8_e4m3fn value (a library
    implementation of the OCP format), NaN patterns included."""
    torch = _torch_fp8()
    b = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(b).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.fp8_e4m3_decode(b)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok]) and np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))
    assert O.fp8_e4m3_decode([0x7E])[0] == 448.0 and O.fp8_e4m3_decode([0x01])[0] == 2.0 ** -9


def test_fp8_encode_matches_torch_rounding():
    """Round-to-nearest-even to e4m3 agrees with torch's conversion on every finite
    value, on every midpoint between neighbours (the ties) and on random values."""
    torch = _torch_fp8()
    vals = O.fp8_e4m3_decode(np.arange(256))
    fin = np.unique(vals[~np.isnan(vals)])
    mids = (fin[:-1] + fin[1:]) / 2.0
    rng = np.random.default_rng(3)
    rnd = np.concatenate([rng.uniform(-448, 448, 4000), rng.standard_normal(4000) * 0.01,
                          rng.standard_normal(2000) * 2.0 ** -8])
    for x in (fin, mids, rnd):
        ref = torch.from_numpy(x.astype(np.float64)).to(torch.float8_e4m3fn).view(torch.uint8).numpy().astype(np.int64)
        got = O.fp8_e4m3_encode(x)
        assert np.array_equal(got, ref)
    # two ties by hand: 1.0625 lies between 1.0 (mantissa 000) and 1.125 (001) -> 1.0;
    # 1.1875 between 1.125 (001) and 1.25 (010) -> 1.25
    assert list(O.fp8_e4m3_encode([1.0625, 1.1875])) == [0x38, 0x3A]


def test_fp8_quantize_clamps_first():
    """Without the clamp a value past 464 would round to NaN; the input conversion
    clamps to +-448 first, and values already on the grid are unchanged."""
    assert list(O.fp8_quantize([500.0, -1e6, 460.0])) == [448.0, -448.0, 448.0]
    grid = O.fp8_e4m3_decode(np.arange(0, 0x7F))
    assert np.array_equal(O.fp8_quantize(grid), grid)


def test_fp8_fold_scale_matches_the_pages_expression():
    """The scale fold equals the page's expression evaluated by torch:
    (t.to(bfloat16) * scale).clamp(-fp8_max, fp8_max).to(float8_e4m3fn)."""
    torch = _torch_fp8()
    rng = np.random.default_rng(5)
    b = rng.integers(0, 256, size=3000).astype(np.uint8)
    b = b[~np.isnan(O.fp8_e4m3_decode(b))]
    vals = O.fp8_e4m3_decode(b)
    for s in (np.float32(2.0), np.float32(1.0 / 3.0), np.float32(4.0), np.float32(0.70710677), np.float32(37.5)):
        t = torch.from_numpy(b).view(torch.float8_e4m3fn)
        ref = (t.to(torch.bfloat16) * float(s)).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).to(torch.float64).numpy()
        got = O.fp8_fold_scale(vals, s)
        assert np.array_equal(got, ref), float(s)


# ------------------------------------------------------- FP8 path, composition
def _fp8_golden_apply():
    g = _load("fp8_case.json")
    a = g["adapter"]
    ad = O.Adapter(rank=a["rank"], A=[np.array(a["A"], dtype=np.float64)], B=[np.array(a["B"], dtype=np.float64)],
                   alpha=a["alpha"], rslora=a["rslora"], adapter_scale=a["adapter_scale"])
    y = O.lora_apply_fp8(np.array(g["x"], dtype=np.float64), np.array(g["y_base"], dtype=np.float64), {0: ad},
                         g["slices"], g["ids"], g["S"], max_rank=g["max_rank"])
    return g, y


def check_fp8_golden():
    g, y = _fp8_golden_apply()
    if not np.array_equal(y, np.array(g["y"], dtype=np.float64)):
        return f"lora_apply_fp8: got {y.tolist()}"
    return None


def test_fp8_golden_inputs_are_on_their_grids():
    """The fixture's weights are e4m3 values, its activations and base outputs bf16
    values, and its converted rows are what the input conversion gives."""
    g = _load("fp8_case.json")
    for w in (g["adapter"]["A"], g["adapter"]["B"]):
        v = np.array(w, dtype=np.float64)
        assert np.array_equal(O.fp8_e4m3_decode(O.fp8_e4m3_encode(v)), v)
    for a in (g["x"], g["y_base"]):
        v = np.array(a, dtype=np.float64)
        assert np.array_equal(O.bf16_bits_to_f64(O.f32_to_bf16_bits(v.astype(np.float32))), v)
    conv = O.fp8_quantize(np.array(g["x"], dtype=np.float64))
    assert np.array_equal(conv[:2], np.array(g["x_converted"]["rows"], dtype=np.float64))


def test_fp8_golden():
    """The FP8 path's composition on a hand-worked case (tests/golden/fp8_case.json):
    activations past +-448, between grid points, at ties and in the subnormal range,
    integer e4m3 weights, an off-grid bf16 base output and a no-LoRA token."""
    assert check_fp8_golden() is None


def _fp8_no_conversion(x):
    return np.asarray(x, dtype=np.float64)


def _fp8_clamp_only(x):
    return np.clip(np.asarray(x, dtype=np.float64), -O.FP8_MAX, O.FP8_MAX)


def _fp8_round_without_clamp(x):
    # a conversion without the clamp: magnitudes past the largest finite value are
    # not e4m3 numbers (NaN in the "fn" format)
    x = np.asarray(x, dtype=np.float64)
    r = O.fp8_e4m3_decode(O.fp8_e4m3_encode(np.clip(x, -O.FP8_MAX, O.FP8_MAX)))
    return np.where(np.abs(x) > O.FP8_MAX, np.nan, r)


def _fp8_round_toward_zero(x):
    # truncation instead of round-to-nearest-even
    x = np.clip(np.asarray(x, dtype=np.float64), -O.FP8_MAX, O.FP8_MAX)
    grid = np.unique(O.fp8_e4m3_decode(np.arange(0, 0x7F)))
    mag = np.array([grid[grid <= abs(v)].max() for v in x.ravel()]).reshape(x.shape)
    return np.sign(x) * mag


@pytest.mark.parametrize("mutant", [_fp8_no_conversion, _fp8_clamp_only, _fp8_round_without_clamp,
                                    _fp8_round_toward_zero], ids=lambda f: f.__name__)
def test_fp8_planted_conversion_mistakes_fail_the_golden(monkeypatch, mutant):
    monkeypatch.setattr(O, "fp8_quantize", mutant)
    assert check_fp8_golden() is not None


def test_fp8_planted_base_conversion_fails_the_golden(monkeypatch):
    """Converting the base output to FP8 as well (the page converts only the input)."""
    real = O.lora_apply

    def converting_base(x, y_base, *a, **k):
        return real(x, O.fp8_quantize(y_base), *a, **k)

    monkeypatch.setattr(O, "lora_apply", converting_base)
    assert check_fp8_golden() is not None


def test_fp8_planted_dropped_scale_fails_the_golden(monkeypatch):
    monkeypatch.setattr(O.Adapter, "scale", lambda self: np.float32(1.0))
    assert check_fp8_golden() is not None
