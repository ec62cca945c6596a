"""Pins of the fp64 oracle against things other than itself (CPU only).

Each check is chosen so that a plausible mistake in the oracle (a dropped
term or scale, a wrong sign, a transposed factor, an off-by-one page index, a
wrong segment order) fails at least one of them; ``test_pins_catch_planted_mistakes``
plants such mistakes in copies of the oracle and shows that they do.
"""
import json
import os
from dataclasses import replace

import numpy as np
import pytest

from oracle import slora_oracle as orc
from synth import generate, small_spec

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _dense(w, a, p=0):
    A, B = w.weights(a, p)
    return A.astype(np.float64), B.astype(np.float64)


# ---------------------------------------------------------------------------
# Hand-worked fixtures


def test_hand_example_fixture():
    g = _load("hand_example.json")
    alloc = orc.AllocatorModel([len(f) for f in g["free_order"]], g["free_order"], n_proj=1,
                             two_classes=True)
    alloc.load(0, g["rank"], g["scale"])
    img = orc.PoolImage([g["h_in"], g["h_out"]], np.float32)
    img.write_adapter(alloc, 0, 0, np.array(g["A"], np.float32), np.array(g["B"], np.float32))
    e = g["expected"]
    assert alloc.table[0].a_pages[0] == e["a_pages"]
    assert alloc.table[0].b_pages[0] == e["b_pages"]
    for key, row in e["page_rows"].items():
        cls, page = map(int, key.split(","))
        np.testing.assert_array_equal(img.row(cls, page), np.array(row, np.float32))
    for cls, page in e["unwritten_pages"]:
        assert np.isnan(img.row(cls, page)).all()
    seg = orc.segment_model(g["ids"], alloc)
    for k in ("perm", "seg_start", "seg_adapter", "seg_rank", "seg_page_off"):
        assert getattr(seg, k).tolist() == e[k], k
    y, _ = orc.lora_delta(alloc, img, g["ids"], np.array(g["x"], np.float32),
                          np.array(g["y_in"], np.float32))
    np.testing.assert_array_equal(y, np.array(e["y"], np.float64))


@pytest.mark.parametrize("case", ["single_class", "two_class_two_proj"])
def test_allocator_fifo_fixture(case):
    g = _load("allocator_fifo.json")[case]
    two = len(g["n_pages"]) == 2
    alloc = orc.AllocatorModel(g["n_pages"], g["free_order"], n_proj=g["n_proj"], two_classes=two)
    for st in g["steps"]:
        if st["op"] == "load":
            e = alloc.load(st["adapter"], st["rank"], 1.0)
            assert e.a_pages == st["a_pages"] and e.b_pages == st["b_pages"]
        elif st["op"] == "load_fail":
            with pytest.raises(orc.OracleError):
                alloc.load(st["adapter"], st["rank"], 1.0)
            assert st["adapter"] not in alloc.table
            assert [list(f) for f in alloc.free] == st["free_after"]
        elif st["op"] == "unload":
            alloc.unload(st["adapter"])
            assert [list(f) for f in alloc.free] == st["free_after"]
        elif st["op"] == "kv":
            assert alloc.alloc(st["cls"], st["n"]) == st["pages"]
        elif st["op"] == "kv_fail":
            with pytest.raises(orc.OracleError):
                alloc.alloc(st["cls"], st["n"])
            assert [list(f) for f in alloc.free] == st["free_after"]


# ---------------------------------------------------------------------------
# Closed form x(W + sAB) - xW, which is the delta by definition of LoRA


def closed_form_check(delta_fn, spec, seed=0, tol=1e-9):
    """True when delta_fn's s*(xA)B matches x(W + sAB) - xW for every token."""
    w = generate(spec, seed)
    st = orc.build_from_workload(w)
    rng = np.random.default_rng(1234)
    W = rng.standard_normal((spec.h_in, spec.h_out))
    ok = True
    for p in range(spec.n_proj):
        x = w.x[spec.proj_x[p]]
        _, sd = delta_fn(st.alloc, st.image, w.ids, x, w.y[p], p)
        for t in range(w.T):
            a = int(w.ids[t])
            xt = x[t].astype(np.float64)
            if a < 0:
                ref = np.zeros(spec.h_out)
            else:
                A, B = _dense(w, a, p)
                s = float(w.scales[a])
                ref = xt @ (W + s * (A @ B)) - xt @ W
            scale = max(1e-30, np.abs(ref).max())
            if not (np.abs(sd[t] - ref).max() <= tol * scale + 1e-12):
                ok = False
    return ok


def _oracle_delta(alloc, image, ids, x, y, p):
    return orc.lora_delta(alloc, image, ids, x, y, proj=p)


CLOSED_FORM_SPECS = [
    small_spec("sq", h_in=48, h_out=48, n_adapters=5, rank_set=(1, 3, 8), dtype="f32"),
    small_spec("nonsq", h_in=40, h_out=24, two_classes=True, n_adapters=4, rank_set=(2, 5, 8)),
    small_spec("proj", h_in=32, h_out=32, n_adapters=3, n_proj=3, proj_x=(0, 1, 1),
               rank_set=(2, 4)),
    small_spec("scales", h_in=64, h_out=16, two_classes=True, n_adapters=6,
               scale_set=(0.5, 1.0, 2.0, 4.0, 0.3), rank_set=(1, 7)),
]


@pytest.mark.parametrize("spec", CLOSED_FORM_SPECS, ids=lambda s: s.name)
def test_closed_form(spec):
    assert closed_form_check(_oracle_delta, spec)


def test_single_adapter_matches_dense_gemm():
    """All tokens on one adapter: y_in + s (X A) B with numpy's fp64 matmul."""
    spec = small_spec("one", h_in=64, h_out=48, two_classes=True, n_adapters=1,
                      rank_set=(8,), batch=("uniform", 20), scale=1.5)
    w = generate(spec, 3)
    st = orc.build_from_workload(w)
    y, _ = orc.workload_delta(st, w)
    A, B = _dense(w, 0)
    ref = w.y[0].astype(np.float64) + 1.5 * ((w.x[0].astype(np.float64) @ A) @ B)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


# ---------------------------------------------------------------------------
# Integer brute force: every partial sum is an integer, so the result is exact


@pytest.mark.parametrize("dtype,h,rank_set", [("f32", 256, (1, 4, 8)), ("f16", 128, (1, 2, 4))])
def test_integer_brute_force(dtype, h, rank_set):
    spec = small_spec("int", dtype=dtype, h_in=h, h_out=h, n_adapters=5, rank_set=rank_set,
                      values="ternary", scale=2.0, batch=("uniform", 12))
    w = generate(spec, 7)
    st = orc.build_from_workload(w)
    y, _ = orc.workload_delta(st, w)
    xi = w.x[0].astype(np.int64)
    for t in range(w.T):
        a = int(w.ids[t])
        A, B = (m.astype(np.int64) for m in w.weights(a))
        exact = w.y[0][t].astype(np.int64) + 2 * ((xi[t] @ A) @ B)
        assert np.array_equal(y[t], exact.astype(np.float64))
        # the exact value is representable, so one rounding to the storage type is exact too
        assert np.array_equal(orc.round_to(y[t], w.np_dtype).astype(np.int64), exact)


# ---------------------------------------------------------------------------
# The one rounding of the result to the output type (reading 6: round to
# nearest, ties to even, straight from the exact value).  Each fixture value is
# a tie or sits next to one, worked out by hand from the IEEE binary16 and
# binary32 formats: in [2048, 4096) binary16 values are 2 apart and in
# [4096, 8192) 4 apart, binary32 values in [2^24, 2^25) are 2 apart, and at a
# tie the result is the neighbour whose last significand bit is 0.

ROUND_PINS = {
    np.float16: [
        (2049.0, 2048.0),             # tie between 2048 (even) and 2050
        (2051.0, 2052.0),             # tie between 2050 and 2052 (even)
        (-2051.0, -2052.0),           # the same, negative
        (4097.0, 4096.0),             # a quarter of the way: nearest, not a tie
        (4098.0, 4096.0),             # tie between 4096 (even) and 4100
        (4102.0, 4104.0),             # tie between 4100 and 4104 (even)
        (4103.0, 4104.0),             # three quarters of the way
        (2049.0 + 2.0 ** -30, 2050.0),  # just above a tie: no detour through binary32
        (2.0 ** -25, 0.0),            # tie between 0 (even) and the least subnormal
        (3 * 2.0 ** -25, 2.0 ** -23), # tie between 2^-24 and 2^-23 (even)
        (65519.0, 65504.0),           # below the tie with 65536: the largest finite value
        (65520.0, np.inf),            # the tie rounds to even, past the largest finite value
    ],
    np.float32: [
        (16777217.0, 16777216.0),     # 2^24 + 1: tie between 2^24 (even) and 2^24 + 2
        (16777219.0, 16777220.0),     # tie between 2^24 + 2 and 2^24 + 4 (even)
        (-16777217.0, -16777216.0),
        (16777217.0 + 2.0 ** -20, 16777218.0),   # just above a tie
        (1.0 + 2.0 ** -24, 1.0),      # half an ulp above 1: tie, to 1 (even)
        (1.0 + 3 * 2.0 ** -24, 1.0 + 2.0 ** -22),  # tie between 1 + 2^-23 and 1 + 2^-22 (even)
    ],
}


def _round_pin_failures(fn):
    bad = []
    for dt, cases in ROUND_PINS.items():
        got = fn(np.array([c[0] for c in cases], np.float64), dt)
        for (val, want), g in zip(cases, np.asarray(got)):
            if not (g == want and np.asarray(g).dtype == np.dtype(dt)):
                bad.append((dt.__name__, val, want, float(g)))
    return bad


def test_round_to_ties_to_even():
    with np.errstate(over="ignore"):
        assert _round_pin_failures(orc.round_to) == []


def _truncate(y, dt):
    r = np.asarray(y, np.float64).astype(dt)
    return np.where(np.abs(r.astype(np.float64)) > np.abs(y), np.nextafter(r, dt(0)), r).astype(dt)


def _half_away(y, dt):
    r = np.asarray(y, np.float64).astype(dt)
    lo = np.where(r.astype(np.float64) > y, np.nextafter(r, dt(-np.inf)), r)
    hi = np.where(r.astype(np.float64) < y, np.nextafter(r, dt(np.inf)), r)
    dlo, dhi = y - lo.astype(np.float64), hi.astype(np.float64) - y
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (y > 0))
    return np.where(pick_hi, hi, lo).astype(dt)


def _via_f32(y, dt):
    return np.asarray(y, np.float64).astype(np.float32).astype(dt)


@pytest.mark.parametrize("planted", [_truncate, _half_away, _via_f32],
                         ids=["truncate", "ties_away", "double_rounding"])
def test_round_pins_catch_planted_roundings(planted):
    with np.errstate(over="ignore", invalid="ignore"):
        assert _round_pin_failures(planted), f"{planted.__name__} passed every rounding pin"


# ---------------------------------------------------------------------------
# Invariants


def test_page_permutation_invariance():
    """Where the pages sit in the pool does not change the result, bit for bit."""
    spec = small_spec("perm", h_in=64, h_out=64, n_adapters=6, rank_set=(2, 4, 8),
                      pool=("occ", 3, 5), batch=("uniform", 30))
    w1 = generate(spec, 11)
    w2 = generate(spec, 11)
    rng = np.random.default_rng(99)
    w2.free_order = [rng.permutation(P).astype(np.int32) for P in w2.n_pages]
    s1, s2 = orc.build_from_workload(w1), orc.build_from_workload(w2)
    a1 = sorted(p for e in s1.alloc.table.values() for p in e.a_pages[0])
    a2 = sorted(p for e in s2.alloc.table.values() for p in e.a_pages[0])
    assert a1 != a2
    y1, _ = orc.workload_delta(s1, w1)
    y2, _ = orc.workload_delta(s2, w2)
    assert np.array_equal(y1, y2)


@pytest.mark.parametrize("what", ["zero_A", "zero_B", "zero_scale"])
def test_no_op_cases(what):
    spec = small_spec("zero", h_in=32, h_out=48, two_classes=True, n_adapters=3,
                      rank_set=(2, 8), scale=0.0 if what == "zero_scale" else 2.0)
    w = generate(spec, 5)
    st = orc.build_from_workload(w, load_weights=False)
    for a in range(spec.n_adapters):
        A, B = w.weights(a)
        if what == "zero_A":
            A = np.zeros_like(A)
        if what == "zero_B":
            B = np.zeros_like(B)
        st.image.write_adapter(st.alloc, a, 0, A, B)
    y, _ = orc.workload_delta(st, w)
    assert np.array_equal(y, w.y[0].astype(np.float64))


def test_rank_padding_invariance():
    """Zero columns appended to A and zero rows to B leave the delta unchanged."""
    spec = small_spec("pad", h_in=48, h_out=48, n_adapters=2, fixed_ranks=(3, 5),
                      batch=("uniform", 10), dtype="f32")
    w = generate(spec, 2)
    st = orc.build_from_workload(w)
    _, sd = orc.workload_delta(st, w)
    alloc = orc.AllocatorModel([64], [None])
    img = orc.PoolImage([48], np.float32)
    for a in range(2):
        A, B = w.weights(a)
        r = A.shape[1]
        alloc.load(a, r + 4, float(w.scales[a]))
        img.write_adapter(alloc, a, 0, np.hstack([A, np.zeros((48, 4), np.float32)]),
                          np.vstack([B, np.zeros((4, 48), np.float32)]))
    _, sd_pad = orc.lora_delta(alloc, img, w.ids, w.x[0], w.y[0])
    np.testing.assert_allclose(sd_pad, sd, rtol=1e-12, atol=1e-14)


def test_token_permutation_equivariance():
    spec = small_spec("tokperm", h_in=32, h_out=32, n_adapters=4, batch=("uniform", 17))
    w = generate(spec, 4)
    st = orc.build_from_workload(w)
    y, _ = orc.workload_delta(st, w)
    q = np.random.default_rng(5).permutation(w.T)
    yq, _ = orc.lora_delta(st.alloc, st.image, w.ids[q], w.x[0][q], w.y[0][q])
    assert np.array_equal(yq, y[q])


def test_linearity_in_x_and_scale():
    spec = small_spec("lin", h_in=32, h_out=24, two_classes=True, n_adapters=3, rank_set=(4,),
                      dtype="f32")
    w = generate(spec, 8)
    st = orc.build_from_workload(w)
    rng = np.random.default_rng(3)
    x1 = rng.standard_normal((w.T, 32))
    x2 = rng.standard_normal((w.T, 32))
    zero = np.zeros((w.T, 24))
    _, d1 = orc.lora_delta(st.alloc, st.image, w.ids, x1, zero)
    _, d2 = orc.lora_delta(st.alloc, st.image, w.ids, x2, zero)
    _, d12 = orc.lora_delta(st.alloc, st.image, w.ids, x1 + x2, zero)
    np.testing.assert_allclose(d12, d1 + d2, rtol=1e-12, atol=1e-12 * np.abs(d12).max())
    for a in st.alloc.table:
        st.alloc.table[a].scale *= 3.0
    _, d3 = orc.lora_delta(st.alloc, st.image, w.ids, x1, zero)
    np.testing.assert_allclose(d3, 3.0 * d1, rtol=1e-12, atol=1e-14)


def test_negative_id_means_no_adapter():
    spec = small_spec("neg", h_in=16, h_out=16, n_adapters=2, rank_set=(2,),
                      batch=("explicit", (1, -1, 0, -1, 1)))
    w = generate(spec, 0)
    st = orc.build_from_workload(w)
    y, sd = orc.workload_delta(st, w)
    for t in (1, 3):
        assert np.array_equal(y[t], w.y[0][t].astype(np.float64))
        assert not sd[t].any()
    seg = orc.segment_model(w.ids, st.alloc)
    assert seg.perm.tolist() == [2, 0, 4]


# ---------------------------------------------------------------------------
# Segment model: brute force over the definition, with plain loops


@pytest.mark.parametrize("seed", range(4))
def test_segment_model_brute_force(seed):
    spec = small_spec("seg", h_in=16, h_out=16, n_adapters=9, rank_set=(1, 2, 3, 5),
                      n_proj=2, proj_x=(0, 0), batch=("zipf", 40, 1.1))
    w = generate(spec, seed)
    ids = w.ids.copy()
    ids[::7] = -1
    st = orc.build_from_workload(w, load_weights=False)
    seg = orc.segment_model(ids, st.alloc)
    # expected order: adapters ascending, tokens ascending within an adapter
    pairs = sorted((int(a), t) for t, a in enumerate(ids) if a >= 0)
    assert seg.perm.tolist() == [t for _, t in pairs]
    adapters = []
    for a, _ in pairs:
        if not adapters or adapters[-1] != a:
            adapters.append(a)
    assert seg.seg_adapter.tolist() == adapters
    starts, i = [], 0
    for a in adapters:
        starts.append(i)
        while i < len(pairs) and pairs[i][0] == a:
            i += 1
    assert seg.seg_start.tolist() == starts + [len(pairs)]
    off = 0
    sum_r = sum(st.alloc.table[a].rank for a in adapters)
    for s, a in enumerate(adapters):
        e = st.alloc.table[a]
        assert seg.seg_rank[s] == e.rank and seg.seg_page_off[s] == off
        assert seg.seg_scale[s] == np.float32(e.scale)
        for p in range(2):
            base = p * sum_r + off
            assert seg.a_pages[base:base + e.rank].tolist() == e.a_pages[p]
            assert seg.b_pages[base:base + e.rank].tolist() == e.b_pages[p]
        off += e.rank
    assert seg.seg_page_off[-1] == sum_r


def test_segment_model_rejects_unloaded_adapter():
    alloc = orc.AllocatorModel([8], [None])
    alloc.load(0, 1, 1.0)
    with pytest.raises(orc.OracleError):
        orc.segment_model([0, 1], alloc)


# ---------------------------------------------------------------------------
# Allocator invariants on the real workload shapes (page sets only; no weights)


@pytest.mark.parametrize("name", ["tiny", "decode7b", "prefill7b"])
def test_allocator_invariants_on_workloads(name):
    from synth import CONFIGS
    w = generate(CONFIGS[name], 0)
    st = orc.build_from_workload(w, load_weights=False)
    seen = set()
    for c, pages in enumerate(st.kv_pages):
        for p in pages:
            assert 0 <= p < w.n_pages[c]
            seen.add((c, p))
    for a, e in st.alloc.table.items():
        assert e.rank == w.ranks[a]
        for p in range(w.spec.n_proj):
            assert len(e.a_pages[p]) == e.rank and len(e.b_pages[p]) == e.rank
            for pg in e.a_pages[p]:
                assert (0, pg) not in seen
                seen.add((0, pg))
            for pg in e.b_pages[p]:
                key = (st.alloc.b_class(), pg)
                assert key not in seen
                seen.add(key)
    used = sum(len(f) for f in st.alloc.free) + len(seen)
    assert used == sum(w.n_pages)


# ---------------------------------------------------------------------------
# The pins have teeth: plant mistakes in copies of the oracle and watch them fail


def _mutant(kind):
    def fn(alloc, image, ids, x, y, p):
        real_row = image.row
        if kind == "page_off_by_one":
            image.row = lambda cls, page: real_row(cls, page + 1)
        try:
            y_ref, sd = orc.lora_delta(alloc, image, ids, x, y, proj=p)
        finally:
            image.row = real_row
        if kind == "dropped_scale":
            for t, a in enumerate(ids):
                if a >= 0 and alloc.table[int(a)].scale != 0:
                    sd[t] = sd[t] / alloc.table[int(a)].scale
        if kind == "wrong_sign":
            sd = -sd
        if kind == "a_for_b":
            # use the A^T pages where the B pages belong (square shapes only)
            saved = {a: e.b_pages for a, e in alloc.table.items()}
            for e in alloc.table.values():
                e.b_pages = e.a_pages
            try:
                _, sd = orc.lora_delta(alloc, image, ids, x, y, proj=p)
            finally:
                for a, e in alloc.table.items():
                    e.b_pages = saved[a]
        if kind == "wrong_projection":
            _, sd = orc.lora_delta(alloc, image, ids, x, y, proj=(p + 1) % alloc.n_proj)
        return y_ref, sd
    return fn


@pytest.mark.parametrize("kind,spec_i", [("page_off_by_one", 0), ("dropped_scale", 0),
                                         ("wrong_sign", 1), ("a_for_b", 0),
                                         ("wrong_projection", 2)])
def test_pins_catch_planted_mistakes(kind, spec_i):
    spec = CLOSED_FORM_SPECS[spec_i]
    if kind == "page_off_by_one":
        spec = replace(spec, pool=("fixed", 4096))
    with np.errstate(invalid="ignore"):
        assert not closed_form_check(_mutant(kind), spec)


# ---------------------------------------------------------------------------
# The base-plus-delta product (lora_forward)


def test_forward_hand_fixture():
    g = _load("hand_example.json")
    f = _load("hand_forward.json")
    alloc = orc.AllocatorModel([len(o) for o in g["free_order"]], g["free_order"], n_proj=1,
                               two_classes=True)
    alloc.load(0, g["rank"], g["scale"])
    img = orc.PoolImage([g["h_in"], g["h_out"]], np.float32)
    img.write_adapter(alloc, 0, 0, np.array(g["A"], np.float32), np.array(g["B"], np.float32))
    h, sd = orc.lora_forward(alloc, img, g["ids"], np.array(g["x"], np.float32),
                             np.array(f["W"], np.float32))
    np.testing.assert_array_equal(h, np.array(f["expected_h"], np.float64))
    np.testing.assert_array_equal(sd[1], [0.0, 0.0])


@pytest.mark.parametrize("dtype,h_in,h_out,rank_set", [("f32", 256, 128, (1, 4, 8)),
                                                       ("f16", 64, 128, (1, 2, 4))])
def test_forward_integer_brute_force(dtype, h_in, h_out, rank_set):
    """{-1, 0, 1} inputs: x W + 2 (x A) B is an integer computed exactly in int64."""
    spec = small_spec("fint", dtype=dtype, h_in=h_in, h_out=h_out, two_classes=True, n_adapters=5,
                      rank_set=rank_set, values="ternary", scale=2.0, batch=("uniform", 12))
    w = generate(spec, 3)
    st = orc.build_from_workload(w)
    h, _ = orc.workload_forward(st, w)
    xi = w.x[0].astype(np.int64)
    Wi = w.base_weight(0).astype(np.int64)
    assert np.abs(Wi).max() == 1
    for t in range(w.T):
        A, B = (m.astype(np.int64) for m in w.weights(int(w.ids[t])))
        exact = xi[t] @ Wi + 2 * ((xi[t] @ A) @ B)
        assert np.array_equal(h[t], exact.astype(np.float64))


@pytest.mark.parametrize("shape", [(64, 64, 1), (48, 80, 2), (96, 32, 3)])
def test_forward_closed_form_combined_weight(shape):
    """Each token's output equals x (W + s A B): one dense product with the
    merged weight, the form the pages contrast with keeping the delta apart."""
    h_in, h_out, n_proj = shape
    spec = small_spec("fcf", h_in=h_in, h_out=h_out, two_classes=h_in != h_out, n_proj=n_proj,
                      proj_x=tuple(range(n_proj)), n_adapters=4, rank_set=(1, 3, 8),
                      scale_set=(0.5, 2.0, -1.5), batch=("uniform", 10))
    w = generate(spec, 1)
    st = orc.build_from_workload(w)
    for p in range(n_proj):
        h, _ = orc.workload_forward(st, w, proj=p)
        x = w.x[p].astype(np.float64)
        W = w.base_weight(p).astype(np.float64)
        for t in range(w.T):
            a = int(w.ids[t])
            A, B = _dense(w, a, p)
            merged = W + np.float64(w.scales[a]) * (A @ B)
            ref = x[t] @ merged
            np.testing.assert_allclose(h[t], ref, rtol=0, atol=1e-12 * max(1.0, np.abs(ref).max()))


def test_forward_zero_base_is_the_delta():
    """With W = 0 the forward output is the adapter output of lora_delta over a
    zero base y, token for token; a negative id gives x W."""
    spec = small_spec("fz", h_in=64, h_out=64, n_adapters=3, rank_set=(2, 5), batch=("uniform", 9))
    w = generate(spec, 2)
    st = orc.build_from_workload(w)
    ids = w.ids.copy()
    ids[4] = -1
    x = w.x[0]
    zero_w = np.zeros((64, 64), np.float16)
    h, sd = orc.lora_forward(st.alloc, st.image, ids, x, zero_w)
    y0 = np.zeros((w.T, 64), np.float16)
    y_d, sd_d = orc.lora_delta(st.alloc, st.image, ids, x, y0)
    np.testing.assert_array_equal(h, y_d)
    np.testing.assert_array_equal(sd, sd_d)
    assert not h[4].any()


def _forward_mutant(kind):
    def f(alloc, image, ids, x, W, proj=0, tokens=None):
        if kind == "dropped_base":
            return orc.lora_forward(alloc, image, ids, x, np.zeros_like(W), proj, tokens)
        if kind == "transposed_base":
            return orc.lora_forward(alloc, image, ids, x, W.T.copy(), proj, tokens)
        if kind == "base_twice":
            h, sd = orc.lora_forward(alloc, image, ids, x, W, proj, tokens)
            return 2 * h - sd, sd
        raise ValueError(kind)
    return f


@pytest.mark.parametrize("kind", ["dropped_base", "transposed_base", "base_twice"])
def test_forward_pins_catch_planted_mistakes(kind):
    spec = small_spec("fm", h_in=64, h_out=64, n_adapters=4, rank_set=(1, 3, 8), batch=("uniform", 10))
    w = generate(spec, 1)
    st = orc.build_from_workload(w)
    h, _ = _forward_mutant(kind)(st.alloc, st.image, w.ids, w.x[0], w.base_weight(0))
    x = w.x[0].astype(np.float64)
    W = w.base_weight(0).astype(np.float64)
    bad = False
    for t in range(w.T):
        a = int(w.ids[t])
        A, B = _dense(w, a)
        ref = x[t] @ (W + np.float64(w.scales[a]) * (A @ B))
        bad |= not np.allclose(h[t], ref, rtol=0, atol=1e-12 * max(1.0, np.abs(ref).max()))
    assert bad, f"the closed form did not catch {kind}"
