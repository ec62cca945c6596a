"""HIP path against the fp64 oracle, through the C ABI, on an MI355X.

Every test puts a seeded synthetic workload on the GPU with NaN in all pages
that are not adapter rows of the batch, runs slora_lora_delta and compares
with the oracle (gates G1 and G2 of tests/gates.py, or bit-exact where the
arithmetic is exact).  Routing is forced both ways where it matters: all
segments on the vector-ALU tiles, all on the MFMA tiles, and the default.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import build_from_workload, round_to, workload_delta  # noqa: E402
from rank_gemm_page_amd import slora as S  # noqa: E402
from rank_gemm_page_amd.device_workload import DeviceWorkload  # noqa: E402
from synth import CONFIGS, generate, small_spec  # noqa: E402
from tests.gates import check_gates  # noqa: E402

pytestmark = pytest.mark.gpu

ROUTES = {"gemv": {S.SLORA_TUNE_MFMA_MIN_TOKENS: 1 << 30},
          "mfma": {S.SLORA_TUNE_MFMA_MIN_TOKENS: 1},
          "mfma_cols_1024": {S.SLORA_TUNE_MFMA_MIN_TOKENS: 1, S.SLORA_TUNE_MFMA_EXPAND_COLS: 1024},
          "default": {}}
LAUNCH = {"fused": {S.SLORA_TUNE_FUSED: 1}, "two": {S.SLORA_TUNE_FUSED: 0}}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.lib()


def run_gpu(w, route="default", tuning=None, projs=None, free_order=None, launch="fused"):
    if free_order is not None:
        w.free_order = free_order
    t = dict(ROUTES[route])
    t.update(LAUNCH[launch])
    t.update(tuning or {})
    print(f"[gpu] {w.spec.name} seed={w.seed} route={route} T={w.T}", flush=True)
    dw = DeviceWorkload(w, "cuda:0", tuning=t)
    try:
        out = []
        for p in projs if projs is not None else range(w.spec.n_proj):
            dw.delta(p)
        torch.cuda.synchronize()
        for p in projs if projs is not None else range(w.spec.n_proj):
            out.append(dw.y[p].cpu().numpy())
        assert S.slora_segments_read_error(dw.seg) == 0
        return out, dw.info
    finally:
        dw.close()


def oracle(w, proj=0, tokens=None):
    return workload_delta(build_from_workload(w), w, proj=proj, tokens=tokens)


def test_tiny_fp32():
    w = generate(CONFIGS["tiny"], 0)
    (y,), info = run_gpu(w)
    assert info["n_mfma_segments"] == 0
    y_ref, sd_ref = oracle(w)
    check_gates(y, y_ref, sd_ref, np.float32, "tiny")


SMALL = [
    small_spec("sq512", h_in=512, h_out=512, n_adapters=9, batch=("zipf", 96, 1.1),
               pool=("occ", 3, 5)),
    small_spec("nonsq", h_in=384, h_out=1288, two_classes=True, n_adapters=6,
               rank_set=(8, 16, 32, 64, 128), batch=("zipf", 80, 1.0), pool=("occ", 4, 5)),
    small_spec("proj3", h_in=256, h_out=256, n_adapters=5, n_proj=3, proj_x=(0, 0, 1),
               batch=("mixed", 2, 40, 17)),
    small_spec("ragged", h_in=136, h_out=200, two_classes=True, n_adapters=4,
               rank_set=(1, 3, 13, 40), batch=("zipf", 50, 1.0)),
    small_spec("scales", h_in=1024, h_out=1024, n_adapters=7, scale_set=(0.5, 1.0, 2.0, 4.0, 0.3),
               batch=("requests", 5, 3, 40)),
    small_spec("f32big", dtype="f32", h_in=2048, h_out=1024, two_classes=True, n_adapters=5,
               rank_set=(4, 16, 64), batch=("zipf", 40, 1.1)),
    # four 16-byte chunks a thread: one-token blocks take the 8-row shrink
    # shape (rank tails of 1 to 7 rows, rows past the tile's end clamped)
    small_spec("f32w", dtype="f32", h_in=3000, h_out=520, two_classes=True, n_adapters=40,
               rank_set=(1, 5, 8, 12, 24), batch=("zipf", 48, 0.7)),
    small_spec("f16w", h_in=6000, h_out=264, two_classes=True, n_adapters=40,
               rank_set=(3, 8, 9, 16, 40), batch=("zipf", 48, 0.7)),
]


@pytest.mark.parametrize("spec", SMALL, ids=lambda s: s.name)
@pytest.mark.parametrize("route", list(ROUTES))
@pytest.mark.parametrize("launch", list(LAUNCH))
def test_small_shapes(spec, route, launch):
    w = generate(spec, 1)
    ys, info = run_gpu(w, route, launch=launch)
    if route.startswith("mfma") and spec.dtype == "f16" and spec.h_in % 32 == 0:
        assert info["n_mfma_segments"] == info["n_segments"]
    for p, y in enumerate(ys):
        y_ref, sd_ref = oracle(w, p)
        check_gates(y, y_ref, sd_ref, w.np_dtype, f"{spec.name}/{route}/p{p}")


@pytest.mark.parametrize("dtype,h,ranks", [("f32", 256, (1, 4, 8)), ("f16", 128, (1, 2, 4)),
                                           ("f16", 256, (3, 8))])
@pytest.mark.parametrize("route", ["gemv", "mfma"])
def test_integer_inputs_bit_exact(dtype, h, ranks, route):
    """{-1,0,1} inputs, s = 2: every partial sum is an integer below 2^24, so the
    fp32 sum is exact whatever its order and the one rounding of y to the output
    type matches the oracle's rounding of its exact result bit for bit (for fp16
    with h = 256 and r = 8, |y| reaches 4097, where that rounding is not trivial)."""
    spec = small_spec("int", dtype=dtype, h_in=h, h_out=h, n_adapters=5, rank_set=ranks,
                      values="ternary", scale=2.0, batch=("zipf", 40, 1.0))
    w = generate(spec, 7)
    (y,), _ = run_gpu(w, route)
    y_ref, _ = oracle(w)
    assert np.array_equal(np.round(y_ref), y_ref)
    np.testing.assert_array_equal(y, round_to(y_ref, w.np_dtype))


def test_page_permutation_invariance_bit_exact():
    spec = small_spec("perm", h_in=512, h_out=512, n_adapters=8, batch=("zipf", 64, 1.1),
                      pool=("occ", 3, 5))
    outs = []
    for k in range(2):
        w = generate(spec, 2)
        rng = np.random.default_rng(100 + k)
        fo = [rng.permutation(P).astype(np.int32) for P in w.n_pages]
        (y,), _ = run_gpu(w, "default", tuning={S.SLORA_TUNE_MFMA_MIN_TOKENS: 8}, free_order=fo)
        outs.append(y)
    assert np.array_equal(outs[0].view(np.uint16), outs[1].view(np.uint16))


@pytest.mark.parametrize("launch", list(LAUNCH))
def test_xcd_placement_and_rank_order_change_nothing(launch):
    """Grouping the shrink tiles by XCD, or clustering tiles by rank, reorders
    the launch, never the arithmetic of a tile: results are bit-identical to
    the default order."""
    spec = small_spec("xcd", h_in=1024, h_out=768, two_classes=True, n_adapters=12,
                      batch=("zipf", 96, 1.1), pool=("occ", 1, 2))
    outs = []
    for xcds, order in ((1, 0), (8, 0), (3, 0), (1, 1), (8, 1), (1, 2)):
        w = generate(spec, 4)
        (y,), _ = run_gpu(w, "default", launch=launch,
                          tuning={S.SLORA_TUNE_MFMA_MIN_TOKENS: 8, S.SLORA_TUNE_XCDS: xcds,
                                  S.SLORA_TUNE_TILE_ORDER: order})
        outs.append(y)
    y_ref, sd_ref = oracle(w)
    check_gates(outs[0], y_ref, sd_ref, w.np_dtype, "xcd")
    assert all(np.array_equal(outs[0].view(np.uint16), o.view(np.uint16)) for o in outs[1:])


def test_epoch_wrap_clears_the_pairs_and_starts_again():
    """Fused launches across the epoch counter's end (2^31 - 1 launches since
    the upload): the launch past it clears the exchange pairs and takes epoch 1
    again.  K-split partials carry the epoch with bit 31 set, so the last
    epochs tag them 0xFFFFFFFF.  Every launch gives the bits of the upload's
    first launch, alone and with four projections in one launch, and no wait
    gives up."""
    spec = small_spec("wrap", h_in=1024, h_out=512, two_classes=True, n_adapters=6, n_proj=2,
                      proj_x=(0, 0), batch=("mixed", 2, 70, 20))
    w = generate(spec, 2)
    dw = DeviceWorkload(w, "cuda:0", tuning={S.SLORA_TUNE_MFMA_MIN_TOKENS: 16})
    try:
        assert dw.info["n_mfma_segments"] > 0
        dw.delta(0)
        dw.delta(1)
        torch.cuda.synchronize()
        ref = [dw.y[p].cpu().numpy().view(np.uint16) for p in range(2)]
        with pytest.raises(S.SloraError):
            S.slora_segments_set_launch_count(dw.seg, 1)          # backwards: refused
        S.slora_segments_set_launch_count(dw.seg, 0x7FFFFFFD)
        # k = 0: epochs 2^31 - 2 and 2^31 - 1; k = 1 (both projections in one
        # launch): the pairs cleared, epoch 1; then epochs 2 and 3, and 4
        for k in range(4):
            dw.reset_y()
            if k % 2:
                dw.delta_multi()
            else:
                dw.delta(0)
                dw.delta(1)
            torch.cuda.synchronize()
            for p in range(2):
                np.testing.assert_array_equal(dw.y[p].cpu().numpy().view(np.uint16), ref[p],
                                              err_msg=f"launch {k} p{p}")
        assert S.slora_segments_read_error(dw.seg) == 0
    finally:
        dw.close()


@pytest.mark.parametrize("route", ["gemv", "mfma"])
def test_deterministic_run_to_run(route):
    """Same result bit for bit from repeated fused launches on one upload (epochs
    1, 2, 3, ...), after a re-upload (epoch reset), from two launches and from
    the two stage entry points."""
    spec = small_spec("det", h_in=1024, h_out=1024, n_adapters=6, batch=("zipf", 70, 1.0))
    w = generate(spec, 3)
    dw = DeviceWorkload(w, "cuda:0", tuning=ROUTES[route])
    try:
        res = []

        def run(fn):
            dw.reset_y()
            fn()
            torch.cuda.synchronize()
            res.append(dw.y[0].cpu().numpy().view(np.uint16).copy())

        for _ in range(3):
            run(lambda: dw.delta(0))
        dw.upload()
        run(lambda: dw.delta(0))
        run(lambda: (dw.shrink(0), dw.expand(0)))
        S.slora_pool_set_tuning(dw.pool, S.SLORA_TUNE_FUSED, 0)
        run(lambda: dw.delta(0))
        assert S.slora_segments_read_error(dw.seg) == 0
        assert all(np.array_equal(res[0], r) for r in res[1:])
    finally:
        dw.close()


@pytest.mark.parametrize("what", ["zero_B", "zero_scale"])
@pytest.mark.parametrize("route", ["gemv", "mfma"])
def test_no_op_leaves_y_unchanged(what, route):
    spec = small_spec("noop", h_in=256, h_out=512, two_classes=True, n_adapters=4,
                      batch=("zipf", 40, 1.0), scale=0.0 if what == "zero_scale" else 2.0)
    w = generate(spec, 4)
    if what == "zero_B":
        for a in range(spec.n_adapters):
            A, B = w.weights(a)
            w._wcache[(a, 0)] = (A, np.zeros_like(B))
    (y,), _ = run_gpu(w, route)
    np.testing.assert_array_equal(y.astype(np.float64), w.y[0].astype(np.float64))


def test_negative_ids_leave_rows_untouched():
    spec = small_spec("neg", h_in=256, h_out=256, n_adapters=3, batch=("zipf", 40, 1.0))
    w = generate(spec, 5)
    w.ids = w.ids.copy()
    w.ids[::3] = -1
    (y,), _ = run_gpu(w, "default", tuning={S.SLORA_TUNE_MFMA_MIN_TOKENS: 4})
    y_ref, sd_ref = oracle(w)
    check_gates(y, y_ref, sd_ref, np.float16, "neg")
    assert np.array_equal(y[::3].view(np.uint16), w.y[0][::3].view(np.uint16))


def test_unload_reload_same_result_other_pages():
    spec = small_spec("reload", h_in=512, h_out=512, n_adapters=5, batch=("zipf", 50, 1.0),
                      pool=("occ", 1, 2))
    w = generate(spec, 6)
    dw = DeviceWorkload(w, "cuda:0", tuning={S.SLORA_TUNE_MFMA_MIN_TOKENS: 8})
    try:
        dw.delta(0)
        torch.cuda.synchronize()
        y1 = dw.y[0].cpu().numpy().copy()
        a = int(w.ids[0])
        before = S.slora_adapter_pages(dw.pool, a)
        # a stale batch is refused, then the adapter comes back on other pages:
        # the KV pages go back to the free list first, so FIFO hands them out next
        S.slora_free_pages(dw.pool, 0, dw.kv[0])
        S.slora_unload_adapter(dw.pool, a)
        with pytest.raises(S.SloraError) as e:
            dw.delta(0)
        assert e.value.status == S.SLORA_E_STALE
        A, B = w.weights(a)
        S.slora_load_adapter(dw.pool, a, int(w.ranks[a]), float(w.scales[a]), [A], [B],
                             torch.cuda.current_stream())
        after = S.slora_adapter_pages(dw.pool, a)
        assert set(before[0].tolist()).isdisjoint(after[0].tolist())
        dw.build(w.ids)
        dw.reset_y()
        dw.delta(0)
        torch.cuda.synchronize()
        y2 = dw.y[0].cpu().numpy()
        assert np.array_equal(y1.view(np.uint16), y2.view(np.uint16))
    finally:
        dw.close()


def test_pool_bytes_match_oracle_image():
    """The loader put every A^T and B row on its page, bit for bit."""
    spec = small_spec("img", h_in=264, h_out=136, two_classes=True, n_adapters=4,
                      rank_set=(1, 5, 9), batch=("uniform", 10))
    w = generate(spec, 8)
    dw = DeviceWorkload(w, "cuda:0")
    try:
        st = build_from_workload(w)
        pages = [p.cpu().numpy() for p in dw.pages]
        for (cls, pg), row in st.image.rows.items():
            assert np.array_equal(pages[cls][pg].view(np.uint16), row.view(np.uint16))
        n_written = len(st.image.rows)
        n_nan = sum(int(np.isnan(p).all(axis=1).sum()) for p in pages)
        assert n_nan == sum(w.n_pages) - n_written
    finally:
        dw.close()


# ---------------------------------------------------------------------------
# The library's maximum sizes: h_in 16384 (fp16) and 8192 (fp32), the widest
# vector-ALU shrink geometry (8 chunks per thread), h_out 65536, rank 256 and
# 8 projections; sampled tokens against the oracle.

MAX_SPECS = [
    small_spec("max_f16", h_in=16384, h_out=65536, two_classes=True, n_adapters=6, n_proj=2,
               proj_x=(0, 0), rank_set=(1, 17, 128, 256), batch=("zipf", 72, 1.0)),
    small_spec("max_f32", dtype="f32", h_in=8192, h_out=8192, n_adapters=5, n_proj=8,
               proj_x=(0,) * 8, rank_set=(3, 64, 256), batch=("zipf", 30, 1.0)),
]


@pytest.mark.parametrize("spec", MAX_SPECS, ids=lambda s: s.name)
@pytest.mark.parametrize("route", ["default", "mfma"])
def test_maximum_sizes(spec, route):
    w = generate(spec, 4)
    assert int(w.ranks.max()) == 256
    ys, info = run_gpu(w, route)
    st = build_from_workload(w)
    toks = sample_tokens(w, 10)
    for p in (0, spec.n_proj - 1):
        y_ref, sd_ref = workload_delta(st, w, p, tokens=toks)
        check_gates(ys[p][toks], y_ref, sd_ref, w.np_dtype, f"{spec.name}/{route}/p{p}")


# ---------------------------------------------------------------------------
# The five benchmark shapes at full size, default routing (as bench.py runs them)


def sample_tokens(w, n, seed=0):
    rng = np.random.default_rng(seed)
    ids = w.ids
    # the first and last token of every segment boundary region, plus random ones
    order = np.argsort(ids, kind="stable")
    picks = set(order[:4].tolist()) | set(order[-4:].tolist())
    picks |= set(rng.choice(w.T, size=min(n, w.T), replace=False).tolist())
    return sorted(picks)


@pytest.mark.parametrize("name", ["decode7b", "prefill7b", "mixed13b", "mlp70b"])
def test_full_size_config(name):
    """Every token of every projection of the benchmark batches against the oracle."""
    full_size_parity(name, 0)


# Other draws of the same workloads (other batches, ranks and page layouts):
# seeds 1-4 of decode, 1-2 of the others.
@pytest.mark.parametrize("name,seed", [("decode7b", 1), ("decode7b", 2), ("decode7b", 3), ("decode7b", 4),
                                       ("mlp70b", 1), ("mlp70b", 2), ("prefill7b", 1), ("prefill7b", 2),
                                       ("mixed13b", 1), ("mixed13b", 2)])
def test_full_size_other_seeds(name, seed):
    full_size_parity(name, seed)


def full_size_parity(name, seed):
    w = generate(CONFIGS[name], seed)
    ys, info = run_gpu(w, "default")
    print(f"[gpu] {name}/seed{seed}: segments={info['n_segments']} mfma_segments={info['n_mfma_segments']} "
          f"shrink_tiles={info['n_shrink_tiles']} expand_tiles={info['n_expand_tiles']}", flush=True)
    st = build_from_workload(w)
    for p, y in enumerate(ys):
        y_ref, sd_ref = workload_delta(st, w, proj=p)
        check_gates(y, y_ref, sd_ref, np.float16, f"{name}/seed{seed}/p{p}")
        print(f"[gpu] {name}/seed{seed}/p{p}: all {w.T} tokens within the gates", flush=True)
