"""Asynchronous adapter fetch on an MI355X, through the C ABI.

A batch of adapters goes to the device as one copy-engine transfer per packed
pinned image into device staging and one scatter launch, all queued on a
stream (slora_load_adapters_async).  The pages it
fills must equal the oracle's page image bit for bit, the page ids must follow
the oracle's FIFO allocator model, and a delta that runs while other adapters
are being fetched on a second stream must still meet the value gates.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import build_from_workload, lora_delta, workload_delta  # noqa: E402
from rank_gemm_page_amd import slora as S  # noqa: E402
from rank_gemm_page_amd.device_workload import DeviceWorkload  # noqa: E402
from synth import generate, small_spec  # noqa: E402
from tests.gates import check_gates  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.lib()


def uint_view(a):
    return a.view(np.uint16 if a.dtype.itemsize == 2 else np.uint32)


def assert_pool_is_oracle_image(dw, st):
    pages = [p.cpu().numpy() for p in dw.pages]
    for (cls, pg), row in st.image.rows.items():
        assert np.array_equal(uint_view(pages[cls][pg]), uint_view(row)), (cls, pg)
    n_nan = sum(int(np.isnan(p).all(axis=1).sum()) for p in pages)
    assert n_nan == sum(dw.w.n_pages) - len(st.image.rows)


@pytest.mark.parametrize("kw", [
    dict(dtype="f32", h_in=264, h_out=264, rank_set=(1, 5, 9)),
    dict(dtype="f16", h_in=264, h_out=136, two_classes=True, n_proj=2, proj_x=(0, 0),
         rank_set=(1, 5, 9, 64)),
], ids=["f32", "f16_two_class"])
def test_async_load_pages_match_oracle(kw):
    spec = small_spec("async_img", n_adapters=6, batch=("uniform", 12), **kw)
    w = generate(spec, 11)
    print(f"[gpu] async pages {spec.dtype} n_proj={spec.n_proj}", flush=True)
    dw = DeviceWorkload(w, "cuda:0", load="async")
    try:
        torch.cuda.synchronize()
        st = build_from_workload(w)
        for a in range(spec.n_adapters):
            for p in range(spec.n_proj):
                pa, pb = S.slora_adapter_pages(dw.pool, a, p)
                assert pa.tolist() == list(st.alloc.table[a].a_pages[p])
                assert pb.tolist() == list(st.alloc.table[a].b_pages[p])
        assert_pool_is_oracle_image(dw, st)
    finally:
        dw.close()


@pytest.mark.parametrize("route", ["gemv", "mfma"])
def test_async_load_then_delta_on_one_stream(route):
    """Loads and the delta queued on one stream with no synchronisation between
    them: stream order alone makes the delta see the fetched rows."""
    spec = small_spec("async_delta", h_in=512, h_out=768, two_classes=True, n_adapters=7,
                      rank_set=(4, 16, 64), batch=("zipf", 150, 1.0))
    w = generate(spec, 12)
    tune = {S.SLORA_TUNE_MFMA_MIN_TOKENS: 1 if route == "mfma" else 1 << 30}
    print(f"[gpu] async then delta route={route}", flush=True)
    dw = DeviceWorkload(w, "cuda:0", tuning=tune, load="async")
    try:
        # reload every batch adapter on the current stream, then run the delta
        cur = torch.cuda.current_stream()
        torch.cuda.synchronize()
        st = build_from_workload(w)
        for a in sorted(set(int(i) for i in w.ids if i >= 0)):
            S.slora_unload_adapter(dw.pool, a)
            st.alloc.unload(a)
        batch = sorted(set(int(i) for i in w.ids if i >= 0))
        dw.load_async(batch, cur)
        for a in batch:
            st.alloc.load(a, int(w.ranks[a]), float(w.scales[a]))
            A, B = w.weights(a, 0)
            st.image.write_adapter(st.alloc, a, 0, A, B)
        dw.build(w.ids)
        dw.delta(0)
        torch.cuda.synchronize()
        assert S.slora_segments_read_error(dw.seg) == 0
        y_ref, sd_ref = workload_delta(st, w, 0)
        check_gates(dw.y[0].cpu().numpy(), y_ref, sd_ref, w.np_dtype, f"async/{route}")
    finally:
        dw.close()


@pytest.mark.parametrize("launch", ["fused", "two"])
def test_fetch_next_batch_while_delta_runs(launch):
    """Walkthrough step 2 on two streams: while batch 1's delta runs, the
    adapters of batch 2 that were evicted are fetched on a side stream into
    free pages; batch 2 then waits for the fetch.  Both batches meet the gates
    and the fetched pages equal the oracle image."""
    spec = small_spec("prefetch", h_in=1024, h_out=1024, n_adapters=40, rank_set=(8, 16, 32, 64),
                      batch=("zipf", 200, 1.1), pool=("occ", 1, 2), full_weights=True)
    w = generate(spec, 13)
    used = sorted(set(int(i) for i in w.ids if i >= 0))
    evicted = [a for a in range(spec.n_adapters) if a not in used][:4]
    assert evicted, "the batch must leave some adapters unreferenced"
    tune = {S.SLORA_TUNE_FUSED: 1 if launch == "fused" else 0}
    print(f"[gpu] prefetch launch={launch} evicted={evicted}", flush=True)
    dw = DeviceWorkload(w, "cuda:0", tuning=tune, load_all_weights=True)
    side = torch.cuda.Stream()
    try:
        st = build_from_workload(w)
        for a in evicted:
            S.slora_unload_adapter(dw.pool, a)
            st.alloc.unload(a)
        images = {a: dw.pack(a) for a in evicted}
        # batch 1 on the current stream, fetches on the side stream meanwhile
        dw.build(w.ids)
        dw.delta(0)
        dw.load_async(evicted, side, images=[images[a] for a in evicted])
        for a in evicted:
            st.alloc.load(a, int(w.ranks[a]), float(w.scales[a]))
            A, B = w.weights(a, 0)
            st.image.write_adapter(st.alloc, a, 0, A, B)
        y1 = dw.y[0].clone()
        fetched = torch.cuda.Event()
        fetched.record(side)
        # batch 2 uses the fetched adapters and half of batch 1's
        rng = np.random.default_rng(5)
        ids2 = rng.choice(np.array(evicted + used[: max(1, len(used) // 2)]), size=w.T).astype(np.int32)
        torch.cuda.current_stream().wait_event(fetched)
        dw.build(ids2)
        dw.reset_y()
        dw.delta(0)
        torch.cuda.synchronize()
        assert S.slora_segments_read_error(dw.seg) == 0
        y_ref, sd_ref = workload_delta(st, w, 0)
        check_gates(y1.cpu().numpy(), y_ref, sd_ref, w.np_dtype, f"prefetch/{launch}/batch1")
        y2_ref, sd2_ref = lora_delta(st.alloc, st.image, ids2, w.x[0], w.y[0], proj=0)
        check_gates(dw.y[0].cpu().numpy(), y2_ref, sd2_ref, w.np_dtype, f"prefetch/{launch}/batch2")
        for a in evicted:
            pa, pb = S.slora_adapter_pages(dw.pool, a)
            assert pa.tolist() == list(st.alloc.table[a].a_pages[0])
            assert pb.tolist() == list(st.alloc.table[a].b_pages[0])
        assert_pool_is_oracle_image(dw, st)
    finally:
        side.synchronize()
        dw.close()


def test_async_load_rejects_bad_batches_and_takes_no_page():
    spec = small_spec("async_err", h_in=256, h_out=256, n_adapters=4, batch=("uniform", 8))
    w = generate(spec, 14)
    dw = DeviceWorkload(w, "cuda:0")
    try:
        S.slora_unload_adapter(dw.pool, 0)
        S.slora_unload_adapter(dw.pool, 1)
        nb = S.slora_adapter_image_bytes(dw.pool, int(max(w.ranks[0], w.ranks[1])))
        free = S.slora_free_count(dw.pool, 0)
        pageable = np.zeros(nb, np.uint8)
        pinned = [torch.zeros(nb, dtype=torch.uint8, pin_memory=True) for _ in range(2)]
        stage = torch.empty(2 * nb, dtype=torch.uint8, device="cuda:0")
        stream = torch.cuda.current_stream()
        cases = [  # (ids, images, dev_stage, dev_stage_bytes, status)
            ([0, 1], [pinned[0], pageable.ctypes.data], stage, 2 * nb, S.SLORA_E_INVAL),
            ([0, 1], [pinned[0], stage], stage, 2 * nb, S.SLORA_E_INVAL),
            ([0, 1], pinned, pinned[0], 2 * nb, S.SLORA_E_INVAL),
            ([0, 1], pinned, stage, nb // 2, S.SLORA_E_INVAL),
            ([0, 0], pinned, stage, 2 * nb, S.SLORA_E_INVAL),
            ([0, 2], pinned, stage, 2 * nb, S.SLORA_E_EXIST),
        ]
        for ids, imgs, dev, dev_bytes, want in cases:
            with pytest.raises(S.SloraError) as e:
                S.slora_load_adapters_async(dw.pool, ids, [int(w.ranks[a]) for a in ids],
                                            [1.0] * len(ids), imgs, dev, dev_bytes, stream)
            assert e.value.status == want, ids
            assert S.slora_free_count(dw.pool, 0) == free
            for a in (0, 1):
                with pytest.raises(S.SloraError):
                    S.slora_adapter_pages(dw.pool, a)
        S.slora_load_adapters_async(dw.pool, [], [], [], [], stage, 0, stream)
        torch.cuda.synchronize()
    finally:
        dw.close()


def test_refetch_same_images_into_new_pages():
    """One pinned image per adapter, fetched, evicted and fetched again three
    times through the same staging buffer: each fetch rewrites the page ids
    inside the image on the host, and the rows must land on the new pages."""
    spec = small_spec("refetch", h_in=512, h_out=640, two_classes=True, n_adapters=24,
                      rank_set=(8, 16, 64), batch=("zipf", 64, 1.1), pool=("fixed", 2000),
                      full_weights=True)
    w = generate(spec, 15)
    used = set(int(i) for i in w.ids if i >= 0)
    evicted = [a for a in range(spec.n_adapters) if a not in used][:5]
    assert len(evicted) >= 2
    print(f"[gpu] refetch evicted={evicted}", flush=True)
    dw = DeviceWorkload(w, "cuda:0", load_all_weights=True)
    side = torch.cuda.Stream()
    try:
        st = build_from_workload(w)
        images = [dw.pack(a) for a in evicted]
        seen = set()
        for rnd in range(3):
            for a in evicted:
                S.slora_unload_adapter(dw.pool, a)
                st.alloc.unload(a)
            dw.load_async(evicted, side, images=images)
            for a in evicted:
                st.alloc.load(a, int(w.ranks[a]), float(w.scales[a]))
                A, B = w.weights(a, 0)
                st.image.write_adapter(st.alloc, a, 0, A, B)
            side.synchronize()
            pages = [p.cpu().numpy() for p in dw.pages]
            for a in evicted:
                pa, pb = S.slora_adapter_pages(dw.pool, a)
                assert pa.tolist() == list(st.alloc.table[a].a_pages[0])
                assert not seen.intersection((0, int(x)) for x in pa), "pages not new"
                seen.update((0, int(x)) for x in pa)
                A, B = w.weights(a, 0)
                for j in range(int(w.ranks[a])):
                    assert np.array_equal(uint_view(pages[0][pa[j]]), uint_view(A[:, j].copy())), (rnd, a, j)
                    assert np.array_equal(uint_view(pages[1][pb[j]]), uint_view(B[j].copy())), (rnd, a, j)
        assert_pool_is_oracle_image(dw, st)
    finally:
        side.synchronize()
        dw.close()
