"""slora_lora_forward_noalloc (the library's own workspace) on an MI355X.

Two calls in a row on one GPU, the second with a smaller batch than the
first, each compared bit for bit with slora_lora_forward given a caller
workspace (same kernels, same workspace layout), and with the oracle's gates.
The first batch has 64-token matrix-core segments split over K, so the array
holds partial sums as well as x A; the second batch runs on whatever the first
left in it.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import build_from_workload, lora_forward  # noqa: E402
from rank_gemm_page_amd import slora as S  # noqa: E402
from rank_gemm_page_amd.device_workload import DeviceWorkload  # noqa: E402
from synth import generate, small_spec  # noqa: E402
from tests.gates import check_forward_gates  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.lib()


def run_both(w, tuning):
    print(f"[gpu] noalloc {w.spec.name} seed={w.seed} T={w.T}", flush=True)
    dw = DeviceWorkload(w, "cuda:0", tuning=tuning)
    try:
        ref = torch.full((w.T, w.spec.h_out), float("nan"), dtype=torch.float16, device="cuda:0")
        dw.forward(0, ref)
        got = torch.full_like(ref, float("nan"))
        S.slora_lora_forward_noalloc(dw.pool, dw.seg, 0, dw.x[0], dw.base_weight(0), got,
                                     torch.cuda.current_stream())
        torch.cuda.synchronize()
        return ref.cpu().numpy(), got.cpu().numpy(), dw.info
    finally:
        dw.close()


def oracle_check(w, y, label):
    st = build_from_workload(w)
    h_ref, sd_ref = lora_forward(st.alloc, st.image, w.ids, w.x[0], w.base_weight(0))
    base_abs = np.abs(w.x[0].astype(np.float64)) @ np.abs(w.base_weight(0).astype(np.float64))
    check_forward_gates(y, h_ref, sd_ref, base_abs, w.spec.h_in, np.float16, label)


def test_noalloc_forward_two_calls_second_smaller():
    big = generate(small_spec("na_big", h_in=512, h_out=512, n_adapters=6, rank_set=(8, 32, 64),
                              batch=("requests", 6, 100, 300)), 5)
    small = generate(small_spec("na_small", h_in=256, h_out=384, two_classes=True, n_adapters=4,
                                rank_set=(1, 13, 40), batch=("zipf", 70, 1.0)), 6)
    tuning = {S.SLORA_TUNE_MFMA_MIN_TOKENS: 64}
    ref1, got1, info1 = run_both(big, tuning)
    assert info1["n_mfma_segments"] > 0 and info1["n_combine_tiles"] > 0   # K-split partials in the array
    ref2, got2, info2 = run_both(small, tuning)
    assert info2["workspace_bytes"] < info1["workspace_bytes"]
    for ref, got, w, label in ((ref1, got1, big, "first call"), (ref2, got2, small, "second call, smaller")):
        assert np.isfinite(got).all(), label
        np.testing.assert_array_equal(got.view(np.uint16), ref.view(np.uint16), err_msg=label)
        oracle_check(w, got, f"noalloc {label}")
