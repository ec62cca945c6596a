"""Several projections in one launch (slora_lora_delta_multi) on an MI355X.

Each projection of a multi-projection launch must equal, bit for bit, the
same projection run alone with slora_lora_delta (same tiles, same summation
order), and both must meet the oracle's gates.  Shapes cover projections that
share x (q, k, v) beside one with its own x (o), batches with matrix-core and
vector-ALU segments, subsets of the projections in any order, repeated
launches, and the two-launch (staged) fallback.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import build_from_workload, workload_delta  # noqa: E402
from rank_gemm_page_amd import slora as S  # noqa: E402
from rank_gemm_page_amd.device_workload import DeviceWorkload  # noqa: E402
from synth import CONFIGS, generate, small_spec  # noqa: E402
from tests.gates import check_gates  # noqa: E402

pytestmark = pytest.mark.gpu

ROUTES = {"gemv": {S.SLORA_TUNE_MFMA_MIN_TOKENS: 1 << 30},
          "mfma": {S.SLORA_TUNE_MFMA_MIN_TOKENS: 1},
          "default": {S.SLORA_TUNE_MFMA_MIN_TOKENS: 16}}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.lib()


SPECS = [
    small_spec("qkvo", h_in=512, h_out=512, n_adapters=7, n_proj=4, proj_x=(0, 0, 0, 1),
               batch=("mixed", 3, 48, 40)),
    small_spec("qkv_nonsq", h_in=384, h_out=1288, two_classes=True, n_adapters=5, n_proj=3,
               proj_x=(0, 0, 0), rank_set=(3, 16, 64, 128), batch=("zipf", 90, 1.0)),
    small_spec("f32_proj3", dtype="f32", h_in=256, h_out=256, n_adapters=4, n_proj=3,
               proj_x=(0, 1, 1), batch=("uniform", 37)),
]


def singles_and_multi(w, tuning, subsets):
    """y of every projection run alone, then of each projection subset run as one launch."""
    print(f"[gpu] multi {w.spec.name} seed={w.seed} T={w.T} tuning={tuning}", flush=True)
    dw = DeviceWorkload(w, "cuda:0", tuning=tuning)
    try:
        singles = {}
        for p in range(w.spec.n_proj):
            dw.delta(p)
        torch.cuda.synchronize()
        for p in range(w.spec.n_proj):
            singles[p] = dw.y[p].cpu().numpy()
        multis = []
        for projs in subsets:
            dw.reset_y()
            dw.delta_multi(projs)
            torch.cuda.synchronize()
            multis.append({p: dw.y[p].cpu().numpy() for p in projs})
        assert S.slora_segments_read_error(dw.seg) == 0
        return singles, multis, dw.info
    finally:
        dw.close()


@pytest.mark.parametrize("spec", SPECS, ids=lambda s: s.name)
@pytest.mark.parametrize("route", list(ROUTES))
@pytest.mark.parametrize("fused", [1, 0])
def test_multi_equals_singles_and_oracle(spec, route, fused):
    w = generate(spec, 3)
    n = spec.n_proj
    subsets = [list(range(n)), list(range(n))[::-1], [n - 1, 0], [1]]
    tuning = dict(ROUTES[route])
    tuning[S.SLORA_TUNE_FUSED] = fused
    singles, multis, info = singles_and_multi(w, tuning, subsets)
    st = build_from_workload(w)
    for p in range(n):
        y_ref, sd_ref = workload_delta(st, w, proj=p)
        check_gates(singles[p], y_ref, sd_ref, w.np_dtype, f"{spec.name}/{route}/single p{p}")
    for projs, got in zip(subsets, multis):
        for p in projs:
            np.testing.assert_array_equal(got[p].view(np.uint16 if w.np_dtype == np.float16 else np.uint32),
                                          singles[p].view(np.uint16 if w.np_dtype == np.float16 else np.uint32),
                                          err_msg=f"{spec.name}/{route}/fused={fused} projs={projs} p{p}")


def test_multi_repeated_launches_and_full_mixed_batch():
    """The 13B mixed batch (q, k, v on one x, o on its own): all four
    projections in one launch, twice in a row from the same y, equal the
    single-projection launches bit for bit."""
    w = generate(CONFIGS["mixed13b"], 0)
    dw = DeviceWorkload(w, "cuda:0")
    try:
        for p in range(4):
            dw.delta(p)
        torch.cuda.synchronize()
        singles = [dw.y[p].cpu().numpy() for p in range(4)]
        for rep in range(2):
            dw.reset_y()
            dw.delta_multi()
            torch.cuda.synchronize()
            for p in range(4):
                np.testing.assert_array_equal(dw.y[p].cpu().numpy().view(np.uint16), singles[p].view(np.uint16),
                                              err_msg=f"mixed13b rep {rep} p{p}")
        assert S.slora_segments_read_error(dw.seg) == 0
        print(f"[gpu] mixed13b: four projections in one launch match the single launches "
              f"(segments={dw.info['n_segments']})", flush=True)
    finally:
        dw.close()


@pytest.mark.parametrize("route", ["gemv", "default"])
def test_multi_eight_projections_the_largest_launch(route):
    """The most projections one launch takes (8), each on an x of its own or
    shared, with ranks up to the pool's largest: every projection equals its
    single launch bit for bit, in one launch and as two launches of four."""
    spec = small_spec("proj8", h_in=320, h_out=448, two_classes=True, n_adapters=9, n_proj=8,
                      proj_x=(0, 1, 1, 2, 3, 3, 3, 4), rank_set=(1, 7, 32, 64, 200),
                      batch=("mixed", 2, 66, 30))
    w = generate(spec, 8)
    tuning = dict(ROUTES[route])
    subsets = [list(range(8)), [7, 6, 5, 4], [3, 2, 1, 0]]
    singles, multis, info = singles_and_multi(w, tuning, subsets)
    st = build_from_workload(w)
    for p in range(8):
        y_ref, sd_ref = workload_delta(st, w, proj=p)
        check_gates(singles[p], y_ref, sd_ref, w.np_dtype, f"proj8/{route}/single p{p}")
    for projs, got in zip(subsets, multis):
        for p in projs:
            np.testing.assert_array_equal(got[p].view(np.uint16), singles[p].view(np.uint16),
                                          err_msg=f"proj8/{route} projs={projs} p{p}")
    print(f"[gpu] proj8/{route}: segments={info['n_segments']} mfma={info['n_mfma_segments']}", flush=True)


@pytest.mark.parametrize("xcds", [3, 8])
def test_multi_with_xcd_placement(xcds):
    """Shrink tiles grouped by XCD interleave the matrix-core and vector-ALU
    shrink kinds, so a launch over several projections runs its three stages
    as phases instead of one phase per tile kind: every projection still equals
    its single launch bit for bit, and the single launches meet the gates."""
    spec = SPECS[0]
    w = generate(spec, 5)
    tuning = dict(ROUTES["default"])
    tuning[S.SLORA_TUNE_XCDS] = xcds
    subsets = [list(range(spec.n_proj)), [3, 1]]
    singles, multis, info = singles_and_multi(w, tuning, subsets)
    assert 0 < info["n_mfma_segments"] < info["n_segments"]
    st = build_from_workload(w)
    for p in range(spec.n_proj):
        y_ref, sd_ref = workload_delta(st, w, proj=p)
        check_gates(singles[p], y_ref, sd_ref, w.np_dtype, f"xcds{xcds}/single p{p}")
    for projs, got in zip(subsets, multis):
        for p in projs:
            np.testing.assert_array_equal(got[p].view(np.uint16), singles[p].view(np.uint16),
                                          err_msg=f"xcds{xcds} projs={projs} p{p}")
