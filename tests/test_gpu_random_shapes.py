"""Seeded random shapes through the C ABI on an MI355X, against the fp64 oracle.

Each case draws a shape the hand-picked tests do not: fp16 or fp32, one or
two page classes, h_in and h_out any multiple of 8 up to 2048 (ragged against
every tile width), one to three projections sharing or not sharing x, ranks
from 1 to 256, a batch of any of the four kinds with some tokens on no
adapter, and the pool's occupancy.  The delta runs fused and as two launches,
with the default routing and with every eligible segment on the matrix-core
tiles; the base product with the delta runs where its shape allows.  Every
output is held to the oracle's gates.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import build_from_workload, lora_forward, workload_delta  # noqa: E402
from rank_gemm_page_amd import slora as S  # noqa: E402
from rank_gemm_page_amd.device_workload import DeviceWorkload  # noqa: E402
from synth import generate, small_spec  # noqa: E402
from tests.gates import check_forward_gates, check_gates  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.lib()


def random_spec(seed):
    rng = np.random.default_rng(1000 + seed)
    f16 = rng.random() < 0.75
    two = bool(rng.random() < 0.6)
    if rng.random() < 0.35:        # a shape the base-plus-delta kernel takes (64 | h_in, 128 | h_out)
        h_in = 128 * int(rng.integers(1, 17))
        h_out = 128 * int(rng.integers(1, 17)) if two else h_in
    else:
        h_in = 8 * int(rng.integers(1, 257))
        h_out = 8 * int(rng.integers(1, 257)) if two else h_in
    n_proj = int(rng.integers(1, 4))
    proj_x = tuple(int(v) for v in rng.integers(0, n_proj, size=n_proj))
    proj_x = tuple(sorted(set(proj_x)).index(v) for v in proj_x)       # x numbers 0, 1, ... in use
    ranks = tuple(sorted(set(int(v) for v in rng.choice([1, 2, 3, 5, 8, 13, 16, 31, 32, 64, 100, 128, 200, 256],
                                                         size=int(rng.integers(1, 5)), replace=False))))
    kind = int(rng.integers(0, 4))
    if kind == 0:
        batch = ("uniform", int(rng.integers(1, 200)))
    elif kind == 1:
        batch = ("zipf", int(rng.integers(1, 300)), float(rng.choice([0.8, 1.1, 1.5])))
    elif kind == 2:
        batch = ("requests", int(rng.integers(1, 6)), int(rng.integers(1, 40)), int(rng.integers(40, 160)))
    else:
        batch = ("mixed", int(rng.integers(1, 4)), int(rng.integers(60, 130)), int(rng.integers(1, 60)))
    occ = int(rng.integers(0, 4))
    spec = small_spec(f"rand{seed}", dtype="f16" if f16 else "f32", h_in=h_in, h_out=h_out, two_classes=two,
                      n_adapters=int(rng.integers(2, 24)), rank_set=ranks, n_proj=n_proj, proj_x=proj_x,
                      scale_set=(0.5, 2.0, -1.5), batch=batch, pool=("occ", occ, 4))
    return spec, rng


def run(w, tuning, fused):
    dw = DeviceWorkload(w, "cuda:0", tuning={**tuning, S.SLORA_TUNE_FUSED: fused})
    try:
        for p in range(w.spec.n_proj):
            dw.delta(p)
        torch.cuda.synchronize()
        ys = [dw.y[p].cpu().numpy() for p in range(w.spec.n_proj)]
        assert S.slora_segments_read_error(dw.seg) == 0
        return ys, dw.info
    finally:
        dw.close()


@pytest.mark.parametrize("seed", range(40))
def test_random_shape_delta(seed):
    spec, rng = random_spec(seed)
    w = generate(spec, seed)
    w.ids = w.ids.copy()
    w.ids[rng.random(w.T) < 0.1] = -1
    print(f"[gpu] random {spec.name}: {spec.dtype} {spec.h_in}x{spec.h_out} two={spec.two_classes} "
          f"proj={spec.n_proj} x={spec.proj_x} ranks={spec.rank_set} batch={spec.batch} T={w.T}", flush=True)
    st = build_from_workload(w)
    refs = [workload_delta(st, w, proj=p) for p in range(spec.n_proj)]
    routes = [{}] + ([{S.SLORA_TUNE_MFMA_MIN_TOKENS: 1}] if spec.dtype == "f16" else [])
    for tuning in routes:
        for fused in (1, 0):
            ys, info = run(w, tuning, fused)
            for p, (y_ref, sd_ref) in enumerate(refs):
                check_gates(ys[p], y_ref, sd_ref, w.np_dtype,
                            f"{spec.name}/{'mfma' if tuning else 'default'}/fused={fused}/p{p}")
    if spec.dtype == "f16" and spec.h_in % 64 == 0 and spec.h_out % 128 == 0:
        dw = DeviceWorkload(w, "cuda:0")
        try:
            out = torch.full((w.T, spec.h_out), float("nan"), dtype=torch.float16, device="cuda:0")
            dw.forward(0, out)
            torch.cuda.synchronize()
            y = out.cpu().numpy()
        finally:
            dw.close()
        x = w.x[spec.proj_x[0]]
        h_ref, sd_ref = lora_forward(st.alloc, st.image, w.ids, x, w.base_weight(0), proj=0)
        base_abs = np.abs(x.astype(np.float64)) @ np.abs(w.base_weight(0).astype(np.float64))
        check_forward_gates(y, h_ref, sd_ref, base_abs, spec.h_in, np.float16, f"{spec.name}/forward")
        w.drop_weight_cache()
