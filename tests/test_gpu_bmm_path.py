"""The padded-BMM comparison path of bench.py against the fp64 oracle.

bench.py times this torch path beside the paged kernels (the pages' Figure 5
ablation); it must compute the same delta, so it meets the same value gates.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from bench import BmmPath  # noqa: E402
from oracle import build_from_workload, workload_delta  # noqa: E402
from rank_gemm_page_amd import slora as S  # noqa: E402
from rank_gemm_page_amd.device_workload import DeviceWorkload  # noqa: E402
from synth import CONFIGS, generate, small_spec  # noqa: E402
from tests.gates import check_gates  # noqa: E402

pytestmark = pytest.mark.gpu

SPECS = [
    CONFIGS["tiny"],
    small_spec("bmm_mixed_ranks", h_in=512, h_out=384, two_classes=True, n_adapters=7,
               rank_set=(1, 8, 40, 64), batch=("zipf", 90, 1.0)),
    small_spec("bmm_proj", h_in=256, h_out=256, n_adapters=5, n_proj=3, proj_x=(0, 0, 1),
               batch=("mixed", 2, 30, 11)),
]


@pytest.mark.parametrize("spec", SPECS, ids=lambda s: s.name)
def test_bmm_path_matches_oracle(spec):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w = generate(spec, 21)
    print(f"[gpu] bmm path {spec.name}", flush=True)
    dw = DeviceWorkload(w, "cuda:0")
    try:
        st = build_from_workload(w)
        for p in range(spec.n_proj):
            BmmPath(dw, p).step(dw.x[spec.proj_x[p]], dw.y[p])
        torch.cuda.synchronize()
        for p in range(spec.n_proj):
            y_ref, sd_ref = workload_delta(st, w, p)
            check_gates(dw.y[p].cpu().numpy(), y_ref, sd_ref, w.np_dtype, f"bmm/{spec.name}/p{p}")
    finally:
        dw.close()
