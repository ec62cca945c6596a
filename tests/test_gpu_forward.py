"""Base product plus delta (slora_lora_forward) against the fp64 oracle, on an MI355X.

Each case puts a seeded synthetic workload on the GPU (NaN in every page that
is not an adapter row of the batch, NaN in the output buffer), runs
slora_lora_forward with the workload's dense base weight W, and compares
y = x W + s (x A) B with the oracle's lora_forward: gates G1 and G2 of
tests/gates.py, with the base product's fp32 summation bound added to G2
(check_forward_gates), or bit for bit where the arithmetic is exact.  The kernel's
tiles hold 128 positions of the batch in segment order, so the shapes put
segment boundaries inside and across tiles, and add tokens with no adapter.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import build_from_workload, lora_forward, round_to  # noqa: E402
from rank_gemm_page_amd import slora as S  # noqa: E402
from rank_gemm_page_amd.device_workload import DeviceWorkload  # noqa: E402
from synth import CONFIGS, generate, small_spec  # noqa: E402
from tests.gates import check_forward_gates  # noqa: E402

pytestmark = pytest.mark.gpu

ROUTES = {"gemv": {S.SLORA_TUNE_MFMA_MIN_TOKENS: 1 << 30},
          "mfma": {S.SLORA_TUNE_MFMA_MIN_TOKENS: 1},
          "default": {}}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.lib()


def run_forward(w, projs=(0,), route="default", repeat=1, tile=0, group=0, ks=0):
    print(f"[gpu] forward {w.spec.name} seed={w.seed} route={route} T={w.T} "
          f"h={w.spec.h_in}x{w.spec.h_out} tile={tile} group={group} ks={ks}", flush=True)
    dw = DeviceWorkload(w, "cuda:0", tuning={**ROUTES[route], S.SLORA_TUNE_FWD_TILE: tile,
                                             S.SLORA_TUNE_FWD_GROUP: group, S.SLORA_TUNE_FWD_KSPLIT: ks})
    try:
        outs = []
        for p in projs:
            runs = []
            for _ in range(repeat):
                out = torch.full((w.T, w.spec.h_out), float("nan"), dtype=torch.float16, device="cuda:0")
                dw.forward(p, out)
                runs.append(out)
            torch.cuda.synchronize()
            outs.append([o.cpu().numpy() for o in runs])
        return outs, dw.info
    finally:
        dw.close()


def oracle_forward(w, proj=0, tokens=None, state=None):
    st = state or build_from_workload(w)
    return lora_forward(st.alloc, st.image, w.ids, w.x[w.spec.proj_x[proj]], w.base_weight(proj),
                        proj=proj, tokens=tokens)


def check(w, y, h_ref, sd_ref, proj=0, tokens=None, label=""):
    x = w.x[w.spec.proj_x[proj]]
    xs = x if tokens is None else x[tokens]
    base_abs = np.abs(xs.astype(np.float64)) @ np.abs(w.base_weight(proj).astype(np.float64))
    return check_forward_gates(y, h_ref, sd_ref, base_abs, w.spec.h_in, np.float16, label)


def drop_some(w, every):
    """Give every `every`-th token no adapter (id -1)."""
    if every:
        w.ids = w.ids.copy()
        w.ids[::every] = -1
    return w


SMALL = {
    # one class, tokens spread over six adapters, two row blocks
    "sq128": dict(h_in=128, h_out=128, n_adapters=6, batch=("uniform", 200)),
    # prefill-like requests: segments of 20..150 tokens crossing row blocks
    "requests": dict(h_in=192, h_out=256, two_classes=True, n_adapters=7, rank_set=(1, 5, 33, 64),
                     batch=("requests", 5, 20, 150)),
    # decode-like: many one-token segments in each row block
    "decode": dict(h_in=256, h_out=384, two_classes=True, n_adapters=60, batch=("zipf", 300, 1.1)),
    # ranks past 64 (several LoRA stages per segment) up to the pool's 256
    "highrank": dict(h_in=128, h_out=128, n_adapters=4, fixed_ranks=(100, 256, 129, 31),
                     batch=("uniform", 70)),
    # one token
    "one": dict(h_in=64, h_out=128, two_classes=True, n_adapters=3, batch=("uniform", 1)),
}


@pytest.mark.parametrize("tile", [0, 32, 64, 128])
@pytest.mark.parametrize("route", ["default", "gemv", "mfma"])
@pytest.mark.parametrize("name", list(SMALL))
def test_forward_small_shapes(name, route, tile):
    spec = small_spec(f"fw_{name}", scale_set=(0.5, 2.0, -1.5, 4.0), **SMALL[name])
    w = drop_some(generate(spec, 11), 7 if name != "one" else 0)
    (ys,), _ = run_forward(w, route=route, tile=tile)
    h_ref, sd_ref = oracle_forward(w)
    check(w, ys[0], h_ref, sd_ref, label=f"forward {name}/{route}/{tile}")


@pytest.mark.parametrize("ks", [1, 2])
@pytest.mark.parametrize("tile", [32, 64])
@pytest.mark.parametrize("name", list(SMALL))
def test_forward_wave_groups_split_steps(name, tile, ks):
    """One or two groups of waves per 32- or 64-row tile.  The shapes give
    odd and even numbers of x W steps (h_in 64, 128, 192, 256) and of LoRA
    steps, so a group's last step is sometimes one it does not own."""
    spec = small_spec(f"fw_{name}", scale_set=(0.5, 2.0, -1.5, 4.0), **SMALL[name])
    w = drop_some(generate(spec, 17), 5 if name != "one" else 0)
    (ys,), _ = run_forward(w, route="mfma", tile=tile, ks=ks)
    h_ref, sd_ref = oracle_forward(w)
    check(w, ys[0], h_ref, sd_ref, label=f"forward {name}/{tile}/ks{ks}")


BIG = {
    # 256 x 256 tiles: ragged last row block, segments across row blocks
    "big_requests": dict(h_in=192, h_out=512, two_classes=True, n_adapters=7, rank_set=(1, 5, 33, 64),
                         batch=("requests", 6, 40, 200)),
    # many one-token segments in one 256-position row block
    "big_decode": dict(h_in=128, h_out=256, two_classes=True, n_adapters=80, batch=("zipf", 250, 1.1)),
    # high ranks, one token past a row block
    "big_highrank": dict(h_in=256, h_out=256, n_adapters=4, fixed_ranks=(100, 256, 129, 31),
                         batch=("uniform", 257)),
}


@pytest.mark.parametrize("name", list(BIG))
def test_forward_big_tiles(name):
    spec = small_spec(f"fw_{name}", scale_set=(0.5, 2.0, -1.5, 4.0), **BIG[name])
    w = drop_some(generate(spec, 13), 6)
    (ys,), info = run_forward(w, tile=256)
    h_ref, sd_ref = oracle_forward(w)
    check(w, ys[0], h_ref, sd_ref, label=f"forward {name}/256")


def test_forward_big_tiles_integer_bit_exact_and_same_as_small():
    spec = small_spec("fw_bigint", h_in=64, h_out=256, two_classes=True, n_adapters=6,
                      rank_set=(1, 2, 4), values="ternary", scale=2.0, batch=("requests", 6, 20, 90))
    w = drop_some(generate(spec, 4), 5)
    h_ref, _ = oracle_forward(w)
    assert np.abs(h_ref).max() < 2048
    outs = {}
    for tile, ks in ((32, 1), (32, 2), (64, 1), (64, 2), (128, 0), (256, 0)):
        (ys,), _ = run_forward(w, route="mfma", tile=tile, ks=ks)
        np.testing.assert_array_equal(ys[0], round_to(h_ref, np.float16))
        outs[tile, ks] = ys[0]
    for key in outs:
        np.testing.assert_array_equal(outs[key], outs[256, 0], err_msg=str(key))


@pytest.mark.parametrize("tile", [32, 64, 128])
def test_forward_tile_order_changes_nothing(tile):
    """The order in which tiles walk the chip (groups of 1, 3, 8 and all row
    blocks, ragged last group) places work, never changes it: bit-identical
    outputs, all within the gates."""
    spec = small_spec("fw_order", h_in=192, h_out=1024, two_classes=True, n_adapters=40,
                      rank_set=(4, 8, 16, 64), batch=("zipf", 700, 1.1))
    w = drop_some(generate(spec, 21), 7)
    h_ref, sd_ref = oracle_forward(w)
    outs = {}
    for group in (0, 1, 3, 8, 64):
        (ys,), _ = run_forward(w, tile=tile, group=group)
        outs[group] = ys[0]
    check(w, outs[0], h_ref, sd_ref, label=f"forward order {tile}")
    for group in (1, 3, 8, 64):
        np.testing.assert_array_equal(outs[group], outs[0])


@pytest.mark.parametrize("batch,n_adapters", [(("requests", 40, 190, 230), 12),
                                               (("mixed", 32, 256, 400), 60)])
def test_forward_big_and_small_tiles_split(batch, n_adapters):
    """Automatic tiles on a batch large enough for one whole round of 256
    big tiles: the leading 8192 positions go in 256 x 256 tiles, the rest in
    128 x 256 tiles of a second launch (with the mixed batch, many one-token
    segments there); every position around the boundary, the first and last
    rows and random ones are checked."""
    spec = small_spec("fw_split", h_in=64, h_out=2048, two_classes=True, n_adapters=n_adapters,
                      rank_set=(8, 16, 32, 64), batch=batch)
    w = drop_some(generate(spec, 21), 11)
    assert w.T > 8192 + 128 and -(-w.T // 256) * 8 >= 256
    (ys,), _ = run_forward(w)
    y = ys[0]
    assert np.isfinite(y).all()
    ids = w.ids
    routed = np.flatnonzero(ids >= 0)
    order = np.concatenate([routed[np.argsort(ids[routed], kind="stable")], np.flatnonzero(ids < 0)])
    rng = np.random.default_rng(0)
    pos = set(range(8192 - 300, min(w.T, 8192 + 300))) | {0, 1, w.T - 1}
    pos |= set(rng.choice(w.T, 200, replace=False).tolist())
    toks = sorted(int(order[p]) for p in pos)
    h_ref, sd_ref = oracle_forward(w, tokens=toks)
    check(w, y[toks], h_ref, sd_ref, tokens=toks, label="forward split 256/128")


# The library's extremes, one dimension at a time (a 16384 x 65536 W would be
# 2 GiB, and its fp64 copy for the oracle 8 GiB on the host): the longest K
# loop (h_in 16384, 256 x W steps per tile) and the widest output (h_out
# 65536: 512 column tiles of 128 or 256 of 256, 128 KB B pages), with rank
# 256 adapters (eight LoRA steps a segment) and a second projection, in both
# tile sizes.
MAX_FWD = [
    small_spec("fw_max_k", h_in=16384, h_out=512, two_classes=True, n_adapters=6, n_proj=2,
               proj_x=(0, 0), rank_set=(1, 17, 128, 256), batch=("zipf", 150, 1.0)),
    small_spec("fw_max_n", h_in=64, h_out=65536, two_classes=True, n_adapters=6, n_proj=2,
               proj_x=(0, 0), rank_set=(1, 17, 128, 256), batch=("zipf", 150, 1.0)),
]


@pytest.mark.parametrize("tile", [32, 64, 128, 256])
@pytest.mark.parametrize("spec", MAX_FWD, ids=lambda s: s.name)
def test_forward_maximum_sizes(spec, tile):
    w = generate(spec, 4)
    assert int(w.ranks.max()) == 256
    ys, _ = run_forward(w, projs=(0, 1), tile=tile)
    st = build_from_workload(w)
    toks = sample_positions(w, 20, bm=min(tile, 128) if tile else 32)
    for p, runs in zip((0, 1), ys):
        assert np.isfinite(runs[0]).all()
        h_ref, sd_ref = oracle_forward(w, p, tokens=toks, state=st)
        check(w, runs[0][toks], h_ref, sd_ref, proj=p, tokens=toks, label=f"{spec.name}/{tile}/p{p}")
    w.drop_weight_cache()


def test_forward_every_projection():
    spec = small_spec("fw_proj", h_in=128, h_out=128, n_proj=3, proj_x=(0, 1, 2), n_adapters=5,
                      batch=("requests", 3, 30, 110))
    w = drop_some(generate(spec, 5), 9)
    ys, _ = run_forward(w, projs=(0, 1, 2))
    st = build_from_workload(w)
    for p in range(3):
        h_ref, sd_ref = oracle_forward(w, p, state=st)
        check(w, ys[p][0], h_ref, sd_ref, proj=p, label=f"forward proj {p}")


def test_forward_integer_bit_exact():
    """{-1, 0, 1} inputs, s = 2: every partial sum is an integer below 2^11, so
    the result is exact whatever the summation order and must equal the
    oracle's bit for bit."""
    spec = small_spec("fw_int", h_in=64, h_out=128, two_classes=True, n_adapters=6,
                      rank_set=(1, 2, 4), values="ternary", scale=2.0, batch=("requests", 6, 10, 60))
    w = drop_some(generate(spec, 4), 5)
    for route in ("gemv", "mfma"):
        (ys,), _ = run_forward(w, route=route)
        h_ref, _ = oracle_forward(w)
        assert np.abs(h_ref).max() < 2048
        np.testing.assert_array_equal(ys[0], round_to(h_ref, np.float16))


def test_forward_no_adapter_tokens_and_repeat():
    """A batch with no routed token is the base product alone; repeated calls
    give bit-identical outputs."""
    spec = small_spec("fw_none", h_in=128, h_out=256, two_classes=True, n_adapters=3,
                      batch=("uniform", 150))
    w = generate(spec, 2)
    w.ids = np.full_like(w.ids, -1)
    (ys,), info = run_forward(w, repeat=2)
    assert info["n_routed"] == 0
    h_ref, sd_ref = oracle_forward(w)
    assert not sd_ref.any()
    check(w, ys[0], h_ref, sd_ref, label="forward, no adapters")
    np.testing.assert_array_equal(ys[0], ys[1])
    w2 = drop_some(generate(small_spec("fw_rep", h_in=128, h_out=128, batch=("uniform", 130)), 3), 4)
    (ys2,), _ = run_forward(w2, repeat=3)
    np.testing.assert_array_equal(ys2[0], ys2[1])
    np.testing.assert_array_equal(ys2[0], ys2[2])


def sample_positions(w, n, bm=128, seed=0):
    """Tokens at sorted positions on both sides of every tile boundary (tiles
    of bm positions), the first and last positions, and random tokens."""
    ids = w.ids
    routed = np.flatnonzero(ids >= 0)
    order = np.concatenate([routed[np.argsort(ids[routed], kind="stable")], np.flatnonzero(ids < 0)])
    picks = {int(order[0]), int(order[-1])}
    for b in range(bm, w.T, bm):
        picks |= {int(order[b - 1]), int(order[b])}
    rng = np.random.default_rng(seed)
    picks |= set(rng.choice(w.T, size=min(n, w.T), replace=False).tolist())
    return sorted(picks)


@pytest.mark.parametrize("name,projs,seed", [("decode7b", (0,), 0), ("prefill7b", (0,), 0),
                                             ("mixed13b", (0, 1, 2, 3), 0), ("mlp70b", (0,), 0),
                                             # other draws: new ranks, token ids, x, W, y and page layout
                                             ("decode7b", (0,), 1), ("mlp70b", (0,), 1)])
def test_forward_full_size(name, projs, seed):
    """Every row of every projection of the benchmark batches against the oracle."""
    w = generate(CONFIGS[name], seed)
    ys, info = run_forward(w, projs=projs)
    print(f"[gpu] {name}/seed{seed}: segments={info['n_segments']} tokens={w.T}", flush=True)
    st = build_from_workload(w)
    for p, runs in zip(projs, ys):
        y = runs[0]
        assert np.isfinite(y).all(), f"{name}/p{p}: a row was not written or a NaN page was read"
        h_ref, sd_ref = oracle_forward(w, p, state=st)
        check(w, y, h_ref, sd_ref, proj=p, label=f"forward {name}/p{p}")
        print(f"[gpu] forward {name}/p{p}: all {w.T} rows within the gates", flush=True)
    w.drop_weight_cache()
