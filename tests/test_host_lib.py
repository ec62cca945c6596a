"""Host side of libslora on the CPU: exports, allocator, segments, tiles, errors.

No GPU is touched: pools get fake (never dereferenced) page addresses, adapters
are loaded without data (pages reserved only), and every check runs on
metadata the library computes on the host.
"""
import json
import os
import re

import numpy as np
import pytest

from oracle import slora_oracle as orc
from rank_gemm_page_amd import slora as S
from synth import CONFIGS, generate, small_spec

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE_BASE = [1 << 40, 1 << 41]


def make_pool(w, base=FAKE_BASE, tuning=None):
    spec = w.spec
    n_classes = 2 if spec.two_classes else 1
    pool = S.slora_pool_create(S.SLORA_F16 if spec.dtype == "f16" else S.SLORA_F32, spec.h_in,
                               spec.h_out, spec.n_proj, spec.n_adapters, int(w.ranks.max()),
                               base[:n_classes], list(w.n_pages), w.free_order)
    for k, v in (tuning or {}).items():
        S.slora_pool_set_tuning(pool, k, v)
    kv = [S.slora_alloc_pages(pool, c, int(n)) for c, n in enumerate(w.kv_pages)]
    for a in range(spec.n_adapters):
        S.slora_load_adapter(pool, a, int(w.ranks[a]), float(w.scales[a]))
    return pool, kv


@pytest.mark.parametrize("header,names", [("slora.h", S.EXPORTED), ("slora_probe.h", S.EXPORTED_PROBE)])
def test_library_exports_every_declared_symbol(header, names):
    text = open(os.path.join(ROOT, "include", header)).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)        # declarations only, not comments
    declared = set(re.findall(r"\b(slora_[a-z_]+)\s*\(", text))
    assert declared == set(names)
    lib = S.lib()
    for name in declared:
        assert hasattr(lib, name), name


def test_every_header_is_covered():
    assert sorted(os.listdir(os.path.join(ROOT, "include"))) == ["slora.h", "slora_probe.h"]


@pytest.mark.parametrize("case", ["single_class", "two_class_two_proj"])
def test_allocator_fixture_through_library(case):
    with open(os.path.join(ROOT, "tests", "golden", "allocator_fifo.json")) as f:
        g = json.load(f)[case]
    n_classes = len(g["n_pages"])
    pool = S.slora_pool_create(S.SLORA_F16, 8, 8 if n_classes == 1 else 16, g["n_proj"], 16, 4,
                               FAKE_BASE[:n_classes], g["n_pages"], g["free_order"])
    try:
        for st in g["steps"]:
            if st["op"] == "load":
                S.slora_load_adapter(pool, st["adapter"], st["rank"], 1.0)
                for p in range(g["n_proj"]):
                    a, b = S.slora_adapter_pages(pool, st["adapter"], p)
                    assert a.tolist() == st["a_pages"][p] and b.tolist() == st["b_pages"][p]
            elif st["op"] == "load_fail":
                before = [S.slora_free_count(pool, c) for c in range(n_classes)]
                with pytest.raises(S.SloraError) as e:
                    S.slora_load_adapter(pool, st["adapter"], st["rank"], 1.0)
                assert e.value.status == S.SLORA_E_NOMEM
                assert [S.slora_free_count(pool, c) for c in range(n_classes)] == before
                assert before == [len(f) for f in st["free_after"]]
            elif st["op"] == "unload":
                S.slora_unload_adapter(pool, st["adapter"])
                assert [S.slora_free_count(pool, c) for c in range(n_classes)] == \
                    [len(f) for f in st["free_after"]]
            elif st["op"] == "kv":
                assert S.slora_alloc_pages(pool, st["cls"], st["n"]).tolist() == st["pages"]
            elif st["op"] == "kv_fail":
                with pytest.raises(S.SloraError) as e:
                    S.slora_alloc_pages(pool, st["cls"], st["n"])
                assert e.value.status == S.SLORA_E_NOMEM
        # the free lists' order, read back by draining them, matches the fixture
        final = g["steps"][-1].get("free_after")
        if final is not None:
            for c in range(n_classes):
                assert S.slora_alloc_pages(pool, c, len(final[c])).tolist() == final[c]
    finally:
        S.slora_pool_destroy(pool)


def oracle_segments(w):
    st = orc.build_from_workload(w, load_weights=False)
    return st, orc.segment_model(w.ids, st.alloc)


@pytest.mark.parametrize("name", list(CONFIGS))
def test_metadata_bit_exact_vs_oracle(name):
    w = generate(CONFIGS[name], 0)
    pool, kv = make_pool(w)
    try:
        st, ref = oracle_segments(w)
        for c in range(len(kv)):
            assert kv[c].tolist() == st.kv_pages[c]
        for a in range(w.spec.n_adapters):
            for p in range(w.spec.n_proj):
                ap, bp = S.slora_adapter_pages(pool, a, p)
                assert ap.tolist() == st.alloc.table[a].a_pages[p]
                assert bp.tolist() == st.alloc.table[a].b_pages[p]
        seg = S.slora_build_segments(pool, w.ids)
        try:
            got = S.slora_segments_export(seg)
            for k in ("perm", "seg_start", "seg_adapter", "seg_rank", "seg_page_off", "a_pages",
                      "b_pages"):
                np.testing.assert_array_equal(got[k], getattr(ref, k), err_msg=k)
            assert got["seg_scale"].view(np.uint32).tolist() == ref.seg_scale.view(np.uint32).tolist()
            info = S.slora_segments_get_info(seg)
            assert info["n_routed"] == w.T and info["n_segments"] == ref.seg_adapter.shape[0]
            assert info["sum_rank_tokens"] == int(w.ranks[w.ids].astype(np.int64).sum())
        finally:
            S.slora_segments_destroy(seg)
    finally:
        S.slora_pool_destroy(pool)


def check_forward_tables(w, pool, ids, tuning_label=""):
    """slora_lora_forward's LoRA stage table, decoded per row block: every
    (segment, rank row) of the segments that own a position of the block
    appears exactly once, with the oracle's B page id; rows with no rank row
    of their own repeat the page before them and, packed, sit in a group whose
    word counts only the real rows (0 for an empty group); the packed fields
    stay within their 23-bit segment and 6-bit row-quad ranges."""
    seg = S.slora_build_segments(pool, ids)
    try:
        L, rb_info, stages = S.slora_segments_forward_tables(seg)
        _, ref = oracle_segments_of(w, ids)
        routed = int(np.count_nonzero(np.asarray(ids) >= 0))
        starts, ranks, page_off = ref.seg_start, ref.seg_rank, ref.seg_page_off
        sum_r = int(page_off[-1])
        pos_seg = np.repeat(np.arange(len(ranks)), np.diff(starts))
        assert L["stage_words"] == 40 and L["n_proj"] == w.spec.n_proj
        assert L["n_rb"] == L["n_rb_big"] + -(-(len(ids) - L["big_rows"]) // L["small_bm"])
        for rb in range(L["n_rb"]):
            big = rb < L["n_rb_big"]
            p0 = rb * 256 if big else L["big_rows"] + (rb - L["n_rb_big"]) * L["small_bm"]
            p1 = min(p0 + (256 if big else L["small_bm"]), routed)
            first, count = (int(v) for v in rb_info[rb])
            want = set()
            if p0 < p1:
                for g in range(int(pos_seg[p0]), int(pos_seg[p1 - 1]) + 1):
                    want |= {(g, j) for j in range(int(ranks[g]))}
            else:
                assert count == 0
            for proj in range(L["n_proj"]):
                seen = []
                bp = ref.b_pages[proj * sum_r:(proj + 1) * sum_r]
                for e in range(first, first + count):
                    ent = stages[proj, e]
                    last = None
                    if L["packed"]:
                        for u in range(8):
                            word = int(ent[32 + u])
                            if word == 0:
                                rows = []
                            else:
                                g, jq, n = word >> 9, (word >> 3) & 63, word & 7
                                assert 1 <= n <= 4 and g < (1 << 23) and jq < 64
                                rows = [(g, 4 * jq + k) for k in range(n)]
                            for k in range(4):
                                pg = int(ent[4 * u + k])
                                if k < len(rows):
                                    g, j = rows[k]
                                    assert pg == bp[page_off[g] + j], (rb, e, u, k)
                                    seen.append((g, j))
                                    last = pg
                                else:
                                    assert last is not None and pg == last, (rb, e, u, k)   # filler row
                    else:
                        g, j0, r = int(ent[32]), int(ent[33]), int(ent[34])
                        assert r == ranks[g] and j0 % 32 == 0
                        for k in range(32):
                            pg = int(ent[k])
                            if j0 + k < r:
                                assert pg == bp[page_off[g] + j0 + k]
                                seen.append((g, j0 + k))
                                last = pg
                            else:
                                assert pg == last
                assert len(seen) == len(set(seen)) and set(seen) == want, (tuning_label, rb, proj)
        return L
    finally:
        S.slora_segments_destroy(seg)


def oracle_segments_of(w, ids):
    st = orc.build_from_workload(w, load_weights=False)
    return st, orc.segment_model(ids, st.alloc)


@pytest.mark.parametrize("name", list(CONFIGS))
@pytest.mark.parametrize("tile", [0, 32, 128, 256])
def test_forward_tables_match_oracle_pages(name, tile):
    w = generate(CONFIGS[name], 0)
    if w.spec.dtype != "f16" or (tile == 256 and w.spec.h_out % 256):
        pytest.skip("slora_lora_forward: fp16 only; 256-wide tiles need h_out a multiple of 256")
    pool, _ = make_pool(w, tuning={S.SLORA_TUNE_FWD_TILE: tile})
    try:
        ids = w.ids.copy()
        ids[::7] = -1                 # tokens with no adapter sort after the routed ones
        L = check_forward_tables(w, pool, ids, f"{name}/tile {tile}")
        assert L["packed"] == (L["n_rb_big"] == 0)
    finally:
        S.slora_pool_destroy(pool)


def check_tiles_cover(w, pool, ids):
    """Every (token, rank row) is shrunk once (MFMA shrink: once per K split,
    the splits' k ranges tiling [0, h_in), summed by exactly one combine tile
    when there are several), every (token, column) expanded once, and every
    expand tile comes after the shrink and combine tiles of its tokens."""
    seg = S.slora_build_segments(pool, ids)
    try:
        info = S.slora_segments_get_info(seg)
        ex = S.slora_segments_export(seg)
        lay, recs = S.slora_segments_tiles(seg)
        spec = w.spec
        n_seg = info["n_segments"]
        hdr, tokcap, pagecap = lay["hdr"], lay["tokcap"], lay["pagecap"]
        assert lay["n_tiles"] == len(recs) == lay["n_shrink"] + lay["n_combine"] + lay["n_expand"]
        assert lay["n_combine"] == info["n_combine_tiles"]
        assert lay["n_shrink"] == info["n_shrink_tiles"] and lay["n_expand"] == info["n_expand_tiles"]
        seg_of = {}
        for s in range(n_seg):
            for i in range(ex["seg_start"][s], ex["seg_start"][s + 1]):
                seg_of[int(ex["perm"][i])] = s
        # where each token's v row lives: prefix over sorted tokens of their ranks
        v_row = {}
        off = 0
        for s in range(n_seg):
            r = int(ex["seg_rank"][s])
            for i in range(ex["seg_start"][s], ex["seg_start"][s + 1]):
                v_row[int(ex["perm"][i])] = off
                off += r
        assert off == info["sum_rank_tokens"]
        shrink_seen = np.zeros(max(off, 1), np.int32)
        combine_seen = np.zeros(max(off, 1), np.int32)
        k_cover = {}                    # MFMA shrink: token -> h_in coverage by k
        last_shrink_of_token = {}
        n_co = 0
        routed = [t for t in range(len(ids)) if ids[t] >= 0]
        cover = {t: np.zeros(spec.h_out, np.int32) for t in routed}
        n_sh = n_ex = 0
        for idx, rec in enumerate(recs):
            kind, ntok, r, pos, length, v0 = (int(v) for v in rec[:6])
            assert kind in (0, 1, 2, 3, 5) and 1 <= ntok <= tokcap and length >= 1
            assert (kind & 1) <= (spec.dtype == "f16")
            toks = rec[hdr:hdr + ntok]
            s = seg_of[int(toks[0])]
            assert rec[8] == s and r == ex["seg_rank"][s]
            for k, t in enumerate(toks):
                assert seg_of[int(t)] == s and v_row[int(t)] == v0 + k * r
            base = [p * info["sum_rank"] + ex["seg_page_off"][s] for p in range(spec.n_proj)]
            if kind == 5:               # combine: after every shrink tile of its tokens
                n_co += 1
                assert idx >= lay["n_shrink"] and ntok <= 16 and length == r
                assert int(rec[7]) == lay["n_splits"] > 1
                for t in toks:
                    assert last_shrink_of_token[int(t)] < idx
                    combine_seen[v_row[int(t)]:v_row[int(t)] + r] += 1
                    last_shrink_of_token[int(t)] = idx
                continue
            if kind == 1:               # MFMA shrink: all r rows over one K split
                n_sh += 1
                assert int(rec[9]) == lay["n_splits"] and 0 <= int(rec[7]) < lay["n_splits"]
                assert pos % 64 == 0 and length % 64 == 0 and pos + length <= spec.h_in
                for t in toks:
                    cov = k_cover.setdefault(int(t), np.zeros(spec.h_in, np.int32))
                    cov[pos:pos + length] += 1
                    if pos == 0:
                        shrink_seen[v_row[int(t)]:v_row[int(t)] + r] += 1
                    last_shrink_of_token[int(t)] = idx
                for p in range(spec.n_proj):
                    pg = rec[hdr + tokcap + p * pagecap:][:r]
                    np.testing.assert_array_equal(pg, ex["a_pages"][base[p]:base[p] + r])
                continue
            if not kind & 2:            # vector-ALU shrink
                n_sh += 1
                assert 0 <= pos and pos + length <= r
                for t in toks:
                    shrink_seen[v_row[int(t)] + pos:v_row[int(t)] + pos + length] += 1
                    last_shrink_of_token[int(t)] = idx
                for p in range(spec.n_proj):
                    pg = rec[hdr + tokcap + p * pagecap:][:length]
                    np.testing.assert_array_equal(pg, ex["a_pages"][base[p] + pos:base[p] + pos + length])
            else:                       # expand
                n_ex += 1
                assert pos % 8 == 0 and length % 8 == 0 and 0 <= pos and pos + length <= spec.h_out
                assert np.float32(rec[6:7].view(np.float32)[0]) == ex["seg_scale"][s]
                for t in toks:
                    cover[int(t)][pos:pos + length] += 1
                    assert last_shrink_of_token[int(t)] < idx   # launch order
                if not kind & 1:
                    width = int(rec[7])
                    vec = 8 if spec.dtype == "f16" else 4
                    assert width % vec == 0 and 256 % (width // vec) == 0 and length <= width
                for p in range(spec.n_proj):
                    pg = rec[hdr + tokcap + p * pagecap:][:r]
                    np.testing.assert_array_equal(pg, ex["b_pages"][base[p]:base[p] + r])
        assert n_sh == lay["n_shrink"] and n_ex == lay["n_expand"] and n_co == lay["n_combine"]
        assert (shrink_seen[:off] == 1).all()
        for cov in k_cover.values():
            assert (cov == 1).all()
        if lay["n_splits"] > 1:         # every MFMA token's v is combined exactly once
            for t in k_cover:
                assert (combine_seen[v_row[t]:v_row[t] + int(ex["seg_rank"][seg_of[t]])] == 1).all()
        for t in routed:
            assert (cover[t] == 1).all(), t
        return info
    finally:
        S.slora_segments_destroy(seg)


@pytest.mark.parametrize("name", ["tiny", "decode7b", "prefill7b", "mixed13b", "mlp70b"])
@pytest.mark.parametrize("route", ["default", "all_gemv", "all_mfma", "xcd_grouped", "rank_order",
                                   "bytes_order", "mfma_cols_1024", "mfma_cols_384"])
def test_tiles_cover_each_output_once(name, route):
    tuning = {"default": {}, "all_gemv": {S.SLORA_TUNE_MFMA_MIN_TOKENS: 1 << 30},
              "all_mfma": {S.SLORA_TUNE_MFMA_MIN_TOKENS: 1},
              "xcd_grouped": {S.SLORA_TUNE_XCDS: 8},
              "rank_order": {S.SLORA_TUNE_TILE_ORDER: 1},
              "bytes_order": {S.SLORA_TUNE_TILE_ORDER: 2},
              "mfma_cols_1024": {S.SLORA_TUNE_MFMA_EXPAND_COLS: 1024},
              "mfma_cols_384": {S.SLORA_TUNE_MFMA_EXPAND_COLS: 384}}[route]
    w = generate(CONFIGS[name], 0)
    pool, _ = make_pool(w, tuning=tuning)
    try:
        info = check_tiles_cover(w, pool, w.ids)
        if route == "all_gemv" or w.spec.dtype == "f32":
            assert info["n_mfma_segments"] == 0
        if route == "all_mfma" and w.spec.dtype == "f16":
            eligible = sum(1 for a in np.unique(w.ids[w.ids >= 0]) if w.ranks[a] <= S.SLORA_MFMA_MAX_RANK)
            assert info["n_mfma_segments"] == eligible
    finally:
        S.slora_pool_destroy(pool)


@pytest.mark.parametrize("name,tuning,want", [
    ("prefill7b", {}, 512),                                  # every segment on the MFMA tiles
    ("mixed13b", {}, 1024),                                  # vector-ALU segments beside them
    ("prefill7b", {S.SLORA_TUNE_MFMA_EXPAND_COLS: 1024}, 1024),   # an explicit width wins
    ("mixed13b", {S.SLORA_TUNE_MFMA_EXPAND_COLS: 384}, 384)])
def test_mfma_expand_width_follows_the_batch(name, tuning, want):
    w = generate(CONFIGS[name], 0)
    pool, _ = make_pool(w, tuning=tuning)
    try:
        seg = S.slora_build_segments(pool, w.ids)
        try:
            _, recs = S.slora_segments_tiles(seg)
            widths = [int(rec[4]) for rec in recs if int(rec[0]) == 3]   # MFMA expand: columns handled
            assert widths and max(widths) == want
            assert all(c == want for c in widths if c != w.spec.h_out % want)
        finally:
            S.slora_segments_destroy(seg)
    finally:
        S.slora_pool_destroy(pool)


@pytest.mark.parametrize("name,tuning,budget,pipelined", [
    ("decode7b", {}, 16384, False),      # light launch: stays within one register set of B rows
    ("mixed13b", {}, 131072, True),      # MFMA tiles beside: budget from all four projections' work
    ("mlp70b", {}, 262144, True),        # deep tiles at any budget: the cap
    ("mlp70b", {S.SLORA_TUNE_GEMV_EXPAND_ELEMS: 32768}, 32768, True)])   # an explicit budget wins
def test_vector_alu_expand_budget_follows_the_launch(name, tuning, budget, pipelined):
    """Vector-ALU expand tiles: rank x width within the chosen budget, and as
    wide as it allows (up to 8 x 256 columns); whether some thread holds more
    B rows than one register set (the pipelined kernel) follows from it."""
    w = generate(CONFIGS[name], 0)
    pool, _ = make_pool(w, tuning=tuning)
    try:
        seg = S.slora_build_segments(pool, w.ids)
        try:
            _, recs = S.slora_segments_tiles(seg)
            gemv = [(int(rec[2]), int(rec[7])) for rec in recs if int(rec[0]) == 2]   # (rank, width)
            assert gemv
            for r, width in gemv:
                assert r * width <= budget or width == 8 * 32
                assert width == 8 * 256 or r * width * 2 > budget
            deep = any(-(-r // (256 // (width // 8))) > 8 for r, width in gemv)
            assert deep == pipelined
        finally:
            S.slora_segments_destroy(seg)
    finally:
        S.slora_pool_destroy(pool)


def test_tiles_with_ragged_shapes_and_no_adapter_tokens():
    spec = small_spec("ragged", h_in=136, h_out=200, two_classes=True, n_adapters=7,
                      rank_set=(1, 3, 13, 40, 100), batch=("zipf", 60, 1.0))
    w = generate(spec, 3)
    ids = w.ids.copy()
    ids[::5] = -1
    for route in (1, 5, 1 << 30):
        pool, _ = make_pool(w, tuning={S.SLORA_TUNE_MFMA_MIN_TOKENS: route,
                                       S.SLORA_TUNE_GEMV_EXPAND_ELEMS: 1000})
        try:
            check_tiles_cover(w, pool, ids)
        finally:
            S.slora_pool_destroy(pool)


# ---------------------------------------------------------------------------
# Errors: every failure is reported and changes nothing


def small_pool(n_pages=64, n_proj=1, max_rank=8, two=False, free_order=None):
    return S.slora_pool_create(S.SLORA_F16, 16, 32 if two else 16, n_proj, 8, max_rank,
                               FAKE_BASE[:2 if two else 1], [n_pages] * (2 if two else 1),
                               free_order)


def status_of(fn, *args, **kw):
    try:
        fn(*args, **kw)
    except S.SloraError as e:
        return e.status
    return S.SLORA_OK


@pytest.mark.parametrize("kw,what", [
    (dict(dtype=7), "dtype"), (dict(h_in=12, h_out=12), "h not multiple of 8"),
    (dict(h_out=24), "one class needs h_in == h_out"), (dict(n_proj=0), "n_proj"),
    (dict(max_rank=0), "max_rank"), (dict(max_rank=300), "max_rank too big"),
    (dict(base=[(1 << 40) + 4]), "unaligned base"), (dict(base=[0]), "NULL base"),
    (dict(free_order=[[0, 0, 1, 2]]), "free order not a permutation"),
    (dict(n_pages=[0]), "no pages"), (dict(h_in=32768, h_out=32768), "h_in too large"),
])
def test_pool_create_rejects(kw, what):
    args = dict(dtype=S.SLORA_F16, h_in=16, h_out=16, n_proj=1, max_adapters=4, max_rank=4,
                base=[1 << 40], n_pages=[4], free_order=None)
    args.update(kw)
    st = status_of(S.slora_pool_create, args["dtype"], args["h_in"], args["h_out"], args["n_proj"],
                   args["max_adapters"], args["max_rank"], args["base"], args["n_pages"],
                   args["free_order"])
    assert st == S.SLORA_E_INVAL, what


def test_load_errors_leave_pool_unchanged():
    pool = small_pool(n_pages=10)
    try:
        S.slora_load_adapter(pool, 0, 4, 1.0)                       # takes 8 pages
        assert status_of(S.slora_load_adapter, pool, 0, 1, 1.0) == S.SLORA_E_EXIST
        assert status_of(S.slora_load_adapter, pool, 1, 2, 1.0) == S.SLORA_E_NOMEM
        assert status_of(S.slora_load_adapter, pool, 9, 1, 1.0) == S.SLORA_E_INVAL
        assert status_of(S.slora_load_adapter, pool, 1, 0, 1.0) == S.SLORA_E_INVAL
        assert status_of(S.slora_load_adapter, pool, 1, 9, 1.0) == S.SLORA_E_INVAL
        assert status_of(S.slora_load_adapter, pool, 1, 1, float("nan")) == S.SLORA_E_INVAL
        assert S.slora_free_count(pool, 0) == 2
        S.slora_load_adapter(pool, 1, 1, 1.0)
        assert S.slora_free_count(pool, 0) == 0
        assert status_of(S.slora_unload_adapter, pool, 2) == S.SLORA_E_NOENT
        assert status_of(S.slora_adapter_pages, pool, 2) == S.SLORA_E_NOENT
        assert "not loaded" in S.slora_last_error()
    finally:
        S.slora_pool_destroy(pool)


def test_free_pages_rejects_non_kv_and_double_free():
    pool = small_pool(n_pages=8)
    try:
        kv = S.slora_alloc_pages(pool, 0, 3)
        S.slora_load_adapter(pool, 0, 1, 1.0)
        a, _ = S.slora_adapter_pages(pool, 0)
        assert status_of(S.slora_free_pages, pool, 0, a) == S.SLORA_E_INVAL
        assert status_of(S.slora_free_pages, pool, 0, [kv[0], kv[0]]) == S.SLORA_E_INVAL
        assert status_of(S.slora_free_pages, pool, 0, [kv[1], 99]) == S.SLORA_E_INVAL
        assert status_of(S.slora_free_pages, pool, 1, [kv[1]]) == S.SLORA_E_INVAL
        assert S.slora_free_count(pool, 0) == 3
        S.slora_free_pages(pool, 0, kv[::-1])
        assert S.slora_free_count(pool, 0) == 6
        assert status_of(S.slora_free_pages, pool, 0, kv[:1]) == S.SLORA_E_INVAL
        # freed pages come back last, in the order they were returned
        assert S.slora_alloc_pages(pool, 0, 6).tolist()[-3:] == kv[::-1].tolist()
    finally:
        S.slora_pool_destroy(pool)


def test_segments_errors_and_staleness():
    pool = small_pool(n_pages=32)
    try:
        for a in range(3):
            S.slora_load_adapter(pool, a, 2, 1.0)
        assert status_of(S.slora_build_segments, pool, [0, 5]) == S.SLORA_E_NOENT
        assert status_of(S.slora_build_segments, pool, [0, 8]) == S.SLORA_E_NOENT
        seg = S.slora_build_segments(pool, [2, -1, 0, 2])
        try:
            fake = 1 << 42
            # not uploaded yet: refused before any device work
            assert status_of(S.slora_lora_delta, pool, seg, 0, fake, fake, fake, 1 << 20) == S.SLORA_E_INVAL
            assert status_of(S.slora_lora_delta, pool, seg, 1, fake, fake, fake, 1 << 20) == S.SLORA_E_INVAL
            S.slora_unload_adapter(pool, 0)
            assert status_of(S.slora_lora_delta, pool, seg, 0, fake, fake, fake, 1 << 20) == S.SLORA_E_STALE
            S.slora_load_adapter(pool, 0, 2, 1.0)   # reloaded: a new generation, still stale
            assert status_of(S.slora_lora_delta, pool, seg, 0, fake, fake, fake, 1 << 20) == S.SLORA_E_STALE
            # the launch count only moves forward and stays below 2^31
            S.slora_segments_set_launch_count(seg, 5)
            assert status_of(S.slora_segments_set_launch_count, seg, 4) == S.SLORA_E_INVAL
            assert status_of(S.slora_segments_set_launch_count, seg, 1 << 31) == S.SLORA_E_INVAL
            S.slora_segments_set_launch_count(seg, 5)
            S.slora_segments_set_launch_count(seg, (1 << 31) - 1)
        finally:
            S.slora_segments_destroy(seg)
        ex = S.slora_segments_export(seg2 := S.slora_build_segments(pool, [2, -1, 0, 2]))
        assert ex["perm"].tolist() == [2, 0, 3] and ex["seg_adapter"].tolist() == [0, 2]
        S.slora_segments_destroy(seg2)
    finally:
        S.slora_pool_destroy(pool)


def test_multi_projection_argument_errors():
    """slora_lora_delta_multi refuses bad projection lists, NULL or unaligned
    buffers and a workspace smaller than n areas before any device work."""
    pool = small_pool(n_pages=64, n_proj=3)
    try:
        for a in range(2):
            S.slora_load_adapter(pool, a, 2, 1.0)
        seg = S.slora_build_segments(pool, [1, 0, 1])
        try:
            ws = S.slora_segments_get_info(seg)["workspace_bytes"]
            fake = 1 << 42
            call = lambda projs, xs=None, ys=None, w=fake, wb=3 * ws: status_of(   # noqa: E731
                S.slora_lora_delta_multi, pool, seg, projs, xs or [fake] * len(projs),
                ys or [fake] * len(projs), w, wb)
            assert call([]) == S.SLORA_E_INVAL                       # n = 0
            assert call([0, 1, 2, 0]) == S.SLORA_E_INVAL             # more than n_proj, and a repeat
            assert call([0, 0]) == S.SLORA_E_INVAL                   # a projection twice
            assert call([0, 3]) == S.SLORA_E_INVAL                   # out of range
            assert call([2, -1]) == S.SLORA_E_INVAL
            assert call([0, 1], xs=[fake, 0]) == S.SLORA_E_INVAL     # NULL x
            assert call([0, 1], ys=[fake + 8, fake]) == S.SLORA_E_INVAL   # unaligned y
            assert call([0, 1], w=0) == S.SLORA_E_INVAL              # NULL workspace
            assert call([0, 1, 2], wb=3 * ws - 1) == S.SLORA_E_NOMEM  # n areas needed
            assert call([0, 1, 2]) == S.SLORA_E_INVAL                # not uploaded yet
            S.slora_unload_adapter(pool, 1)
            assert call([0, 1]) == S.SLORA_E_STALE
        finally:
            S.slora_segments_destroy(seg)
    finally:
        S.slora_pool_destroy(pool)


def test_empty_and_unrouted_batches_launch_nothing():
    pool = small_pool()
    try:
        S.slora_load_adapter(pool, 0, 2, 1.0)
        for ids in ([], [-1, -1, -3]):
            seg = S.slora_build_segments(pool, ids)
            try:
                info = S.slora_segments_get_info(seg)
                assert info["n_routed"] == 0 and info["n_shrink_tiles"] == 0 and info["n_expand_tiles"] == 0
                # no routed token: returns before touching the device or the pointers
                S.slora_lora_delta(pool, seg, 0, 0, 0, 0, 0)
            finally:
                S.slora_segments_destroy(seg)
    finally:
        S.slora_pool_destroy(pool)


def test_tuning_validation():
    pool = small_pool()
    try:
        assert status_of(S.slora_pool_set_tuning, pool, 0, 0) == S.SLORA_E_INVAL
        assert status_of(S.slora_pool_set_tuning, pool, S.SLORA_TUNE_GEMV_EXPAND_ELEMS, -1) == S.SLORA_E_INVAL
        S.slora_pool_set_tuning(pool, S.SLORA_TUNE_GEMV_EXPAND_ELEMS, 0)
        assert status_of(S.slora_pool_set_tuning, pool, 2, 300) == S.SLORA_E_INVAL
        assert status_of(S.slora_pool_set_tuning, pool, S.SLORA_TUNE_MFMA_EXPAND_COLS, -128) == S.SLORA_E_INVAL
        assert status_of(S.slora_pool_set_tuning, pool, S.SLORA_TUNE_MFMA_EXPAND_COLS, 65536 + 128) == S.SLORA_E_INVAL
        S.slora_pool_set_tuning(pool, S.SLORA_TUNE_MFMA_EXPAND_COLS, 512)
        S.slora_pool_set_tuning(pool, S.SLORA_TUNE_MFMA_EXPAND_COLS, 0)
        assert status_of(S.slora_pool_set_tuning, pool, 11, 1) == S.SLORA_E_INVAL
        assert status_of(S.slora_pool_set_tuning, pool, S.SLORA_TUNE_FWD_KSPLIT, 3) == S.SLORA_E_INVAL
        assert status_of(S.slora_pool_set_tuning, pool, S.SLORA_TUNE_FWD_KSPLIT, -1) == S.SLORA_E_INVAL
        S.slora_pool_set_tuning(pool, S.SLORA_TUNE_FWD_KSPLIT, 2)
        assert status_of(S.slora_pool_set_tuning, pool, S.SLORA_TUNE_SHRINK_ROWS, 17) == S.SLORA_E_INVAL
        S.slora_pool_set_tuning(pool, S.SLORA_TUNE_SHRINK_ROWS, 2)
        assert status_of(S.slora_pool_set_tuning, pool, 99, 1) == S.SLORA_E_INVAL
        assert status_of(S.slora_pool_set_tuning, pool, S.SLORA_TUNE_FUSED, 2) == S.SLORA_E_INVAL
        assert status_of(S.slora_pool_set_tuning, pool, S.SLORA_TUNE_XCDS, 65) == S.SLORA_E_INVAL
        assert status_of(S.slora_pool_set_tuning, pool, S.SLORA_TUNE_XCDS, 0) == S.SLORA_E_INVAL
        S.slora_pool_set_tuning(pool, S.SLORA_TUNE_XCDS, 8)
        assert status_of(S.slora_pool_set_tuning, pool, S.SLORA_TUNE_TILE_ORDER, 3) == S.SLORA_E_INVAL
        S.slora_pool_set_tuning(pool, S.SLORA_TUNE_TILE_ORDER, 1)
        assert status_of(S.slora_pool_set_tuning, pool, S.SLORA_TUNE_FWD_TILE, 48) == S.SLORA_E_INVAL
        assert status_of(S.slora_pool_set_tuning, pool, S.SLORA_TUNE_FWD_TILE, 16) == S.SLORA_E_INVAL
        S.slora_pool_set_tuning(pool, S.SLORA_TUNE_FWD_TILE, 32)
        S.slora_pool_set_tuning(pool, S.SLORA_TUNE_FWD_TILE, 64)
        assert status_of(S.slora_pool_set_tuning, pool, S.SLORA_TUNE_FWD_GROUP, -1) == S.SLORA_E_INVAL
        S.slora_pool_set_tuning(pool, S.SLORA_TUNE_FWD_TILE, 256)
        S.slora_pool_set_tuning(pool, S.SLORA_TUNE_FWD_GROUP, 4)
        S.slora_pool_set_tuning(pool, 2, 1024)
    finally:
        S.slora_pool_destroy(pool)


def test_unload_reload_lands_on_other_pages():
    """Unloading returns pages to the tail, so a reload takes different pages."""
    pool = small_pool(n_pages=16)
    try:
        S.slora_load_adapter(pool, 0, 2, 1.0)
        a1, b1 = S.slora_adapter_pages(pool, 0)
        S.slora_unload_adapter(pool, 0)
        S.slora_load_adapter(pool, 0, 2, 1.0)
        a2, b2 = S.slora_adapter_pages(pool, 0)
        assert set(a1.tolist() + b1.tolist()).isdisjoint(a2.tolist() + b2.tolist())
    finally:
        S.slora_pool_destroy(pool)


def test_no_mfma_under_partial_exec_mask(tmp_path):
    """Every matrix instruction sits in wave-uniform control flow (see build.masked_mfma_lines)."""
    from rank_gemm_page_amd import build
    for src in ("slora_kernels.hip", "slora_forward.hip"):
        asm = build.device_assembly(str(tmp_path), src)
        with open(asm) as f:
            assert sum(1 for line in f if line.strip().startswith("v_mfma")) > 0, src
        assert build.masked_mfma_lines(asm) == [], src


@pytest.mark.parametrize("kw", [dict(dtype="f32", rank_set=(4, 8)),
                                dict(dtype="f16", h_out=384, two_classes=True, n_proj=2,
                                     proj_x=(0, 0), rank_set=(1, 8, 16))])
def test_adapter_image_matches_oracle_pages(kw):
    """Each row of a packed image equals the oracle's pool row of the page the
    allocator gives it (A^T row j = column j of A; B row j = row j of B)."""
    w = generate(small_spec("image", **kw), seed=3)
    st = orc.build_from_workload(w)
    pool, _ = make_pool(w)
    spec, e = w.spec, np.dtype(w.np_dtype).itemsize
    uint = np.uint16 if e == 2 else np.uint32
    try:
        for a in range(spec.n_adapters):
            r = int(w.ranks[a])
            nb = S.slora_adapter_image_bytes(pool, r)
            rows = spec.n_proj * r
            used = rows * (spec.h_in + spec.h_out) * e + 2 * rows * 4
            assert nb == (used + 255) // 256 * 256
            img = np.zeros(nb, np.uint8)
            A = [w.weights(a, p)[0] for p in range(spec.n_proj)]
            B = [w.weights(a, p)[1] for p in range(spec.n_proj)]
            S.slora_pack_adapter(pool, r, A, B, img.ctypes.data, nb)
            a_bytes = rows * spec.h_in * e
            ent = st.alloc.table[a]
            for p in range(spec.n_proj):
                for j in range(r):
                    off = ((p * r) + j) * spec.h_in * e
                    got = img[off:off + spec.h_in * e].view(uint)
                    assert np.array_equal(got, st.image.row(0, ent.a_pages[p][j]).view(uint)), (a, p, j)
                    off = a_bytes + ((p * r) + j) * spec.h_out * e
                    got = img[off:off + spec.h_out * e].view(uint)
                    want = st.image.row(st.alloc.b_class(), ent.b_pages[p][j]).view(uint)
                    assert np.array_equal(got, want), (a, p, j)
    finally:
        S.slora_pool_destroy(pool)


def test_async_load_argument_errors_leave_pool_unchanged():
    """Every batch-level check of slora_load_adapters_async runs before any
    device call, and a refused batch takes no page."""
    pool = small_pool(n_pages=10)
    img = np.zeros(1 << 16, np.uint8)
    im = img.ctypes.data
    dev, big = 1 << 40, 1 << 20
    try:
        assert S.slora_adapter_image_bytes(pool, 0) == 0
        assert S.slora_adapter_image_bytes(pool, 9) == 0
        assert status_of(S.slora_pack_adapter, pool, 2, [np.zeros((16, 2), np.float16)],
                         [np.zeros((2, 16), np.float16)], im, 64) == S.SLORA_E_INVAL
        S.slora_load_adapter(pool, 0, 4, 1.0)                       # 2 pages stay free
        bad = [([0], [1], [1.0], [im], dev, big, S.SLORA_E_EXIST),
               ([1], [2], [1.0], [im], dev, big, S.SLORA_E_NOMEM),
               ([1, 2], [1, 1], [1.0, 1.0], [im, im], dev, big, S.SLORA_E_NOMEM),
               ([9], [1], [1.0], [im], dev, big, S.SLORA_E_INVAL),
               ([1], [0], [1.0], [im], dev, big, S.SLORA_E_INVAL),
               ([1], [1], [float("inf")], [im], dev, big, S.SLORA_E_INVAL),
               ([1], [1], [1.0], [0], dev, big, S.SLORA_E_INVAL),
               ([1], [1], [1.0], [im], 0, big, S.SLORA_E_INVAL),
               ([1, 1], [1, 1], [1.0, 1.0], [im, im], dev, big, S.SLORA_E_INVAL),
               ([1], [1], [1.0], [im], dev, 16, S.SLORA_E_INVAL)]
        for ids, ranks, scales, ims, d, nb, want in bad:
            got = status_of(S.slora_load_adapters_async, pool, ids, ranks, scales, ims, d, nb)
            assert got == want, (ids, ranks)
            assert S.slora_free_count(pool, 0) == 2
        S.slora_load_adapters_async(pool, [], [], [], [], dev, 0)    # empty batch: nothing
        assert S.slora_free_count(pool, 0) == 2
    finally:
        S.slora_pool_destroy(pool)


def test_forward_noalloc_refuses_batches_beyond_its_array():
    """The no-allocation forward's workspace is an 8 MiB device array: a batch
    whose workspace_bytes exceed it is refused before any device work."""
    pool = S.slora_pool_create(S.SLORA_F16, 512, 512, 1, 4, 64, FAKE_BASE[:1], [256], None)
    try:
        S.slora_load_adapter(pool, 0, 64, 1.0)
        seg = S.slora_build_segments(pool, [0] * 10000)    # 64-token MFMA blocks split over K
        try:
            info = S.slora_segments_get_info(seg)
            assert info["workspace_bytes"] > 8 << 20
            fake = 1 << 42
            assert status_of(S.slora_lora_forward_noalloc, pool, seg, 0, fake, fake, fake) == S.SLORA_E_NOMEM
            assert "8388608" in S.slora_last_error()
        finally:
            S.slora_segments_destroy(seg)
        assert status_of(S.slora_lora_forward_noalloc, None, None, 0, 0, 0, 0) == S.SLORA_E_INVAL
    finally:
        S.slora_pool_destroy(pool)


def test_forward_argument_errors():
    """slora_lora_forward refuses what its kernel cannot do before any device work."""
    fake = 1 << 42
    # fp32 pools and shapes off the 64 / 128 grid
    p32 = S.slora_pool_create(S.SLORA_F32, 64, 128, 1, 4, 8, FAKE_BASE, [16, 16], None)
    p16_bad = S.slora_pool_create(S.SLORA_F16, 64, 64 + 8, 1, 4, 8, FAKE_BASE, [16, 16], None)
    p16 = S.slora_pool_create(S.SLORA_F16, 64, 128, 1, 4, 8, FAKE_BASE, [16, 16], None)
    try:
        for pool in (p32, p16_bad, p16):
            S.slora_load_adapter(pool, 0, 3, 1.0)
        for pool in (p32, p16_bad):
            seg = S.slora_build_segments(pool, [0, -1])
            try:
                assert status_of(S.slora_lora_forward, pool, seg, 0, fake, fake, fake, fake, 1 << 20) == S.SLORA_E_INVAL
            finally:
                S.slora_segments_destroy(seg)
        seg = S.slora_build_segments(p16, [0, -1, 0])
        try:
            args = dict(x=fake, w=fake, y=fake, workspace=fake, workspace_bytes=1 << 20)
            call = lambda **kw: status_of(S.slora_lora_forward, p16, seg, kw.pop("proj", 0),
                                          **{**args, **kw})
            assert call() == S.SLORA_E_INVAL                      # not uploaded
            assert call(proj=1) == S.SLORA_E_INVAL                # no such projection
            assert call(w=0) == S.SLORA_E_INVAL                   # NULL weight
            assert call(y=fake + 4) == S.SLORA_E_INVAL            # unaligned output
            assert call(workspace_bytes=4) == S.SLORA_E_NOMEM     # workspace too small
            S.slora_unload_adapter(p16, 0)
            assert call() == S.SLORA_E_STALE
        finally:
            S.slora_segments_destroy(seg)
        # an empty batch launches nothing and touches no pointer
        seg = S.slora_build_segments(p16, [])
        try:
            S.slora_lora_forward(p16, seg, 0, 0, 0, 0, 0, 0)
        finally:
            S.slora_segments_destroy(seg)
    finally:
        for pool in (p32, p16_bad, p16):
            S.slora_pool_destroy(pool)


def test_probe_argument_errors():
    """The bandwidth probes refuse bad arguments before any launch."""
    fake = 1 << 42
    read = lambda **kw: status_of(S.slora_probe_read, **{**dict(src=fake, nbytes=4096, items=4,
                                                                   nontemporal=True, sink=fake), **kw})
    assert read(items=3) == S.SLORA_E_INVAL
    assert read(nbytes=4100) == S.SLORA_E_INVAL
    assert read(nbytes=0) == S.SLORA_E_INVAL
    assert read(src=fake + 8) == S.SLORA_E_INVAL
    assert read(sink=0) == S.SLORA_E_INVAL
    row = (fake, 8192, 8192, fake, 4)
    gather = lambda arrays, items=4, sink=fake: status_of(S.slora_probe_gather, arrays, items, sink)
    assert gather([row], items=5) == S.SLORA_E_INVAL
    assert gather([(fake, 8192, 8200, fake, 4)]) == S.SLORA_E_INVAL       # row longer than its stride
    assert gather([(fake, 8192, 8184, fake, 4)]) == S.SLORA_E_INVAL       # row not whole 16-byte chunks
    assert gather([(fake, 8192, 8192, 0, 4)]) == S.SLORA_E_INVAL          # NULL row ids
    assert gather([(fake, 8192, 8192, fake, 0)]) == S.SLORA_E_INVAL       # no rows
    assert gather([row, (0, 8192, 8192, fake, 2)]) == S.SLORA_E_INVAL     # NULL second array
    assert gather([row], sink=0) == S.SLORA_E_INVAL


@pytest.mark.parametrize("seed", range(12))
def test_allocator_random_operations_match_oracle(seed):
    """Random sequences of adapter loads and unloads and KV allocations and
    frees, one or two page classes, one to three projections: after every
    operation the library's block table and free counts equal the oracle's
    allocator model, failed operations leave both unchanged, and the free
    lists drain in the same order at the end.  Every few operations a random
    batch's segment metadata is compared with the oracle's segment model."""
    rng = np.random.default_rng(seed)
    two = bool(seed % 2)
    n_proj = 1 + seed % 3
    n_pages = [int(rng.integers(40, 160))] + ([int(rng.integers(40, 160))] if two else [])
    orders = [rng.permutation(P).astype(np.int32) for P in n_pages]
    n_adapters, max_rank = 12, 9
    model = orc.AllocatorModel(n_pages, [o.tolist() for o in orders], n_proj=n_proj, two_classes=two)
    pool = S.slora_pool_create(S.SLORA_F16, 8, 16 if two else 8, n_proj, n_adapters, max_rank,
                               FAKE_BASE[:len(n_pages)], n_pages, orders)
    kv = [[] for _ in n_pages]          # KV pages held, per class
    try:
        for step in range(160):
            op = rng.integers(0, 5)
            if op <= 1:                                      # load
                a = int(rng.integers(0, n_adapters))
                r = int(rng.integers(1, max_rank + 1))
                s = float(rng.choice([0.5, 1.0, 2.0]))
                if a in model.table:
                    assert status_of(S.slora_load_adapter, pool, a, r, s) == S.SLORA_E_EXIST
                    continue
                try:
                    entry = model.load(a, r, s)
                except orc.OracleError:
                    assert status_of(S.slora_load_adapter, pool, a, r, s) == S.SLORA_E_NOMEM
                else:
                    S.slora_load_adapter(pool, a, r, s)
                    for p in range(n_proj):
                        ga, gb = S.slora_adapter_pages(pool, a, p)
                        assert ga.tolist() == entry.a_pages[p] and gb.tolist() == entry.b_pages[p], (seed, step)
            elif op == 2:                                    # unload
                a = int(rng.integers(0, n_adapters))
                if a in model.table:
                    model.unload(a)
                    S.slora_unload_adapter(pool, a)
                else:
                    assert status_of(S.slora_unload_adapter, pool, a) == S.SLORA_E_NOENT
            elif op == 3:                                    # KV allocation
                c = int(rng.integers(0, len(n_pages)))
                n = int(rng.integers(1, 12))
                if n > len(model.free[c]):
                    assert status_of(S.slora_alloc_pages, pool, c, n) == S.SLORA_E_NOMEM
                else:
                    want = model.alloc(c, n)
                    assert S.slora_alloc_pages(pool, c, n).tolist() == want, (seed, step)
                    kv[c].extend(want)
            else:                                            # KV free, a random subset in random order
                c = int(rng.integers(0, len(n_pages)))
                if kv[c]:
                    k = int(rng.integers(1, len(kv[c]) + 1))
                    pick = [kv[c][i] for i in rng.permutation(len(kv[c]))[:k]]
                    for p in pick:
                        kv[c].remove(p)
                    model.release(c, pick)
                    S.slora_free_pages(pool, c, pick)
            assert [S.slora_free_count(pool, c) for c in range(len(n_pages))] == \
                [len(f) for f in model.free], (seed, step)
            if step % 20 == 19 and model.table:              # a batch over the loaded adapters
                loaded = sorted(model.table)
                ids = rng.choice(loaded + [-1], size=int(rng.integers(1, 40))).astype(np.int32)
                ref = orc.segment_model(ids, model)
                seg = S.slora_build_segments(pool, ids)
                try:
                    ex = S.slora_segments_export(seg)
                    np.testing.assert_array_equal(ex["perm"], ref.perm)
                    np.testing.assert_array_equal(ex["seg_start"], ref.seg_start)
                    np.testing.assert_array_equal(ex["seg_adapter"], ref.seg_adapter)
                    np.testing.assert_array_equal(ex["seg_rank"], ref.seg_rank)
                    np.testing.assert_array_equal(ex["a_pages"], ref.a_pages)
                    np.testing.assert_array_equal(ex["b_pages"], ref.b_pages)
                finally:
                    S.slora_segments_destroy(seg)
        for c in range(len(n_pages)):                        # the free lists drain in the same order
            assert S.slora_alloc_pages(pool, c, len(model.free[c])).tolist() == list(model.free[c])
    finally:
        S.slora_pool_destroy(pool)


def test_missing_library_fails_loudly(tmp_path):
    """With no built library the binding raises on first use; nothing falls
    back to a CPU computation."""
    import subprocess
    import sys
    code = ("from rank_gemm_page_amd import slora as S\n"
            "try:\n"
            "    S.slora_pool_create(S.SLORA_F16, 8, 8, 1, 2, 2, [1 << 40], [16], None)\n"
            "except ImportError as e:\n"
            "    print('raised:', e)\n"
            "else:\n"
            "    print('no error')\n")
    env = dict(os.environ, SLORA_LIB=str(tmp_path / "libslora_absent.so"))
    res = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                         timeout=120)
    assert res.returncode == 0, res.stderr
    assert "raised:" in res.stdout and "is missing" in res.stdout, res.stdout
