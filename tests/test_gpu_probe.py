"""The bandwidth probes (include/slora_probe.h) on an MI355X: every 16-byte
chunk they are asked to read is read, and nothing else.

The probes xor what each thread loads and store it only when it equals one
fixed pattern.  With all memory zero and that pattern planted in one chunk,
the store runs exactly when the chunk is read: a planted chunk inside the
requested range (or a listed row) must show up in the sink, one outside it
must not.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from rank_gemm_page_amd import slora as S  # noqa: E402

pytestmark = pytest.mark.gpu

MAGIC = np.array([0x5A5A5A5A, 0xA5A5A5A5, 0x0F0F0F0F, 0xF0F0F0F0], dtype=np.uint32).view(np.int32)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.lib()


def planted(buf_i32, chunk):
    buf_i32.zero_()
    buf_i32[chunk * 4:(chunk + 1) * 4] = torch.from_numpy(MAGIC).to(buf_i32.device)


def sink_hit(sink):
    torch.cuda.synchronize()
    got = sink.cpu().numpy()
    if not got.any():
        return False
    np.testing.assert_array_equal(got, MAGIC)
    return True


@pytest.mark.parametrize("items", [1, 4, 16])
@pytest.mark.parametrize("nt", [False, True])
def test_read_probe_reads_exactly_its_range(items, nt):
    n_chunks = 256 * items * 3 + 37                     # a ragged last workgroup
    buf = torch.zeros((n_chunks + 64) * 4, dtype=torch.int32, device="cuda:0")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda:0")
    print(f"[gpu] probe read items={items} nt={nt} chunks={n_chunks}", flush=True)
    for chunk, inside in ((0, True), (n_chunks - 1, True), (n_chunks // 2 + 5, True), (n_chunks, False),
                          (n_chunks + 63, False)):
        planted(buf, chunk)
        sink.zero_()
        S.slora_probe_read(buf, n_chunks * 16, items, nt, sink)
        assert sink_hit(sink) == inside, (chunk, inside)


@pytest.mark.parametrize("items", [1, 2, 8, 16])
def test_gather_probe_reads_exactly_the_listed_rows(items):
    """Two arrays: short rows (several per workgroup) and long ragged rows
    (pieces of one row per workgroup at small items), rows listed out of order."""
    dev = "cuda:0"
    rng = np.random.default_rng(items)
    shapes = [(40, 8192 + 256, 8192), (12, 3600 * 16, 3590 * 16)]   # (rows, stride bytes, row bytes)
    bufs = [torch.zeros(n * st // 4, dtype=torch.int32, device=dev) for n, st, _ in shapes]
    lists = [rng.choice(shapes[0][0], size=23, replace=False), rng.choice(shapes[1][0], size=5, replace=False)]
    rows = [torch.from_numpy(l.astype(np.int32)).to(dev) for l in lists]
    arrays = [(bufs[a], shapes[a][1], shapes[a][2], rows[a], len(lists[a])) for a in range(2)]
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    print(f"[gpu] probe gather items={items}", flush=True)
    for a in range(2):
        n, st, rb = shapes[a]
        listed = set(int(r) for r in lists[a])
        unlisted = sorted(set(range(n)) - listed)
        cases = [(int(lists[a][0]), 0, True), (int(lists[a][-1]), rb // 16 - 1, True),
                 (int(lists[a][len(lists[a]) // 2]), rb // 32 + 3, True),
                 (unlisted[0], 0, False), (int(lists[a][0]), rb // 16, False)]   # past the row's end
        for row, col, inside in cases:
            for b in bufs:
                b.zero_()
            planted(bufs[a], (row * st) // 16 + col)
            sink.zero_()
            S.slora_probe_gather(arrays, items, sink)
            assert sink_hit(sink) == inside, (a, row, col, inside)
        # one array alone
        planted(bufs[a], (int(lists[a][0]) * st) // 16)
        sink.zero_()
        S.slora_probe_gather([arrays[a]], items, sink)
        assert sink_hit(sink)
