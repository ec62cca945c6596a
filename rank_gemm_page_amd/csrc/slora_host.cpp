// Host runtime of the paged LoRA delta: unified page pool with FIFO free lists
// and a block table, the adapter loader, the segment builder and tile lists,
// and the C ABI declared in include/slora.h.
//
// S-LoRA pages this follows:
//  * one pool hands out pages to KV blocks and to LoRA factors of varying
//    rank, and a block table maps logical tensors to physical pages (summary
//    page "S-LoRA: Serving Thousands of Concurrent LoRA Adapters", "Unified
//    Paging"; blog page section 2: adapter weights in non-contiguous blocks);
//  * adapters stay in host memory and only those a batch needs are copied to
//    the device; unused ones leave it (summary page, "Host-resident adapter
//    store" and walkthrough steps 2 and 4);
//  * a batch mixes adapters and ranks and is computed by kernels that gather
//    non-contiguous pages (summary page, "Heterogeneous batching kernels";
//    blog page section 3: the kernel matches each request's hidden state to
//    its adapter's pages in the paging table).
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <array>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "slora.h"
#include "slora_internal.h"

using namespace slora;

namespace {

thread_local std::string g_last_error;

slora_status fail(slora_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

slora_status hip_fail(hipError_t e, const char* what) {
  return fail(SLORA_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

int elem_bytes(int32_t dtype) { return dtype == SLORA_F16 ? 2 : 4; }

// FIFO free list of one page class as a ring over [0, capacity).
struct FreeRing {
  std::vector<int32_t> buf;
  int64_t head = 0, count = 0;
  int64_t cap() const { return (int64_t)buf.size(); }
  int32_t pop_front() {
    const int32_t v = buf[head];
    head = (head + 1 == cap()) ? 0 : head + 1;
    --count;
    return v;
  }
  void push_back(int32_t v) {
    int64_t pos = head + count;
    if (pos >= cap()) pos -= cap();
    buf[pos] = v;
    ++count;
  }
  void push_front(int32_t v) {
    head = (head == 0) ? cap() - 1 : head - 1;
    buf[head] = v;
    ++count;
  }
};

enum : uint8_t { PAGE_FREE = 0, PAGE_KV = 1, PAGE_ADAPTER = 2 };

struct AdapterRec {
  bool loaded = false;
  int32_t rank = 0;
  float scale = 0.f;
  uint64_t gen = 0;
  std::vector<int32_t> a_pages;  // [n_proj][rank]
  std::vector<int32_t> b_pages;  // [n_proj][rank]
};

// Defaults chosen by measurement on MI355X (decode, prefill and 70B-MLP
// shapes): segments below 64 tokens stream faster through the vector-ALU
// tiles, which cut their work finer; long segments need the matrix cores.
struct Tuning {
  int64_t mfma_min_tokens = 64;
  int64_t gemv_expand_elems = 0;   // 0: sized from the batch (auto_expand_elems)
  int64_t mfma_expand_cols = 0;    // 0: 512 when every segment takes the MFMA tiles, else 1024
  int64_t mfma_shrink_splits = 0;   // K splits per MFMA shrink block (0: automatic)
  int64_t fused = 1;
  int64_t xcds = 1;             // XCD groups of the shrink placement (1: none)
  int64_t tile_order = 2;       // 0: segment order, 1: rank-descending, 2: bytes-descending
  int64_t fwd_group = 0;        // row blocks per group of the base-plus-delta tile order (0: automatic)
  int64_t fwd_tile = 0;         // base-plus-delta tile rows: 32, 64, 128, 256, or 0 (automatic)
  int64_t fwd_ksplit = 0;       // wave groups splitting a base-plus-delta tile's steps: 1, 2, or 0 (automatic)
  int64_t shrink_rows = 0;      // rank rows per vector-ALU shrink tile (0: as many as fit)
};

// GEMV shrink geometry: chunks of 16 bytes per thread per row, as a power of
// two (the kernel instantiates 1, 2, 4, 8), and the rank rows per tile.
int shrink_nck(int32_t dtype, int32_t h_in) {
  const int vec = dtype == SLORA_F16 ? 8 : 4;
  const int per = (h_in / vec + kThreads - 1) / kThreads;
  int nck = 1;
  while (nck < per) nck *= 2;
  return nck;
}

}  // namespace

void slora::set_last_error(const char* msg) { g_last_error = msg; }

struct slora_pool {
  slora_pool_desc d{};
  int elem = 2;
  int64_t page_elems[2] = {0, 0};
  int64_t page_bytes[2] = {0, 0};
  FreeRing free_list[2];
  std::vector<uint8_t> state[2];
  std::vector<AdapterRec> adapters;
  uint64_t gen_counter = 0;
  Tuning tune;
  // synchronous-load staging: one adapter image of max_rank, pinned on the
  // host and on the device (allocated on the first load with data)
  int device = -1;
  char* h_stage = nullptr;
  char* d_stage = nullptr;
  size_t stage_bytes = 0;
  // metadata upload arena (pinned, two slots used in turn)
  char* h_meta[2] = {nullptr, nullptr};
  size_t h_meta_bytes[2] = {0, 0};
  hipEvent_t meta_done[2] = {nullptr, nullptr};
  int meta_slot = 0;
  // counting-sort scratch, all zero between builds
  std::vector<int32_t> count_scratch;

  int n_classes() const { return d.n_classes; }
  int b_class() const { return d.n_classes == 2 ? 1 : 0; }
};

struct slora_segments {
  slora_pool* pool = nullptr;
  int32_t n_tokens = 0;
  int32_t n_proj = 1;
  std::vector<int32_t> perm, seg_start, seg_adapter, seg_rank, seg_page_off, a_pages, b_pages;
  std::vector<float> seg_scale;
  std::vector<uint64_t> seg_gen;
  std::vector<int64_t> seg_v_off;
  int64_t sum_r = 0, sum_rt = 0;
  int32_t n_mfma_segments = 0;
  int32_t n_combine = 0;           // combine tiles (MFMA shrink blocks split over K)
  int32_t n_splits = 1;            // K splits of the MFMA shrink blocks (1: none)
  // tile records: shrink records, then expand records
  std::vector<int32_t> blob;
  int32_t n_tiles = 0, n_shrink = 0, n_expand = 0;
  int32_t stride = 0, tokcap = 0, pagecap = 0;
  int64_t shrink_idx_off_words = 0, expand_idx_off_words = 0;
  std::vector<int32_t> phase_rec;   // record runs of one tile kind (fused launch phases), with the end
  int64_t records_words = 0;       // records and index lists (the uploaded part)
  // Base-plus-delta table (uploaded after the index lists): batch order of
  // the sorted positions, segment of each routed position, per-segment
  // start, rank, scale and v offset, per row block its LoRA stages, and the
  // LoRA stage entries of every projection.
  int64_t fw_order_off = 0, fw_pos_seg_off = 0, fw_seg_start_off = 0, fw_seg_rank_off = 0;
  int64_t fw_seg_scale_off = 0, fw_seg_v_off = 0, fw_rb_info_off = 0, fw_stages_off = 0;
  int32_t fw_n_rb = 0, fw_n_stages = 0;
  // Sorted positions 0 .. fw_big_rows go in 256 x 256 tiles (fw_n_rb_big row
  // blocks), the rest in 128 x 128 tiles; fw_n_rb counts both kinds.
  int32_t fw_big_rows = 0, fw_n_rb_big = 0;
  int32_t fw_small_bm = kFwdBM;    // rows of the small tiles (128, or 64 / 32 for batches below one tile per CU)
  bool fw_packed = false;          // LoRA stages in the packed layout (batches without 256-row tiles)
  int64_t error_off_words = 0;     // one error word (zeroed on device at upload), padding
  int64_t vtag_off_words = 0;      // fused-launch v pairs (zeroed on device at upload)
  int32_t gemv_rows = 0;
  bool pipe_expand = false;        // a vector-ALU expand thread holds more than kExpandRowSet B rows
  const int32_t* dev_meta = nullptr;
  mutable uint32_t epoch = 0;      // fused launches since the last upload
};

namespace {

// Device metadata: the tile records, an error word, then 8 bytes per
// (token, rank row) of v pairs for the fused launch.
// One exchange area of n_splits x sum_rt pairs per projection.
int64_t vtag_words_of(const slora_segments* s) { return (int64_t)s->n_proj * s->n_splits * s->sum_rt * 2; }

// Workspace of one projection: the x A products and their K-split partials.
size_t workspace_bytes_of(const slora_segments* s) {
  return std::max<size_t>(16, (size_t)s->n_splits * s->sum_rt * sizeof(float));
}

size_t meta_bytes_of(const slora_segments* s) {
  return (size_t)(s->vtag_off_words + vtag_words_of(s)) * 4;
}

slora_status set_device(slora_pool* p) {
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (p->device < 0) p->device = cur;
  if (cur != p->device) {
    e = hipSetDevice(p->device);
    if (e != hipSuccess) return hip_fail(e, "hipSetDevice");
  }
  return SLORA_OK;
}

// Adapter image: the byte layout shared by the synchronous load's pinned
// staging buffer and the caller's images for slora_load_adapters_async.
struct ImageLayout {
  size_t a_bytes;     // n_proj x rank A^T rows of h_in elements
  size_t rows_bytes;  // + n_proj x rank B rows of h_out elements
  size_t ids_off;     // 2 x n_proj x rank int32 page ids (A^T pages, then B pages)
  size_t used;        // bytes the load copies to the device
  size_t total;       // used, rounded up to 256
};

ImageLayout image_layout(const slora_pool* p, int32_t rank) {
  ImageLayout L;
  const size_t rows = (size_t)p->d.n_proj * (size_t)rank;
  L.a_bytes = rows * (size_t)p->d.h_in * (size_t)p->elem;
  L.rows_bytes = L.a_bytes + rows * (size_t)p->d.h_out * (size_t)p->elem;
  L.ids_off = L.rows_bytes;   // a multiple of 16: h_in and h_out are multiples of 8
  L.used = L.ids_off + 2 * rows * sizeof(int32_t);
  L.total = (L.used + 255) / 256 * 256;
  return L;
}

slora_status ensure_stage(slora_pool* p) {
  if (p->h_stage) return SLORA_OK;
  slora_status st = set_device(p);
  if (st != SLORA_OK) return st;
  const size_t bytes = image_layout(p, p->d.max_rank).total;
  hipError_t e = hipHostMalloc((void**)&p->h_stage, bytes, hipHostMallocDefault);
  if (e != hipSuccess) { p->h_stage = nullptr; return hip_fail(e, "hipHostMalloc(load staging)"); }
  e = hipMalloc((void**)&p->d_stage, bytes);
  if (e != hipSuccess) {
    (void)hipHostFree(p->h_stage);
    p->h_stage = nullptr; p->d_stage = nullptr;
    return hip_fail(e, "hipMalloc(load staging)");
  }
  p->stage_bytes = bytes;
  return SLORA_OK;
}

// A^T row j of projection p is column j of the h_in x rank row-major A[p];
// the transpose goes in blocks of 64 source rows to stay in cache.
template <typename E>
void transpose_into(E* dst, const E* src, int64_t hin, int32_t r) {
  constexpr int64_t KB = 64;
  for (int64_t k0 = 0; k0 < hin; k0 += KB) {
    const int64_t k1 = std::min(hin, k0 + KB);
    for (int32_t j = 0; j < r; ++j) {
      E* d = dst + (size_t)j * hin;
      for (int64_t k = k0; k < k1; ++k) d[k] = src[(size_t)k * r + j];
    }
  }
}

slora_status pack_image(const slora_pool* p, int32_t r, const void* const* A, const void* const* B,
                        char* image, const char* fn) {
  const int np = p->d.n_proj, e = p->elem;
  const int64_t hin = p->d.h_in, hout = p->d.h_out;
  const ImageLayout L = image_layout(p, r);
  for (int pr = 0; pr < np; ++pr)
    if (!A[pr] || !B[pr]) return fail(SLORA_E_INVAL, std::string(fn) + ": NULL A[p] or B[p]");
  for (int pr = 0; pr < np; ++pr) {
    char* dst = image + (size_t)pr * r * hin * e;
    if (e == 2)
      transpose_into(reinterpret_cast<uint16_t*>(dst), static_cast<const uint16_t*>(A[pr]), hin, r);
    else
      transpose_into(reinterpret_cast<uint32_t*>(dst), static_cast<const uint32_t*>(A[pr]), hin, r);
    std::memcpy(image + L.a_bytes + (size_t)pr * r * hout * e, B[pr], (size_t)r * hout * e);
  }
  return SLORA_OK;
}

// Put pages taken for a failed load back at the head, newest first, so the
// free list is exactly as before.
void rollback_pages(slora_pool* p, const AdapterRec& rec) {
  for (int pr = p->d.n_proj - 1; pr >= 0; --pr) {
    for (int j = rec.rank - 1; j >= 0; --j) {
      const int32_t b = rec.b_pages[(size_t)pr * rec.rank + j];
      p->state[p->b_class()][b] = PAGE_FREE;
      p->free_list[p->b_class()].push_front(b);
    }
    for (int j = rec.rank - 1; j >= 0; --j) {
      const int32_t a = rec.a_pages[(size_t)pr * rec.rank + j];
      p->state[0][a] = PAGE_FREE;
      p->free_list[0].push_front(a);
    }
  }
}

// For each adapter k: write its page ids into images[k] and queue on `stream`
// the copy of the image to dev_stage + (sum of the earlier images' sizes);
// then queue the scatters of all rows into their pages, kMaxFetch adapters
// per launch.  All copies go first so the copy engine runs them back to back.
// On a failure, whatever was already queued is waited for before returning,
// so that the caller can give the pages back (and reuse the staging) without
// a queued copy or scatter still reading or writing them.
slora_status enqueue_images(slora_pool* p, const std::vector<const AdapterRec*>& recs,
                            char* const* images, char* dev_stage, hipStream_t stream) {
  bool queued = false;
  auto failed = [&](hipError_t he, const char* what) {
    if (queued) {
      (void)hipStreamSynchronize(stream);
      (void)hipGetLastError();
    }
    return hip_fail(he, what);
  };
  const int np = p->d.n_proj;
  const size_t n = recs.size();
  std::vector<size_t> off(n + 1, 0);
  for (size_t k = 0; k < n; ++k) {
    const AdapterRec& rec = *recs[k];
    const int r = rec.rank;
    const ImageLayout L = image_layout(p, r);
    int32_t* ids = reinterpret_cast<int32_t*>(images[k] + L.ids_off);
    std::memcpy(ids, rec.a_pages.data(), (size_t)np * r * sizeof(int32_t));
    std::memcpy(ids + (size_t)np * r, rec.b_pages.data(), (size_t)np * r * sizeof(int32_t));
    hipError_t he = hipMemcpyAsync(dev_stage + off[k], images[k], L.used, hipMemcpyHostToDevice, stream);
    if (he != hipSuccess) return failed(he, "hipMemcpyAsync(adapter image)");
    queued = true;
    off[k + 1] = off[k] + L.total;
  }
  for (size_t k0 = 0; k0 < n; k0 += kMaxFetch) {
    ScatterLaunch S{};
    S.stage = dev_stage;
    S.n = (int32_t)std::min<size_t>(kMaxFetch, n - k0);
    S.n_proj = np;
    S.a_row_bytes = p->d.h_in * (int64_t)p->elem;
    S.b_row_bytes = p->d.h_out * (int64_t)p->elem;
    S.a_base = static_cast<char*>(p->d.class_base[0]);
    S.b_base = static_cast<char*>(p->d.class_base[p->b_class()]);
    S.a_page_bytes = p->page_bytes[0];
    S.b_page_bytes = p->page_bytes[p->b_class()];
    S.row_start[0] = 0;
    for (int i = 0; i < S.n; ++i) {
      S.rank[i] = recs[k0 + i]->rank;
      S.img_off[i] = (int64_t)off[k0 + i];
      S.row_start[i + 1] = S.row_start[i] + 2 * np * S.rank[i];
    }
    hipError_t he = launch_scatter_pages(S, stream);
    if (he != hipSuccess) return failed(he, "scatter adapter rows");
  }
  return SLORA_OK;
}

slora_status upload_adapter(slora_pool* p, const AdapterRec& rec, const void* const* A,
                            const void* const* B, hipStream_t stream) {
  slora_status st = ensure_stage(p);
  if (st != SLORA_OK) return st;
  st = pack_image(p, rec.rank, A, B, p->h_stage, "slora_load_adapter");
  if (st != SLORA_OK) return st;
  char* img = p->h_stage;
  st = enqueue_images(p, {&rec}, &img, p->d_stage, stream);
  if (st != SLORA_OK) return st;
  hipError_t he = hipStreamSynchronize(stream);
  if (he != hipSuccess) return hip_fail(he, "hipStreamSynchronize(adapter load)");
  return SLORA_OK;
}

// Argument checks shared by the two loads (no device call).
slora_status check_load(const slora_pool* p, int32_t id, int32_t rank, float scale, const char* fn) {
  const std::string f(fn);
  if (!p) return fail(SLORA_E_INVAL, f + ": NULL pool");
  if (id < 0 || id >= p->d.max_adapters) return fail(SLORA_E_INVAL, f + ": id out of range");
  if (rank < 1 || rank > p->d.max_rank) return fail(SLORA_E_INVAL, f + ": rank out of range");
  if (!std::isfinite(scale)) return fail(SLORA_E_INVAL, f + ": scale must be finite");
  if (p->adapters[id].loaded) return fail(SLORA_E_EXIST, f + ": adapter already loaded");
  const int64_t need = (int64_t)rank * p->d.n_proj;
  if (p->d.n_classes == 2) {
    if (need > p->free_list[0].count || need > p->free_list[1].count)
      return fail(SLORA_E_NOMEM, f + ": not enough free pages");
  } else if (2 * need > p->free_list[0].count) {
    return fail(SLORA_E_NOMEM, f + ": not enough free pages");
  }
  return SLORA_OK;
}

// Take the adapter's pages from the head of the free list: per projection,
// rank pages for the A^T rows, then rank pages for the B rows.
AdapterRec take_pages(slora_pool* p, int32_t rank, float scale) {
  const int np = p->d.n_proj;
  AdapterRec rec;
  rec.rank = rank;
  rec.scale = scale;
  rec.a_pages.resize((size_t)rank * np);
  rec.b_pages.resize((size_t)rank * np);
  for (int pr = 0; pr < np; ++pr) {
    for (int j = 0; j < rank; ++j) {
      const int32_t a = p->free_list[0].pop_front();
      p->state[0][a] = PAGE_ADAPTER;
      rec.a_pages[(size_t)pr * rank + j] = a;
    }
    for (int j = 0; j < rank; ++j) {
      const int32_t b = p->free_list[p->b_class()].pop_front();
      p->state[p->b_class()][b] = PAGE_ADAPTER;
      rec.b_pages[(size_t)pr * rank + j] = b;
    }
  }
  return rec;
}

void commit_adapter(slora_pool* p, int32_t id, AdapterRec&& rec) {
  rec.loaded = true;
  rec.gen = ++p->gen_counter;
  p->adapters[id] = std::move(rec);
}

// ---------------------------------------------------------------------------
// Tiles.  Each segment's tokens are cut into token blocks; the shrink work of
// a block into rank-row blocks, the expand work into column blocks.

struct TileSpec {
  int32_t kind, seg, i0, ntok, pos, len, aux;
  int32_t grp;   // token group for the XCD placement (tiles sharing x rows)
};

void split_tokens(int32_t c, int32_t cap, std::vector<std::pair<int32_t, int32_t>>& out) {
  // ceil(c / cap) blocks of near-equal size
  out.clear();
  const int32_t nb = (c + cap - 1) / cap;
  int32_t start = 0;
  for (int32_t b = 0; b < nb; ++b) {
    const int32_t len = (c - start) / (nb - b);
    out.emplace_back(start, len);
    start += len;
  }
}

void build_tiles(slora_segments* s) {
  const slora_pool* p = s->pool;
  const int32_t S = (int32_t)s->seg_adapter.size();
  const int32_t hin = p->d.h_in, hout = p->d.h_out;
  const bool f16 = p->d.dtype == SLORA_F16;
  const int vec = f16 ? 8 : 4;
  const int nck = shrink_nck(p->d.dtype, hin);

  // Matrix-core tiles need fp16, h_in a multiple of 64 and a y that the
  // expand can address through one buffer descriptor.
  const bool mfma_ok = f16 && hin % kShrinkKc == 0 && (int64_t)s->n_tokens * hout * 2 <= kMaxBufferBytes;

  // Work per vector-ALU expand tile (rank x columns).  A small batch needs
  // many small tiles to keep enough loads in flight; a large one runs faster
  // with fewer, larger tiles (less per-tile setup).  Measured on MI355X the
  // best budget tracks the batch's vector-ALU expand work / 1024, rounded
  // down to a power of two and clamped to [16K, 256K] elements: 16K for 256
  // Llama-7B decode tokens, 32K for the 13B mixed batch, 256K for 512 tokens
  // of the 70B MLP projection (257.9-258.3 against 261.2-262.5 us at 128K;
  // above 256K a rank-128 tile is already at its widest, 2048 columns).
  // K splits of the MFMA shrink: enough tiles to give every CU about two
  // (512), at most kMaxSplits; with more than one, a combine tile per 16
  // tokens sums the splits' partial x A in a fixed order.
  int64_t mfma_blocks = 0;
  for (int32_t g = 0; g < S; ++g) {
    const int32_t c = s->seg_start[g + 1] - s->seg_start[g];
    if (mfma_ok && c >= p->tune.mfma_min_tokens && s->seg_rank[g] <= kMaxRankMfma)
      mfma_blocks += (c + kMfmaExpandTok - 1) / kMfmaExpandTok;
  }
  int32_t splits = 1;
  const int32_t n_kc = hin / kShrinkKc;
  if (p->tune.mfma_shrink_splits > 0) {
    splits = (int32_t)std::min<int64_t>(p->tune.mfma_shrink_splits, n_kc);
  } else {
    while (splits < kMaxSplits && splits * 2 <= n_kc && mfma_blocks * splits < 512) splits *= 2;
  }
  if (mfma_blocks == 0) splits = 1;
  s->n_splits = splits;
  const int gemv_rows = p->tune.shrink_rows > 0 ? (int)std::min<int64_t>(p->tune.shrink_rows, kShrinkRowBudget / nck)
                                                : kShrinkRowBudget / nck;
  s->gemv_rows = gemv_rows;
  // One-token blocks at four 16-byte chunks a thread take tiles of
  // kShrinkRowsOne rows (the kernel's one-token shape) unless the rows are
  // set by hand.
  const int gemv_rows_one = (nck == kShrinkOneNck && p->tune.shrink_rows == 0) ? kShrinkRowsOne : gemv_rows;

  // Width of a vector-ALU expand tile of rank r under a budget: the largest
  // of vec * {256, 128, 64, 32} columns with r x width within it; a thread
  // of it holds more than kExpandRowSet B rows (the pipelined variant) when
  // the 256 / (width / vec) row groups leave it more rows than that.
  auto gemv_width = [&](int32_t r, int64_t budget) {
    int32_t width = vec * 256;
    while (width > vec * 32 && (int64_t)r * width > budget) width /= 2;
    return width;
  };
  auto gemv_pipelined = [&](int32_t r, int64_t budget) {
    const int32_t groups = kThreads / (gemv_width(r, budget) / vec);
    return (r + groups - 1) / groups > kExpandRowSet;
  };
  int64_t expand_elems = p->tune.gemv_expand_elems;
  if (expand_elems == 0) {
    int64_t work = 0;
    bool heavy = false;   // the launch runs a variant with three workgroups per CU anyway
    for (int32_t g = 0; g < S; ++g) {
      const int32_t c = s->seg_start[g + 1] - s->seg_start[g];
      const bool mfma_seg = mfma_ok && c >= p->tune.mfma_min_tokens && s->seg_rank[g] <= kMaxRankMfma;
      if (!mfma_seg) work += (int64_t)((c + kGemvMaxTok - 1) / kGemvMaxTok) * s->seg_rank[g] * hout;
      heavy = heavy || mfma_seg;
    }
    auto budget_of = [](int64_t w) {
      int64_t b = 16384;
      while (b < 262144 && b * 2 <= w / 1024) b *= 2;
      return b;
    };
    expand_elems = budget_of(work);
    for (int32_t g = 0; g < S && !heavy; ++g) {
      const int32_t c = s->seg_start[g + 1] - s->seg_start[g];
      const bool mfma_seg = mfma_ok && c >= p->tune.mfma_min_tokens && s->seg_rank[g] <= kMaxRankMfma;
      heavy = !mfma_seg && gemv_pipelined(s->seg_rank[g], expand_elems);
    }
    // A launch whose registers already leave three workgroups per CU (matrix-
    // core tiles, or vector-ALU tiles deeper than one register set) loses no
    // residency to larger expand tiles, so there the budget follows the work
    // of a launch over all projections (slora_lora_delta_multi): the 13B
    // mixed step 218.7-219.2 against 223.6-224.0 us at its one-projection
    // budget of 32K (one projection per launch it is 3 % slower: each launch
    // holds a quarter of the tiles).  A batch that would become pipelined
    // keeps the small budget (7B decode 21.2-21.4 us at 16K against 22.4 at
    // 32K and 26.4 at 64K).
    if (heavy) expand_elems = budget_of(work * s->n_proj);
  }

  // MFMA expand width.  Measured on MI355X: a batch whose segments all take
  // the MFMA tiles (the 7B prefill batch) runs 3 % faster with 512 columns
  // (twice the expand tiles: the chip holds them all at once), while a batch
  // whose vector-ALU tiles already fill the chip (the 13B mixed batch) runs
  // 5 % faster with 1024 (each staged B slice serves twice the columns).
  int64_t mfma_cols = p->tune.mfma_expand_cols;
  if (mfma_cols == 0) {
    bool all_mfma = mfma_ok;
    for (int32_t g = 0; g < S && all_mfma; ++g) {
      const int32_t c = s->seg_start[g + 1] - s->seg_start[g];
      all_mfma = c >= p->tune.mfma_min_tokens && s->seg_rank[g] <= kMaxRankMfma;
    }
    mfma_cols = all_mfma ? 512 : 1024;
  }

  std::vector<TileSpec> tiles;
  std::vector<std::pair<int32_t, int32_t>> eblocks;   // token blocks of a segment
  int32_t max_rank = 1;
  int32_t n_groups = 0;
  s->n_mfma_segments = 0;
  s->n_shrink = s->n_expand = s->n_combine = 0;
  for (int32_t g = 0; g < S; ++g) {
    const int32_t c = s->seg_start[g + 1] - s->seg_start[g];
    const int32_t r = s->seg_rank[g];
    max_rank = std::max(max_rank, r);
    const bool mfma = mfma_ok && c >= p->tune.mfma_min_tokens && r <= kMaxRankMfma;
    if (mfma) ++s->n_mfma_segments;
    split_tokens(c, mfma ? kMfmaExpandTok : kGemvMaxTok, eblocks);
    const int32_t width = gemv_width(r, expand_elems);
    const int32_t cols = mfma ? (int32_t)mfma_cols : width;
    if (!mfma && gemv_pipelined(r, expand_elems)) s->pipe_expand = true;
    for (size_t b = 0; b < eblocks.size(); ++b) {
      const auto& tb = eblocks[b];
      const int32_t grp = n_groups + (int32_t)b;
      if (mfma) {
        // 64-token shrink tiles over all r rows, one per K split
        for (int32_t sp = 0; sp < splits; ++sp, ++s->n_shrink) {
          const int32_t c0 = (int32_t)((int64_t)sp * n_kc / splits), c1 = (int32_t)((int64_t)(sp + 1) * n_kc / splits);
          tiles.push_back({KIND_SHRINK_MFMA, g, tb.first, tb.second, c0 * kShrinkKc, (c1 - c0) * kShrinkKc, sp, grp});
        }
        if (splits > 1)
          for (int32_t k = 0; k < tb.second; k += kCombineTok, ++s->n_combine)
            tiles.push_back({KIND_COMBINE, g, tb.first + k, std::min(kCombineTok, tb.second - k), 0, r, splits, grp});
      } else {
        const int32_t rows = tb.second == 1 ? gemv_rows_one : gemv_rows;
        for (int32_t j0 = 0; j0 < r; j0 += rows, ++s->n_shrink)
          tiles.push_back({KIND_SHRINK_GEMV, g, tb.first, tb.second, j0, std::min(rows, r - j0), 0, grp});
      }
      for (int32_t o0 = 0; o0 < hout; o0 += cols, ++s->n_expand)
        tiles.push_back({mfma ? KIND_EXPAND_MFMA : KIND_EXPAND_GEMV, g, tb.first, tb.second, o0,
                         std::min(cols, hout - o0), mfma ? 0 : width, grp});
    }
    n_groups += (int32_t)eblocks.size();
  }

  // Launch order: every shrink tile, then the combine tiles, then every
  // expand tile; within each stage the matrix-core
  // tiles (the heavier ones) first within each stage, segment order otherwise.
  // Producers first keeps the waiting expand tiles of a fused launch from
  // holding the workgroup slots the shrink tiles need (measured: putting each
  // token block's expand tiles right after its shrink tiles is 20-50 % slower).
  // SLORA_TUNE_TILE_ORDER reorders tiles within a stage (segment order among
  // equals): 1 clusters them by rank, highest first; 2 (default) puts the
  // tiles that move the most bytes first (longest-processing-time order), so
  // the long tiles start early and the short ones fill the end of the launch.
  // Measured on MI355X against segment order: 3.5 % faster on the 7B prefill
  // batch, 1 % on the 13B mixed batch, 5 % on the 70B MLP projection, and the
  // same on the 7B decode batch, whose vector-ALU tiles all move about as
  // much (rank order, 1, costs that batch 4 %).
  auto launch_rank = [](const TileSpec& t) {
    if (t.kind & KIND_COMBINE_BIT) return 2;
    return ((t.kind & KIND_EXPAND_BIT) ? 3 : 0) + ((t.kind & KIND_MFMA_BIT) ? 0 : 1);
  };
  auto tile_bytes = [&](const TileSpec& t) -> int64_t {
    const int64_t r = s->seg_rank[t.seg];
    switch (t.kind) {
      case KIND_SHRINK_GEMV: return (int64_t)t.len * hin;                  // page rows (x from L2)
      case KIND_SHRINK_MFMA: return ((int64_t)t.ntok + r) * t.len;         // x and A^T over the K range
      case KIND_COMBINE: return (int64_t)t.ntok * r * t.aux;               // partials
      default: return (r + 2 * (int64_t)t.ntok) * t.len;                   // B rows, y read and written
    }
  };
  const int64_t order = p->tune.tile_order;
  std::stable_sort(tiles.begin(), tiles.end(), [&](const TileSpec& a, const TileSpec& b) {
    const int ra = launch_rank(a), rb = launch_rank(b);
    if (ra != rb) return ra < rb;
    if (order == 1) return s->seg_rank[a.seg] > s->seg_rank[b.seg];
    if (order == 2) return tile_bytes(a) > tile_bytes(b);
    return false;
  });

  // Optional XCD-aware placement of the shrink tiles (SLORA_TUNE_XCDS > 1).
  // Workgroup i of a launch runs on XCD i mod 8 (checked on MI355X), and each
  // XCD has its own L2.  The shrink tiles of one token block all read the
  // block's x rows; they are given one XCD (greedily, by the bytes they move)
  // and laid out so that position i holds a tile of XCD i mod n.  Measured,
  // it does not pay on the benchmark batches: the 7B decode is 1.5 us slower
  // (the stage no longer spreads evenly over all XCDs) and the 70B MLP
  // projection shows no change beyond its +-8 % run-to-run spread, so it is
  // off by default.
  const int nx = (int)p->tune.xcds;
  if (nx > 1 && s->n_shrink > 0) {
    const int e = f16 ? 2 : 4;
    std::vector<double> grp_work(n_groups, 0.0);
    for (int32_t i = 0; i < s->n_shrink; ++i)
      grp_work[tiles[i].grp] += (double)e * hin * (tiles[i].len + (double)tiles[i].ntok);
    std::vector<int32_t> order(n_groups);
    for (int32_t k = 0; k < n_groups; ++k) order[k] = k;
    std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) { return grp_work[a] > grp_work[b]; });
    std::vector<double> load(nx, 0.0);
    std::vector<int> grp_xcd(n_groups, 0);
    for (int32_t k : order) {
      const int x = (int)(std::min_element(load.begin(), load.end()) - load.begin());
      grp_xcd[k] = x;
      load[x] += grp_work[k];
    }
    std::vector<TileSpec> placed;
    placed.reserve(tiles.size());
    std::vector<std::vector<TileSpec>> q(nx);
    std::vector<size_t> head(nx, 0);
    for (int32_t i = 0; i < s->n_shrink; ++i) q[grp_xcd[tiles[i].grp]].push_back(tiles[i]);
    for (int32_t pos = 0; pos < s->n_shrink; ++pos) {
      int x = pos % nx;
      if (head[x] == q[x].size()) {   // this XCD's queue is spent: take from the longest remaining
        size_t best = 0;
        for (int y = 0; y < nx; ++y)
          if (q[y].size() - head[y] > best) best = q[y].size() - head[y], x = y;
      }
      placed.push_back(q[x][head[x]++]);
    }
    placed.insert(placed.end(), tiles.begin() + s->n_shrink, tiles.end());
    tiles.swap(placed);
  }

  const int np = s->n_proj;
  s->n_tiles = (int32_t)tiles.size();
  // Phases of a fused launch over several projections: each run of one tile
  // kind, every projection's copies of it before the next run, so that
  // matrix-core tiles of the last projection do not queue behind the other
  // projections' vector-ALU tiles.  With one projection this is the record
  // order itself.  Should the runs outnumber kMaxPhases (tiles placed by XCD)
  // the three stages serve as phases.
  s->phase_rec.assign(1, 0);
  for (int32_t i = 1; i < s->n_tiles; ++i)
    if (launch_rank(tiles[i]) != launch_rank(tiles[i - 1])) s->phase_rec.push_back(i);
  if ((int)s->phase_rec.size() > kMaxPhases) {
    s->phase_rec.assign(1, 0);
    for (int32_t edge : {s->n_shrink, s->n_shrink + s->n_combine})
      if (edge > s->phase_rec.back() && edge < s->n_tiles) s->phase_rec.push_back(edge);
  }
  s->phase_rec.push_back(s->n_tiles);
  // Token slots of a record: the most tokens any tile of the batch holds,
  // rounded up to 4 (4 for batches of vector-ALU tiles only, 64 with MFMA
  // tiles), so a decode batch's records are 80 words instead of 140.
  int32_t max_tok = 1;
  for (const TileSpec& t : tiles) max_tok = std::max(max_tok, t.ntok);
  s->tokcap = std::min<int32_t>(kTokCap, (max_tok + 3) & ~3);
  s->pagecap = (std::max(gemv_rows, max_rank) + 3) & ~3;   // <= kMaxPageCap
  s->stride = (REC_HDR + s->tokcap + np * s->pagecap + 3) & ~3;
  s->shrink_idx_off_words = (int64_t)s->n_tiles * s->stride;
  s->expand_idx_off_words = s->shrink_idx_off_words + s->n_shrink;
  s->records_words = (s->expand_idx_off_words + s->n_expand + 3) & ~(int64_t)3;

  // Base-plus-delta table.  A 256 x 256 tile reads x and W half as often
  // per flop as a 128 x 128 one but holds a whole CU (one workgroup per CU,
  // 256 CUs), so big tiles are used only in whole rounds of 256: the leading
  // row blocks that fill complete rounds take big tiles, the remaining
  // positions 128 x 256 tiles (half the work of a big tile), which spread a
  // partial round over the chip (for the 7B prefill batch: 512 big tiles and
  // 160 half tiles instead of 592 big tiles in three rounds, the last a third
  // full).  Batches too small for one round use 128 x 128 tiles only.  Row block rb holds sorted positions
  // start(rb) .. +tile; its LoRA stages are, for every segment that owns one
  // of those positions, one stage per kFwdLoraRows rank rows.
  const int32_t T = s->n_tokens, routed = (int32_t)s->perm.size();
  const bool big_ok = hout % kFwdBig == 0;
  const int64_t cb_big = hout / kFwdBig;
  const int64_t rb_big_all = (T + kFwdBig - 1) / kFwdBig;
  int32_t n_rb_big = 0;
  if (big_ok && p->tune.fwd_tile == kFwdBig) {
    n_rb_big = (int32_t)rb_big_all;
  } else if (big_ok && p->tune.fwd_tile == 0 && rb_big_all * cb_big >= 256) {
    const int64_t rounds = rb_big_all * cb_big / 256;
    n_rb_big = (int32_t)std::min<int64_t>(rb_big_all, rounds * 256 / cb_big);
  }
  s->fw_n_rb_big = n_rb_big;
  s->fw_big_rows = std::min<int32_t>(T, n_rb_big * kFwdBig);
  // Without big tiles, 64 x 128 tiles (twice the workgroups, half the LoRA
  // steps each) when a batch gives fewer than 256 tiles of 128 x 128 (one per
  // CU; the 7B decode batch: 128 tiles instead of 64), or when its LoRA steps
  // per 128-position block would outnumber the x W steps of a tile (the 70B
  // MLP batch: about 160 against 128, 6 % faster; the 13B mixed batch, about
  // 24 against 80, is 7 % slower with them); 32 x 128 tiles when even the
  // 64 x 128 tiles number fewer than 256 (the 7B decode batch: 256 tiles
  // instead of 128, each with about half the LoRA steps).
  const int64_t small128 = (int64_t)((T + kFwdBM - 1) / kFwdBM) * (hout / kFwdBN);
  int64_t lora_steps = 0;
  for (int32_t g = 0; g < S; ++g) lora_steps += (s->seg_rank[g] + kFwdLoraRows - 1) / kFwdLoraRows;
  const int64_t blocks128 = std::max<int64_t>(1, (T + kFwdBM - 1) / kFwdBM);
  const bool lora_heavy = lora_steps > (int64_t)(hin / kFwdBK) * blocks128;
  s->fw_small_bm = kFwdBM;
  if (n_rb_big == 0) {
    if (p->tune.fwd_tile == kFwdTiny || (p->tune.fwd_tile == 0 && 2 * small128 < 256))
      s->fw_small_bm = kFwdTiny;
    else if (p->tune.fwd_tile == kFwdSmall || (p->tune.fwd_tile == 0 && (small128 < 256 || lora_heavy)))
      s->fw_small_bm = kFwdSmall;
  }
  const int32_t SBM = s->fw_small_bm;
  const int32_t n_rb_small = (T - s->fw_big_rows + SBM - 1) / SBM;
  s->fw_n_rb = n_rb_big + n_rb_small;
  std::vector<int32_t> pos_seg(routed);
  for (int32_t g = 0; g < S; ++g)
    for (int32_t i = s->seg_start[g]; i < s->seg_start[g + 1]; ++i) pos_seg[i] = g;
  std::vector<int32_t> rb_info(2 * (size_t)s->fw_n_rb, 0);
  // LoRA stages as 8 groups of 4 rank rows (segment, first row, rows).  On
  // batches with 256-row tiles every tile takes one segment per stage (32
  // rank rows of it, groups past its rank empty); the 128-column tiles of
  // the other batches pack the groups of all their segments 8 to a stage, so
  // ranks of 8 or 16 no longer leave most of a stage empty (the 7B decode
  // batch: 116 stages instead of 150).
  const bool pack = n_rb_big == 0;
  s->fw_packed = pack;
  struct Group { int32_t g = 0, j0 = 0, n = 0; };
  using Stage = std::array<Group, kFwdLoraRows / 4>;
  std::vector<Stage> fw_stages;
  for (int32_t rb = 0; rb < s->fw_n_rb; ++rb) {
    const bool big = rb < n_rb_big;
    const int32_t p0 = big ? rb * kFwdBig : s->fw_big_rows + (rb - n_rb_big) * SBM;
    const int32_t p1 = std::min(p0 + (big ? kFwdBig : SBM), routed);
    rb_info[2 * rb] = (int32_t)fw_stages.size();
    if (p0 < p1) {
      size_t u = Stage().size();
      for (int32_t g = pos_seg[p0]; g <= pos_seg[p1 - 1]; ++g) {
        const int32_t r = s->seg_rank[g];
        if (pack) {
          for (int32_t j0 = 0; j0 < r; j0 += 4) {
            if (u == Stage().size()) fw_stages.emplace_back(), u = 0;
            fw_stages.back()[u++] = Group{g, j0, std::min(4, r - j0)};
          }
        } else {
          for (int32_t j0 = 0; j0 < r; j0 += kFwdLoraRows) {
            Stage st;
            for (size_t v = 0; v < st.size(); ++v) {
              const int32_t jg = j0 + 4 * (int32_t)v;
              st[v] = Group{g, jg, std::max(0, std::min(4, r - jg))};
            }
            fw_stages.push_back(st);
          }
        }
      }
    }
    rb_info[2 * rb + 1] = (int32_t)fw_stages.size() - rb_info[2 * rb];
  }
  s->fw_n_stages = (int32_t)fw_stages.size();
  auto take = [](int64_t& cur, int64_t words) { const int64_t at = cur; cur = (cur + words + 3) & ~(int64_t)3; return at; };
  int64_t cur = s->records_words;
  s->fw_order_off = take(cur, T);
  s->fw_pos_seg_off = take(cur, routed);
  s->fw_seg_start_off = take(cur, S + 1);
  s->fw_seg_rank_off = take(cur, S);
  s->fw_seg_scale_off = take(cur, S);
  s->fw_seg_v_off = take(cur, S);
  s->fw_rb_info_off = take(cur, 2 * (int64_t)s->fw_n_rb);
  s->fw_stages_off = take(cur, (int64_t)np * s->fw_n_stages * kFwdStageWords);

  s->error_off_words = cur;                         // 16-byte aligned
  s->vtag_off_words = s->error_off_words + 4;       // 8-byte pairs, 16-byte aligned
  s->blob.assign((size_t)cur, 0);
  {
    int32_t* b = s->blob.data();
    // copies of possibly empty arrays (an empty vector's data() may be NULL,
    // which memcpy may not be given even for zero bytes)
    auto copy_words = [](int32_t* dst, const void* src, size_t n) { if (n) std::memcpy(dst, src, n * 4); };
    copy_words(b + s->fw_order_off, s->perm.data(), (size_t)routed);
    // then the tokens with no adapter, in batch order
    std::vector<uint8_t> is_routed(T, 0);
    for (int32_t t : s->perm) is_routed[t] = 1;
    int32_t k = routed;
    for (int32_t t = 0; t < T; ++t)
      if (!is_routed[t]) b[s->fw_order_off + k++] = t;
    copy_words(b + s->fw_pos_seg_off, pos_seg.data(), (size_t)routed);
    copy_words(b + s->fw_seg_start_off, s->seg_start.data(), (size_t)(S + 1));
    copy_words(b + s->fw_seg_rank_off, s->seg_rank.data(), (size_t)S);
    copy_words(b + s->fw_seg_scale_off, s->seg_scale.data(), (size_t)S);
    for (int32_t g = 0; g < S; ++g) b[s->fw_seg_v_off + g] = (int32_t)s->seg_v_off[g];
    copy_words(b + s->fw_rb_info_off, rb_info.data(), rb_info.size());
    for (int pr = 0; pr < np; ++pr)
      for (int32_t e = 0; e < s->fw_n_stages; ++e) {
        const Stage& st = fw_stages[e];
        int32_t* ent = b + s->fw_stages_off + ((int64_t)pr * s->fw_n_stages + e) * kFwdStageWords;
        const int32_t* bp = s->b_pages.data() + (size_t)pr * s->sum_r;
        // Rows with no rank row of their own (past a group's rows, or in an
        // empty group) repeat the page of the last row before them; their
        // A column is zero.  Group 0 always holds rows.
        int32_t last = bp[s->seg_page_off[st[0].g] + st[0].j0];
        for (size_t v = 0; v < st.size(); ++v) {
          const Group& q = st[v];
          for (int32_t k = 0; k < 4; ++k) {
            if (k < q.n) last = bp[s->seg_page_off[q.g] + q.j0 + k];
            ent[4 * v + k] = last;
          }
          if (pack)
            ent[FWS_GROUP + v] = q.n > 0 ? (int32_t)(((uint32_t)q.g << 9) | ((uint32_t)(q.j0 >> 2) << 3) | (uint32_t)q.n)
                                         : 0;
        }
        if (!pack) {
          ent[FWS_SEG] = st[0].g;
          ent[FWS_J0] = st[0].j0;
          ent[FWS_RANK] = s->seg_rank[st[0].g];
        }
      }
  }

  int32_t* shrink_idx = s->blob.data() + s->shrink_idx_off_words;
  int32_t* expand_idx = s->blob.data() + s->expand_idx_off_words;
  int32_t ns = 0, ne = 0;
  for (int32_t i = 0; i < s->n_tiles; ++i) {
    const TileSpec& t = tiles[i];
    int32_t* rec = s->blob.data() + (size_t)i * s->stride;
    const bool expand = (t.kind & KIND_EXPAND_BIT) != 0;
    const bool combine = (t.kind & KIND_COMBINE_BIT) != 0;
    if (!combine) (expand ? expand_idx[ne++] : shrink_idx[ns++]) = i;
    const int32_t g = t.seg;
    const int32_t r = s->seg_rank[g];
    rec[REC_KIND] = t.kind;
    rec[REC_NTOK] = t.ntok;
    rec[REC_RANK] = r;
    rec[REC_POS] = t.pos;
    rec[REC_LEN] = t.len;
    rec[REC_V0] = (int32_t)(s->seg_v_off[g] + (int64_t)t.i0 * r);
    float sc = s->seg_scale[g];
    std::memcpy(&rec[REC_SCALE], &sc, 4);
    rec[REC_AUX] = t.aux;
    rec[REC_SEG] = g;
    rec[REC_NSPLIT] = (t.kind == KIND_SHRINK_MFMA) ? s->n_splits : 0;
    const int32_t first = s->seg_start[g] + t.i0;
    for (int32_t k = 0; k < t.ntok; ++k) rec[REC_HDR + k] = s->perm[first + k];
    for (int pr = 0; pr < np; ++pr) {
      int32_t* pg = rec + REC_HDR + s->tokcap + pr * s->pagecap;
      const int32_t* src = (expand ? s->b_pages.data() : s->a_pages.data()) +
                           (size_t)pr * s->sum_r + s->seg_page_off[g];
      if (combine) continue;
      if (expand || t.kind == KIND_SHRINK_MFMA)
        for (int32_t j = 0; j < r; ++j) pg[j] = src[j];
      else
        for (int32_t j = 0; j < t.len; ++j) pg[j] = src[t.pos + j];
    }
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI

extern "C" {

const char* slora_last_error(void) { return g_last_error.c_str(); }

slora_status slora_pool_create(const slora_pool_desc* desc, slora_pool** out) {
  if (!desc || !out) return fail(SLORA_E_INVAL, "slora_pool_create: NULL argument");
  const slora_pool_desc& d = *desc;
  if (d.dtype != SLORA_F32 && d.dtype != SLORA_F16)
    return fail(SLORA_E_INVAL, "slora_pool_create: dtype must be SLORA_F32 or SLORA_F16");
  if (d.h_in <= 0 || d.h_out <= 0 || d.h_in % 8 || d.h_out % 8 || d.h_in > 65536 || d.h_out > 65536)
    return fail(SLORA_E_INVAL, "slora_pool_create: h_in and h_out must be positive multiples of 8, at most 65536");
  const int vec = d.dtype == SLORA_F16 ? 8 : 4;
  if ((d.h_in / vec + kThreads - 1) / kThreads > 8)
    return fail(SLORA_E_INVAL, "slora_pool_create: h_in too large for the shrink kernel (max 16384 fp16, 8192 fp32)");
  if (d.n_proj < 1 || d.n_proj > 8) return fail(SLORA_E_INVAL, "slora_pool_create: n_proj must be 1..8");
  if (d.max_adapters < 1) return fail(SLORA_E_INVAL, "slora_pool_create: max_adapters must be >= 1");
  if (d.max_rank < 1 || d.max_rank > 256) return fail(SLORA_E_INVAL, "slora_pool_create: max_rank must be 1..256");
  if (d.n_classes != 1 && d.n_classes != 2) return fail(SLORA_E_INVAL, "slora_pool_create: n_classes must be 1 or 2");
  if (d.n_classes == 1 && d.h_in != d.h_out)
    return fail(SLORA_E_INVAL, "slora_pool_create: one page class needs h_in == h_out");
  if (d.reserved0 != 0) return fail(SLORA_E_INVAL, "slora_pool_create: reserved0 must be 0");
  for (int c = 0; c < d.n_classes; ++c) {
    if (d.n_pages[c] < 1 || d.n_pages[c] > INT32_MAX)
      return fail(SLORA_E_INVAL, "slora_pool_create: n_pages must be 1..2^31-1");
    if (!d.class_base[c] || (reinterpret_cast<uintptr_t>(d.class_base[c]) & 15))
      return fail(SLORA_E_INVAL, "slora_pool_create: class_base must be non-NULL and 16-byte aligned");
  }
  slora_pool* p = new (std::nothrow) slora_pool();
  if (!p) return fail(SLORA_E_NOMEM, "slora_pool_create: out of host memory");
  try {
    p->d = d;
    p->elem = elem_bytes(d.dtype);
    p->page_elems[0] = d.h_in;
    p->page_elems[1] = d.n_classes == 2 ? d.h_out : 0;
    for (int c = 0; c < d.n_classes; ++c) {
      p->page_bytes[c] = p->page_elems[c] * p->elem;
      const int64_t P = d.n_pages[c];
      p->free_list[c].buf.resize((size_t)P);
      p->state[c].assign((size_t)P, PAGE_FREE);
      if (d.free_order[c]) {
        std::vector<uint8_t> seen((size_t)P, 0);
        for (int64_t i = 0; i < P; ++i) {
          const int32_t id = d.free_order[c][i];
          if (id < 0 || id >= P || seen[id]) {
            delete p;
            return fail(SLORA_E_INVAL, "slora_pool_create: free_order must be a permutation of [0, n_pages)");
          }
          seen[id] = 1;
          p->free_list[c].buf[(size_t)i] = id;
        }
      } else {
        for (int64_t i = 0; i < P; ++i) p->free_list[c].buf[(size_t)i] = (int32_t)i;
      }
      p->free_list[c].head = 0;
      p->free_list[c].count = P;
    }
    p->adapters.resize((size_t)d.max_adapters);
    p->count_scratch.assign((size_t)d.max_adapters, 0);
  } catch (const std::bad_alloc&) {
    delete p;
    return fail(SLORA_E_NOMEM, "slora_pool_create: out of host memory");
  }
  *out = p;
  return SLORA_OK;
}

void slora_pool_destroy(slora_pool* p) {
  if (!p) return;
  for (int i = 0; i < 2; ++i) {
    if (p->meta_done[i]) {
      (void)hipEventSynchronize(p->meta_done[i]);
      (void)hipEventDestroy(p->meta_done[i]);
    }
    if (p->h_meta[i]) (void)hipHostFree(p->h_meta[i]);
  }
  if (p->d_stage) (void)hipFree(p->d_stage);
  if (p->h_stage) (void)hipHostFree(p->h_stage);
  delete p;
}

slora_status slora_pool_set_tuning(slora_pool* p, int32_t key, int64_t value) {
  if (!p) return fail(SLORA_E_INVAL, "slora_pool_set_tuning: NULL pool");
  switch (key) {
    case SLORA_TUNE_MFMA_MIN_TOKENS:
      if (value < 1) return fail(SLORA_E_INVAL, "mfma_min_tokens must be >= 1");
      p->tune.mfma_min_tokens = value;
      return SLORA_OK;
    case SLORA_TUNE_GEMV_EXPAND_ELEMS:
      if (value < 0) return fail(SLORA_E_INVAL, "gemv_expand_elems must be >= 0 (0: automatic)");
      p->tune.gemv_expand_elems = value;
      return SLORA_OK;
    case SLORA_TUNE_MFMA_EXPAND_COLS:
      if (value < 0 || value % kMfmaPass || value > 65536)
        return fail(SLORA_E_INVAL, "mfma_expand_cols must be 0 (automatic) or a multiple of 128, at most 65536");
      p->tune.mfma_expand_cols = value;
      return SLORA_OK;
    case SLORA_TUNE_XCDS:
      if (value < 1 || value > 64) return fail(SLORA_E_INVAL, "xcds must be 1..64");
      p->tune.xcds = value;
      return SLORA_OK;
    case SLORA_TUNE_TILE_ORDER:
      if (value < 0 || value > 2) return fail(SLORA_E_INVAL, "tile_order must be 0, 1 or 2");
      p->tune.tile_order = value;
      return SLORA_OK;
    case SLORA_TUNE_FUSED:
      if (value != 0 && value != 1) return fail(SLORA_E_INVAL, "fused must be 0 or 1");
      p->tune.fused = value;
      return SLORA_OK;
    case SLORA_TUNE_FWD_GROUP:
      if (value < 0 || value > 65536) return fail(SLORA_E_INVAL, "fwd_group must be 0..65536 (0: automatic)");
      p->tune.fwd_group = value;
      return SLORA_OK;
    case SLORA_TUNE_FWD_TILE:
      if (value != 0 && value != kFwdTiny && value != kFwdSmall && value != kFwdBM && value != kFwdBig)
        return fail(SLORA_E_INVAL, "fwd_tile must be 0 (automatic), 32, 64, 128 or 256");
      p->tune.fwd_tile = value;
      return SLORA_OK;
    case SLORA_TUNE_MFMA_SHRINK_SPLITS:
      if (value < 0 || value > kMaxSplits) return fail(SLORA_E_INVAL, "mfma_shrink_splits must be 0..4 (0: automatic)");
      p->tune.mfma_shrink_splits = value;
      return SLORA_OK;
    case SLORA_TUNE_SHRINK_ROWS:
      if (value < 0 || value > kShrinkRowBudget) return fail(SLORA_E_INVAL, "shrink_rows must be 0..16 (0: automatic)");
      p->tune.shrink_rows = value;
      return SLORA_OK;
    case SLORA_TUNE_FWD_KSPLIT:
      if (value < 0 || value > 2) return fail(SLORA_E_INVAL, "fwd_ksplit must be 0 (automatic), 1 or 2");
      p->tune.fwd_ksplit = value;
      return SLORA_OK;
    default:
      return fail(SLORA_E_INVAL, "slora_pool_set_tuning: unknown key");
  }
}

int64_t slora_free_count(const slora_pool* p, int32_t cls) {
  if (!p || cls < 0 || cls >= p->d.n_classes) return -1;
  return p->free_list[cls].count;
}

slora_status slora_alloc_pages(slora_pool* p, int32_t cls, int64_t n, int32_t* out_ids) {
  if (!p) return fail(SLORA_E_INVAL, "slora_alloc_pages: NULL pool");
  if (cls < 0 || cls >= p->d.n_classes) return fail(SLORA_E_INVAL, "slora_alloc_pages: bad class");
  if (n < 0 || (n > 0 && !out_ids)) return fail(SLORA_E_INVAL, "slora_alloc_pages: bad count or NULL out_ids");
  if (n > p->free_list[cls].count) return fail(SLORA_E_NOMEM, "slora_alloc_pages: not enough free pages");
  for (int64_t i = 0; i < n; ++i) {
    const int32_t id = p->free_list[cls].pop_front();
    p->state[cls][id] = PAGE_KV;
    out_ids[i] = id;
  }
  return SLORA_OK;
}

slora_status slora_free_pages(slora_pool* p, int32_t cls, int64_t n, const int32_t* ids) {
  if (!p) return fail(SLORA_E_INVAL, "slora_free_pages: NULL pool");
  if (cls < 0 || cls >= p->d.n_classes) return fail(SLORA_E_INVAL, "slora_free_pages: bad class");
  if (n < 0 || (n > 0 && !ids)) return fail(SLORA_E_INVAL, "slora_free_pages: bad count or NULL ids");
  const int64_t P = p->d.n_pages[cls];
  // validate everything first (including duplicates within ids) so failure changes nothing
  std::vector<int32_t> touched;
  slora_status st = SLORA_OK;
  for (int64_t i = 0; i < n; ++i) {
    const int32_t id = ids[i];
    if (id < 0 || id >= P || p->state[cls][id] != PAGE_KV) {
      st = fail(SLORA_E_INVAL, "slora_free_pages: page " + std::to_string(id) + " is not an allocated KV page");
      break;
    }
    p->state[cls][id] = PAGE_FREE;  // marks duplicates
    touched.push_back(id);
  }
  if (st != SLORA_OK) {
    for (int32_t id : touched) p->state[cls][id] = PAGE_KV;
    return st;
  }
  for (int64_t i = 0; i < n; ++i) p->free_list[cls].push_back(ids[i]);
  return SLORA_OK;
}

slora_status slora_load_adapter(slora_pool* p, int32_t id, int32_t rank, float scale,
                                const void* const* A, const void* const* B, void* stream) {
  slora_status st = check_load(p, id, rank, scale, "slora_load_adapter");
  if (st != SLORA_OK) return st;
  if ((A == nullptr) != (B == nullptr))
    return fail(SLORA_E_INVAL, "slora_load_adapter: A and B must both be given or both be NULL");
  AdapterRec rec = take_pages(p, rank, scale);
  if (A) {
    st = upload_adapter(p, rec, A, B, static_cast<hipStream_t>(stream));
    if (st != SLORA_OK) {
      rollback_pages(p, rec);
      return st;
    }
  }
  commit_adapter(p, id, std::move(rec));
  return SLORA_OK;
}

size_t slora_adapter_image_bytes(const slora_pool* p, int32_t rank) {
  if (!p || rank < 1 || rank > p->d.max_rank) return 0;
  return image_layout(p, rank).total;
}

slora_status slora_pack_adapter(const slora_pool* p, int32_t rank, const void* const* A,
                                const void* const* B, void* image, size_t image_bytes) {
  if (!p) return fail(SLORA_E_INVAL, "slora_pack_adapter: NULL pool");
  if (rank < 1 || rank > p->d.max_rank) return fail(SLORA_E_INVAL, "slora_pack_adapter: rank out of range");
  if (!A || !B || !image) return fail(SLORA_E_INVAL, "slora_pack_adapter: NULL A, B or image");
  if (image_bytes < image_layout(p, rank).total)
    return fail(SLORA_E_INVAL, "slora_pack_adapter: image smaller than slora_adapter_image_bytes(rank)");
  return pack_image(p, rank, A, B, static_cast<char*>(image), "slora_pack_adapter");
}

slora_status slora_load_adapters_async(slora_pool* p, int32_t n, const int32_t* ids,
                                       const int32_t* ranks, const float* scales, void* const* images,
                                       void* dev_stage, size_t dev_stage_bytes, void* stream) {
  const char* fn = "slora_load_adapters_async";
  if (!p) return fail(SLORA_E_INVAL, std::string(fn) + ": NULL pool");
  if (n < 0) return fail(SLORA_E_INVAL, std::string(fn) + ": n must be >= 0");
  if (n == 0) return SLORA_OK;
  if (!ids || !ranks || !scales || !images || !dev_stage)
    return fail(SLORA_E_INVAL, std::string(fn) + ": NULL ids, ranks, scales, images or dev_stage");
  // Every check before any page is taken: ids, ranks, scales, duplicates,
  // free pages for the whole batch, staging size, then the buffers' kinds.
  std::vector<char> seen((size_t)p->d.max_adapters, 0);
  int64_t need[2] = {0, 0};
  size_t stage_need = 0;
  for (int32_t k = 0; k < n; ++k) {
    const int32_t id = ids[k], r = ranks[k];
    if (id < 0 || id >= p->d.max_adapters) return fail(SLORA_E_INVAL, std::string(fn) + ": id out of range");
    if (r < 1 || r > p->d.max_rank) return fail(SLORA_E_INVAL, std::string(fn) + ": rank out of range");
    if (!std::isfinite(scales[k])) return fail(SLORA_E_INVAL, std::string(fn) + ": scale must be finite");
    if (!images[k]) return fail(SLORA_E_INVAL, std::string(fn) + ": NULL image");
    if (seen[id]) return fail(SLORA_E_INVAL, std::string(fn) + ": an id appears twice");
    seen[id] = 1;
    if (p->adapters[id].loaded) return fail(SLORA_E_EXIST, std::string(fn) + ": adapter already loaded");
    need[0] += (int64_t)r * p->d.n_proj;
    need[p->b_class()] += (int64_t)r * p->d.n_proj;
    stage_need += image_layout(p, r).total;
  }
  for (int c = 0; c < p->d.n_classes; ++c)
    if (need[c] > p->free_list[c].count) return fail(SLORA_E_NOMEM, std::string(fn) + ": not enough free pages");
  if (dev_stage_bytes < stage_need)
    return fail(SLORA_E_INVAL, std::string(fn) + ": dev_stage smaller than the images' total size");
  slora_status st = set_device(p);
  if (st != SLORA_OK) return st;
  // The copies are asynchronous only from pinned memory, and the scatter reads
  // dev_stage on the pool's device.
  for (int32_t k = 0; k < n; ++k) {
    hipPointerAttribute_t at{};
    hipError_t he = hipPointerGetAttributes(&at, images[k]);
    if (he != hipSuccess || at.type != hipMemoryTypeHost) {
      (void)hipGetLastError();
      return fail(SLORA_E_INVAL, std::string(fn) + ": an image is not pinned host memory");
    }
  }
  hipPointerAttribute_t at{};
  hipError_t he = hipPointerGetAttributes(&at, dev_stage);
  if (he != hipSuccess || at.type != hipMemoryTypeDevice || at.device != p->device) {
    (void)hipGetLastError();
    return fail(SLORA_E_INVAL, std::string(fn) + ": dev_stage is not device memory of the pool's device");
  }
  std::vector<AdapterRec> recs;
  recs.reserve((size_t)n);
  for (int32_t k = 0; k < n; ++k) recs.push_back(take_pages(p, ranks[k], scales[k]));
  std::vector<const AdapterRec*> rp;
  for (const AdapterRec& r : recs) rp.push_back(&r);
  st = enqueue_images(p, rp, reinterpret_cast<char* const*>(images), static_cast<char*>(dev_stage),
                      static_cast<hipStream_t>(stream));
  if (st != SLORA_OK) {
    for (int32_t k = n - 1; k >= 0; --k) rollback_pages(p, recs[(size_t)k]);
    return st;
  }
  for (int32_t k = 0; k < n; ++k) commit_adapter(p, ids[k], std::move(recs[(size_t)k]));
  return SLORA_OK;
}

slora_status slora_unload_adapter(slora_pool* p, int32_t id) {
  if (!p) return fail(SLORA_E_INVAL, "slora_unload_adapter: NULL pool");
  if (id < 0 || id >= p->d.max_adapters) return fail(SLORA_E_INVAL, "slora_unload_adapter: id out of range");
  AdapterRec& rec = p->adapters[id];
  if (!rec.loaded) return fail(SLORA_E_NOENT, "slora_unload_adapter: adapter not loaded");
  for (int pr = 0; pr < p->d.n_proj; ++pr) {
    for (int j = 0; j < rec.rank; ++j) {
      const int32_t a = rec.a_pages[(size_t)pr * rec.rank + j];
      p->state[0][a] = PAGE_FREE;
      p->free_list[0].push_back(a);
    }
    for (int j = 0; j < rec.rank; ++j) {
      const int32_t b = rec.b_pages[(size_t)pr * rec.rank + j];
      p->state[p->b_class()][b] = PAGE_FREE;
      p->free_list[p->b_class()].push_back(b);
    }
  }
  rec = AdapterRec();
  return SLORA_OK;
}

slora_status slora_adapter_pages(const slora_pool* p, int32_t id, int32_t proj, int32_t* a_ids,
                                 int32_t* b_ids, int32_t* rank_out) {
  if (!p) return fail(SLORA_E_INVAL, "slora_adapter_pages: NULL pool");
  if (id < 0 || id >= p->d.max_adapters) return fail(SLORA_E_INVAL, "slora_adapter_pages: id out of range");
  if (proj < 0 || proj >= p->d.n_proj) return fail(SLORA_E_INVAL, "slora_adapter_pages: proj out of range");
  const AdapterRec& rec = p->adapters[id];
  if (!rec.loaded) return fail(SLORA_E_NOENT, "slora_adapter_pages: adapter not loaded");
  if (a_ids) std::memcpy(a_ids, rec.a_pages.data() + (size_t)proj * rec.rank, rec.rank * sizeof(int32_t));
  if (b_ids) std::memcpy(b_ids, rec.b_pages.data() + (size_t)proj * rec.rank, rec.rank * sizeof(int32_t));
  if (rank_out) *rank_out = rec.rank;
  return SLORA_OK;
}

slora_status slora_build_segments(slora_pool* p, int32_t n_tokens, const int32_t* ids,
                                  slora_segments** out) {
  if (!p || !out) return fail(SLORA_E_INVAL, "slora_build_segments: NULL argument");
  if (n_tokens < 0 || (n_tokens > 0 && !ids)) return fail(SLORA_E_INVAL, "slora_build_segments: bad token count or NULL ids");
  for (int32_t t = 0; t < n_tokens; ++t) {
    const int32_t a = ids[t];
    if (a < 0) continue;
    if (a >= p->d.max_adapters || !p->adapters[a].loaded)
      return fail(SLORA_E_NOENT, "slora_build_segments: token " + std::to_string(t) + " names adapter " +
                                     std::to_string(a) + " which is not loaded");
  }
  slora_segments* s = new (std::nothrow) slora_segments();
  if (!s) return fail(SLORA_E_NOMEM, "slora_build_segments: out of host memory");
  try {
    s->pool = p;
    s->n_tokens = n_tokens;
    s->n_proj = p->d.n_proj;
    // Stable counting sort by adapter id; segments in ascending id order.
    std::vector<int32_t>& cnt = p->count_scratch;
    std::vector<int32_t> distinct;
    int32_t routed = 0;
    for (int32_t t = 0; t < n_tokens; ++t) {
      const int32_t a = ids[t];
      if (a < 0) continue;
      if (cnt[a]++ == 0) distinct.push_back(a);
      ++routed;
    }
    std::sort(distinct.begin(), distinct.end());
    const int32_t S = (int32_t)distinct.size();
    s->seg_start.resize(S + 1);
    s->seg_adapter = distinct;
    s->seg_rank.resize(S);
    s->seg_scale.resize(S);
    s->seg_gen.resize(S);
    s->seg_page_off.resize(S + 1);
    s->seg_v_off.resize(S + 1);
    int32_t cursor = 0;
    int64_t page_off = 0, v_off = 0;
    for (int32_t g = 0; g < S; ++g) {
      const int32_t a = distinct[g];
      const AdapterRec& rec = p->adapters[a];
      const int32_t c = cnt[a];
      s->seg_start[g] = cursor;
      s->seg_rank[g] = rec.rank;
      s->seg_scale[g] = rec.scale;
      s->seg_gen[g] = rec.gen;
      s->seg_page_off[g] = (int32_t)page_off;
      s->seg_v_off[g] = v_off;
      cnt[a] = cursor;  // becomes the write cursor of adapter a
      cursor += c;
      page_off += rec.rank;
      v_off += (int64_t)c * rec.rank;
    }
    s->seg_start[S] = cursor;
    s->seg_page_off[S] = (int32_t)page_off;
    s->seg_v_off[S] = v_off;
    s->sum_r = page_off;
    s->sum_rt = v_off;
    s->perm.resize(routed);
    for (int32_t t = 0; t < n_tokens; ++t) {
      const int32_t a = ids[t];
      if (a >= 0) s->perm[cnt[a]++] = t;
    }
    for (int32_t a : distinct) cnt[a] = 0;
    const int np = p->d.n_proj;
    s->a_pages.resize((size_t)np * s->sum_r);
    s->b_pages.resize((size_t)np * s->sum_r);
    for (int pr = 0; pr < np; ++pr) {
      for (int32_t g = 0; g < S; ++g) {
        const AdapterRec& rec = p->adapters[distinct[g]];
        const size_t dst = (size_t)pr * s->sum_r + s->seg_page_off[g];
        std::memcpy(&s->a_pages[dst], rec.a_pages.data() + (size_t)pr * rec.rank, rec.rank * sizeof(int32_t));
        std::memcpy(&s->b_pages[dst], rec.b_pages.data() + (size_t)pr * rec.rank, rec.rank * sizeof(int32_t));
      }
    }
    if (s->sum_rt > INT32_MAX) {
      delete s;
      return fail(SLORA_E_INVAL, "slora_build_segments: batch too large (sum of token ranks >= 2^31)");
    }
    build_tiles(s);
  } catch (const std::bad_alloc&) {
    for (auto& c : p->count_scratch) c = 0;
    delete s;
    return fail(SLORA_E_NOMEM, "slora_build_segments: out of host memory");
  }
  *out = s;
  return SLORA_OK;
}

void slora_segments_destroy(slora_segments* s) { delete s; }

slora_status slora_segments_get_info(const slora_segments* s, slora_segments_info* info) {
  if (!s || !info) return fail(SLORA_E_INVAL, "slora_segments_get_info: NULL argument");
  std::memset(info, 0, sizeof(*info));
  info->n_tokens = s->n_tokens;
  info->n_routed = (int32_t)s->perm.size();
  info->n_segments = (int32_t)s->seg_adapter.size();
  info->n_proj = s->n_proj;
  info->sum_rank = s->sum_r;
  info->sum_rank_tokens = s->sum_rt;
  info->n_shrink_tiles = s->n_shrink;
  info->n_expand_tiles = s->n_expand;
  info->n_mfma_segments = s->n_mfma_segments;
  info->n_combine_tiles = s->n_combine;
  info->meta_bytes = meta_bytes_of(s);
  info->workspace_bytes = workspace_bytes_of(s);
  return SLORA_OK;
}

slora_status slora_segments_export(const slora_segments* s, int32_t* perm, int32_t* seg_start,
                                   int32_t* seg_adapter, int32_t* seg_rank, float* seg_scale,
                                   int32_t* seg_page_off, int32_t* a_pages, int32_t* b_pages) {
  if (!s) return fail(SLORA_E_INVAL, "slora_segments_export: NULL segments");
  auto cp = [](void* dst, const void* src, size_t n) { if (dst && n) std::memcpy(dst, src, n); };
  cp(perm, s->perm.data(), s->perm.size() * 4);
  cp(seg_start, s->seg_start.data(), s->seg_start.size() * 4);
  cp(seg_adapter, s->seg_adapter.data(), s->seg_adapter.size() * 4);
  cp(seg_rank, s->seg_rank.data(), s->seg_rank.size() * 4);
  cp(seg_scale, s->seg_scale.data(), s->seg_scale.size() * 4);
  cp(seg_page_off, s->seg_page_off.data(), s->seg_page_off.size() * 4);
  cp(a_pages, s->a_pages.data(), s->a_pages.size() * 4);
  cp(b_pages, s->b_pages.data(), s->b_pages.size() * 4);
  return SLORA_OK;
}

slora_status slora_segments_tiles(const slora_segments* s, int32_t* layout, int32_t* records,
                                  size_t records_words) {
  if (!s || !layout) return fail(SLORA_E_INVAL, "slora_segments_tiles: NULL argument");
  const int32_t lay[9] = {s->n_tiles, s->stride, s->tokcap, s->pagecap, s->n_shrink, s->n_expand,
                          REC_HDR, s->n_combine, s->n_splits};
  std::memcpy(layout, lay, sizeof(lay));
  if (records) {
    const size_t words = (size_t)s->n_tiles * s->stride;
    if (records_words < words) return fail(SLORA_E_NOMEM, "slora_segments_tiles: records buffer too small");
    std::memcpy(records, s->blob.data(), words * sizeof(int32_t));
  }
  return SLORA_OK;
}

slora_status slora_segments_forward_tables(const slora_segments* s, int32_t* layout, int32_t* rb_info,
                                           size_t rb_words, int32_t* stages, size_t stage_words) {
  if (!s || !layout) return fail(SLORA_E_INVAL, "slora_segments_forward_tables: NULL argument");
  const int32_t lay[8] = {s->fw_n_rb, s->fw_n_rb_big, s->fw_big_rows, s->fw_small_bm, s->fw_n_stages,
                          s->fw_packed ? 1 : 0, kFwdStageWords, s->n_proj};
  std::memcpy(layout, lay, sizeof(lay));
  const size_t rbw = 2 * (size_t)s->fw_n_rb;
  const size_t stw = (size_t)s->n_proj * s->fw_n_stages * kFwdStageWords;
  if (rb_info) {
    if (rb_words < rbw) return fail(SLORA_E_NOMEM, "slora_segments_forward_tables: rb_info buffer too small");
    if (rbw) std::memcpy(rb_info, s->blob.data() + s->fw_rb_info_off, rbw * sizeof(int32_t));
  }
  if (stages) {
    if (stage_words < stw) return fail(SLORA_E_NOMEM, "slora_segments_forward_tables: stages buffer too small");
    if (stw) std::memcpy(stages, s->blob.data() + s->fw_stages_off, stw * sizeof(int32_t));
  }
  return SLORA_OK;
}

slora_status slora_segments_upload(slora_segments* s, void* dev_meta, size_t dev_meta_bytes, void* stream) {
  if (!s || !dev_meta) return fail(SLORA_E_INVAL, "slora_segments_upload: NULL argument");
  if (reinterpret_cast<uintptr_t>(dev_meta) & 15) return fail(SLORA_E_INVAL, "slora_segments_upload: dev_meta must be 16-byte aligned");
  const size_t bytes = s->blob.size() * sizeof(int32_t);
  if (dev_meta_bytes < meta_bytes_of(s)) return fail(SLORA_E_NOMEM, "slora_segments_upload: dev_meta smaller than meta_bytes");
  slora_pool* p = s->pool;
  if (bytes > 0) {
    slora_status st = set_device(p);
    if (st != SLORA_OK) return st;
    const int slot = p->meta_slot;
    hipError_t e = hipSuccess;
    if (p->meta_done[slot]) {
      e = hipEventSynchronize(p->meta_done[slot]);  // the slot's previous copy has finished
      if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize(metadata slot)");
    } else {
      e = hipEventCreateWithFlags(&p->meta_done[slot], hipEventDisableTiming);
      if (e != hipSuccess) { p->meta_done[slot] = nullptr; return hip_fail(e, "hipEventCreate"); }
    }
    if (p->h_meta_bytes[slot] < bytes) {
      if (p->h_meta[slot]) (void)hipHostFree(p->h_meta[slot]);
      p->h_meta[slot] = nullptr;
      p->h_meta_bytes[slot] = 0;
      const size_t want = std::max<size_t>(bytes, 1 << 20);
      e = hipHostMalloc((void**)&p->h_meta[slot], want, hipHostMallocDefault);
      if (e != hipSuccess) { p->h_meta[slot] = nullptr; return hip_fail(e, "hipHostMalloc(metadata)"); }
      p->h_meta_bytes[slot] = want;
    }
    std::memcpy(p->h_meta[slot], s->blob.data(), bytes);
    hipStream_t st_ = static_cast<hipStream_t>(stream);
    e = hipMemcpyAsync(dev_meta, p->h_meta[slot], bytes, hipMemcpyHostToDevice, st_);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(metadata)");
    e = hipEventRecord(p->meta_done[slot], st_);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord(metadata)");
    p->meta_slot ^= 1;
    // error word and v pairs start at zero; fused launches count epochs from 1
    e = launch_zero_words(static_cast<int32_t*>(dev_meta) + s->error_off_words,
                          (int64_t)(meta_bytes_of(s) / 4) - s->error_off_words, st_);
    if (e != hipSuccess) return hip_fail(e, "zeroing the fused-launch area");
  }
  s->dev_meta = static_cast<const int32_t*>(dev_meta);
  s->epoch = 0;
  return SLORA_OK;
}

slora_status slora_segments_set_launch_count(slora_segments* s, int64_t launches) {
  if (!s) return fail(SLORA_E_INVAL, "slora_segments_set_launch_count: NULL segments");
  if (launches < (int64_t)s->epoch || launches > 0x7FFFFFFF)
    return fail(SLORA_E_INVAL, "slora_segments_set_launch_count: launches must be at least the current count "
                               "and at most 2^31 - 1");
  s->epoch = (uint32_t)launches;
  return SLORA_OK;
}

slora_status slora_segments_read_error(const slora_segments* s, void* stream, int32_t* flag) {
  if (!s || !flag) return fail(SLORA_E_INVAL, "slora_segments_read_error: NULL argument");
  *flag = 0;
  if (!s->dev_meta || s->blob.empty()) return SLORA_OK;
  slora_status st = set_device(s->pool);
  if (st != SLORA_OK) return st;
  const int32_t* src = s->dev_meta + s->error_off_words;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(flag, src, sizeof(int32_t), hipMemcpyDeviceToHost, hs);
  if (e == hipSuccess) e = hipStreamSynchronize(hs);
  if (e != hipSuccess) return hip_fail(e, "slora_segments_read_error");
  return SLORA_OK;
}

}  // extern "C"

slora_status slora::pool_device_current(slora_pool* p) {
  if (!p) return fail(SLORA_E_INVAL, "NULL pool");
  return set_device(p);
}

size_t slora::segments_workspace_bytes(const slora_segments* s) { return workspace_bytes_of(s); }

namespace {

// The launch description of projections projs[0 .. n) of a batch, with
// inputs xs[i] and outputs ys[i] (no checks).
DeltaLaunch make_delta_launch(const slora_pool* p, const slora_segments* s, int32_t n, const int32_t* projs,
                              const void* const* xs, void* const* ys, const void* workspace) {
  DeltaLaunch L{};
  L.pool.base_a = static_cast<const char*>(p->d.class_base[0]);
  L.pool.base_b = static_cast<const char*>(p->d.class_base[p->b_class()]);
  L.pool.page_bytes_a = p->page_bytes[0];
  L.pool.page_bytes_b = p->page_bytes[p->b_class()];
  L.dtype = p->d.dtype;
  L.h_in = p->d.h_in;
  L.h_out = p->d.h_out;
  L.n_slots = n;
  for (int32_t i = 0; i < n; ++i) {
    L.projs[i] = projs[i];
    L.xs[i] = xs ? xs[i] : nullptr;
    L.ys[i] = ys ? ys[i] : nullptr;
  }
  L.v = static_cast<float*>(const_cast<void*>(workspace));
  L.rec = s->dev_meta;
  L.stride = s->stride;
  L.tokcap = s->tokcap;
  L.pagecap = s->pagecap;
  L.n_tiles = s->n_tiles;
  L.n_shrink = s->n_shrink;
  L.n_expand = s->n_expand;
  L.shrink_idx = s->dev_meta + s->shrink_idx_off_words;
  L.expand_idx = s->dev_meta + s->expand_idx_off_words;
  L.gemv_rows = s->gemv_rows;
  L.has_mfma = s->n_mfma_segments > 0;
  L.error_flag = reinterpret_cast<uint32_t*>(const_cast<int32_t*>(s->dev_meta + s->error_off_words));
  L.vtag = reinterpret_cast<unsigned long long*>(const_cast<int32_t*>(s->dev_meta + s->vtag_off_words));
  L.y_bytes = (uint32_t)std::min<int64_t>((int64_t)s->n_tokens * p->d.h_out * elem_bytes(p->d.dtype), kMaxBufferBytes);
  L.sum_rt = (int32_t)s->sum_rt;
  L.n_splits = s->n_splits;
  L.n_combine = s->n_combine;
  L.pipe_expand = s->pipe_expand ? 1 : 0;
  L.x_shared = 0;
  for (int32_t i = 0; i < n && xs; ++i)
    for (int32_t j = i + 1; j < n; ++j)
      if (xs[i] && xs[i] == xs[j]) L.x_shared = 1;
  L.n_phases = (int32_t)s->phase_rec.size() - 1;
  for (int32_t k = 0; k <= L.n_phases; ++k) L.phase_rec[k] = s->phase_rec[(size_t)k];
  return L;
}

// Checks shared by every compute entry point: pool and segments match, the
// projection exists, and no adapter of the batch changed since the build.
slora_status check_batch(const std::string& f, const slora_pool* p, const slora_segments* s, int32_t proj) {
  if (!p || !s) return fail(SLORA_E_INVAL, f + ": NULL pool or segments");
  if (s->pool != p) return fail(SLORA_E_INVAL, f + ": segments belong to another pool");
  if (proj < 0 || proj >= p->d.n_proj) return fail(SLORA_E_INVAL, f + ": proj out of range");
  const int32_t S = (int32_t)s->seg_adapter.size();
  for (int32_t g = 0; g < S; ++g) {
    const AdapterRec& rec = p->adapters[s->seg_adapter[g]];
    if (!rec.loaded || rec.gen != s->seg_gen[g])
      return fail(SLORA_E_STALE, f + ": adapter " + std::to_string(s->seg_adapter[g]) +
                                     " changed since the segments were built");
  }
  return SLORA_OK;
}

// Projections projs[0 .. n) of one batch: in one fused launch (slots of
// one grid), or staged, one projection at a time.  stages: STAGE_SHRINK,
// STAGE_EXPAND or both.
slora_status run_delta(const char* fn, int stages, slora_pool* p, const slora_segments* s, int32_t n,
                       const int32_t* projs, const void* const* xs, void* const* ys, const void* workspace,
                       size_t workspace_bytes, void* stream, void* ev_start = nullptr, void* ev_stop = nullptr) {
  const std::string f(fn);
  if (n < 1 || n > kMaxSlots || !projs) return fail(SLORA_E_INVAL, f + ": n must be 1..8 with a projs array");
  if (p && (n > p->d.n_proj)) return fail(SLORA_E_INVAL, f + ": more projections than the pool has");
  for (int32_t i = 0; i < n; ++i) {
    slora_status chk = check_batch(f, p, s, projs[i]);
    if (chk != SLORA_OK) return chk;
    for (int32_t k = 0; k < i; ++k)
      if (projs[k] == projs[i]) return fail(SLORA_E_INVAL, f + ": a projection is named twice");
  }
  if (s->perm.empty()) return SLORA_OK;
  if (!workspace || reinterpret_cast<uintptr_t>(workspace) & 15)
    return fail(SLORA_E_INVAL, f + ": workspace must be non-NULL and 16-byte aligned");
  for (int32_t i = 0; i < n; ++i) {
    const void* x = xs ? xs[i] : nullptr;
    const void* y = ys ? ys[i] : nullptr;
    if (((stages & STAGE_SHRINK) && !x) || ((stages & STAGE_EXPAND) && !y))
      return fail(SLORA_E_INVAL, f + ": NULL x or y");
    if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(y)) & 15)
      return fail(SLORA_E_INVAL, f + ": x and y must be 16-byte aligned");
  }
  const size_t area = (size_t)s->n_splits * s->sum_rt * sizeof(float);
  if (workspace_bytes < (size_t)n * area)
    return fail(SLORA_E_NOMEM, f + ": workspace smaller than " + (n > 1 ? "n x " : "") + "workspace_bytes");
  if (!s->dev_meta) return fail(SLORA_E_INVAL, f + ": segments not uploaded (call slora_segments_upload)");
  slora_status st = set_device(p);
  if (st != SLORA_OK) return st;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (stages == (STAGE_SHRINK | STAGE_EXPAND) && p->tune.fused) {
    DeltaLaunch L = make_delta_launch(p, s, n, projs, xs, ys, workspace);
    // Epochs run 1 .. 2^31 - 1 (partial sums of K-split shrink tiles carry the
    // epoch with bit 31 set); before they would wrap, clear the pairs so that
    // no stale pair can match a new epoch.
    if (s->epoch == 0x7FFFFFFFu) {
      hipError_t z = launch_zero_words(const_cast<int32_t*>(s->dev_meta) + s->vtag_off_words, vtag_words_of(s), hs);
      if (z != hipSuccess) return hip_fail(z, (f + " clearing v pairs").c_str());
      s->epoch = 0;
    }
    L.epoch = ++s->epoch;
    hipError_t e = launch_delta(L, STAGE_FUSED, hs, static_cast<hipEvent_t>(ev_start),
                                static_cast<hipEvent_t>(ev_stop));
    if (e != hipSuccess) return hip_fail(e, (f + " launch").c_str());
    return SLORA_OK;
  }
  for (int32_t i = 0; i < n; ++i) {
    const void* x1[1] = {xs ? xs[i] : nullptr};
    void* y1[1] = {ys ? ys[i] : nullptr};
    const char* ws = static_cast<const char*>(workspace) + i * area;
    const DeltaLaunch L = make_delta_launch(p, s, 1, projs + i, x1, y1, ws);
    hipError_t e = launch_delta(L, stages, hs, i == 0 ? static_cast<hipEvent_t>(ev_start) : nullptr,
                                i == n - 1 ? static_cast<hipEvent_t>(ev_stop) : nullptr);
    if (e != hipSuccess) return hip_fail(e, (f + " launch").c_str());
  }
  return SLORA_OK;
}

slora_status run_stages(const char* fn, int stages, slora_pool* p, const slora_segments* s,
                        int32_t proj, const void* x, void* y, const void* workspace,
                        size_t workspace_bytes, void* stream, void* ev_start = nullptr,
                        void* ev_stop = nullptr) {
  return run_delta(fn, stages, p, s, 1, &proj, &x, &y, workspace, workspace_bytes, stream, ev_start, ev_stop);
}


// Base product plus delta: the shrink stage (v = x A into the workspace), then
// one launch of the base-plus-delta kernel over every token of the batch.
slora_status run_forward(const char* fn, slora_pool* p, const slora_segments* s, int32_t proj,
                         const void* x, const void* w, void* y, void* workspace, size_t workspace_bytes,
                         void* stream, void* ev_start, void* ev_stop) {
  const std::string f(fn);
  slora_status chk = check_batch(f, p, s, proj);
  if (chk != SLORA_OK) return chk;
  if (p->d.dtype != SLORA_F16) return fail(SLORA_E_INVAL, f + ": fp16 pools only");
  if (p->d.h_in % kFwdBK != 0 || p->d.h_out % kFwdBN != 0)
    return fail(SLORA_E_INVAL, f + ": needs h_in a multiple of " + std::to_string(kFwdBK) +
                                   " and h_out a multiple of " + std::to_string(kFwdBN));
  if (s->n_tokens == 0) return SLORA_OK;
  if (s->fw_packed && s->seg_adapter.size() >= ((size_t)1 << 23))
    return fail(SLORA_E_INVAL, f + ": more than 2^23 - 1 segments in a batch without 256-row tiles");
  const bool routed = !s->perm.empty();
  if (!x || !w || !y || (routed && !workspace)) return fail(SLORA_E_INVAL, f + ": NULL x, w, y or workspace");
  if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(w) | reinterpret_cast<uintptr_t>(y) |
       reinterpret_cast<uintptr_t>(workspace)) & 15)
    return fail(SLORA_E_INVAL, f + ": x, w, y and workspace must be 16-byte aligned");
  if (routed && workspace_bytes < (size_t)s->n_splits * s->sum_rt * sizeof(float))
    return fail(SLORA_E_NOMEM, f + ": workspace smaller than workspace_bytes");
  if (!s->dev_meta) return fail(SLORA_E_INVAL, f + ": segments not uploaded (call slora_segments_upload)");
  slora_status st = set_device(p);
  if (st != SLORA_OK) return st;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (routed) {
    const DeltaLaunch L = make_delta_launch(p, s, 1, &proj, &x, nullptr, workspace);
    hipError_t e = launch_delta(L, STAGE_SHRINK, hs, static_cast<hipEvent_t>(ev_start), nullptr);
    if (e != hipSuccess) return hip_fail(e, (f + " shrink launch").c_str());
  }
  const int32_t* m = s->dev_meta;
  ForwardLaunch F{};
  F.base_b = static_cast<const char*>(p->d.class_base[p->b_class()]);
  F.page_bytes_b = p->page_bytes[p->b_class()];
  F.h_in = p->d.h_in;
  F.h_out = p->d.h_out;
  F.n_tokens = s->n_tokens;
  F.n_routed = (int32_t)s->perm.size();
  F.x = x;
  F.w = w;
  F.y = y;
  F.v = static_cast<const float*>(workspace);
  F.order = m + s->fw_order_off;
  F.pos_seg = m + s->fw_pos_seg_off;
  F.seg_start = m + s->fw_seg_start_off;
  F.seg_rank = m + s->fw_seg_rank_off;
  F.seg_scale = m + s->fw_seg_scale_off;
  F.seg_v_off = m + s->fw_seg_v_off;
  F.stages = m + s->fw_stages_off + (int64_t)proj * s->fw_n_stages * kFwdStageWords;
  F.v4 = std::all_of(s->seg_rank.begin(), s->seg_rank.end(), [](int32_t r) { return r % 4 == 0; }) ? 1 : 0;
  // Big tiles over the leading positions, then small tiles over the rest; the
  // start event goes with the first launch, the stop event with the last.
  const int32_t n_small = s->fw_n_rb - s->fw_n_rb_big;
  hipError_t e = hipSuccess;
  ForwardLaunch parts[2];
  for (int part = 0; part < 2; ++part) {
    const int32_t n_rb = part == 0 ? s->fw_n_rb_big : n_small;
    parts[part] = F;
    if (n_rb == 0) continue;
    // the remainder of a batch whose bulk takes big tiles: 128 positions x
    // 256 columns (half a big tile's work, one round over the CUs)
    F.bm = part == 0 ? kFwdBig : s->fw_small_bm;
    F.bn = (part == 0 || s->fw_n_rb_big > 0) ? kFwdBig : kFwdBN;
    F.pos0 = part == 0 ? 0 : s->fw_big_rows;
    F.rb_info = m + s->fw_rb_info_off + (part == 0 ? 0 : 2 * (int64_t)s->fw_n_rb_big);
    F.n_rb = n_rb;
    F.n_cb = p->d.h_out / F.bn;
    F.n_tiles = F.n_rb * F.n_cb;
    F.per_xcd = (F.n_tiles + 7) / 8;
    // Tile order (automatic): the 32- and 64-row tiles go in groups of 8 row
    // blocks, column by column inside a group, so the 32 tiles an XCD holds
    // at once share 4 column blocks of W (and 8 blocks of x) in its L2
    // instead of each reading a column block of W of its own (measured: the
    // 7B decode batch 76.2 -> 68.4 us, the 70B MLP batch 930 -> 878 us).  The
    // 256-column tiles too: row-block major, an XCD's 32 tiles of a round
    // span 2 row blocks and all 16 column blocks of the 7B prefill batch, so
    // each XCD streams the whole W every round; in groups of 8 they span 4 x
    // 8 (the prefill forward's memory reads 907 -> 549 MB, 435 -> 425 us).
    // The 128 x 128 tiles stay row-block major: grouped, the 13B mixed batch
    // ran 428 us against 332 us (its tiles on one XCD then read B page rows
    // of different segments instead of neighbouring columns of the same rows).
    const int64_t auto_group = (F.bm <= kFwdSmall || F.bn == kFwdBig) ? 8 : 1;
    F.group_m = (int32_t)std::min<int64_t>(p->tune.fwd_group > 0 ? p->tune.fwd_group : auto_group, F.n_rb);
    // Two wave groups per tile, splitting its steps (automatic for the 32-
    // and 64-row tiles, which have the variant: the decode batch's 32-row
    // tiles are one workgroup per CU, whose step chains otherwise run alone
    // on their SIMDs, 63.0 -> 54.4 us; the 70B MLP's 64-row tiles 869-897 ->
    // 826-871 us over four boxes).  On 128 x 128 tiles it was slower (the 13B
    // mixed batch 336 against 308-316 us).
    F.ks = (int32_t)(p->tune.fwd_ksplit > 0 ? p->tune.fwd_ksplit : (F.bm <= kFwdSmall ? 2 : 1));
    if (F.bn != kFwdBN || F.bm > kFwdSmall) F.ks = 1;
    parts[part] = F;
  }
  // The remainder after the big tiles, in a launch of its own: in one grid
  // with the big tiles (remainder first) it ran beside the first round of big
  // tiles and saved the launch gap (1-2 %), but the two shapes then shared
  // each XCD's L2 and the forward's memory reads rose from 549 to 855 MB.
  for (int part = 0; part < 2 && e == hipSuccess; ++part) {
    if ((part == 0 ? s->fw_n_rb_big : n_small) == 0) continue;
    const bool first = part == 0 || s->fw_n_rb_big == 0;
    const bool last = part == 1 || n_small == 0;
    e = launch_forward(parts[part], hs, (first && !routed) ? static_cast<hipEvent_t>(ev_start) : nullptr,
                       last ? static_cast<hipEvent_t>(ev_stop) : nullptr);
  }
  if (e != hipSuccess) return hip_fail(e, (f + " launch").c_str());
  return SLORA_OK;
}

}  // namespace

extern "C" {

slora_status slora_lora_delta(slora_pool* p, const slora_segments* s, int32_t proj, const void* x, void* y,
                              void* workspace, size_t workspace_bytes, void* stream) {
  return run_stages("slora_lora_delta", STAGE_SHRINK | STAGE_EXPAND, p, s, proj, x, y, workspace,
                    workspace_bytes, stream);
}

slora_status slora_lora_delta_timed(slora_pool* p, const slora_segments* s, int32_t proj,
                                    const void* x, void* y, void* workspace, size_t workspace_bytes,
                                    void* stream, void* ev_start, void* ev_stop) {
  return run_stages("slora_lora_delta_timed", STAGE_SHRINK | STAGE_EXPAND, p, s, proj, x, y,
                    workspace, workspace_bytes, stream, ev_start, ev_stop);
}

slora_status slora_lora_delta_multi(slora_pool* p, const slora_segments* s, int32_t n, const int32_t* projs,
                                    const void* const* xs, void* const* ys, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  return run_delta("slora_lora_delta_multi", STAGE_SHRINK | STAGE_EXPAND, p, s, n, projs, xs, ys, workspace,
                   workspace_bytes, stream);
}

slora_status slora_lora_delta_multi_timed(slora_pool* p, const slora_segments* s, int32_t n,
                                          const int32_t* projs, const void* const* xs, void* const* ys,
                                          void* workspace, size_t workspace_bytes, void* stream,
                                          void* ev_start, void* ev_stop) {
  return run_delta("slora_lora_delta_multi_timed", STAGE_SHRINK | STAGE_EXPAND, p, s, n, projs, xs, ys,
                   workspace, workspace_bytes, stream, ev_start, ev_stop);
}

slora_status slora_lora_shrink(slora_pool* p, const slora_segments* s, int32_t proj, const void* x,
                               void* workspace, size_t workspace_bytes, void* stream) {
  return run_stages("slora_lora_shrink", STAGE_SHRINK, p, s, proj, x, nullptr, workspace,
                    workspace_bytes, stream);
}

slora_status slora_lora_expand(slora_pool* p, const slora_segments* s, int32_t proj, void* y,
                               const void* workspace, size_t workspace_bytes, void* stream) {
  return run_stages("slora_lora_expand", STAGE_EXPAND, p, s, proj, nullptr, y, workspace,
                    workspace_bytes, stream);
}

slora_status slora_lora_forward(slora_pool* p, const slora_segments* s, int32_t proj, const void* x,
                                const void* w, void* y, void* workspace, size_t workspace_bytes,
                                void* stream) {
  return run_forward("slora_lora_forward", p, s, proj, x, w, y, workspace, workspace_bytes, stream,
                     nullptr, nullptr);
}

slora_status slora_lora_forward_timed(slora_pool* p, const slora_segments* s, int32_t proj,
                                      const void* x, const void* w, void* y, void* workspace,
                                      size_t workspace_bytes, void* stream, void* ev_start,
                                      void* ev_stop) {
  return run_forward("slora_lora_forward_timed", p, s, proj, x, w, y, workspace, workspace_bytes,
                     stream, ev_start, ev_stop);
}

}  // extern "C"
