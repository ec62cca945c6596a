// Internal interface between the host runtime (slora_host.cpp) and the HIP
// kernels (slora_kernels.hip): the tile-record layout written by the segment
// builder and read by the kernels, and the launch entry points.
#pragma once

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "slora.h"

namespace slora {

// Record the calling thread's message for slora_last_error() (for sources
// other than the host runtime's C ABI).
void set_last_error(const char* msg);
// Make the pool's device current (the device of its first HIP call).
slora_status pool_device_current(slora_pool* pool);
// Workspace bytes one projection of the batch needs (slora_segments_info.workspace_bytes).
size_t segments_workspace_bytes(const slora_segments* seg);

// A tile record is a run of int32 words:
//   [0] kind        KIND_{SHRINK,EXPAND}_{GEMV,MFMA}: bit 0 set for the
//                   matrix-core (MFMA) tiles, bit 1 set for expand tiles
//   [1] ntok        tokens in the tile (all of one segment)
//   [2] rank        the segment's rank r (row stride of its v block)
//   [3] pos         shrink: first rank row j0 (MFMA: first k)   expand: first column o0
//   [4] len         shrink: rank rows handled (MFMA: k extent)  expand: columns handled
//   [5] v0          workspace offset of the tile's first token's v row
//   [6] scale       the segment's scale, float bits
//   [7] aux         expand GEMV: nominal column width of the tile (thread map);
//                   MFMA shrink: its K split; combine: the number of splits
//   [8] seg         index of the tile's segment
//   [9] nsplit      MFMA shrink: the K splits of its token block (1: writes v
//                   itself; more: a combine tile sums the splits' partials)
//   [10..11]        reserved
//   [HDR .. HDR+tokcap)                   batch indices of the tokens
//   [HDR+tokcap + p*pagecap .. +npages)   page ids of projection p: GEMV
//                                         shrink holds the A^T pages of rows
//                                         pos..pos+len, MFMA shrink all r A^T
//                                         pages, expand all r B pages
// All records share one stride (a multiple of 4 words) and sit in launch
// order: every shrink tile, then every combine tile, then every expand tile.
// Two index lists give the shrink and the expand records for launches that
// run the stages separately; combine records follow the shrink records.
enum : int32_t {
  REC_KIND = 0, REC_NTOK = 1, REC_RANK = 2, REC_POS = 3, REC_LEN = 4,
  REC_V0 = 5, REC_SCALE = 6, REC_AUX = 7, REC_SEG = 8, REC_NSPLIT = 9, REC_HDR = 12
};
enum : int32_t {
  KIND_SHRINK_GEMV = 0, KIND_SHRINK_MFMA = 1, KIND_EXPAND_GEMV = 2, KIND_EXPAND_MFMA = 3,
  KIND_COMBINE = 5,
  KIND_MFMA_BIT = 1, KIND_EXPAND_BIT = 2, KIND_COMBINE_BIT = 4
};

// Fixed tile geometry shared by the builder and the kernels.
constexpr int kThreads = 256;           // every tile kernel runs 4 waves of 64
constexpr int kMfmaExpandTok = 64;      // tokens per MFMA shrink / expand tile (four waves of 16)
constexpr int kCombineTok = 16;         // tokens per combine tile
constexpr int kMaxSplits = 4;           // K splits of an MFMA shrink token block
constexpr int kShrinkKc = 64;           // k elements per staged MFMA shrink chunk
constexpr int kMaxRankMfma = SLORA_MFMA_MAX_RANK;   // rank limit of MFMA segments
constexpr int kTokCap = 64;             // most token slots of a record (>= every tile kind's)
constexpr int kMaxPageCap = 256;        // page slots per projection (max_rank <= 256)
constexpr int kMfmaPass = 128;          // columns per MFMA expand pass
// The MFMA expand addresses y through a buffer descriptor (stores past its
// extent are dropped by the hardware): MFMA tiles are used only while y fits
// in this many bytes.
constexpr int64_t kMaxBufferBytes = 0xFFFFFF00LL;
constexpr int kGemvMaxTok = 4;          // tokens per vector-ALU tile
constexpr int kShrinkRowBudget = 16;    // rows x 16-byte chunks per thread (GEMV shrink)
constexpr int kShrinkOneNck = 4;        // chunks per thread of the one-token GEMV shrink shape
constexpr int kShrinkRowsOne = 8;       // its rows (twice the general tile's at four chunks)
constexpr int kExpandRowSet = 8;        // B rows a vector-ALU expand thread loads at once
static_assert(kTokCap >= kGemvMaxTok && kTokCap >= kMfmaExpandTok && kTokCap >= kCombineTok, "token slots");
static_assert(kMaxRankMfma <= 64, "the MFMA shrink holds at most four 16-row blocks of A^T");

struct PoolView {
  const char* base_a;     // class of the A^T pages
  const char* base_b;     // class of the B pages
  int64_t page_bytes_a;
  int64_t page_bytes_b;
};

// A launch covers n_slots projections of one batch (slora_lora_delta: one;
// slora_lora_delta_multi: up to n_proj, e.g. q, k and v with their shared x,
// and o with its own).  Slot s is projection projs[s] with input xs[s],
// output ys[s] and, in a staged launch, the x A products at v + s * n_splits
// * sum_rt; a fused launch passes them through the exchange area of its
// projection, vtag + projs[s] * n_splits * sum_rt.
constexpr int kMaxSlots = 8;
constexpr int kMaxPhases = 6;    // runs of one tile kind in the launch order (at most 5 kinds)

struct DeltaLaunch {
  PoolView pool;
  int32_t dtype;          // 0 fp32, 1 fp16
  int32_t h_in, h_out;
  int32_t n_slots;
  int32_t projs[kMaxSlots];
  const void* xs[kMaxSlots];
  void* ys[kMaxSlots];
  float* v;
  const int32_t* rec;             // all tile records, launch order
  int32_t stride, tokcap, pagecap;
  int32_t n_tiles, n_shrink, n_expand;
  const int32_t* shrink_idx;      // record index of each shrink tile
  const int32_t* expand_idx;      // record index of each expand tile
  int32_t gemv_rows;      // rank rows per GEMV shrink tile (host choice)
  int32_t has_mfma;       // some tile of this launch is an MFMA tile
  // fused launch: v as (value, epoch) pairs in the metadata buffer (zeroed at
  // upload), the launch's epoch (1, 2, ... per upload) and a flag raised if a
  // wait gave up
  unsigned long long* vtag;
  uint32_t* error_flag;
  int32_t sum_rt;         // v values of the batch (stride between the K-split partial areas)
  int32_t n_splits;       // K splits of the MFMA shrink blocks (areas per projection)
  int32_t n_combine;      // combine tiles (records n_shrink .. n_shrink + n_combine)
  uint32_t y_bytes;       // extent of y (n_tokens x h_out x element), < kMaxBufferBytes when has_mfma
  uint32_t epoch;
  int32_t pipe_expand;    // some vector-ALU expand thread holds more B rows than one register set
  int32_t x_shared;       // two slots of the launch read the same x
  // Fused launch order: phase k runs records phase_rec[k] .. phase_rec[k+1]
  // - 1 of every slot, slot by slot; the phases cover the records in order.
  int32_t n_phases;
  int32_t phase_rec[kMaxPhases + 1];
};

// Launch the shrink kernel (stages & 1) then the expand kernel (stages & 2) on
// `stream`, or both in one launch (STAGE_FUSED) in which each expand tile waits
// for the shrink tiles of its segment.
enum : int { STAGE_SHRINK = 1, STAGE_EXPAND = 2, STAGE_FUSED = 4 };
// Optional start/stop events are recorded by the dispatch itself (start when
// the first kernel begins, stop when the last one ends).
hipError_t launch_delta(const DeltaLaunch& L, int stages, hipStream_t stream,
                        hipEvent_t start = nullptr, hipEvent_t stop = nullptr);

// Base product with the LoRA delta folded into its tiles (fp16 only):
//   y[t, o] = round( sum_k x[t, k] W[k, o]  +  s_a sum_j v[t, j] B_j[o] )
// over the batch in segment order (routed tokens sorted by adapter, then the
// tokens with no adapter), in tiles of sorted positions x columns: 128 x 128
// (kFwdBM x kFwdBN), 256 x 256 and 128 x 256 on large batches, 64 x 128 and
// 32 x 128 on small ones.  Each tile first runs one LoRA stage per 32 rank
// rows of every segment its positions touch (the B page rows against s v,
// split into fp16 high and low parts), then the x W stages of kFwdBK rows of
// W, and writes y once.  v = x A comes from the shrink kernels (workspace).
constexpr int kFwdBM = 128;
constexpr int kFwdBN = 128;
constexpr int kFwdBig = 256;       // the large tile's rows and columns
constexpr int kFwdSmall = 64;      // rows of the tile for batches below one 128 x 128 tile per CU
constexpr int kFwdTiny = 32;       // rows of the tile for batches below one 64 x 128 tile per CU
constexpr int kFwdBK = 64;
constexpr int kFwdLoraRows = 32;   // B page rows per LoRA stage
// LoRA stage table entry (int32 words): the stage's 32 B page ids (rows with
// no rank row of their own repeat the page of the row before), then, on
// batches with 256-row tiles (one segment per stage), segment, first rank row
// and rank; otherwise (packed: rows 4u .. 4u+3 hold group u, up to 4 rank
// rows of any segment of the row block), one word per group,
// segment << 9 | first rank row / 4 << 3 | rows (0: an empty group).
constexpr int kFwdStageWords = 40;
enum : int32_t { FWS_SEG = 32, FWS_J0 = 33, FWS_RANK = 34, FWS_GROUP = 32 };

struct ForwardLaunch {
  const char* base_b;        // class of the B pages
  int64_t page_bytes_b;
  int32_t h_in, h_out;
  int32_t n_tokens, n_routed;
  const void* x;             // n_tokens x h_in, batch order
  const void* w;             // h_in x h_out, row-major
  void* y;                   // n_tokens x h_out, batch order (written)
  const float* v;            // x A of the routed tokens (segment order)
  const int32_t* order;      // [n_tokens] batch index of sorted position i
  const int32_t* pos_seg;    // [n_routed] segment of routed position i
  const int32_t* seg_start;  // [S + 1]
  const int32_t* seg_rank;   // [S]
  const int32_t* seg_scale;  // [S] float bits
  const int32_t* seg_v_off;  // [S] workspace offset of the segment's first v row
  const int32_t* rb_info;    // [n_rb][2] of this launch: first LoRA stage entry, LoRA stages
  const int32_t* stages;     // LoRA stage table of this projection
  int32_t n_rb, n_cb, n_tiles, per_xcd;
  int32_t group_m;           // tile order: groups of group_m row blocks, column-major inside a group
  int32_t bm, bn;            // tile shape: 256 x 256, 128 x 256, 128 x 128, 64 x 128 or 32 x 128
  int32_t pos0;              // first sorted position of row block 0 of this launch
  int32_t v4;                // every segment's rank is a multiple of 4 (v rows 16-byte aligned)
  int32_t ks;                // wave groups splitting each tile's steps: 1, or 2 (32- and 64-row tiles)
};

// Launch the base-plus-delta kernel (one launch, n_tiles workgroups placed
// XCD by XCD); start/stop events as for launch_delta.
hipError_t launch_forward(const ForwardLaunch& F, hipStream_t stream, hipEvent_t start = nullptr,
                          hipEvent_t stop = nullptr);

// Zero n_words 32-bit words at p (a fill kernel; no memset node in the stream).
hipError_t launch_zero_words(void* p, int64_t n_words, hipStream_t stream);

// Adapter images staged on the device for one scatter launch.  Image i sits
// at stage + img_off[i]: n_proj x rank[i] A^T rows of a_row_bytes, then as many
// B rows of b_row_bytes, then the 2 x n_proj x rank[i] destination page ids
// (A^T pages, then B pages).  Workgroup g moves global row g; adapter i owns
// rows row_start[i] .. row_start[i + 1].
constexpr int kMaxFetch = 64;
struct ScatterLaunch {
  const char* stage;
  int32_t n, n_proj;
  int64_t a_row_bytes, b_row_bytes;
  char* a_base;
  char* b_base;
  int64_t a_page_bytes, b_page_bytes;
  int32_t row_start[kMaxFetch + 1];
  int32_t rank[kMaxFetch];
  int64_t img_off[kMaxFetch];
};

// Copy every row of the staged images into its page (one launch).
hipError_t launch_scatter_pages(const ScatterLaunch& S, hipStream_t stream);

}  // namespace slora
