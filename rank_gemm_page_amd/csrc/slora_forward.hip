// Base product with the LoRA delta folded into its tiles, for MI355X (gfx950).
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "slora_device.h"

namespace slora {

// Base product with the LoRA delta in the same tiles: the summary page's
// "How to read the paper" item 2 (h = xW + xAB) evaluated as one fp32 sum per
// output element, and the blog page's section-2 interface (base output plus
// adapter output in one call).  y is written once, so the delta costs no
// extra pass over y.
//
// One workgroup per tile of BM sorted positions x BN columns, 2 x (BN / 64)
// waves, each BM / 2 positions x 64 columns (blocks of
// v_mfma_f32_16x16x32_f16).  Five shapes: 128 x 128 (four waves of
// 64 x 64), 256 x 256 (eight waves of 128 x 64), 128 x 256 (eight waves of
// 64 x 64, the remainder of a batch whose bulk takes 256 x 256 tiles),
// 64 x 128 (four waves of 32 x 64, for batches too small to give every CU a
// 128 x 128 tile or heavy in LoRA steps) and 32 x 128 (four waves of
// 16 x 64, for batches too small to give every CU a 64 x 128 tile); the
// 32- and 64-row tiles run two such groups of waves that split the tile's
// steps (KS = 2, below).  The
// larger tiles read x and W half as often per flop: x is read once per column
// block and W once per row block, and at 128 x 128 that traffic, not the
// matrix cores, bounds the kernel on large batches.  Per step the tile stages in LDS (two buffers, one
// barrier per step):
//   A  BM rows x 64 k of fp16 (16-byte chunks XOR-swizzled by row)
//   B  64 rows x BN columns, as BN / 128 slices of 128 columns (the
//      expand's slice layout, read with the transposing ds_read_b64_tr_b16)
// An x W step holds the positions' x rows (k0 .. k0+63) in A and W rows
// k0 .. k0+63 in B; its two 32-k halves are two MFMA sub-steps.  A LoRA step
// of segment g and rank rows j0 .. j0+31 holds the B page rows j0 .. j0+31 of
// g in B rows 0..31 and, in A, s v[t, j] 2^-e_t for the positions t of g
// (zero for the others) split into an fp16 high part (k 0..31) and the
// rounding remainder (k 32..63); both sub-steps multiply the same B rows, so
// the matrix cores see s v with about 22 significant bits.  The 128-column
// tiles pack their steps: B rows 4u .. 4u+3 hold up to 4 rank rows of any of
// the tile's segments (group u), and the A column of such a row is nonzero
// only for the positions of that row's segment.  e_t puts the
// position's largest |s v| in [2^14, 2^15); the accumulators are scaled back
// by 2^e_t (exact) after the LoRA steps, before the x W steps.

template <int BM, int BN, int KS = 1>
struct FwdTile {
  static constexpr int WN = BN / 64;                 // waves along the columns
  static constexpr int GT = 128 * WN;                // threads of one group (2 x WN waves)
  static constexpr int NT = GT * KS;                 // threads: KS groups
  static constexpr int RW = BM / 2;                  // positions per wave
  static constexpr int RB = RW / 16;                 // 16-row MFMA blocks per wave
  static constexpr int NSL = BN / 128;               // 128-column B slices
  static constexpr int CH = BN / 8;                  // 16-byte chunks per B row
  static constexpr int ADw = BM * (kFwdBK / 2);
  static constexpr int SliceDw = kFwdBK * kSliceRowDw;
  static constexpr int StageDw = ADw + NSL * SliceDw;
  static constexpr int EpiPitchDw = BN / 2 + 4;      // one fp16 output row, padded
  static constexpr int GroupDw = 2 * StageDw;        // one group's two stage buffers
  static constexpr int LdsDw = KS * GroupDw + 5 * BM;
  static constexpr int TPR = GT / BM;                // threads per position (prologue, LoRA staging)
  static constexpr int KL = kFwdLoraRows / TPR;      // rank rows of a LoRA step per thread
  static constexpr int XL = BM * 8 / GT;             // 16-byte x loads per thread per step
  static_assert(TPR == 2 || TPR == 4 || TPR == 8, "two, four or eight threads per position");
  // LoRA steps with page rows two steps ahead and stage tables four ahead
  // where the registers allow; the 256 x 256 tile keeps one step ahead.
  static constexpr bool DEEP = BM * BN <= 128 * 256;
  // The 128-column tiles (32, 64 and 128 rows: batches without 256-row
  // tiles) read the packed stage table (groups of 4 rank rows of any
  // segment); the 256-column tiles one segment per stage.
  static constexpr bool PACK = BN == kFwdBN;
  static constexpr int EP = BM < 128 ? BM : 128;    // rows per epilogue pass
  static_assert(EP * EpiPitchDw <= 2 * StageDw, "an epilogue pass reuses the stage buffers");
  static_assert(RW <= EP && EP % RW == 0, "epilogue passes hold whole waves");
  static_assert(kShrinkKc == kFwdBK && kFwdLoraRows == 32, "stage layouts");
  static_assert(KS == 1 || (KS == 2 && BM * BN <= GroupDw), "the second group's partial sums fit its buffers");
  static_assert(EP * CH % NT == 0, "epilogue stores: whole passes of the workgroup");
};

// V4: every rank of the batch is a multiple of 4, so v rows start on 16-byte
// boundaries and a LoRA step reads a thread's v values four at a time.
// KS = 2: two groups of 2 x WN waves share the tile and split its steps, the
// LoRA steps and the x W steps alike, group k taking steps k, k + 2, ...
// into accumulators of its own (its own stage buffers; both groups pass the
// same barriers, a group without a step of its own in the last round
// staging zeros); group 1's sums join group 0's through LDS before the
// epilogue.  For tiles with one workgroup per CU (the 32-row tiles), where
// each step's chain of load, LDS store, barrier and MFMAs otherwise runs with
// nothing beside it on its SIMD.
template <int BM, int BN, bool V4, int KS>
__device__ __forceinline__ void forward_tile(const ForwardLaunch& F, const int b, uint32_t* lds) {
  using C = FwdTile<BM, BN, KS>;
  // Workgroup b runs on XCD b mod 8; XCD x takes tiles x * per_xcd .. +per_xcd
  // in the tile order below, so the tiles resident on one XCD at a time share
  // x rows and W columns through its L2.
  const int tile = uni((b & 7) * F.per_xcd + (b >> 3));
  if (tile >= F.n_tiles) return;
  // groups of group_m row blocks, column by column inside a group
  const int gsize = F.group_m * F.n_cb;
  const int grp = tile / gsize, within = tile - grp * gsize;
  const int gm = min(F.group_m, F.n_rb - grp * F.group_m);
  const int rb = grp * F.group_m + within % gm;
  const int r0 = F.pos0 + rb * BM, c0 = (within / gm) * BN;
  const int kg = KS > 1 ? uni((int)threadIdx.x / C::GT) : 0;    // this thread's group
  const int tid = (int)threadIdx.x - kg * C::GT, lane = tid & 63, wave = uni(tid >> 6);
  const int m = lane & 15, g = lane >> 4;
  const int wm = wave / C::WN, wn = wave % C::WN;
  uint32_t* const stg = lds + kg * C::GroupDw;                   // this group's stage buffers

  int32_t* tok_l = reinterpret_cast<int32_t*>(lds + KS * C::GroupDw);
  int32_t* seg_l = tok_l + BM;
  int32_t* voff_l = seg_l + BM;
  float* mul_l = reinterpret_cast<float*>(voff_l + BM);
  float* up_l = mul_l + BM;

  // Per position of the tile: batch index, segment (-1: no adapter), v row
  // offset, s 2^-e and 2^e.  Positions past the batch take the last token's
  // row (loaded, never stored).  TPR threads per position scan its v row for
  // the largest |v|, eight independent loads each at a time (group 0).
  if (kg == 0) {
    const int row = tid / C::TPR, part = tid % C::TPR;
    const int p = r0 + row;
    int seg = -1, voff = 0, rank = 0;
    float scale = 0.f;
    if (p < F.n_routed) {
      seg = F.pos_seg[p];
      rank = F.seg_rank[seg];
      scale = __int_as_float(F.seg_scale[seg]);
      voff = F.seg_v_off[seg] + (p - F.seg_start[seg]) * rank;
    }
    float amax = 0.f;
    for (int j0 = part; j0 < rank; j0 += 8 * C::TPR) {
      float t[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j = j0 + C::TPR * u;
        t[u] = F.v[j < rank ? voff + j : voff];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) amax = fmaxf(amax, fabsf(t[u]));
    }
#pragma unroll
    for (int o = 1; o < C::TPR; o *= 2) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
    amax *= fabsf(scale);
    int ex = 0;
    if (amax > 0.f) {
      (void)frexpf(amax, &ex);
      ex = max(ex - 15, -100);
    }
    if (part == 0) {
      tok_l[row] = F.order[min(p, F.n_tokens - 1)];
      seg_l[row] = seg;
      voff_l[row] = voff;
      mul_l[row] = seg >= 0 ? scale * ldexpf(1.f, -ex) : 0.f;
      up_l[row] = seg >= 0 ? ldexpf(1.f, ex) : 1.f;
    }
  }
  __syncthreads();

  // Thread maps.  LoRA staging: A row ar = tid / TPR, rank rows
  // KL ah .. KL ah + KL - 1 (ah = tid % TPR).  B rows (W or pages): rows
  // brow + 16h, one 16-byte chunk bch of the BN columns (slice bch / 16).
  // x rows: chunk xch of rows xrow + (NT / 8) i, so one wave instruction
  // reads 8 whole 128-byte row segments.
  const int ar = tid / C::TPR, ah = tid % C::TPR;
  const int brow = tid / C::CH, bch = tid % C::CH;
  const int bsl = bch >> 4, bquad = 2 * (bch & 15);
  const int xrow = tid >> 3, xch = tid & 7;
  const _Float16* xb = static_cast<const _Float16*>(F.x);
  const _Float16* wb = static_cast<const _Float16*>(F.w);
  const int n_w = F.h_in / kFwdBK;

  float4v acc[C::RB][4];
#pragma unroll
  for (int i = 0; i < C::RB; ++i)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[i][c] = float4v{0.f, 0.f, 0.f, 0.f};

  // One MFMA sub-step: A chunks 4h .. 4h+3 against B rows brow0 .. brow0+31.
  auto mfma_step = [&](const uint32_t* S, int h, int brow0) {
    const uint32_t* A = S;
    const uint32_t* B = S + C::ADw + (wn >> 1) * C::SliceDw;
    half8 bf[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int q = 16 * (wn & 1) + 4 * c + (m & 3);
      const short4v r0v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) short4v*)(B + quad_dw(brow0 + 8 * g + (m >> 2), q)));
      const short4v r1v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) short4v*)(B + quad_dw(brow0 + 8 * g + 4 + (m >> 2), q)));
      bf[c] = __builtin_bit_cast(half8, __builtin_shufflevector(r0v, r1v, 0, 1, 2, 3, 4, 5, 6, 7));
    }
#pragma unroll
    for (int i = 0; i < C::RB; ++i) {
      const half8 af = __builtin_bit_cast(
          half8, *reinterpret_cast<const uint4*>(A + chunk_dw(C::RW * wm + 16 * i + m, 4 * h + g)));
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[i][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf[c], acc[i][c], 0, 0, 0);
    }
  };

  // x W steps: every load unconditional (a step past the end reloads the last).
  auto w_load = [&](int i, uint4 (&aq)[C::XL], uint4 (&bq)[4]) {
    int s = KS * i + kg;
    s = s < n_w ? s : n_w - 1;
    const int k0 = s * kFwdBK;
#pragma unroll
    for (int i = 0; i < C::XL; ++i)
      aq[i] = ld16(xb + (int64_t)tok_l[xrow + (C::GT / 8) * i] * F.h_in + k0 + 8 * xch);
#pragma unroll
    for (int h = 0; h < 4; ++h) bq[h] = ld16(wb + (int64_t)(k0 + brow + 16 * h) * F.h_out + c0 + 8 * bch);
  };
  // Local step j of a group is step KS j + kg; past the last step (a group's
  // share in the last round) it stages zero x rows.
  auto w_store = [&](uint32_t* S, const uint4 (&aq)[C::XL], const uint4 (&bq)[4], int j) {
    const bool ok = KS == 1 || KS * j + kg < n_w;
#pragma unroll
    for (int i = 0; i < C::XL; ++i)
      *reinterpret_cast<uint4*>(S + chunk_dw(xrow + (C::GT / 8) * i, xch)) = ok ? aq[i] : uint4{0u, 0u, 0u, 0u};
    uint32_t* B = S + C::ADw + bsl * C::SliceDw;
#pragma unroll
    for (int h = 0; h < 4; ++h) *reinterpret_cast<uint4*>(B + quad_dw(brow + 16 * h, bquad)) = bq[h];
  };

  const int n_lora = uni(F.rb_info[2 * rb + 1]);
  const int n_it = (n_lora + KS - 1) / KS;       // LoRA steps of each group
  if (n_lora > 0) {
    const int32_t* tab = F.stages + (int64_t)uni(F.rb_info[2 * rb]) * kFwdStageWords;
    // Stage table entry of LoRA step q (clamped): this thread's two B page
    // ids and one word of the step's header (segment, first rank row, rank
    // in lanes 0, 1, 2 of each wave).  The header is read with vector loads
    // on purpose: as a scalar load it would share the counter of the LDS
    // reads, and scalar loads complete out of order, so every LDS wait of the
    // step (the MFMA operands included) would wait for it as well.
    // Packed: this thread's rank rows KL ah .. KL ah + KL - 1 are groups
    // NG ah .. NG ah + NG - 1, one table word each.
    constexpr int NG = C::PACK ? C::KL / 4 : 1;
    struct Tab { int id0, id1, hw[NG]; bool ok; };
    const int hlane = lane & 3;
    // local step i of this group: step KS i + kg, ok = whether it exists
    auto tab_load = [&](int i, Tab& t) {
      int q = KS * i + kg;
      t.ok = KS == 1 || q < n_lora;
      q = q < n_lora ? q : n_lora - 1;
      const int32_t* e = tab + (int64_t)q * kFwdStageWords;
      t.id0 = e[brow];
      t.id1 = e[16 + brow];
      if constexpr (C::PACK) {
#pragma unroll
        for (int u = 0; u < NG; ++u) t.hw[u] = e[FWS_GROUP + NG * ah + u];
      } else {
        t.hw[0] = e[FWS_SEG + hlane];
      }
    };
    auto t_seg = [](const Tab& t) { return __builtin_amdgcn_readlane(t.hw[0], 0); };
    auto t_j0 = [](const Tab& t) { return __builtin_amdgcn_readlane(t.hw[0], 1); };
    auto t_rank = [](const Tab& t) { return __builtin_amdgcn_readlane(t.hw[0], 2); };
    // this thread's position: fixed for the tile, kept in registers
    const int my_seg = seg_l[ar], my_voff = voff_l[ar];
    const float my_mul = mul_l[ar];
    // A step's header as this thread needs it: the packed group words, or
    // (one segment per step) whether the step's segment is this thread's,
    // its first rank row of this thread and the rank, read once per step.
    struct View { bool in; int j, rank; };
    auto view_of = [&](const Tab& t) -> View {
      if constexpr (C::PACK) {
        return View{false, 0, 0};
      } else {
        return View{t.ok && my_seg == t_seg(t), t_j0(t) + C::KL * ah, t_rank(t)};
      }
    };
    // Rank row KL ah + i of a step: whether it is a row of this thread's
    // segment, and the index of its v value.
    struct Row { bool ok; int at; };
    auto row_of = [&](const Tab& t, const View& vw, int i) -> Row {
      if constexpr (C::PACK) {
        const uint32_t w = (uint32_t)t.hw[i >> 2];
        const int k = i & 3;
        return Row{t.ok && (int)(w & 7u) > k && (int)(w >> 9) == my_seg, my_voff + 4 * (int)((w >> 3) & 63u) + k};
      } else {
        return Row{vw.in && vw.j + i < vw.rank, my_voff + vw.j + i};
      }
    };
    auto lora_load = [&](const Tab& t, uint4 (&lb)[2], float (&vv)[C::KL]) {
      // Page ids are never negative: zero-extending them (unlike a sign
      // extension) needs no instruction on the loaded value, so the compiler
      // does not place one right behind the id loads of a later step, where
      // its wait would drain every load in flight.
      const int64_t col = (int64_t)(c0 + 8 * bch) * 2;
      lb[0] = ld16(F.base_b + (uint64_t)(uint32_t)t.id0 * (uint64_t)F.page_bytes_b + col);
      lb[1] = ld16(F.base_b + (uint64_t)(uint32_t)t.id1 * (uint64_t)F.page_bytes_b + col);
      const View vw = view_of(t);
      if constexpr (V4) {
        // a chunk of 4 values lies wholly inside the row or wholly past its
        // rank (rank % 4 == 0); one past it reads v[0 .. 3] instead
#pragma unroll
        for (int c = 0; c < C::KL / 4; ++c) {
          const Row r = row_of(t, vw, 4 * c);
          const uint4 q = ld16(F.v + (r.ok ? r.at : 0));
          vv[4 * c] = __uint_as_float(q.x);
          vv[4 * c + 1] = __uint_as_float(q.y);
          vv[4 * c + 2] = __uint_as_float(q.z);
          vv[4 * c + 3] = __uint_as_float(q.w);
        }
      } else {
#pragma unroll
        for (int i = 0; i < C::KL; ++i) {
          const Row r = row_of(t, vw, i);
          vv[i] = F.v[r.ok ? r.at : 0];
        }
      }
    };
    auto lora_store = [&](uint32_t* S, const Tab& t, const uint4 (&lb)[2], const float (&vv)[C::KL]) {
      uint32_t* B = S + C::ADw + bsl * C::SliceDw;
      *reinterpret_cast<uint4*>(B + quad_dw(brow, bquad)) = lb[0];
      *reinterpret_cast<uint4*>(B + quad_dw(16 + brow, bquad)) = lb[1];
      const float mul = my_mul;
      const View vw = view_of(t);
      if constexpr (C::KL >= 8) {
        constexpr int NC = C::KL / 8;           // 16-byte chunks of this thread's rank rows
        half8 hi[NC], lo[NC];
#pragma unroll
        for (int i = 0; i < C::KL; ++i) {
          const float f = row_of(t, vw, i).ok ? vv[i] * mul : 0.f;
          const _Float16 hv = (_Float16)f;
          hi[i >> 3][i & 7] = hv;
          lo[i >> 3][i & 7] = (_Float16)(f - (float)hv);
        }
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          *reinterpret_cast<uint4*>(S + chunk_dw(ar, NC * ah + c)) = __builtin_bit_cast(uint4, hi[c]);
          *reinterpret_cast<uint4*>(S + chunk_dw(ar, 4 + NC * ah + c)) = __builtin_bit_cast(uint4, lo[c]);
        }
      } else {
        // four rank rows per thread: half of a 16-byte chunk (dwords 0-1 or 2-3)
        static_assert(C::KL == 4, "four rank rows per thread");
        short4v hi, lo;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float f = row_of(t, vw, i).ok ? vv[i] * mul : 0.f;
          const _Float16 hv = (_Float16)f;
          hi[i] = __builtin_bit_cast(short, hv);
          lo[i] = __builtin_bit_cast(short, (_Float16)(f - (float)hv));
        }
        const int half = 2 * (ah & 1);
        *reinterpret_cast<uint2*>(S + chunk_dw(ar, ah >> 1) + half) = __builtin_bit_cast(uint2, hi);
        *reinterpret_cast<uint2*>(S + chunk_dw(ar, 4 + (ah >> 1)) + half) = __builtin_bit_cast(uint2, lo);
      }
    };
    if constexpr (C::DEEP) {
      // Step q: store its rows, issue the table of step q + 4, then issue
      // step q + 2's rows into the freed register set.  Step q + 2's table
      // was issued two steps earlier, ahead of the rows of steps q and q + 1,
      // so waiting for it neither drains rows still in flight nor waits a
      // full load latency.  Unrolled by two so that the register sets and
      // LDS buffers are static.
      Tab t0, t1, ta, tb, tx;
      uint4 lb0[2], lb1[2];
      float vv0[C::KL], vv1[C::KL];
      tab_load(0, t0);
      tab_load(1, t1);
      tab_load(2, ta);
      tab_load(3, tb);
      lora_load(t0, lb0, vv0);
      lora_load(t1, lb1, vv1);
      for (int q = 0;; q += 2) {
        lora_store(stg, t0, lb0, vv0);
        lds_barrier();
        tab_load(q + 4, tx);
        __builtin_amdgcn_sched_barrier(0);   // keep the table loads ahead of the rows
        lora_load(ta, lb0, vv0);
        t0 = ta;
        ta = tb;
        tb = tx;
        mfma_step(stg, 0, 0);
        mfma_step(stg, 1, 0);
        if (q + 1 >= n_it) break;
        lora_store(stg + C::StageDw, t1, lb1, vv1);
        lds_barrier();
        tab_load(q + 5, tx);
        __builtin_amdgcn_sched_barrier(0);
        lora_load(ta, lb1, vv1);
        t1 = ta;
        ta = tb;
        tb = tx;
        mfma_step(stg + C::StageDw, 0, 0);
        mfma_step(stg + C::StageDw, 1, 0);
        if (q + 2 >= n_it) break;
      }
    } else {
      Tab tc, tn;
      uint4 lb[2];
      float vv[C::KL];
      tab_load(0, tc);
      lora_load(tc, lb, vv);
      tab_load(1, tn);
      for (int q = 0; q < n_it; ++q) {
        uint32_t* S = stg + (q & 1) * C::StageDw;
        lora_store(S, tc, lb, vv);
        lds_barrier();
        tc = tn;
        lora_load(tc, lb, vv);
        tab_load(q + 2, tn);
        mfma_step(S, 0, 0);
        mfma_step(S, 1, 0);
      }
    }
    lds_barrier();   // the x W steps reuse both buffers
#pragma unroll
    for (int i = 0; i < C::RB; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float u = up_l[C::RW * wm + 16 * i + 4 * g + e];
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[i][c][e] *= u;
      }
  }

  // The first two x W steps (issued after the LoRA steps, whose registers
  // they would otherwise compete with).
  uint4 wa0[C::XL], wb0[4], wa1[C::XL], wb1[4];
  w_load(0, wa0, wb0);
  w_load(1, wa1, wb1);

  // x W steps, unrolled by two so that each register set and LDS buffer is
  // static: step s stores set s & 1 into buffer s & 1, then refills the set
  // with step s + 2.  A buffer is written again only after every wave has
  // passed the barrier of the step that followed its last read.
  const int n_wit = (n_w + KS - 1) / KS;         // x W steps of each group
  for (int s = 0;; s += 2) {
    w_store(stg, wa0, wb0, s);
    lds_barrier();
    w_load(s + 2, wa0, wb0);
    mfma_step(stg, 0, 0);
    mfma_step(stg, 1, 32);
    if (s + 1 >= n_wit) break;
    w_store(stg + C::StageDw, wa1, wb1, s + 1);
    lds_barrier();
    w_load(s + 3, wa1, wb1);
    mfma_step(stg + C::StageDw, 0, 0);
    mfma_step(stg + C::StageDw, 1, 32);
    if (s + 2 >= n_wit) break;
  }

  if constexpr (KS > 1) {
    // group 1's sums, through its own stage buffers, into group 0's
    float4v* R = reinterpret_cast<float4v*>(lds + C::GroupDw);
    lds_barrier();
    if (kg == 1) {
#pragma unroll
      for (int i = 0; i < C::RB; ++i)
#pragma unroll
        for (int c = 0; c < 4; ++c) R[(4 * i + c) * C::GT + tid] = acc[i][c];
    }
    lds_barrier();
    if (kg == 0) {
#pragma unroll
      for (int i = 0; i < C::RB; ++i)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[i][c] += R[(4 * i + c) * C::GT + tid];
    }
  }

  // Epilogue, EP rows at a time: fp16 results of group 0 through LDS, then
  // whole 16-byte chunks of y rows, stored by every thread of the workgroup.
  _Float16* E = reinterpret_cast<_Float16*>(lds);
  _Float16* yb = static_cast<_Float16*>(F.y);
  const int erow = (int)threadIdx.x / C::CH, ech = (int)threadIdx.x % C::CH;
#pragma unroll
  for (int pass = 0; pass < BM / C::EP; ++pass) {
    lds_barrier();   // every wave is done with the stage buffers / the previous pass
    if (kg == 0 && C::RW * wm / C::EP == pass) {
      const int rbase = C::RW * wm - C::EP * pass;
#pragma unroll
      for (int i = 0; i < C::RB; ++i)
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            E[(rbase + 16 * i + 4 * g + e) * (2 * C::EpiPitchDw) + 64 * wn + 16 * c + m] = (_Float16)acc[i][c][e];
    }
    lds_barrier();
#pragma unroll
    for (int k = 0; k < C::EP * C::CH / C::NT; ++k) {
      const int row = erow + (C::NT / C::CH) * k;
      const uint4 val = *reinterpret_cast<const uint4*>(lds + row * C::EpiPitchDw + 4 * ech);
      const int p = C::EP * pass + row;
      if (r0 + p < F.n_tokens) st16(yb + (int64_t)tok_l[p] * F.h_out + c0 + 8 * ech, val);
    }
  }
}

template <int BM, int BN, bool V4, int KS>
__global__ __launch_bounds__(128 * (BN / 64) * KS) __attribute__((amdgpu_waves_per_eu(2)))
void forward_kernel(ForwardLaunch F) {
  __shared__ __attribute__((aligned(16))) uint32_t lds[FwdTile<BM, BN, KS>::LdsDw];
  forward_tile<BM, BN, V4, KS>(F, blockIdx.x, lds);
}

template <int BM, int BN, int KS>
static const void* forward_fn(bool v4, int& nt) {
  nt = FwdTile<BM, BN, KS>::NT;
  return v4 ? reinterpret_cast<const void*>(&forward_kernel<BM, BN, true, KS>)
            : reinterpret_cast<const void*>(&forward_kernel<BM, BN, false, KS>);
}

hipError_t launch_forward(const ForwardLaunch& F, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  if (F.n_tiles <= 0) return hipSuccess;
  void* args[] = {const_cast<ForwardLaunch*>(&F)};
  const void* k;
  int nt;
  const bool v4 = F.v4 != 0;
  if (F.bm == 256 && F.bn == 256 && F.ks == 1) k = forward_fn<256, 256, 1>(v4, nt);
  else if (F.bm == 128 && F.bn == 256 && F.ks == 1) k = forward_fn<128, 256, 1>(v4, nt);
  else if (F.bm == 128 && F.bn == 128 && F.ks == 1) k = forward_fn<128, 128, 1>(v4, nt);
  else if (F.bm == 64 && F.bn == 128 && F.ks == 1) k = forward_fn<64, 128, 1>(v4, nt);
  else if (F.bm == 64 && F.bn == 128 && F.ks == 2) k = forward_fn<64, 128, 2>(v4, nt);
  else if (F.bm == 32 && F.bn == 128 && F.ks == 1) k = forward_fn<32, 128, 1>(v4, nt);
  else if (F.bm == 32 && F.bn == 128 && F.ks == 2) k = forward_fn<32, 128, 2>(v4, nt);
  else return hipErrorInvalidValue;
  const dim3 grid((unsigned)(8 * F.per_xcd));
  if (!start && !stop) return hipLaunchKernel(k, grid, dim3(nt), args, 0, stream);
  return hipExtLaunchKernel(k, grid, dim3(nt), args, 0, stream, start, stop, 0);
}

}  // namespace slora
