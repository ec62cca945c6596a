// HIP kernels of the paged, heterogeneous-batch LoRA delta for MI355X (gfx950).
//
// The delta (S-LoRA summary page, "The mechanism": keep one base W and
// compute x A B per request on the fly; blog page, section 2 pseudocode: the
// per-token product times a scaling factor) is split in two stages:
//
//   shrink  v[t, j] = sum_k x[t, k] * AT_j[k]           AT_j = page of row j of A^T
//   expand  y[t, o] = round(y[t, o] + s * sum_j v[t, j] * B_j[o])
//
// where the pages are gathered through the per-tile page lists the host
// segment builder resolved (summary page, "Heterogeneous batching kernels":
// gather non-contiguous adapter pages, ranks differ across the batch).
//
// Each kernel walks a list of self-contained tile records (one record per
// workgroup, 256 threads), of two kinds:
//   * GEMV tiles (vector ALU) for segments with few tokens: the decode case is
//     a bandwidth-bound matrix-vector product, so rows stream from HBM in
//     16-byte coalesced loads, fp16 pairs go through v_dot2_f32_f16, and the
//     rank-row partial sums are reduced with a butterfly reduce-scatter over
//     the wavefront followed by one LDS pass across the four waves.
//   * MFMA tiles (matrix cores, fp16 only) for segments where at least a
//     block of 16 tokens share an adapter: the shrink is a 16 x K x rank GEMM
//     fed straight from global memory (x rows and A^T page rows are both
//     K-contiguous), the expand stages 32-row slices of the B pages in LDS and
//     multiplies the fp32 v split into an fp16 high and low part, so the
//     matrix cores see v with about 22 significant bits and accumulate in fp32.
// Every output element is written by exactly one thread, once, with one
// rounding; no atomics, so results are deterministic run to run and do not
// depend on where the pages sit in the pool.
#include <type_traits>

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "slora_device.h"

namespace slora {

typedef _Float16 half2v __attribute__((ext_vector_type(2)));

template <typename T> struct VecN;
template <> struct VecN<_Float16> { static constexpr int N = 8; };
template <> struct VecN<float> { static constexpr int N = 4; };


// Streaming (non-temporal) 16-byte load and store, for data read once per
// launch: page rows of the vector-ALU tiles, x rows of the MFMA shrink (each
// K split of a 64-token block reads its own k range once), and y.  Measured
// on MI355X, row gathers of 60-240 MB stream 1.5-1.7x faster with the
// non-temporal hint than with ordinary loads.  The A^T rows of the MFMA
// shrink and the B slices of the MFMA expand, read again by every token block
// of the segment, keep ordinary loads, and the MFMA expand stores y with
// ordinary stores (measured faster there).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_nt(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st16_nt(void* p, uint4 v) {
  __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(p));
}
#ifndef SLORA_NT_A
#define SLORA_NT_A 1
#endif
#ifndef SLORA_NT_B
#define SLORA_NT_B 1
#endif
#ifndef SLORA_NT_Y
#define SLORA_NT_Y 1
#endif
#ifndef SLORA_NT_X
#define SLORA_NT_X 1
#endif
template <bool NT> __device__ __forceinline__ uint4 ldsel(const void* p) { return NT ? ld16_nt(p) : ld16(p); }
template <bool NT> __device__ __forceinline__ void stsel(void* p, uint4 v) { if (NT) st16_nt(p, v); else st16(p, v); }

__device__ __forceinline__ float dot16(uint4 a, uint4 b, float acc, _Float16) {
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, a.x), __builtin_bit_cast(half2v, b.x), acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, a.y), __builtin_bit_cast(half2v, b.y), acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, a.z), __builtin_bit_cast(half2v, b.z), acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, a.w), __builtin_bit_cast(half2v, b.w), acc, false);
  return acc;
}
__device__ __forceinline__ float dot16(uint4 a, uint4 b, float acc, float) {
  acc = fmaf(__uint_as_float(a.x), __uint_as_float(b.x), acc);
  acc = fmaf(__uint_as_float(a.y), __uint_as_float(b.y), acc);
  acc = fmaf(__uint_as_float(a.z), __uint_as_float(b.z), acc);
  acc = fmaf(__uint_as_float(a.w), __uint_as_float(b.w), acc);
  return acc;
}

// 16 bytes of T -> VecN<T>::N floats (exact conversions).
__device__ __forceinline__ void to_float(uint4 v, float (&f)[8], _Float16) {
  half8 h = __builtin_bit_cast(half8, v);
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = (float)h[e];
}
__device__ __forceinline__ void to_float(uint4 v, float (&f)[4], float) {
  f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
  f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
}
// y chunk + delta -> one rounding per element back to T.
__device__ __forceinline__ uint4 add_round(uint4 y, const float (&d)[8], _Float16) {
  half8 h = __builtin_bit_cast(half8, y);
  half8 o;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = (_Float16)((float)h[e] + d[e]);
  return __builtin_bit_cast(uint4, o);
}
__device__ __forceinline__ uint4 add_round(uint4 y, const float (&d)[4], float) {
  uint4 o;
  o.x = __float_as_uint(__uint_as_float(y.x) + d[0]);
  o.y = __float_as_uint(__uint_as_float(y.y) + d[1]);
  o.z = __float_as_uint(__uint_as_float(y.z) + d[2]);
  o.w = __float_as_uint(__uint_as_float(y.w) + d[3]);
  return o;
}

// Select by mask on the values themselves (a plain ?: on two array elements
// can be folded into one dynamically indexed load, which spills the array).
__device__ __forceinline__ float pick(bool c, float a, float b) {
  const uint32_t m = 0u - (uint32_t)c;
  return __uint_as_float((__float_as_uint(a) & m) | (__float_as_uint(b) & ~m));
}

// Butterfly reduce-scatter over a wavefront of 64 lanes: on return, lane l
// holds the wave-wide sum of p[l / (64 / N)] (N a power of two, N <= 64).
// Each halving step swaps half of the still-live partials with the partner
// lane, so N partials cost N-1 exchanges instead of N * log2(64).
template <int N>
__device__ __forceinline__ float wave_reduce_scatter(float (&p)[N], int lane) {
  static_assert(N >= 1 && N <= 64 && (N & (N - 1)) == 0, "power of two");
#pragma unroll
  for (int s = 0; s < 6; ++s) {
    const int off = 32 >> s;
    const int n = (N >> s) > 0 ? (N >> s) : 1;  // live partials before this step
    if (n > 1) {
      const int half = n / 2;
      const bool upper = (lane & off) != 0;
#pragma unroll
      for (int i = 0; i < N / 2; ++i) {
        if (i < half) {
          const float lo = p[i], hi = p[i + half];
          const float send = pick(upper, lo, hi);
          const float keep = pick(upper, hi, lo);
          p[i] = keep + __shfl_xor(send, off, 64);
        }
      }
    } else {
      p[0] += __shfl_xor(p[0], off, 64);
    }
  }
  return p[0];
}




// Copy the part of a tile record this launch needs (header, tokens and the
// page list of projection `proj`) into LDS with one batch of independent
// loads, so that page ids and token ids come from LDS instead of a chain of
// dependent global loads.  Layout in LDS: [HDR][tokcap][pagecap].
constexpr int kMaxRecWords = REC_HDR + kTokCap + kMaxPageCap;

__device__ __forceinline__ void record_to_lds(const int32_t* rec, int tokcap, int pagecap, int proj,
                                              int32_t* srec) {
  const int head = REC_HDR + tokcap;
  const int n = head + pagecap;
  for (int i = threadIdx.x; i < n; i += kThreads) srec[i] = rec[i < head ? i : i + proj * pagecap];
  __syncthreads();
}

// The projection a workgroup works on: its x, its y, where its x A values go
// (staged launches: the workspace; fused launches: the exchange pairs) and
// which page list of the tile record it reads.
struct Slot {
  const void* x;
  void* y;
  float* v;
  unsigned long long* vtag;
  int32_t proj;
};

__device__ __forceinline__ Slot make_slot(const DeltaLaunch& L, int s) {
  const int64_t area = (int64_t)L.n_splits * L.sum_rt;
  const int p = L.projs[s];
  return Slot{L.xs[s], L.ys[s], L.v + s * area, L.vtag + p * area, p};
}

// Fused launch: shrink tiles and expand tiles run in one grid, and v passes
// from one to the other as self-validating (value, epoch) pairs.  A shrink
// tile stores each v value together with the launch's epoch in one 64-bit
// agent-scope atomic store; an expand tile loads its tokens' v pairs with
// agent-scope atomic loads and goes on once every pair carries the current
// epoch, polling again otherwise.  Agent-scope atomics are coherent across the
// XCDs by themselves (they leave no dirty or stale copy in an XCD's L2) and a
// 64-bit aligned store is seen whole or not at all, so no fence, counter or
// completion wait is needed on either side.  The pairs live in the metadata
// buffer, which the upload zeroes, and epochs count 1, 2, ... from there, so
// no stale pair can carry the current epoch.
//
// A 64-token MFMA shrink block split over K writes partial sums tagged with
// the epoch and bit 31 set (kPartialTag), each split into its own area of
// sum_rt pairs; a combine tile waits for all of a block's partials, adds them
// in split order and writes the value with the plain epoch into area 0, where
// the expand tiles look.  A partial can therefore never pass for a value.
//
// Progress: shrink tiles occupy the lower block indices and never wait, and
// workgroups are dispatched in index order, so every shrink tile a waiting
// expand tile depends on has been dispatched and finishes.  The wait is
// bounded all the same: past kMaxSpins polls it raises error_flag and goes on,
// so every wave of the grid always exits.
constexpr uint32_t kMaxSpins = 1u << 20;
constexpr uint32_t kPartialTag = 0x80000000u;

template <bool FUSED>
__device__ __forceinline__ void store_v(const Slot& S, int64_t idx, float x, uint32_t tag) {
  if constexpr (FUSED) {
    const unsigned long long pair = ((unsigned long long)tag << 32) | __float_as_uint(x);
    __hip_atomic_store(S.vtag + idx, pair, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    S.v[idx] = x;
  }
}

// Loads v[idx] of every (valid) slot this thread owns, polling until all
// threads of the workgroup hold current values (pairs tagged `want`).  get(q)
// gives slot q's index (or -1), put(q, value) receives the value; the first nq
// (uniform, <= N) slots of each thread are in use.  All loads of a poll are issued before
// any is consumed, at index `safe` (any valid v index) for a slot with no
// value, so they travel to memory together instead of one round trip each.
template <bool FUSED, int N, typename Get, typename Put>
__device__ __forceinline__ void load_v(const DeltaLaunch& L, const Slot& S, int nq, int safe, Get get, Put put,
                                       uint32_t want) {
  int idx[N];
#pragma unroll
  for (int q = 0; q < N; ++q) idx[q] = q < nq ? get(q) : -1;
  if constexpr (!FUSED) {
    float val[N];
#pragma unroll
    for (int q = 0; q < N; ++q)
      if (q < nq) val[q] = S.v[idx[q] >= 0 ? idx[q] : safe];
#pragma unroll
    for (int q = 0; q < N; ++q)
      if (q < nq) put(q, idx[q] >= 0 ? val[q] : 0.f);
  } else {
    for (uint32_t spins = 0;; ++spins) {
      unsigned long long pair[N];
#pragma unroll
      for (int q = 0; q < N; ++q)
        if (q < nq)
          pair[q] = __hip_atomic_load(S.vtag + (idx[q] >= 0 ? idx[q] : safe), __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
      bool ok = true;
#pragma unroll
      for (int q = 0; q < N; ++q) {
        if (q < nq) {
          ok = ok && (idx[q] < 0 || (uint32_t)(pair[q] >> 32) == want);
          put(q, idx[q] >= 0 ? __uint_as_float((uint32_t)pair[q]) : 0.f);
        }
      }
      if (__syncthreads_and(ok)) break;
      if (spins >= kMaxSpins) {
        if (threadIdx.x == 0) __hip_atomic_store(L.error_flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
}

// ---------------------------------------------------------------------------
// Shrink, vector-ALU tile: up to TB tokens x RB rank rows, whole h_in.
// Thread tid owns the 16-byte chunks tid, tid+256, ... of every row; the A^T
// rows stay in registers while each token's x chunks are dotted against them.
// The general tile holds kGemvMaxTok tokens.  A tile of one token needs a
// quarter of the x registers; at four chunks a thread the registers saved
// hold twice the rows (kShrinkRowsOne): half the tiles, each with twice the
// bytes in flight.

template <typename T, int NCK, bool FUSED, int RB = kShrinkRowBudget / NCK, int TB = kGemvMaxTok>
__device__ void shrink_gemv_tile(const DeltaLaunch& L, const Slot& S, const int32_t* srec, float* red) {
  constexpr int VEC = VecN<T>::N;
  const int ntok = uni(srec[REC_NTOK]);
  const int rank = uni(srec[REC_RANK]);
  const int j0 = uni(srec[REC_POS]);
  const int nrows = uni(srec[REC_LEN]);
  const int v0 = uni(srec[REC_V0]);
  const int32_t* toks = srec + REC_HDR;
  const int32_t* pages = srec + REC_HDR + L.tokcap;
  const int tid = threadIdx.x, lane = tid & 63, wave = uni(tid >> 6);
  const int nchunks = L.h_in / VEC;
  const T* x = reinterpret_cast<const T*>(S.x);

  // All row and token addresses first, then every load of the tile in one batch.
  const char* arow[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r)
    arow[r] = L.pool.base_a + (int64_t)pages[r < nrows ? r : 0] * L.pool.page_bytes_a;
  const T* xrow[TB];
#pragma unroll
  for (int k = 0; k < TB; ++k) xrow[k] = x + (int64_t)toks[k < ntok ? k : 0] * L.h_in;

  uint4 a[RB][NCK];
  uint4 xv[TB][NCK];
#pragma unroll
  for (int ck = 0; ck < NCK; ++ck) {
    const int c = tid + ck * kThreads;
    const bool inb = c < nchunks;
#pragma unroll
    for (int r = 0; r < RB; ++r)
      a[r][ck] = (inb && r < nrows) ? ldsel<SLORA_NT_A>(arow[r] + (int64_t)c * 16) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int k = 0; k < TB; ++k)
      xv[k][ck] = (inb && k < ntok) ? ld16(xrow[k] + (int64_t)c * VEC) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int k = 0; k < TB; ++k) {
    if (k < ntok) {
      float p[RB];
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        float acc = 0.f;
#pragma unroll
        for (int ck = 0; ck < NCK; ++ck) acc = dot16(a[r][ck], xv[k][ck], acc, T());
        p[r] = acc;
      }
      const float s = wave_reduce_scatter<RB>(p, lane);
      constexpr int LPR = 64 / RB;  // lanes per reduced row
      if ((lane & (LPR - 1)) == 0) red[(k * 4 + wave) * RB + lane / LPR] = s;
    }
  }
  __syncthreads();
  for (int i = tid; i < ntok * nrows; i += kThreads) {
    const int k = i / nrows, r = i - k * nrows;
    const float* q = red + (k * 4) * RB + r;
    const float sum = ((q[0] + q[RB]) + q[2 * RB]) + q[3 * RB];
    store_v<FUSED>(S, v0 + (int64_t)k * rank + j0 + r, sum, L.epoch);
  }
}

// The vector-ALU shrink tile a record asks for: one token with more rows than
// the general tile holds takes the one-token shape.
template <typename T, int NCK, bool FUSED>
__device__ __forceinline__ void shrink_gemv_any(const DeltaLaunch& L, const Slot& S, const int32_t* srec, float* red) {
  if constexpr (NCK == kShrinkOneNck) {
    if (uni(srec[REC_NTOK]) == 1 && uni(srec[REC_LEN]) > kShrinkRowBudget / NCK) {
      shrink_gemv_tile<T, NCK, FUSED, kShrinkRowsOne, 1>(L, S, srec, red);
      return;
    }
  }
  shrink_gemv_tile<T, NCK, FUSED>(L, S, srec, red);
}

// ---------------------------------------------------------------------------
// Shrink, MFMA tile (fp16): up to 64 tokens x all r rows (r <= 64) over the
// k range [pos, pos + len) of one K split.  C[t][j] = sum_k x[t][k] AT_j[k]
// with v_mfma_f32_16x16x32_f16: wave w owns tokens 16w .. 16w+15 and all
// rank rows, so the four waves share each staged chunk of A^T.  x and A^T
// stream through LDS in chunks of 64 k (128 bytes per row): a wave loads 8
// whole rows per instruction, and a lane's MFMA operand (8 consecutive k of
// one row) is one 16-byte LDS read; the 16-byte chunks of a row are
// XOR-swizzled by row.  Three chunks of loads run ahead of the matrix cores
// in registers; the LDS chunks alternate between two buffers, one barrier per
// chunk.

constexpr int kShrinkStageDw = 2 * kMfmaExpandTok * (kShrinkKc / 2);   // x and A^T rows of one chunk
constexpr int kShrinkLdsFloats = 2 * kShrinkStageDw;                   // two chunks (32 KB)


// NTX: x rows with the streaming hint (x read by this launch once), or, when
// several projections of a launch share one x (q, k and v), with ordinary
// loads so that the other projections' tiles find the rows in cache (13B
// mixed step 223.8 against 226.6 us; the 7B prefill batch, one projection,
// 67.5-68.0 with the hint against 72.1-72.9 without).
template <bool FUSED, bool NTX = SLORA_NT_X>
__device__ void shrink_mfma_tile(const DeltaLaunch& L, const Slot& S, const int32_t* srec, float* lds) {
  const int ntok = uni(srec[REC_NTOK]);
  const int rank = uni(srec[REC_RANK]);
  const int k0 = uni(srec[REC_POS]);
  const int klen = uni(srec[REC_LEN]);
  const int v0 = uni(srec[REC_V0]);
  const int split = uni(srec[REC_AUX]);
  const int nsplit = uni(srec[REC_NSPLIT]);
  const int32_t* toks = srec + REC_HDR;
  const int32_t* pages = srec + REC_HDR + L.tokcap;
  const int tid = threadIdx.x, lane = tid & 63, wave = uni(tid >> 6);
  const int m = lane & 15, g = lane >> 4;
  const int nb = (rank + 15) >> 4;                   // 16-row blocks of A^T
  const int nkc = klen / kShrinkKc;
  uint32_t* stage = reinterpret_cast<uint32_t*>(lds);

  // Loader: thread tid moves the 16-byte chunk tid & 7 of rows tid >> 3 and
  // 32 + (tid >> 3) of x and of A^T; rows past ntok / rank repeat the last
  // one (their results are never stored).
  const int lr = tid >> 3, lc = tid & 7;
  const _Float16* xr[2];
  const char* ar[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int row = lr + 32 * h;
    xr[h] = reinterpret_cast<const _Float16*>(S.x) + (int64_t)toks[min(row, ntok - 1)] * L.h_in + k0 + 8 * lc;
    ar[h] = L.pool.base_a + (int64_t)pages[min(row, rank - 1)] * L.pool.page_bytes_a + (int64_t)(k0 + 8 * lc) * 2;
  }
  auto load_chunk = [&](int kc, uint4 (&r)[4]) {
    kc = kc < nkc ? kc : nkc - 1;   // loads past the end re-read the last chunk, unused
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      r[h] = ldsel<NTX>(xr[h] + kShrinkKc * kc);
      r[2 + h] = ld16(ar[h] + 2 * kShrinkKc * kc);
    }
  };
  auto store_chunk = [&](uint32_t* buf, const uint4 (&r)[4]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = lr + 32 * h;
      *reinterpret_cast<uint4*>(buf + chunk_dw(row, lc)) = r[h];
      *reinterpret_cast<uint4*>(buf + kShrinkStageDw / 2 + chunk_dw(row, lc)) = r[2 + h];
    }
  };

  float4v acc[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) acc[b] = float4v{0.f, 0.f, 0.f, 0.f};
  // Ring of three chunks in registers, filled in order (no reordering across
  // the scheduling barriers), so each wait covers only the oldest chunk.  All
  // loads, LDS stores and barriers run for every slot of the last round too;
  // only the matrix work of chunks past the end is skipped.
  constexpr int D = 3;
  uint4 ring[D][4];
#pragma unroll
  for (int slot = 0; slot < D; ++slot) {
    load_chunk(slot, ring[slot]);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int kc0 = 0; kc0 < nkc; kc0 += D) {
#pragma unroll
    for (int slot = 0; slot < D; ++slot) {
      const int kc = kc0 + slot;
      uint32_t* buf = stage + (kc & 1) * kShrinkStageDw;
      store_chunk(buf, ring[slot]);
      lds_barrier();
      load_chunk(kc + D, ring[slot]);
      __builtin_amdgcn_sched_barrier(0);
      if (kc < nkc) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int rx = 16 * wave + m;
          const half8 xop = __builtin_bit_cast(half8, *reinterpret_cast<const uint4*>(buf + chunk_dw(rx, 4 * ks + g)));
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            if (b < nb) {
              const int ra = 16 * b + m;
              const half8 aop = __builtin_bit_cast(
                  half8, *reinterpret_cast<const uint4*>(buf + kShrinkStageDw / 2 + chunk_dw(ra, 4 * ks + g)));
              acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xop, aop, acc[b], 0, 0, 0);
            }
          }
        }
      }
    }
  }
  // acc[b][i] = C[token 16 wave + 4g + i][rank row 16b + m]
  const uint32_t tag = nsplit > 1 ? (L.epoch | kPartialTag) : L.epoch;
  const int64_t area = (int64_t)split * L.sum_rt;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * wave + 4 * g + i, j = 16 * b + m;
      if (b < nb && t < ntok && j < rank) store_v<FUSED>(S, area + v0 + (int64_t)t * rank + j, acc[b][i], tag);
    }
  }
}

// ---------------------------------------------------------------------------
// Combine tile: up to 16 tokens of a 64-token MFMA shrink block split over K.
// v = sum over splits s = 0, 1, ... of the partial in area s, added in that
// order (deterministic), written to area 0 with the plain epoch.
template <bool FUSED>
__device__ void combine_tile(const DeltaLaunch& L, const Slot& S, const int32_t* srec) {
  const int ntok = uni(srec[REC_NTOK]);
  const int rank = uni(srec[REC_RANK]);
  const int v0 = uni(srec[REC_V0]);
  const int nsplit = uni(srec[REC_AUX]);
  const int tid = threadIdx.x;
  const int n = ntok * rank;                           // <= 16 x 64 = 4 per thread
  constexpr int Q = kCombineTok * kMaxRankMfma / kThreads;
  // slot q * kMaxSplits + s: value tid + 256 q of split s
  float part[Q * kMaxSplits];
  load_v<FUSED, Q * kMaxSplits>(
      L, S, Q * kMaxSplits, v0,
      [&](int qs) -> int {
        const int q = qs / kMaxSplits, sp = qs % kMaxSplits, i = tid + q * kThreads;
        return (i < n && sp < nsplit) ? sp * L.sum_rt + v0 + i : -1;
      },
      [&](int qs, float val) { part[qs] = val; }, L.epoch | kPartialTag);
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int i = tid + q * kThreads;
    float sum = 0.f;
#pragma unroll
    for (int sp = 0; sp < kMaxSplits; ++sp)
      if (sp < nsplit) sum += part[q * kMaxSplits + sp];
    if (i < n) store_v<FUSED>(S, v0 + i, sum, L.epoch);
  }
}

template <typename T, int NCK>
__global__ __launch_bounds__(kThreads) void shrink_kernel(DeltaLaunch L) {
  __shared__ float red[sizeof(T) == 2 ? kShrinkLdsFloats : 4 * 4 * 16];
  __shared__ int32_t srec[kMaxRecWords];
  const Slot S = make_slot(L, 0);   // staged launches run one projection
  const int32_t* rec = L.rec + (int64_t)L.shrink_idx[blockIdx.x] * L.stride;
  record_to_lds(rec, L.tokcap, L.pagecap, S.proj, srec);
  if constexpr (sizeof(T) == 2) {
    if (uni(srec[REC_KIND]) & KIND_MFMA_BIT) {
      shrink_mfma_tile<false>(L, S, srec, red);
      return;
    }
  }
  shrink_gemv_any<T, NCK, false>(L, S, srec, red);
}

// Staged launches: the combine tiles, records n_shrink .. n_shrink + n_combine.
__global__ __launch_bounds__(kThreads) void combine_kernel(DeltaLaunch L) {
  __shared__ int32_t srec[kMaxRecWords];
  const Slot S = make_slot(L, 0);
  record_to_lds(L.rec + (int64_t)(L.n_shrink + blockIdx.x) * L.stride, L.tokcap, L.pagecap, S.proj, srec);
  combine_tile<false>(L, S, srec);
}

// ---------------------------------------------------------------------------
// Expand, vector-ALU tile: up to kGemvMaxTok tokens x `width` columns, all r
// rows.  width/VEC threads cover the columns with one 16-byte chunk each and
// G = 256 / (width/VEC) groups of them split the r rows; the groups' partial
// sums meet in LDS and group 0 applies y += s * d with one rounding.

template <typename T, bool FUSED, bool PIPE>
__device__ void expand_gemv_tile(const DeltaLaunch& L, const Slot& S, const int32_t* srec, float* lds) {
  constexpr int VEC = VecN<T>::N;
  constexpr int TB = kGemvMaxTok;
  constexpr int RCH = kExpandRowSet;  // B rows per thread issued together
  const int ntok = uni(srec[REC_NTOK]);
  const int rank = uni(srec[REC_RANK]);
  const int o0 = uni(srec[REC_POS]);
  const int ncol = uni(srec[REC_LEN]);
  const int v0 = uni(srec[REC_V0]);
  const float scale = __int_as_float(uni(srec[REC_SCALE]));
  const int width = uni(srec[REC_AUX]);
  const int32_t* toks = srec + REC_HDR;
  const int32_t* pages = srec + REC_HDR + L.tokcap;
  const int tid = threadIdx.x;
  const int nct = width / VEC;
  const int G = kThreads / nct;
  const int ct = tid % nct, g = tid / nct;

  float* sv = lds;                   // [TB][rank] v of the tile's tokens
  float* part = lds + TB * 256;      // [G-1][TB][nct][VEC] partial sums of groups 1..G-1
  T* y = reinterpret_cast<T*>(S.y);

  // Issue everything the tile reads before waiting on any of it: the first
  // RCH B rows of this thread, (group 0) the y chunks of the epilogue, and v
  // (in a fused launch, once the segment's shrink tiles are done).  With PIPE
  // (batches whose threads hold more than RCH B rows) the rows are
  // software-pipelined: the next RCH rows are in flight while the current
  // ones are used, every B load issued unconditionally at a clamped row (rows
  // past this thread's last one re-read it, threads with no row read row 0 at
  // column o0) so that the compiler's wait counts cover exactly the rows in
  // use.  Without PIPE (at most RCH rows a thread, the decode batches) the
  // second register set is not needed and more workgroups stay resident.
  const bool active = ct * VEC < ncol;
  const int nrt = (active && g < rank) ? (rank - g + G - 1) / G : 0;   // rows of this thread
  const bool has = nrt > 0;
  const int64_t col_byte = (int64_t)(o0 + (has ? ct * VEC : 0)) * sizeof(T);
  auto brow = [&](int i) -> const char* {
    const int slot = has ? g + min(i, nrt - 1) * G : 0;
    return L.pool.base_b + (int64_t)pages[slot] * L.pool.page_bytes_b + col_byte;
  };
  uint4 bq[RCH];
#pragma unroll
  for (int i = 0; i < RCH; ++i) {
    if constexpr (PIPE) bq[i] = ldsel<SLORA_NT_B>(brow(i));
    else bq[i] = i < nrt ? ldsel<SLORA_NT_B>(brow(i)) : make_uint4(0, 0, 0, 0);
  }
  uint4 yv[TB];
#pragma unroll
  for (int k = 0; k < TB; ++k)
    yv[k] = (g == 0 && active && k < ntok) ? ldsel<SLORA_NT_Y>(y + (int64_t)toks[k] * L.h_out + o0 + ct * VEC)
                                           : make_uint4(0, 0, 0, 0);
  load_v<FUSED, TB>(
      L, S, (ntok * rank + kThreads - 1) / kThreads, v0,
      [&](int q) -> int { const int i = tid + q * kThreads; return i < ntok * rank ? v0 + i : -1; },
      [&](int q, float val) { const int i = tid + q * kThreads; if (i < ntok * rank) sv[i] = val; }, L.epoch);
  __syncthreads();

  float acc[TB][VEC];
#pragma unroll
  for (int k = 0; k < TB; ++k)
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[k][e] = 0.f;
  auto use_rows = [&](int i0) {
#pragma unroll
    for (int i = 0; i < RCH; ++i) {
      if (i0 + i < nrt) {
        const int j = g + (i0 + i) * G;
        float bf[VEC];
        to_float(bq[i], bf, T());
#pragma unroll
        for (int k = 0; k < TB; ++k) {
          if (k < ntok) {
            const float vk = sv[k * rank + j];
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc[k][e] = fmaf(vk, bf[e], acc[k][e]);
          }
        }
      }
    }
  };
  if constexpr (PIPE) {
    const int nrt_u = (rank + G - 1) / G;   // rows of group 0, the most any thread has
    for (int i0 = 0; i0 < nrt_u; i0 += RCH) {
      uint4 nq[RCH];
      const bool more = i0 + RCH < nrt_u;
      if (more) {
        // The next set's loads go out at raised wave priority, ahead of the
        // other waves' arithmetic on the SIMD, so they are in flight sooner
        // (70B MLP: 263 -> 256 us; the same at the first set, or around the
        // shrink tile's loads, was slower or no faster).
        __builtin_amdgcn_s_setprio(3);
#pragma unroll
        for (int i = 0; i < RCH; ++i) nq[i] = ldsel<SLORA_NT_B>(brow(i0 + RCH + i));
        __builtin_amdgcn_s_setprio(0);
      }
      use_rows(i0);
      if (more) {
#pragma unroll
        for (int i = 0; i < RCH; ++i) bq[i] = nq[i];
      }
    }
  } else {
    for (int i0 = 0; i0 < nrt; i0 += RCH) {
      if (i0 > 0) {
#pragma unroll
        for (int i = 0; i < RCH; ++i)
          bq[i] = i0 + i < nrt ? ldsel<SLORA_NT_B>(brow(i0 + i)) : make_uint4(0, 0, 0, 0);
      }
      use_rows(i0);
    }
  }
  if (G > 1) {
    if (g > 0) {
#pragma unroll
      for (int k = 0; k < TB; ++k) {
        if (k < ntok) {
          float* q = part + (((int64_t)(g - 1) * TB + k) * nct + ct) * VEC;
#pragma unroll
          for (int e = 0; e < VEC; ++e) q[e] = acc[k][e];
        }
      }
    }
    __syncthreads();
    if (g == 0) {
      for (int gg = 1; gg < G; ++gg) {
#pragma unroll
        for (int k = 0; k < TB; ++k) {
          if (k < ntok) {
            const float* q = part + (((int64_t)(gg - 1) * TB + k) * nct + ct) * VEC;
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc[k][e] += q[e];
          }
        }
      }
    }
  }
  if (g == 0 && active) {
#pragma unroll
    for (int k = 0; k < TB; ++k) {
      if (k < ntok) {
        T* yp = y + (int64_t)toks[k] * L.h_out + o0 + ct * VEC;
        float d[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) d[e] = scale * acc[k][e];
        stsel<SLORA_NT_Y>(yp, add_round(yv[k], d, T()));
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Expand, MFMA tile (fp16): up to 64 tokens x `len` columns, all r rows
// (r <= kMaxRankMfma).  Y[t][o] += sum_j (s v)[t][j] * B_j[o] with
// v_mfma_f32_16x16x32_f16: the A operand is 16 tokens x 32 rows of s*v, split
// into an fp16 high and low part after a per-token power-of-two
// normalisation (about 22 significant bits, registers); the B operand is 32
// rows x 16 columns of a B slice staged row-major in LDS and read with
// ds_read_b64_tr_b16, which hands each lane 4 rows of one column.  Wave w
// owns tokens 16w .. 16w+15 and every column of a pass, so the four waves
// share each staged slice (a quarter of the B reads of 16-token tiles).  The
// accumulators leave through LDS, so y is read and written in whole
// 128-byte lines.

constexpr int kSliceDw = 32 * kSliceRowDw;      // one staged 32-row slice (8 KB)
constexpr int kEpiPitch = kMfmaPass + 4;        // floats per epilogue row
constexpr int kMfmaExpandLds = 2 * kSliceDw + kMfmaExpandTok * kEpiPitch + kMfmaExpandTok;

constexpr int kBufferFormat = 0x00020000;   // descriptor word 3: raw 32-bit buffer

template <bool FUSED, int KS>   // KS: 32-row k slices of the rank (1 or 2), fixed per instantiation
__device__ void expand_mfma_tile(const DeltaLaunch& L, const Slot& S, const int32_t* srec, float* lds) {
  const int ntok = uni(srec[REC_NTOK]);
  const int rank = uni(srec[REC_RANK]);
  const int o0 = uni(srec[REC_POS]);
  const int ncol = uni(srec[REC_LEN]);
  const int v0 = uni(srec[REC_V0]);
  const float scale = __int_as_float(uni(srec[REC_SCALE]));
  const int32_t* toks = srec + REC_HDR;
  const int32_t* pages = srec + REC_HDR + L.tokcap;
  const int tid = threadIdx.x, lane = tid & 63, wave = uni(tid >> 6);
  const int m = lane & 15, g = lane >> 4;
  constexpr int ks_n = KS;                             // (rank + 31) / 32
  const int n_pass = (ncol + kMfmaPass - 1) / kMfmaPass;
  const int n_steps = n_pass * ks_n;                   // (pass, k slice), pass-major
  uint32_t* slice = reinterpret_cast<uint32_t*>(lds);  // two slices, used in turn
  float* epi = lds + 2 * kSliceDw;                     // [64][kEpiPitch]
  float* up_tok = epi + kMfmaExpandTok * kEpiPitch;    // per-token scale back
  _Float16* yb = reinterpret_cast<_Float16*>(S.y);
  const __amdgpu_buffer_rsrc_t yrsrc = __builtin_amdgcn_make_buffer_rsrc(S.y, 0, (int)L.y_bytes, kBufferFormat);

  // Every global access below is issued unconditionally (loads at a clamped
  // address where they fall outside the tile), so that each wait covers only
  // the operands it is for.  A clamped B row (j >= rank) meets a zero s*v.
  //
  // Staging: thread tid moves 8 columns (chunk tid & 15) of rows tid >> 4 and
  // 16 + (tid >> 4) of a slice: 16 threads cover a row's 256 bytes.
  const int s_chunk = tid & 15, s_row = tid >> 4;
  auto stage_load = [&](int step, uint4 (&r)[2]) {
    step = step < n_steps ? step : n_steps - 1;
    const int pass = step / ks_n, ks = step - pass * ks_n;
    const int col = min(pass * kMfmaPass + 8 * s_chunk, ncol - 8);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int j = min(32 * ks + s_row + 16 * h, rank - 1);
      r[h] = ld16(L.pool.base_b + (int64_t)pages[j] * L.pool.page_bytes_b + (int64_t)(o0 + col) * 2);
    }
  };
  auto stage_store = [&](uint32_t* dst, const uint4 (&r)[2]) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
      *reinterpret_cast<uint4*>(dst + quad_dw(s_row + 16 * h, 2 * s_chunk)) = r[h];
  };
  // y chunks of a pass: thread tid takes 8 columns (chunk tid & 15) of tile
  // rows (tid >> 4) + 16k, k = 0..3.
  auto y_row = [&](int k) { return (tid >> 4) + 16 * k; };
  auto y_col = [&](int pass) { return pass * kMfmaPass + 8 * (tid & 15); };
  auto load_y = [&](int pass, uint4 (&yq)[4]) {
    pass = pass < n_pass ? pass : n_pass - 1;
    const int col = min(y_col(pass), ncol - 8);
#pragma unroll
    for (int k = 0; k < 4; ++k)
      yq[k] = ldsel<SLORA_NT_Y>(yb + (int64_t)toks[min(y_row(k), ntok - 1)] * L.h_out + o0 + col);
  };

  // Two staged slices in flight in registers (steps s and s+1), so each wait
  // covers a load issued two steps earlier.
  uint4 bs0[2], bs1[2];
  stage_load(0, bs0);
  stage_load(1, bs1);
  uint4 y0[4], y1[4];
  load_y(0, y0);

  // s*v of this lane's token (16 wave + m) at rows 32ks + 8g + i, zero past
  // ntok / rank.
  const int tok = 16 * wave + m;
  float sv[8 * KS];
  load_v<FUSED, 8 * KS>(
      L, S, 8 * ks_n, v0,
      [&](int q) -> int {
        const int j = 32 * (q >> 3) + 8 * g + (q & 7);
        return (tok < ntok && j < rank) ? v0 + tok * rank + j : -1;
      },
      [&](int q, float val) { sv[q] = scale * val; }, L.epoch);
  float amax = 0.f;
#pragma unroll
  for (int q = 0; q < 8 * KS; ++q)
    if (q < 8 * ks_n) amax = fmaxf(amax, fabsf(sv[q]));
  amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
  // Bring the token's largest |s v| into [2^14, 2^15) so hi and lo stay normal fp16.
  int ex = 0;
  if (amax > 0.f) {
    (void)frexpf(amax, &ex);
    ex = max(ex - 15, -100);
  }
  const float down = ldexpf(1.f, -ex);
  if (g == 0) up_tok[tok] = ldexpf(1.f, ex);
  half8 vhi[KS], vlo[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float f = sv[8 * ks + i] * down;
      const _Float16 h = (_Float16)f;
      vhi[ks][i] = h;
      vlo[ks][i] = (_Float16)(f - (float)h);
    }
  }

  // One pass: kMfmaPass columns, all k slices, then the epilogue.  yc holds
  // this pass's y (fetched a pass earlier), yn receives the next pass's; the
  // two register sets swap roles from pass to pass.  Step s (pass-major)
  // stages register slot and LDS buffer s & 1 -- static here, since the pass
  // loop is unrolled by two and KS is fixed.  Slices alternate between two LDS
  // buffers, so one barrier per slice suffices: a buffer is written again only
  // after every wave has passed the barrier of the slice that followed its
  // last read.
  auto pass_body = [&](auto par, int pass, uint4 (&yc)[4], uint4 (&yn)[4]) {
    float4v acc[kMfmaPass / 16];
#pragma unroll
    for (int c = 0; c < kMfmaPass / 16; ++c) acc[c] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int step = pass * ks_n + ks;
      constexpr int kpar = decltype(par)::value;
      const int slot = KS == 2 ? ks : kpar;             // == step & 1
      uint4 (&cur)[2] = slot ? bs1 : bs0;
      uint32_t* buf = slice + slot * kSliceDw;
      stage_store(buf, cur);
      lds_barrier();
      stage_load(step + 2, cur);
      if (ks == 0) load_y(pass + 1, yn);
#pragma unroll
      for (int cb = 0; cb < kMfmaPass / 16; ++cb) {
        // lane (m, g) reads row 8g + m/4 (+4), columns 16cb + 4(m%4) .. +3;
        // the transposing read returns rows 8g .. 8g+3 (+4) of column 16cb + m.
        const uint32_t* p0 = buf + quad_dw(8 * g + (m >> 2), 4 * cb + (m & 3));
        const uint32_t* p1 = buf + quad_dw(8 * g + 4 + (m >> 2), 4 * cb + (m & 3));
        const short4v r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) short4v*)(p0));
        const short4v r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) short4v*)(p1));
        const half8 bop = __builtin_bit_cast(half8, __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7));
        acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vhi[ks], bop, acc[cb], 0, 0, 0);
        acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vlo[ks], bop, acc[cb], 0, 0, 0);
      }
    }
    // acc[cb][i] = Y[token 16 wave + 4g + i][column 16cb + m] (before the scale back)
#pragma unroll
    for (int cb = 0; cb < kMfmaPass / 16; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) epi[(16 * wave + 4 * g + i) * kEpiPitch + 16 * cb + m] = acc[cb][i];
    lds_barrier();
    const int col = y_col(pass);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int row = y_row(k);
      const float* e = epi + row * kEpiPitch + 8 * (tid & 15);
      const float u = up_tok[row];
      float d[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) d[i] = e[i] * u;
      const uint4 out = add_round(yc[k], d, _Float16());
      // A row or column outside the tile stores past the descriptor's extent,
      // which the hardware drops: no branch, no traffic.  An ordinary store,
      // not a streaming one (7B prefill: 68.3-69.0 against 70.1-71.1 us; the
      // vector-ALU expand's y stores measured the same either way and keep
      // the streaming hint).
      const uint32_t off = (row < ntok && col < ncol) ? 2u * ((uint32_t)toks[row] * L.h_out + o0 + col) : 0xFFFFFFF0u;
      __builtin_amdgcn_raw_buffer_store_b128(u32x4{out.x, out.y, out.z, out.w}, yrsrc, off, 0, 0);
    }
  };
  for (int pass = 0;; pass += 2) {
    pass_body(std::integral_constant<int, 0>{}, pass, y0, y1);
    if (pass + 1 >= n_pass) break;
    pass_body(std::integral_constant<int, 1>{}, pass + 1, y1, y0);
    if (pass + 2 >= n_pass) break;
  }
}

template <bool FUSED>
__device__ __forceinline__ void expand_mfma_dispatch(const DeltaLaunch& L, const Slot& S, const int32_t* srec, float* lds) {
  static_assert(kMaxRankMfma == 64, "two instantiations cover ranks 1..64");
  if (uni(srec[REC_RANK]) <= 32)
    expand_mfma_tile<FUSED, 1>(L, S, srec, lds);
  else
    expand_mfma_tile<FUSED, 2>(L, S, srec, lds);
}

// LDS of the expand tiles: the vector-ALU tiles need kGemvLdsFloats, the
// MFMA tiles kMfmaExpandLds.  Kernels that never run an MFMA tile allocate
// the smaller size, which keeps four of them resident per CU.
constexpr int kGemvLdsFloats = kGemvMaxTok * 256 + 7 * kGemvMaxTok * 256;
constexpr int kExpandLdsFloats = kMfmaExpandLds > kGemvLdsFloats ? kMfmaExpandLds : kGemvLdsFloats;
static_assert(kShrinkLdsFloats <= kExpandLdsFloats, "the fused kernel's LDS holds the MFMA shrink stages");

template <typename T, bool PIPE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3))) void expand_kernel(DeltaLaunch L) {
  __shared__ float lds[sizeof(T) == 2 ? kExpandLdsFloats : kGemvLdsFloats];
  __shared__ int32_t srec[kMaxRecWords];
  const Slot S = make_slot(L, 0);
  const int32_t* rec = L.rec + (int64_t)L.expand_idx[blockIdx.x] * L.stride;
  record_to_lds(rec, L.tokcap, L.pagecap, S.proj, srec);
  if constexpr (sizeof(T) == 2) {
    if (uni(srec[REC_KIND]) & KIND_MFMA_BIT) {
      expand_mfma_dispatch<false>(L, S, srec, lds);
      return;
    }
  }
  expand_gemv_tile<T, false, PIPE>(L, S, srec, lds);
}

// Both stages in one launch over the records in launch order: shrink tiles
// and expand tiles that wait for their tokens' v (see store_v / load_v).
// With several projections (slots) the grid runs the records in phases, each
// a run of one tile kind (matrix-core shrink, vector-ALU shrink, combine,
// matrix-core expand, vector-ALU expand), every slot's copy of a phase before
// the next phase, so every tile a workgroup waits for still has a lower block
// index.
// MFMA=false leaves the matrix-core tiles out (a batch without them), which
// keeps the register budget, and so the workgroups resident per CU, of the
// vector-ALU tiles alone.
// Three workgroups per CU fit the matrix-core tiles' registers without
// spilling (fewer would leave slots empty); the widest vector-ALU shrink
// (h_in above 8192) needs more registers and runs two.
template <typename T, int NCK, bool MFMA, bool PIPE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(NCK == 8 ? 2 : 3)))
void fused_kernel(DeltaLaunch L) {
  __shared__ float lds[sizeof(T) == 2 && MFMA ? kExpandLdsFloats : kGemvLdsFloats];
  __shared__ int32_t srec[kMaxRecWords];
  // block -> (slot, record): phase k holds blocks n_slots * phase_rec[k] ..
  // n_slots * phase_rec[k+1] - 1, slot-major
  const int b = blockIdx.x;
  int k = 0;
#pragma unroll
  for (int i = 1; i < kMaxPhases; ++i)
    if (i < L.n_phases && b >= L.n_slots * L.phase_rec[i]) k = i;
  const int r0 = L.phase_rec[k], len = L.phase_rec[k + 1] - r0;
  const int off = b - L.n_slots * r0;
  const int slot = off / len;
  const int rec = r0 + (off - slot * len);
  const Slot S = make_slot(L, uni(slot));
  record_to_lds(L.rec + (int64_t)uni(rec) * L.stride, L.tokcap, L.pagecap, S.proj, srec);
  const int kind = uni(srec[REC_KIND]);
  if (!(kind & KIND_EXPAND_BIT)) {
    if constexpr (sizeof(T) == 2 && MFMA) {
      if (kind & KIND_COMBINE_BIT) {
        combine_tile<true>(L, S, srec);
        return;
      }
      if (kind & KIND_MFMA_BIT) {
        if (L.x_shared) shrink_mfma_tile<true, false>(L, S, srec, lds);
        else shrink_mfma_tile<true>(L, S, srec, lds);
        return;
      }
    }
    shrink_gemv_any<T, NCK, true>(L, S, srec, lds);
    return;
  }
  if constexpr (sizeof(T) == 2 && MFMA) {
    if (kind & KIND_MFMA_BIT) {
      expand_mfma_dispatch<true>(L, S, srec, lds);
      return;
    }
  }
  expand_gemv_tile<T, true, PIPE>(L, S, srec, lds);
}

// ---------------------------------------------------------------------------

// One launch of `kernel` over `blocks` workgroups; with events, through
// hipExtLaunchKernel so that the timestamps come from the dispatch itself.
static hipError_t launch_one(const void* kernel, int blocks, const DeltaLaunch& L, hipStream_t stream,
                             hipEvent_t start, hipEvent_t stop) {
  void* args[] = {const_cast<DeltaLaunch*>(&L)};
  if (!start && !stop)
    return hipLaunchKernel(kernel, dim3(blocks), dim3(kThreads), args, 0, stream);
  return hipExtLaunchKernel(kernel, dim3(blocks), dim3(kThreads), args, 0, stream, start, stop, 0);
}

// Instantiation for the GEMV shrink geometry: 16-byte chunks per thread per
// row, rounded up to a power of two.
template <typename T>
static int chunks_per_thread(int h_in) {
  const int per = (h_in / VecN<T>::N + kThreads - 1) / kThreads;
  return per <= 1 ? 1 : per <= 2 ? 2 : per <= 4 ? 4 : per <= 8 ? 8 : 0;
}

template <typename T>
static const void* shrink_fn(int nck) {
  switch (nck) {
    case 1: return reinterpret_cast<const void*>(&shrink_kernel<T, 1>);
    case 2: return reinterpret_cast<const void*>(&shrink_kernel<T, 2>);
    case 4: return reinterpret_cast<const void*>(&shrink_kernel<T, 4>);
    case 8: return reinterpret_cast<const void*>(&shrink_kernel<T, 8>);
    default: return nullptr;
  }
}

template <typename T, bool MFMA, bool PIPE>
static const void* fused_fn(int nck) {
  switch (nck) {
    case 1: return reinterpret_cast<const void*>(&fused_kernel<T, 1, MFMA, PIPE>);
    case 2: return reinterpret_cast<const void*>(&fused_kernel<T, 2, MFMA, PIPE>);
    case 4: return reinterpret_cast<const void*>(&fused_kernel<T, 4, MFMA, PIPE>);
    case 8: return reinterpret_cast<const void*>(&fused_kernel<T, 8, MFMA, PIPE>);
    default: return nullptr;
  }
}

template <typename T>
static const void* fused_pick(int nck, bool mfma, bool pipe) {
  if (mfma) return pipe ? fused_fn<T, true, true>(nck) : fused_fn<T, true, false>(nck);
  return pipe ? fused_fn<T, false, true>(nck) : fused_fn<T, false, false>(nck);
}

template <typename T>
static hipError_t launch_delta_t(const DeltaLaunch& L, int stages, hipStream_t stream,
                                 hipEvent_t start, hipEvent_t stop) {
  const int nck = chunks_per_thread<T>(L.h_in);
  if (stages & STAGE_FUSED) {
    const int blocks = L.n_tiles * L.n_slots;
    if (blocks == 0) return hipSuccess;
    const void* k = fused_pick<T>(nck, sizeof(T) == 2 && L.has_mfma, L.pipe_expand != 0);
    if (!k) return hipErrorInvalidValue;
    return launch_one(k, blocks, L, stream, start, stop);
  }
  // Staged: shrink, combine (K-split MFMA blocks), expand; the events bracket
  // whichever launches run.
  const bool sh = (stages & STAGE_SHRINK) && L.n_shrink > 0;
  const bool co = (stages & STAGE_SHRINK) && L.n_combine > 0;
  const bool ex = (stages & STAGE_EXPAND) && L.n_expand > 0;
  if (sh) {
    const void* k = shrink_fn<T>(nck);
    if (!k) return hipErrorInvalidValue;
    hipError_t e = launch_one(k, L.n_shrink, L, stream, start, (co || ex) ? nullptr : stop);
    if (e != hipSuccess) return e;
  }
  if (co) {
    hipError_t e = launch_one(reinterpret_cast<const void*>(&combine_kernel), L.n_combine, L, stream,
                              sh ? nullptr : start, ex ? nullptr : stop);
    if (e != hipSuccess) return e;
  }
  if (ex) {
    const void* k = L.pipe_expand ? reinterpret_cast<const void*>(&expand_kernel<T, true>)
                                  : reinterpret_cast<const void*>(&expand_kernel<T, false>);
    return launch_one(k, L.n_expand, L, stream, (sh || co) ? nullptr : start, stop);
  }
  return hipSuccess;
}

hipError_t launch_delta(const DeltaLaunch& L, int stages, hipStream_t stream, hipEvent_t start,
                        hipEvent_t stop) {
  return L.dtype == 1 ? launch_delta_t<_Float16>(L, stages, stream, start, stop)
                      : launch_delta_t<float>(L, stages, stream, start, stop);
}

__global__ __launch_bounds__(kThreads) void zero_words_kernel(uint32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads)
    p[i] = 0u;
}

hipError_t launch_zero_words(void* p, int64_t n_words, hipStream_t stream) {
  if (n_words <= 0) return hipSuccess;
  int64_t blocks = (n_words + kThreads - 1) / kThreads;
  if (blocks > 1024) blocks = 1024;
  zero_words_kernel<<<dim3((unsigned)blocks), dim3(kThreads), 0, stream>>>(static_cast<uint32_t*>(p), n_words);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Adapter fetch, second half: the images are already in device staging (one
// copy-engine transfer each); one workgroup per row moves the row into its
// page.  Row sizes are multiples of 16 bytes (h_in and h_out are multiples of
// 8 elements).

__global__ __launch_bounds__(kThreads) void scatter_pages_kernel(ScatterLaunch S) {
  const int32_t g = blockIdx.x;
  int lo = 0, hi = S.n - 1;          // adapter i with row_start[i] <= g < row_start[i + 1]
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (S.row_start[mid] <= g) lo = mid; else hi = mid - 1;
  }
  const int64_t q = g - S.row_start[lo];
  const int64_t n_a = (int64_t)S.n_proj * S.rank[lo];
  const char* img = S.stage + S.img_off[lo];
  const int32_t* ids = reinterpret_cast<const int32_t*>(img + n_a * (S.a_row_bytes + S.b_row_bytes));
  const bool is_a = q < n_a;
  const int64_t n16 = (is_a ? S.a_row_bytes : S.b_row_bytes) / 16;
  const uint4* src = reinterpret_cast<const uint4*>(
      img + (is_a ? q * S.a_row_bytes : n_a * S.a_row_bytes + (q - n_a) * S.b_row_bytes));
  uint4* dst = reinterpret_cast<uint4*>(is_a ? S.a_base + (int64_t)ids[q] * S.a_page_bytes
                                             : S.b_base + (int64_t)ids[q] * S.b_page_bytes);
  for (int64_t i = threadIdx.x; i < n16; i += kThreads) dst[i] = src[i];
}

hipError_t launch_scatter_pages(const ScatterLaunch& S, hipStream_t stream) {
  if (S.n <= 0 || S.row_start[S.n] <= 0) return hipSuccess;
  scatter_pages_kernel<<<dim3((unsigned)S.row_start[S.n]), dim3(kThreads), 0, stream>>>(S);
  return hipGetLastError();
}


}  // namespace slora
