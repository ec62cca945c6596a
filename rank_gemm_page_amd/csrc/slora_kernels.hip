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
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "slora_internal.h"

namespace slora {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));

template <typename T> struct VecN;
template <> struct VecN<_Float16> { static constexpr int N = 8; };
template <> struct VecN<float> { static constexpr int N = 4; };

__device__ __forceinline__ uint4 ld16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}
__device__ __forceinline__ void st16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

// Streaming (non-temporal) 16-byte load and store, for data read once per
// launch or nearly so: page rows of the vector-ALU tiles and y.  Measured on
// MI355X, row gathers of 60-240 MB stream 1.5-1.7x faster with the
// non-temporal hint than with ordinary loads.  The x rows of the MFMA shrink
// (read by every rank block of the token block, and across XCDs) and the B
// slices of the MFMA expand (read by every token block of the segment) keep
// ordinary loads: with the hint, the re-reads miss and the launch is slower.
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
#define SLORA_NT_X 0
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


// Values every lane of a wavefront holds alike (tile header fields, the wave
// index) are moved to scalar registers.  Control flow on them then branches
// instead of masking lanes, which matters for MFMA: a matrix instruction runs
// on the whole wavefront whatever the EXEC mask says, so it must never sit
// behind a lane mask to be skipped.
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Workgroup barrier that orders LDS accesses only.  __syncthreads() also
// orders global memory, which makes every wave wait for all of its global
// loads still in flight (prefetches included) before the barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
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
// Progress: shrink tiles occupy the lower block indices and never wait, and
// workgroups are dispatched in index order, so every shrink tile a waiting
// expand tile depends on has been dispatched and finishes.  The wait is
// bounded all the same: past kMaxSpins polls it raises error_flag and goes on,
// so every wave of the grid always exits.
constexpr uint32_t kMaxSpins = 1u << 20;

template <bool FUSED>
__device__ __forceinline__ void store_v(const DeltaLaunch& L, int64_t idx, float x) {
  if constexpr (FUSED) {
    const unsigned long long pair = ((unsigned long long)L.epoch << 32) | __float_as_uint(x);
    __hip_atomic_store(L.vtag + idx, pair, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    L.v[idx] = x;
  }
}

// Loads v[idx] of every (valid) slot this thread owns, polling until all
// threads of the workgroup hold current values.  get(q) gives slot q's index
// (or -1), put(q, value) receives the value; the first nq (uniform, <= N)
// slots of each thread are in use.  All loads of a poll are issued before
// any is consumed, at index `safe` (any valid v index) for a slot with no
// value, so they travel to memory together instead of one round trip each.
template <bool FUSED, int N, typename Get, typename Put>
__device__ __forceinline__ void load_v(const DeltaLaunch& L, int nq, int safe, Get get, Put put) {
  int idx[N];
#pragma unroll
  for (int q = 0; q < N; ++q) idx[q] = q < nq ? get(q) : -1;
  if constexpr (!FUSED) {
    float val[N];
#pragma unroll
    for (int q = 0; q < N; ++q)
      if (q < nq) val[q] = L.v[idx[q] >= 0 ? idx[q] : safe];
#pragma unroll
    for (int q = 0; q < N; ++q)
      if (q < nq) put(q, idx[q] >= 0 ? val[q] : 0.f);
  } else {
    for (uint32_t spins = 0;; ++spins) {
      unsigned long long pair[N];
#pragma unroll
      for (int q = 0; q < N; ++q)
        if (q < nq)
          pair[q] = __hip_atomic_load(L.vtag + (idx[q] >= 0 ? idx[q] : safe), __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
      bool ok = true;
#pragma unroll
      for (int q = 0; q < N; ++q) {
        if (q < nq) {
          ok = ok && (idx[q] < 0 || (uint32_t)(pair[q] >> 32) == L.epoch);
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
// Shrink, vector-ALU tile: up to kGemvMaxTok tokens x RB rank rows, whole h_in.
// Thread tid owns the 16-byte chunks tid, tid+256, ... of every row; the A^T
// rows stay in registers while each token's x chunks are dotted against them.

template <typename T, int NCK, bool FUSED>
__device__ void shrink_gemv_tile(const DeltaLaunch& L, const int32_t* srec, float* red) {
  constexpr int VEC = VecN<T>::N;
  constexpr int RB = kShrinkRowBudget / NCK;
  constexpr int TB = kGemvMaxTok;
  const int ntok = uni(srec[REC_NTOK]);
  const int rank = uni(srec[REC_RANK]);
  const int j0 = uni(srec[REC_POS]);
  const int nrows = uni(srec[REC_LEN]);
  const int v0 = uni(srec[REC_V0]);
  const int32_t* toks = srec + REC_HDR;
  const int32_t* pages = srec + REC_HDR + L.tokcap;
  const int tid = threadIdx.x, lane = tid & 63, wave = uni(tid >> 6);
  const int nchunks = L.h_in / VEC;
  const T* x = reinterpret_cast<const T*>(L.x);

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
    store_v<FUSED>(L, v0 + (int64_t)k * rank + j0 + r, sum);
  }
}

// ---------------------------------------------------------------------------
// Shrink, MFMA tile: 16 tokens x up to 64 rank rows, whole h_in (fp16).
// C[m][n] = sum_k X[m][k] * AT_n[k] with v_mfma_f32_16x16x32_f16: lane l feeds
// row m = l%16 of X and row n = l%16 of A^T, 8 consecutive k at 8*(l/16); the
// four waves take interleaved 32-wide k steps and are summed through LDS.

#ifndef SLORA_SHRINK_RING
#define SLORA_SHRINK_RING 16
#endif
// Register ring of the MFMA shrink, in 16-byte loads per lane (D stages of
// 1 + NB loads each).
constexpr int kShrinkRingHalf8 = SLORA_SHRINK_RING;

template <int NB, bool FUSED>
__device__ void shrink_mfma_tile(const DeltaLaunch& L, const int32_t* srec, float* red) {
  const int ntok = uni(srec[REC_NTOK]);
  const int rank = uni(srec[REC_RANK]);
  const int j0 = uni(srec[REC_POS]);
  const int nrows = uni(srec[REC_LEN]);
  const int v0 = uni(srec[REC_V0]);
  const int32_t* toks = srec + REC_HDR;
  const int32_t* pages = srec + REC_HDR + L.tokcap;
  const int tid = threadIdx.x, lane = tid & 63, wave = uni(tid >> 6);
  const int m = lane & 15, g = lane >> 4;

  // Rows past ntok / nrows repeat the last valid row (same cache lines); their
  // outputs are never stored.
  const _Float16* xrow = reinterpret_cast<const _Float16*>(L.x) +
                         (int64_t)toks[m < ntok ? m : ntok - 1] * L.h_in + 8 * g;
  const _Float16* arow[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int j = b * 16 + m;
    arow[b] = reinterpret_cast<const _Float16*>(
                  L.pool.base_a + (int64_t)pages[j < nrows ? j : nrows - 1] * L.pool.page_bytes_a) + 8 * g;
  }
  float4v acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = float4v{0.f, 0.f, 0.f, 0.f};

  // Wave w takes the 32-wide k steps w, w+4, w+8, ...: n_it of them.  Loads
  // run D steps ahead of the matrix cores in a ring of registers.  Every load
  // is issued unconditionally (a step past the end re-reads the wave's last
  // step and is never multiplied), so the same number of loads is in flight
  // on every path and the wait before a step covers that step's loads only;
  // a load behind a branch would make the compiler wait for all of them.
  const int n_it = (L.h_in - wave * 32 + 127) >> 7;
  const int last = n_it > 0 ? n_it - 1 : 0;
  const int kbase = n_it > 0 ? wave * 32 : 0;   // a wave with no step re-reads k = 0
  constexpr int D = kShrinkRingHalf8 / (1 + NB) < 2 ? 2 : kShrinkRingHalf8 / (1 + NB);
  half8 xs[D], as[D][NB];
  auto load = [&](int slot, int it) {
    const int k = kbase + (it < last ? it : last) * 128;
    xs[slot] = __builtin_bit_cast(half8, ldsel<SLORA_NT_X>(xrow + k));
#pragma unroll
    for (int b = 0; b < NB; ++b) as[slot][b] = __builtin_bit_cast(half8, ld16(arow[b] + k));
  };
  // The ring is filled in slot order and kept in that order (no reordering
  // across the barriers): the wait before slot s then only needs the loads
  // older than slot s + 1's.
#pragma unroll
  for (int slot = 0; slot < D; ++slot) {
    load(slot, slot);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int it0 = 0; it0 < n_it; it0 += D) {
#pragma unroll
    for (int slot = 0; slot < D; ++slot) {
      if (it0 + slot < n_it) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
          acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xs[slot], as[slot][b], acc[b], 0, 0, 0);
      }
      load(slot, it0 + slot + D);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // acc[b][i] is C[token 4g + i][rank row b*16 + l%16]; sum the four waves in LDS.
#pragma unroll
  for (int b = 0; b < NB; ++b) {
#pragma unroll
    for (int i = 0; i < 4; ++i) red[((wave * 4 + b) * 16 + (4 * g + i)) * 16 + m] = acc[b][i];
  }
  __syncthreads();
  for (int i = tid; i < ntok * nrows; i += kThreads) {
    const int mm = i / nrows, j = i - mm * nrows;
    const int b = j >> 4, n = j & 15;
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) sum += red[((w * 4 + b) * 16 + mm) * 16 + n];
    store_v<FUSED>(L, v0 + (int64_t)mm * rank + j0 + j, sum);
  }
}

template <bool FUSED>
__device__ __forceinline__ void shrink_mfma_dispatch(const DeltaLaunch& L, const int32_t* srec, float* red) {
  switch ((uni(srec[REC_LEN]) + 15) >> 4) {
    case 1: shrink_mfma_tile<1, FUSED>(L, srec, red); break;
    case 2: shrink_mfma_tile<2, FUSED>(L, srec, red); break;
    case 3: shrink_mfma_tile<3, FUSED>(L, srec, red); break;
    default: shrink_mfma_tile<4, FUSED>(L, srec, red); break;
  }
}

template <typename T, int NCK>
__global__ __launch_bounds__(kThreads) void shrink_kernel(DeltaLaunch L) {
  __shared__ float red[4 * 4 * 16 * 16];  // MFMA: 4 waves x 4 blocks x 16 x 16
  __shared__ int32_t srec[kMaxRecWords];
  const int32_t* rec = L.rec + (int64_t)L.shrink_idx[blockIdx.x] * L.stride;
  record_to_lds(rec, L.tokcap, L.pagecap, L.proj, srec);
  if constexpr (sizeof(T) == 2) {
    if (uni(srec[REC_KIND]) & KIND_MFMA_BIT) {
      shrink_mfma_dispatch<false>(L, srec, red);
      return;
    }
  }
  shrink_gemv_tile<T, NCK, false>(L, srec, red);
}

// ---------------------------------------------------------------------------
// Expand, vector-ALU tile: up to kGemvMaxTok tokens x `width` columns, all r
// rows.  width/VEC threads cover the columns with one 16-byte chunk each and
// G = 256 / (width/VEC) groups of them split the r rows; the groups' partial
// sums meet in LDS and group 0 applies y += s * d with one rounding.

template <typename T, bool FUSED>
__device__ void expand_gemv_tile(const DeltaLaunch& L, const int32_t* srec, float* lds) {
  constexpr int VEC = VecN<T>::N;
  constexpr int TB = kGemvMaxTok;
  constexpr int RCH = 8;  // B rows per thread issued together
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
  T* y = reinterpret_cast<T*>(L.y);

  // Issue everything the tile reads before waiting on any of it: the first
  // RCH B rows of this thread, (group 0) the y chunks of the epilogue, and v
  // (in a fused launch, once the segment's shrink tiles are done).
  const bool active = ct * VEC < ncol;
  const int nrt = (active && g < rank) ? (rank - g + G - 1) / G : 0;   // rows of this thread
  const int64_t col_byte = (int64_t)(o0 + ct * VEC) * sizeof(T);
  uint4 bq[RCH];
#pragma unroll
  for (int i = 0; i < RCH; ++i)
    bq[i] = i < nrt ? ldsel<SLORA_NT_B>(L.pool.base_b + (int64_t)pages[g + i * G] * L.pool.page_bytes_b + col_byte)
                    : make_uint4(0, 0, 0, 0);
  uint4 yv[TB];
#pragma unroll
  for (int k = 0; k < TB; ++k)
    yv[k] = (g == 0 && active && k < ntok) ? ldsel<SLORA_NT_Y>(y + (int64_t)toks[k] * L.h_out + o0 + ct * VEC)
                                           : make_uint4(0, 0, 0, 0);
  load_v<FUSED, TB>(
      L, (ntok * rank + kThreads - 1) / kThreads, v0,
      [&](int q) -> int { const int i = tid + q * kThreads; return i < ntok * rank ? v0 + i : -1; },
      [&](int q, float val) { const int i = tid + q * kThreads; if (i < ntok * rank) sv[i] = val; });
  __syncthreads();

  float acc[TB][VEC];
#pragma unroll
  for (int k = 0; k < TB; ++k)
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[k][e] = 0.f;
  for (int i0 = 0; i0 < nrt; i0 += RCH) {
    if (i0 > 0) {
#pragma unroll
      for (int i = 0; i < RCH; ++i)
        bq[i] = i0 + i < nrt ? ldsel<SLORA_NT_B>(L.pool.base_b + (int64_t)pages[g + (i0 + i) * G] * L.pool.page_bytes_b + col_byte)
                             : make_uint4(0, 0, 0, 0);
    }
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

constexpr int kSliceRowDw = kMfmaPass / 2;      // dwords per 128-column row
constexpr int kSliceDw = 32 * kSliceRowDw;      // one staged 32-row slice (8 KB)
constexpr int kEpiPitch = kMfmaPass + 4;        // floats per epilogue row
constexpr int kMfmaExpandLds = 2 * kSliceDw + kMfmaExpandTok * kEpiPitch + kMfmaExpandTok;

// Dword offset of column quad q (4 columns) of row r of a staged slice.  The
// quads are XOR-swizzled by row so that the 8 rows the two lane groups of a
// half-wave read together (8g + t, t = 0..3) land in distinct banks.
__device__ __forceinline__ int quad_dw(int r, int q) {
  return r * kSliceRowDw + 2 * (q ^ (4 * ((r & 3) + 4 * ((r >> 3) & 1))));
}

typedef short short4v __attribute__((ext_vector_type(4)));
constexpr int kBufferFormat = 0x00020000;   // descriptor word 3: raw 32-bit buffer

template <bool FUSED, int KS>
__device__ void expand_mfma_tile(const DeltaLaunch& L, const int32_t* srec, float* lds) {
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
  const int ks_n = (rank + 31) >> 5;                   // <= KS
  const int n_pass = (ncol + kMfmaPass - 1) / kMfmaPass;
  const int n_steps = n_pass * ks_n;                   // (pass, k slice), pass-major
  uint32_t* slice = reinterpret_cast<uint32_t*>(lds);  // two slices, used in turn
  float* epi = lds + 2 * kSliceDw;                     // [64][kEpiPitch]
  float* up_tok = epi + kMfmaExpandTok * kEpiPitch;    // per-token scale back
  _Float16* yb = reinterpret_cast<_Float16*>(L.y);
  const __amdgpu_buffer_rsrc_t yrsrc = __builtin_amdgcn_make_buffer_rsrc(L.y, 0, (int)L.y_bytes, kBufferFormat);

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

  uint4 bnext[2];
  stage_load(0, bnext);
  uint4 y0[4], y1[4];
  load_y(0, y0);

  // s*v of this lane's token (16 wave + m) at rows 32ks + 8g + i, zero past
  // ntok / rank.
  const int tok = 16 * wave + m;
  float sv[8 * KS];
  load_v<FUSED, 8 * KS>(
      L, 8 * ks_n, v0,
      [&](int q) -> int {
        const int j = 32 * (q >> 3) + 8 * g + (q & 7);
        return (tok < ntok && j < rank) ? v0 + tok * rank + j : -1;
      },
      [&](int q, float val) { sv[q] = scale * val; });
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
  // two register sets swap roles from pass to pass.  Slices alternate between
  // two LDS buffers, so one barrier per slice suffices: a buffer is written
  // again only after every wave has passed the barrier of the slice that
  // followed its last read.
  auto pass_body = [&](int pass, uint4 (&yc)[4], uint4 (&yn)[4]) {
    float4v acc[kMfmaPass / 16];
#pragma unroll
    for (int c = 0; c < kMfmaPass / 16; ++c) acc[c] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks >= ks_n) break;
      const int step = pass * ks_n + ks;
      uint32_t* buf = slice + (step & 1) * kSliceDw;
      stage_store(buf, bnext);
      lds_barrier();
      stage_load(step + 1, bnext);
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
      // which the hardware drops: no branch, no traffic.
      const uint32_t off = (row < ntok && col < ncol) ? 2u * ((uint32_t)toks[row] * L.h_out + o0 + col) : 0xFFFFFFF0u;
      __builtin_amdgcn_raw_buffer_store_b128(u32x4{out.x, out.y, out.z, out.w}, yrsrc, off, 0, SLORA_NT_Y ? 2 : 0);
    }
  };
  for (int pass = 0;; pass += 2) {
    pass_body(pass, y0, y1);
    if (pass + 1 >= n_pass) break;
    pass_body(pass + 1, y1, y0);
    if (pass + 2 >= n_pass) break;
  }
}

template <bool FUSED>
__device__ __forceinline__ void expand_mfma_dispatch(const DeltaLaunch& L, const int32_t* srec, float* lds) {
  expand_mfma_tile<FUSED, kMaxRankMfma / 32>(L, srec, lds);
}

// LDS of the expand tiles: the vector-ALU tiles need kGemvLdsFloats, the
// MFMA tiles kMfmaExpandLds.  Kernels that never run an MFMA tile allocate
// the smaller size, which keeps four of them resident per CU.
constexpr int kGemvLdsFloats = kGemvMaxTok * 256 + 7 * kGemvMaxTok * 256;
constexpr int kExpandLdsFloats = kMfmaExpandLds > kGemvLdsFloats ? kMfmaExpandLds : kGemvLdsFloats;

template <typename T>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3))) void expand_kernel(DeltaLaunch L) {
  __shared__ float lds[sizeof(T) == 2 ? kExpandLdsFloats : kGemvLdsFloats];
  __shared__ int32_t srec[kMaxRecWords];
  const int32_t* rec = L.rec + (int64_t)L.expand_idx[blockIdx.x] * L.stride;
  record_to_lds(rec, L.tokcap, L.pagecap, L.proj, srec);
  if constexpr (sizeof(T) == 2) {
    if (uni(srec[REC_KIND]) & KIND_MFMA_BIT) {
      expand_mfma_dispatch<false>(L, srec, lds);
      return;
    }
  }
  expand_gemv_tile<T, false>(L, srec, lds);
}

// Both stages in one launch over the records in launch order: shrink tiles
// and expand tiles that wait for their tokens' v (see store_v / load_v).
// MFMA=false leaves the matrix-core tiles out (a batch without them), which
// keeps the register budget, and so the workgroups resident per CU, of the
// vector-ALU tiles alone.
// Three workgroups per CU fit the matrix-core tiles' registers without
// spilling (fewer would leave slots empty); the widest vector-ALU shrink
// (h_in above 8192) needs more registers and runs two.
template <typename T, int NCK, bool MFMA>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(NCK == 8 ? 2 : 3)))
void fused_kernel(DeltaLaunch L) {
  __shared__ float lds[sizeof(T) == 2 && MFMA ? kExpandLdsFloats : kGemvLdsFloats];
  __shared__ int32_t srec[kMaxRecWords];
  record_to_lds(L.rec + (int64_t)blockIdx.x * L.stride, L.tokcap, L.pagecap, L.proj, srec);
  const int kind = uni(srec[REC_KIND]);
  if (!(kind & KIND_EXPAND_BIT)) {
    if constexpr (sizeof(T) == 2 && MFMA) {
      if (kind & KIND_MFMA_BIT) {
        shrink_mfma_dispatch<true>(L, srec, lds);
        return;
      }
    }
    shrink_gemv_tile<T, NCK, true>(L, srec, lds);
    return;
  }
  if constexpr (sizeof(T) == 2 && MFMA) {
    if (kind & KIND_MFMA_BIT) {
      expand_mfma_dispatch<true>(L, srec, lds);
      return;
    }
  }
  expand_gemv_tile<T, true>(L, srec, lds);
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

template <typename T, bool MFMA>
static const void* fused_fn(int nck) {
  switch (nck) {
    case 1: return reinterpret_cast<const void*>(&fused_kernel<T, 1, MFMA>);
    case 2: return reinterpret_cast<const void*>(&fused_kernel<T, 2, MFMA>);
    case 4: return reinterpret_cast<const void*>(&fused_kernel<T, 4, MFMA>);
    case 8: return reinterpret_cast<const void*>(&fused_kernel<T, 8, MFMA>);
    default: return nullptr;
  }
}

template <typename T>
static hipError_t launch_delta_t(const DeltaLaunch& L, int stages, hipStream_t stream,
                                 hipEvent_t start, hipEvent_t stop) {
  const int nck = chunks_per_thread<T>(L.h_in);
  if (stages & STAGE_FUSED) {
    const int blocks = L.n_tiles;
    if (blocks == 0) return hipSuccess;
    const void* k = (sizeof(T) == 2 && L.has_mfma) ? fused_fn<T, true>(nck) : fused_fn<T, false>(nck);
    if (!k) return hipErrorInvalidValue;
    return launch_one(k, blocks, L, stream, start, stop);
  }
  const bool sh = (stages & STAGE_SHRINK) && L.n_shrink > 0;
  const bool ex = (stages & STAGE_EXPAND) && L.n_expand > 0;
  if (sh) {
    const void* k = shrink_fn<T>(nck);
    if (!k) return hipErrorInvalidValue;
    hipError_t e = launch_one(k, L.n_shrink, L, stream, start, ex ? nullptr : stop);
    if (e != hipSuccess) return e;
  }
  if (ex) {
    const void* k = reinterpret_cast<const void*>(&expand_kernel<T>);
    return launch_one(k, L.n_expand, L, stream, sh ? nullptr : start, stop);
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
// Adapter load: copy packed staging rows into their pages (one block per row).

__global__ __launch_bounds__(kThreads) void scatter_rows_kernel(const char* src, int64_t row_bytes,
                                                                const int32_t* page_ids, char* base,
                                                                int64_t page_bytes) {
  const int64_t row = blockIdx.x;
  const uint4* s = reinterpret_cast<const uint4*>(src + row * row_bytes);
  uint4* d = reinterpret_cast<uint4*>(base + (int64_t)page_ids[row] * page_bytes);
  const int64_t n = row_bytes / 16;
  for (int64_t i = threadIdx.x; i < n; i += kThreads) d[i] = s[i];
}

hipError_t launch_scatter_rows(const char* src, int32_t n_rows, int64_t row_bytes,
                               const int32_t* page_ids, char* base, int64_t page_bytes,
                               hipStream_t stream) {
  if (n_rows <= 0) return hipSuccess;
  scatter_rows_kernel<<<dim3(n_rows), dim3(kThreads), 0, stream>>>(src, row_bytes, page_ids, base,
                                                                  page_bytes);
  return hipGetLastError();
}

}  // namespace slora
