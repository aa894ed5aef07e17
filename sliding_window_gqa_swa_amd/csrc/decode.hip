// decode.hip -- one query token per sequence against its compact ring cache.
//
// Pages cited (title; section):
//   [SPYRE]  "Enable compact sliding-window attention for Gemma 3 and Gemma 4
//            variants" (torch-spyre/hf-adapters pull request 496)
//   [BONSAI] "Gemma3 Local Attention Cache" (jax-ml/bonsai issue 124)
//
// [SPYRE] Compilation behavior / Performance: decode scans only the compact
// (window + slack)-row allocation and every position-dependent value is
// tensor data, so one launch shape serves every step.  [BONSAI] Step 3: the
// window mask is made to follow the modulo wrap.  Here the mask of physical
// row r is computed in the kernel from ring_meta:
//   a = anchor + ((r - start) mod R);  read iff max(lo, pos-W+1, 0) <= a <= pos.
// Rows that fail it are never loaded, so HBM traffic is the valid rows only.
//
// Work split (HBM-bound, arithmetic intensity ~ g flop/byte):
//   block = (split s of the R rows, kv head [, head block], sequence b).
//   One pass: a row is spread over LPR lanes that each own 16 bytes; every
//   lane keeps U rows of K and V in flight (buffer loads: masked rows use an
//   out-of-range offset, so they return zeros and move no bytes), forms the
//   query dot products with a lane-group butterfly and folds the rows into a
//   running (max, sum, weighted V) state, online-softmax style.  The states
//   of the row groups and waves are merged in a fixed order.  A ring of at
//   most 2048 rows on a grid of about one block per CU or more is one split:
//   the block writes the output itself.  Otherwise partials (m, l, o) go to
//   the workspace; the last split block of each sequence and head block (a
//   device-scope counter in the workspace) combines the splits in a fixed
//   order (deterministic), so one launch does the whole decode.
//
// Decode step (STEP = true): the same kernel also performs the per-token
// cache work of the sequence first, so one launch serves a whole decode
// step.  Every block derives the same new state from ring_meta: position
// p = pos + 1; if the ring is full (p - anchor >= R) it is rolled by
// metadata alone (anchor += A, start += A mod R, A = R - W: each position
// keeps its physical row, the A oldest rows become free); the token is
// appended at slot(p) unless the ring is still full (then nothing is
// written and the sticky flag is set, as for swa_cache_append).  Blocks
// whose rows include slot(p) use that row from k_new / v_new, never the
// ring's copy, and exactly one of them writes it to the ring after its row
// loop.  The last block of a sequence (a second device-scope counter)
// stores the new ring_meta after every block of the sequence has read the
// old one.
//
// Small grids (at most about one block per CU: a single sequence, or a few)
// are bound by the chain of memory latencies, not by bandwidth.  There the
// kernel (LA = true) requests every row of its split before ring_meta has
// arrived and applies the mask to the loaded rows, so the ring_meta load
// and the first row loads are in flight together (the masked rows' bytes,
// at most the 64 slack rows of a ring, are read for nothing; a decode
// step's appended row is loaded and replaced by the step's input).
#include <type_traits>

#include "swa_common.h"
#include "swa_internal.h"

namespace swa {
namespace {

// Threads per block: 8 waves on streaming grids, where one block per CU
// (a 64-sequence batch takes one block per ring) keeps 16 rows per wave step
// in flight (48.6 us for the 64-sequence D = 256 decode against 51.4 us
// with two 4-wave blocks of 544 rows and a combine per ring); 4 waves on
// small grids, whose 64-row splits give each wave 16 rows (8.5 against 8.7
// us average launch for one sequence in a kernel trace).
constexpr int dec_threads(bool load_all) { return load_all ? 256 : 512; }
// bounds the work of one block: a ring of up to 2048 rows is one split on
// grids of at least one block per CU (no partials, no combine: the block
// writes the output itself)
constexpr int kMaxRowsPerSplit = 2048;
constexpr int kTargetBlocks = 256;  // about one block per CU before the row cap adds more
constexpr int kMaxSplits = 256;      // (m, l) of every split fit the combine's LDS
constexpr int kLoadAllRows = 64;     // minimum rows per split of a small grid
constexpr int kLoadAllMaxRows = 256; // larger splits stream: the row mask saves their bytes
constexpr float kLog2e = 1.4426950408889634f;
// Cache policy of the streamed ring-row loads: non-temporal (nt).  Every
// row of a large grid is read once, so nothing is gained by keeping it in
// L2; the streaming loads give 42.8-43.6 us for the 64-sequence D = 256
// decode against 48.7 us with the default policy (measured).  Small grids
// keep the default: their decode step took 0.4 us longer with nt.
constexpr int kStreamPolicy = 2;

// 16-byte chunk of a row as fp32.
template <typename T>
__device__ __forceinline__ void load_chunk(const T* p, float* f);
template <>
__device__ __forceinline__ void load_chunk<__bf16>(const __bf16* p, float* f) {
  unpack8(*reinterpret_cast<const u32x4*>(p), f);
}
template <>
__device__ __forceinline__ void load_chunk<float>(const float* p, float* f) {
  const floatx4 x = *reinterpret_cast<const floatx4*>(p);
  f[0] = x[0];
  f[1] = x[1];
  f[2] = x[2];
  f[3] = x[3];
}

// 16 raw bytes of a row as fp32.
template <typename T>
__device__ __forceinline__ void unpack_chunk(const u32x4 w, float* f);
template <>
__device__ __forceinline__ void unpack_chunk<__bf16>(const u32x4 w, float* f) {
  unpack8(w, f);
}
template <>
__device__ __forceinline__ void unpack_chunk<float>(const u32x4 w, float* f) {
  f[0] = __uint_as_float(w[0]);
  f[1] = __uint_as_float(w[1]);
  f[2] = __uint_as_float(w[2]);
  f[3] = __uint_as_float(w[3]);
}

// Device-coherent (agent-scope, relaxed) 4-byte store / load.
__device__ __forceinline__ void st_agent(float* p, float x) {
  __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

constexpr int pow2_at_least(int x) { return x <= 1 ? 1 : 2 * pow2_at_least((x + 1) / 2); }

// A row of CH 16-byte chunks is spread over LPR lanes (the power of two at
// or above CH, at most 64); with CH not a power of two (head size 320:
// 40 chunks of bf16, 80 of fp32) the lanes past the last chunk load
// nothing and add zeros to the lane-group sums.
template <int D, typename T, int NWV>
struct DecGeom {
  static constexpr int VEC = 16 / (int)sizeof(T);  // elements per 16 bytes
  static constexpr int CH = D / VEC;                // chunks per row
  static constexpr int LPR = pow2_at_least(CH) < kWave ? pow2_at_least(CH) : kWave;  // lanes per row
  static constexpr int CPL = (CH + LPR - 1) / LPR;  // chunks per lane per row
  static constexpr int RPW = kWave / LPR;           // rows per wave step
  static constexpr int RPI = RPW * NWV;       // rows per block step
  static constexpr int ELT = CPL * VEC;             // elements per lane
  static constexpr bool FULL = CH % LPR == 0;       // every lane's chunks exist
  static_assert(D % VEC == 0, "whole 16-byte chunks per row");
};

template <int D, typename T, int GB, bool STEP, bool LA>
__global__ __launch_bounds__(dec_threads(LA)) void decode_split_kernel(
    const T* __restrict__ q, T* __restrict__ k_ring, T* __restrict__ v_ring,
    int32_t* __restrict__ meta, int W, int R, int hq, int hkv, int head_blocks,
    int rows_per_split, float qk_scale_log2, float* ws_o, float* ws_ml, int splits,
    uint32_t* counters, T* __restrict__ out, const T* __restrict__ k_new,
    const T* __restrict__ v_new) {
  constexpr int NT = dec_threads(LA);  // threads per block
  constexpr int NWV = NT / kWave;      // waves per block
  using G = DecGeom<D, T, NWV>;
  __shared__ float red_o[NWV][GB][D];
  __shared__ float red_m[NWV][GB], red_l[NWV][GB];

  const int s = blockIdx.x;
  const int kvh = blockIdx.y / head_blocks;
  const int hb = blockIdx.y - kvh * head_blocks;
  const int b = blockIdx.z;
  const int g = hq / hkv;
  const int h0 = kvh * g + hb * GB;
  const int nh = min(GB, g - hb * GB);
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int rg = lane / G::LPR;       // row within the wave step
  const int li = lane - rg * G::LPR;  // lane within the row

  const int r0 = s * rows_per_split;
  const int r1 = min(R, r0 + rows_per_split);

  // ring state; the physical -> position map needs no division per row:
  // j = r - start (+R if negative), a = anchor + j
  const int32_t* m = meta + 4 * (size_t)b;
  int64_t pos = m[0], anchor = m[1];
  int start = (int)pos_mod(m[2], R);
  const int32_t lo_raw = m[3];
  const int64_t lo = lo_raw & 0x7fffffff;
  // decode step: metadata roll, then the append slot (-1: refused)
  int slot_p = -1;
  if constexpr (STEP) {
    const int64_t p = pos + 1;
    const int A = R - W;  // > 0 (checked on the host)
    if (p - anchor >= R) {
      anchor += A;
      start = (int)pos_mod((int64_t)start + A, R);
    }
    if (p - anchor < R && p >= anchor) {
      slot_p = (int)pos_mod((int64_t)start + (p - anchor), R);
      pos = p;
    }
  }
  int64_t low = max(lo, (int64_t)0);
  if (W > 0) low = max(low, pos - W + 1);
  const int64_t high = pos;

  // query chunks of every head of this block: bf16 queries stay packed (the
  // scores are bf16 pair dot products, scaled into the log2 domain after
  // the sum); fp32 queries are pre-scaled
  constexpr bool kBf = !std::is_same<T, float>::value;
  float qv[GB][kBf ? 1 : G::ELT];
  u32x4 qw[GB][kBf ? G::CPL : 1];
  auto load_q = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < GB; ++j) {
      const int h = h0 + min(j, nh - 1);
#pragma unroll
      for (int c = 0; c < G::CPL; ++c) {
        const bool have = G::FULL || li + c * G::LPR < G::CH;
        const T* src = q + ((size_t)b * hq + h) * D + (size_t)(li + c * G::LPR) * G::VEC;
        if constexpr (kBf) {
          qw[j][c] = have ? *reinterpret_cast<const u32x4*>(src) : u32x4{0u, 0u, 0u, 0u};
        } else {
          float f[G::VEC];
          if (have) {
            load_chunk<T>(src, f);
          } else {
#pragma unroll
            for (int e = 0; e < G::VEC; ++e) f[e] = 0.f;
          }
#pragma unroll
          for (int e = 0; e < G::VEC; ++e) qv[j][c * G::VEC + e] = f[e] * qk_scale_log2;
        }
      }
    }
  };

  // one buffer descriptor per ring: masked rows load from an out-of-range
  // offset, which returns zeros without touching memory
  const size_t ring_off = ((size_t)b * hkv + kvh) * (size_t)R * D;
  const uint32_t ring_bytes = (uint32_t)((size_t)R * D * sizeof(T));
  const i32x4 krs = make_buffer_rsrc(k_ring + ring_off, ring_bytes);
  const i32x4 vrs = make_buffer_rsrc(v_ring + ring_off, ring_bytes);
  const size_t new_off = ((size_t)b * hkv + kvh) * D;  // row of k_new / v_new
  // LA decode step: this lane's chunks of the appended row, requested with
  // the first row loads (they replace the ring's copy of the row in consume)
  u32x4 kn_c[G::CPL], vn_c[G::CPL];
  if constexpr (STEP && LA) {
#pragma unroll
    for (int c = 0; c < G::CPL; ++c) {
      const size_t e0 = new_off + (size_t)(li + c * G::LPR) * G::VEC;
      const bool have = G::FULL || li + c * G::LPR < G::CH;
      kn_c[c] = have ? *reinterpret_cast<const u32x4*>(k_new + e0) : u32x4{0u, 0u, 0u, 0u};
      vn_c[c] = have ? *reinterpret_cast<const u32x4*>(v_new + e0) : u32x4{0u, 0u, 0u, 0u};
    }
  }

  float mrun[GB], lrun[GB], acc[GB][G::ELT];
#pragma unroll
  for (int j = 0; j < GB; ++j) {
    mrun[j] = -INFINITY;
    lrun[j] = 0.f;
#pragma unroll
    for (int e = 0; e < G::ELT; ++e) acc[j][e] = 0.f;
  }

  // row steps per batch of K and V loads (2 rather than 4 on large grids:
  // fewer registers per batch, more waves in flight; 50 vs 53.5 us at two
  // splits, measured; 4 on small grids, whose blocks each take more rows)
  constexpr int U = LA ? 4 : 2;
  constexpr int STEPR = G::RPI * U;  // rows per batch
  // One batch of row loads: every lane issues U rows x CPL chunks of K and
  // V.  Batches past r1 issue only out-of-range offsets (zeros, no memory
  // access), so the pipeline below needs no branch around a load.
  // (LA: every row below r1 is loaded; ok is then only r < r1, and consume
  // applies the window mask.)
  auto issue = [&](int base, u32x4 (&kw)[U][G::CPL], u32x4 (&vw)[U][G::CPL], bool (&ok)[U])
      __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = base + u * G::RPI + wave * G::RPW + rg;
      const int32_t row_byte = r * (int32_t)(D * sizeof(T));
      if constexpr (LA) {
        ok[u] = r < r1;
#pragma unroll
        for (int c = 0; c < G::CPL; ++c) {
          const bool have = G::FULL || li + c * G::LPR < G::CH;
          const int32_t off = ok[u] && have ? row_byte + (li + c * G::LPR) * 16 : kBufferOob;
          kw[u][c] = buffer_load16(krs, off);
          vw[u][c] = buffer_load16(vrs, off);
        }
        continue;
      }
      int jj = r - start;
      jj += jj < 0 ? R : 0;
      const int64_t a = anchor + jj;
      ok[u] = r < r1 && a >= low && a <= high;
#pragma unroll
      for (int c = 0; c < G::CPL; ++c) {
        const bool have = G::FULL || li + c * G::LPR < G::CH;
        const int32_t off = ok[u] && have ? row_byte + (li + c * G::LPR) * 16 : kBufferOob;
        if (STEP && r == slot_p) {  // the appended row, from the step's input
          const size_t e0 = new_off + (size_t)(li + c * G::LPR) * G::VEC;
          kw[u][c] = have ? *reinterpret_cast<const u32x4*>(k_new + e0) : u32x4{0u, 0u, 0u, 0u};
          vw[u][c] = have ? *reinterpret_cast<const u32x4*>(v_new + e0) : u32x4{0u, 0u, 0u, 0u};
        } else {
          kw[u][c] = llvm_raw_buffer_load_v4i32(krs, off, 0, kStreamPolicy);
          vw[u][c] = llvm_raw_buffer_load_v4i32(vrs, off, 0, kStreamPolicy);
        }
      }
    }
  };
  // scores, online softmax over the batch, then the weighted V rows
  auto consume = [&](int base, u32x4 (&kw)[U][G::CPL], u32x4 (&vw)[U][G::CPL], bool (&ok)[U])
      __attribute__((always_inline)) {
    if constexpr (LA) {
      // the window mask of the rows loaded unconditionally; the appended
      // row of a decode step comes from the step's input
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int r = base + u * G::RPI + wave * G::RPW + rg;
        int jj = r - start;
        jj += jj < 0 ? R : 0;
        const int64_t a = anchor + jj;
        ok[u] = ok[u] && a >= low && a <= high;
        if constexpr (STEP) {
          if (r == slot_p) {
#pragma unroll
            for (int c = 0; c < G::CPL; ++c) {
              kw[u][c] = kn_c[c];
              vw[u][c] = vn_c[c];
            }
          }
        }
      }
    }
    // scores (identical in every lane of a row group)
    float sc[U][GB];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if constexpr (kBf) {
        typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
#pragma unroll
        for (int j = 0; j < GB; ++j) {
          float x = 0.f;
#pragma unroll
          for (int c = 0; c < G::CPL; ++c)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              // (through scalars: a bit cast of a vector element reads
              // element 0 whatever the index, in this compiler)
              const uint32_t kx = kw[u][c][w], qx = qw[j][c][w];
              x = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, kx),
                                                  __builtin_bit_cast(bf16x2v, qx), x, false);
            }
          x = group_sum<G::LPR>(x) * qk_scale_log2;
          sc[u][j] = ok[u] ? x : -INFINITY;
        }
      } else {
        float kf[G::ELT];
#pragma unroll
        for (int c = 0; c < G::CPL; ++c) unpack_chunk<T>(kw[u][c], &kf[c * G::VEC]);
#pragma unroll
        for (int j = 0; j < GB; ++j) {
          float x = 0.f;
#pragma unroll
          for (int e = 0; e < G::ELT; ++e) x = fmaf(qv[j][e], kf[e], x);
          x = group_sum<G::LPR>(x);
          sc[u][j] = ok[u] ? x : -INFINITY;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < GB; ++j) {
      float bm = sc[0][j];
#pragma unroll
      for (int u = 1; u < U; ++u) bm = fmaxf(bm, sc[u][j]);
      const float mnew = fmaxf(mrun[j], bm);
      const float mref = mnew == -INFINITY ? 0.f : mnew;
      const float alpha = __builtin_amdgcn_exp2f(mrun[j] - mref);
      mrun[j] = mnew;
      float p[U];
      float psum = 0.f;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        p[u] = __builtin_amdgcn_exp2f(sc[u][j] - mref);
        psum += p[u];
      }
      lrun[j] = lrun[j] * alpha + psum;
#pragma unroll
      for (int e = 0; e < G::ELT; ++e) acc[j][e] *= alpha;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float vf[G::ELT];
#pragma unroll
        for (int c = 0; c < G::CPL; ++c) unpack_chunk<T>(vw[u][c], &vf[c * G::VEC]);
#pragma unroll
        for (int e = 0; e < G::ELT; ++e) acc[j][e] = fmaf(p[u], vf[e], acc[j][e]);
      }
    }
  };
  // two batches in flight: the next batch's loads go out before the current
  // batch is consumed, so a wave waits for memory once per split, not once
  // per batch.  LA: the query loads go out after the first two batches
  // (loads complete in order: waiting for the query earlier would wait for
  // it alone and leave the batches for a second round trip).
  {
    u32x4 kA[U][G::CPL], vA[U][G::CPL], kB[U][G::CPL], vB[U][G::CPL];
    bool okA[U], okB[U];
    int base = r0;
    if constexpr (!LA) load_q();
    issue(base, kA, vA, okA);
    issue(base + STEPR, kB, vB, okB);
    if constexpr (LA) {
      asm volatile("" ::: "memory");
      load_q();
    }
    while (base < r1) {
      consume(base, kA, vA, okA);
      base += STEPR;
      if (base >= r1) break;
      issue(base + STEPR, kA, vA, okA);
      consume(base, kB, vB, okB);
      base += STEPR;
      if (base >= r1) break;
      issue(base + STEPR, kB, vB, okB);
    }
  }
  if constexpr (STEP) {
    // one writer of the appended row: head block 0 of the split holding it
    if (hb == 0 && slot_p >= r0 && slot_p < r1) {
      for (int c = threadIdx.x; c < D / G::VEC; c += NT) {
        const size_t dst = ring_off + (size_t)slot_p * D + (size_t)c * G::VEC;
        *reinterpret_cast<u32x4*>(k_ring + dst) =
            *reinterpret_cast<const u32x4*>(k_new + new_off + (size_t)c * G::VEC);
        *reinterpret_cast<u32x4*>(v_ring + dst) =
            *reinterpret_cast<const u32x4*>(v_new + new_off + (size_t)c * G::VEC);
      }
    }
  }

  // merge the row groups of the wave (lanes that differ above LPR)
  auto merge_rows = [&](auto oc) __attribute__((always_inline)) {
    constexpr int o = decltype(oc)::value;
#pragma unroll
    for (int j = 0; j < GB; ++j) {
      const float m2 = lane_xor<o>(mrun[j]);
      const float l2 = lane_xor<o>(lrun[j]);
      const float M = fmaxf(mrun[j], m2);
      const float Mr = M == -INFINITY ? 0.f : M;
      const float e1 = __builtin_amdgcn_exp2f(mrun[j] - Mr);
      const float e2 = __builtin_amdgcn_exp2f(m2 - Mr);
      lrun[j] = lrun[j] * e1 + l2 * e2;
#pragma unroll
      for (int e = 0; e < G::ELT; ++e) {
        const float a2 = lane_xor<o>(acc[j][e]);
        acc[j][e] = acc[j][e] * e1 + a2 * e2;
      }
      mrun[j] = M;
    }
  };
  static_assert(G::LPR >= 8, "row groups are 8, 16, 32 or 64 lanes");
  if constexpr (G::LPR <= 8) merge_rows(std::integral_constant<int, 8>{});
  if constexpr (G::LPR <= 16) merge_rows(std::integral_constant<int, 16>{});
  if constexpr (G::LPR <= 32) merge_rows(std::integral_constant<int, 32>{});
  if (rg == 0) {
#pragma unroll
    for (int j = 0; j < GB; ++j) {
#pragma unroll
      for (int c = 0; c < G::CPL; ++c) {
        if (!G::FULL && li + c * G::LPR >= G::CH) continue;  // no such chunk
#pragma unroll
        for (int e = 0; e < G::VEC; ++e)
          red_o[wave][j][(li + c * G::LPR) * G::VEC + e] = acc[j][c * G::VEC + e];
      }
      if (li == 0) {
        red_m[wave][j] = mrun[j];
        red_l[wave][j] = lrun[j];
      }
    }
  }
  __syncthreads();
  // merge the waves in a fixed order and write the split partial
  for (int idx = threadIdx.x; idx < nh * D; idx += NT) {
    const int j = idx / D, dd = idx - j * D;
    float M = red_m[0][j];
#pragma unroll
    for (int w = 1; w < NWV; ++w) M = fmaxf(M, red_m[w][j]);
    const float Mr = M == -INFINITY ? 0.f : M;
    float x = 0.f, l = 0.f;
#pragma unroll
    for (int w = 0; w < NWV; ++w) {
      const float e = __builtin_amdgcn_exp2f(red_m[w][j] - Mr);
      x += red_o[w][j][dd] * e;
      l += red_l[w][j] * e;
    }
    if (splits == 1) {  // the block holds the whole ring: the output itself
      const float o = l > 0.f ? x / l : 0.f;
      const size_t oo = ((size_t)b * hq + h0 + j) * D + dd;
      if constexpr (std::is_same<T, float>::value) out[oo] = o;
      else reinterpret_cast<uint16_t*>(out)[oo] = (uint16_t)float_to_bf16_bits(o);
      continue;
    }
    // agent-scope stores write through to the device coherence point, so
    // the combining block (possibly on another XCD) reads them back
    st_agent(&ws_o[(((size_t)b * hq + h0 + j) * splits + s) * D + dd], x);
    if (dd == 0) {
      float* ml = ws_ml + (((size_t)b * hq + h0 + j) * splits + s) * 2;
      st_agent(&ml[0], M);
      st_agent(&ml[1], l);
    }
  }

  // The last split block of this (sequence, head block) combines all splits
  // in a fixed order.  Publication, in three steps:
  //  1. the partials above are agent-scope stores, which write through this
  //     XCD's L2 to the device coherence point;
  //  2. every wave waits until its own stores are acknowledged (vmcnt(0):
  //     __syncthreads() alone orders LDS at work-group scope and leaves
  //     global stores in flight), then the barrier, so all of the block's
  //     partials are at the coherence point before thread 0 moves the
  //     counter (a release at agent scope, without the L2 write-back a
  //     fence would add: only these write-through stores need publishing);
  //  3. the block that reads the final count issues its loads after that
  //     atomic has returned (barrier), as agent-scope loads, which are served
  //     from the coherence point and never from a stale line of its own L2.
  // The counter goes back to zero for the next call.
  // Decode step: every block of the sequence has read ring_meta (its loads
  // returned before any of its work, and every thread of the block passed
  // the barrier above): the last one to get here (a second counter, one per
  // sequence) stores the new state.  The next launch reads it (and the
  // appended ring row, written above by one block with plain stores) after
  // the kernel boundary, which makes every store of this launch visible.
  auto publish_state = [&]() __attribute__((always_inline)) {
    uint32_t* scnt = counters + (size_t)gridDim.z * gridDim.y + b;
    const uint32_t nblk = (uint32_t)splits * gridDim.y;
    if (__hip_atomic_fetch_add(scnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == nblk - 1) {
      int32_t* mw = meta + 4 * (size_t)b;
      mw[0] = (int32_t)pos;
      mw[1] = (int32_t)anchor;
      mw[2] = start;
      mw[3] = slot_p >= 0 ? lo_raw : (int32_t)((uint32_t)lo_raw | 0x80000000u);
      __hip_atomic_store(scnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  };
  if (splits == 1) {  // output written above; no partials, no combine
    if constexpr (STEP) {
      if (threadIdx.x == 0) publish_state();
    }
    return;
  }
  __shared__ int is_last;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  uint32_t* cnt = counters + (size_t)b * gridDim.y + blockIdx.y;
  if (threadIdx.x == 0) {
    is_last = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
              (uint32_t)(splits - 1);
    if constexpr (STEP) publish_state();
  }
  __syncthreads();
  if (!is_last) return;
  // Combine, in split order.  Every partial this block reads is requested
  // in one batch of independent agent-scope loads before any is used (16
  // bytes of o per split and thread, the (m, l) pairs of all splits), so
  // the combine waits for memory once instead of once per split.  Thread
  // (part, item): item = (head j, 4 columns), part p takes the splits
  // p, p + PARTS, ...; the parts' sums are added in order through LDS.
  constexpr int C4 = D / 4;
  constexpr int ITEMS = GB * C4;
  constexpr int PARTS = ITEMS >= NT ? 1 : (NT / ITEMS > 4 ? 4 : NT / ITEMS);
  constexpr int IPT = (ITEMS * PARTS + NT - 1) / NT;  // items per thread
  // splits per load batch and item (large grids have few splits; the
  // registers would cost them occupancy)
  constexpr int NB = IPT == 1 ? (LA ? 18 : 4) : (LA ? 9 : 2);
  constexpr int MLN = (GB * kMaxSplits + NT - 1) / NT;
  __shared__ float cm[GB][kMaxSplits], cl[GB][kMaxSplits];
  // o partials of this (sequence, head block): [nh][splits][D] fp32
  const size_t o_base = ((size_t)b * hq + h0) * splits * D;
  const i32x4 ors = make_buffer_rsrc(ws_o + o_base, (uint32_t)((size_t)nh * splits * D * 4));
  constexpr int kAgent = 16;  // cache policy of an agent-scope load (sc1)
  int it_j[IPT], it_c[IPT], it_p[IPT];
  bool it_ok[IPT];
  u32x4 ob[IPT][NB];
#pragma unroll
  for (int i = 0; i < IPT; ++i) {
    const int t = threadIdx.x + i * NT;
    it_p[i] = t / ITEMS;
    const int item = t - it_p[i] * ITEMS;
    it_j[i] = item / C4;
    it_c[i] = item - it_j[i] * C4;
    it_ok[i] = it_p[i] < PARTS && it_j[i] < nh;
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      const int ss = it_p[i] + n * PARTS;
      const int32_t off = it_ok[i] && ss < splits ? ((it_j[i] * splits + ss) * D + it_c[i] * 4) * 4
                                                 : kBufferOob;
      ob[i][n] = llvm_raw_buffer_load_v4i32(ors, off, 0, kAgent);
    }
  }
  float mlv[MLN][2];
#pragma unroll
  for (int n = 0; n < MLN; ++n) {
    const int idx = threadIdx.x + n * NT;
    if (idx < nh * splits) {
      const int j = idx / splits, ss = idx - j * splits;
      const float* ml = ws_ml + (((size_t)b * hq + h0 + j) * splits + ss) * 2;
      mlv[n][0] = ld_agent(&ml[0]);
      mlv[n][1] = ld_agent(&ml[1]);
    }
  }
#pragma unroll
  for (int n = 0; n < MLN; ++n) {
    const int idx = threadIdx.x + n * NT;
    if (idx < nh * splits) {
      const int j = idx / splits, ss = idx - j * splits;
      cm[j][ss] = mlv[n][0];
      cl[j][ss] = mlv[n][1];
    }
  }
  __syncthreads();
  float4* red4 = reinterpret_cast<float4*>(&red_o[0][0][0]);  // [PARTS][ITEMS]
  float Lsum[IPT];
#pragma unroll
  for (int i = 0; i < IPT; ++i) {
    const int j = it_ok[i] ? it_j[i] : 0;
    // (unrolled so that the LDS reads of several splits are in flight at once)
    float M = -INFINITY;
#pragma unroll 8
    for (int ss = 0; ss < splits; ++ss) M = fmaxf(M, cm[j][ss]);
    const float Mref = M == -INFINITY ? 0.f : M;
    float L = 0.f;
#pragma unroll 8
    for (int ss = 0; ss < splits; ++ss) L += __builtin_amdgcn_exp2f(cm[j][ss] - Mref) * cl[j][ss];
    Lsum[i] = L;
    float4 x = {0.f, 0.f, 0.f, 0.f};
    for (int c0 = 0; c0 < splits; c0 += NB * PARTS) {
      if (c0 > 0) {  // splits beyond the first batch (more than NB * PARTS)
#pragma unroll
        for (int n = 0; n < NB; ++n) {
          const int ss = c0 + it_p[i] + n * PARTS;
          const int32_t off = it_ok[i] && ss < splits
                                  ? ((it_j[i] * splits + ss) * D + it_c[i] * 4) * 4
                                  : kBufferOob;
          ob[i][n] = llvm_raw_buffer_load_v4i32(ors, off, 0, kAgent);
        }
      }
#pragma unroll
      for (int n = 0; n < NB; ++n) {
        const int ss = c0 + it_p[i] + n * PARTS;
        if (ss < splits) {
          const float e = __builtin_amdgcn_exp2f(cm[j][ss] - Mref);
          x.x += e * __uint_as_float(ob[i][n][0]);
          x.y += e * __uint_as_float(ob[i][n][1]);
          x.z += e * __uint_as_float(ob[i][n][2]);
          x.w += e * __uint_as_float(ob[i][n][3]);
        }
      }
    }
    if (it_p[i] < PARTS) red4[it_p[i] * ITEMS + (threadIdx.x + i * NT) % ITEMS] = x;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < IPT; ++i) {
    if (!it_ok[i] || it_p[i] != 0) continue;
    const int item = threadIdx.x + i * NT;
    float4 x = red4[item];
#pragma unroll
    for (int pp = 1; pp < PARTS; ++pp) {
      const float4 y = red4[pp * ITEMS + item];
      x.x += y.x;
      x.y += y.y;
      x.z += y.z;
      x.w += y.w;
    }
    const float L = Lsum[i];
    const size_t o = ((size_t)b * hq + h0 + it_j[i]) * D + it_c[i] * 4;
    const float r4[4] = {L > 0.f ? x.x / L : 0.f, L > 0.f ? x.y / L : 0.f,
                         L > 0.f ? x.z / L : 0.f, L > 0.f ? x.w / L : 0.f};
    if constexpr (std::is_same<T, float>::value) {
      *reinterpret_cast<float4*>(out + o) = float4{r4[0], r4[1], r4[2], r4[3]};
    } else {
      uint2 w;
      w.x = float_to_bf16_bits(r4[0]) | (float_to_bf16_bits(r4[1]) << 16);
      w.y = float_to_bf16_bits(r4[2]) | (float_to_bf16_bits(r4[3]) << 16);
      *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + o) = w;
    }
  }
  if (threadIdx.x == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int D, typename T, int GB>
int launch_decode_t(const void* q, const void* k_new, const void* v_new, void* k_ring,
                    void* v_ring, int32_t* meta, int window, void* out, int batch,
                    int ring_rows, int hq, int hkv, float scale,
                    void* workspace, const DecodePlan& p, hipStream_t stream) {
  uint32_t* counters = (uint32_t*)workspace;
  float* ws_ml = (float*)((char*)workspace + p.counter_bytes);
  float* ws_o = ws_ml + (size_t)batch * hq * p.splits * 2;
  dim3 grid(p.splits, hkv * p.head_blocks, batch);
  const bool step = k_new != nullptr;
  auto kern = step ? (p.load_all ? decode_split_kernel<D, T, GB, true, true>
                                 : decode_split_kernel<D, T, GB, true, false>)
                   : (p.load_all ? decode_split_kernel<D, T, GB, false, true>
                                 : decode_split_kernel<D, T, GB, false, false>);
  hipLaunchKernelGGL(kern, grid, dim3(dec_threads(p.load_all)), 0, stream, (const T*)q, (T*)k_ring,
                     (T*)v_ring, meta, window, ring_rows, hq, hkv, p.head_blocks,
                     p.rows_per_split, scale * kLog2e, ws_o, ws_ml, p.splits, counters,
                     (T*)out, (const T*)k_new, (const T*)v_new);
  return hipGetLastError() == hipSuccess ? SWA_OK : SWA_ELAUNCH;
}

// heads per block: bounded so the cross-wave reduction buffer stays <= 64 KB
// (32 KB with 4 waves)
int heads_per_block_for(int d, int g) {
  int cap = 2048 / d;
  if (cap > 8) cap = 8;
  int hb = 1;
  while (hb * 2 <= cap && hb < g) hb *= 2;
  return hb;
}

}  // namespace

DecodePlan plan_decode(int batch, int hq, int hkv, int d, int ring_rows) {
  DecodePlan p;
  const int g = hq / hkv;
  p.heads_per_block = heads_per_block_for(d, g);
  p.head_blocks = (g + p.heads_per_block - 1) / p.heads_per_block;
  const long long units = (long long)batch * hkv * p.head_blocks;
  long long want = (kTargetBlocks + units - 1) / (units > 0 ? units : 1);
  long long max_splits = (ring_rows + 31) / 32;
  if (max_splits > kMaxSplits) max_splits = kMaxSplits;
  const long long min_splits = (ring_rows + kMaxRowsPerSplit - 1) / kMaxRowsPerSplit;
  if (want > max_splits) want = max_splits;
  if (want < min_splits) want = min_splits;
  if (want < 1) want = 1;
  int rps = (int)((ring_rows + want - 1) / want);
  rps = (rps + 31) / 32 * 32;
  // at most kMaxSplits splits: rows per split >= ring_rows / kMaxSplits
  const int rps_min = (int)(((ring_rows + kMaxSplits - 1) / kMaxSplits + 31) / 32 * 32);
  if (rps < rps_min) rps = rps_min;
  p.rows_per_split = rps;
  p.splits = (ring_rows + rps - 1) / rps;
  // latency-bound grids (no more blocks than CUs, short splits) load whole
  // splits ahead of the ring state, at least 64 rows per block; a grid whose
  // blocks each stream a long split (a large batch, one split per ring)
  // waits for the ring state once and loads only the window's rows (51.3
  // against 48.2 us for the 64-sequence D = 256 decode, measured)
  p.load_all = units * p.splits <= kTargetBlocks && p.rows_per_split <= kLoadAllMaxRows;
  if (p.load_all && p.rows_per_split < kLoadAllRows) {
    p.rows_per_split = kLoadAllRows;
    p.splits = (ring_rows + kLoadAllRows - 1) / kLoadAllRows;
  }
  // [counters: one uint32 per (sequence, kv head, head block), then one per
  //  sequence (decode step), 256-byte padded][(m, l) per (sequence, query
  //  head, split)][o per ... and d]
  p.counter_bytes =
      ((size_t)batch * (hkv * p.head_blocks + 1) * sizeof(uint32_t) + 255) / 256 * 256;
  p.workspace_bytes =
      p.counter_bytes + (size_t)batch * hq * p.splits * ((size_t)d + 2) * sizeof(float);
  return p;
}

int launch_decode(const void* q, const void* k_new, const void* v_new, void* k_ring,
                  void* v_ring, int32_t* meta, int window, void* out, int batch,
                  int ring_rows, int hq, int hkv, int d, int dtype,
                  float scale, void* workspace, const DecodePlan& p,
                  hipStream_t stream) {
#define SWA_DEC_CASE(DD, TT, GBV)                                                     \
  if (d == DD && p.heads_per_block == GBV)                                            \
    return launch_decode_t<DD, TT, GBV>(q, k_new, v_new, k_ring, v_ring, meta, window, \
                                        out, batch, ring_rows, hq, hkv, scale, workspace, \
                                        p, stream);
#define SWA_DEC_D(DD, TT) \
  SWA_DEC_CASE(DD, TT, 1) SWA_DEC_CASE(DD, TT, 2) SWA_DEC_CASE(DD, TT, 4) SWA_DEC_CASE(DD, TT, 8)
  // (head sizes above 256 take at most 4 heads per block: heads_per_block_for)
#define SWA_DEC_D4(DD, TT) SWA_DEC_CASE(DD, TT, 1) SWA_DEC_CASE(DD, TT, 2) SWA_DEC_CASE(DD, TT, 4)
  if (dtype == SWA_BF16) {
    SWA_DEC_D(64, __bf16)
    SWA_DEC_D(128, __bf16)
    SWA_DEC_D(192, __bf16)
    SWA_DEC_D(256, __bf16)
    SWA_DEC_D4(320, __bf16)
    SWA_DEC_D4(384, __bf16)
    SWA_DEC_D4(448, __bf16)
    SWA_DEC_D4(512, __bf16)
  } else {
    SWA_DEC_D(64, float)
    SWA_DEC_D(128, float)
    SWA_DEC_D(192, float)
    SWA_DEC_D(256, float)
    SWA_DEC_D4(320, float)
    SWA_DEC_D4(384, float)
    SWA_DEC_D4(448, float)
    SWA_DEC_D4(512, float)
  }
#undef SWA_DEC_D4
#undef SWA_DEC_D
#undef SWA_DEC_CASE
  return SWA_EUNSUPPORTED;
}

}  // namespace swa
