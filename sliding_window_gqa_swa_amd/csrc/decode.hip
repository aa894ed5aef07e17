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
//   block = (split s of the R rows, kv head [, head block], sequence b);
//   phase 1 streams K rows with 16-byte loads, each row spread over
//   LPR lanes that each own 16 bytes, and forms the g query dot products with
//   a lane-group butterfly; phase 2 turns the split's scores into
//   exp2(x - m) with block max / sum; phase 3 streams V rows and accumulates
//   the weighted sum.  Partials (m, l, o) go to the workspace and a second
//   kernel combines the splits in a fixed order (deterministic).
#include <type_traits>

#include "swa_common.h"
#include "swa_internal.h"

namespace swa {
namespace {

constexpr int kDecThreads = 256;
constexpr int kDecWaves = kDecThreads / kWave;
constexpr int kMaxRowsPerSplit = 512;  // score buffer <= 16 KB at 8 heads
constexpr int kTargetBlocks = 1024;  // 4 resident blocks per CU on 256 CUs
constexpr float kLog2e = 1.4426950408889634f;

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

template <int D, typename T>
struct DecGeom {
  static constexpr int VEC = 16 / (int)sizeof(T);  // elements per 16 bytes
  static constexpr int CH = D / VEC;                // chunks per row
  static constexpr int LPR = CH < kWave ? CH : kWave;  // lanes per row
  static constexpr int CPL = CH / LPR;              // chunks per lane per row
  static constexpr int RPW = kWave / LPR;           // rows per wave step
  static constexpr int RPI = RPW * kDecWaves;       // rows per block step
  static constexpr int ELT = CPL * VEC;             // elements per lane
};

template <int D, typename T, int GB>
__global__ __launch_bounds__(kDecThreads) void decode_split_kernel(
    const T* __restrict__ q, const T* __restrict__ k_ring,
    const T* __restrict__ v_ring, const int32_t* __restrict__ meta, int W,
    int R, int hq, int hkv, int head_blocks, int rows_per_split,
    float qk_scale_log2, float* __restrict__ ws_o, float* __restrict__ ws_ml,
    int splits) {
  using G = DecGeom<D, T>;
  extern __shared__ float smem[];
  float* sc = smem;                                 // [rows_per_split][GB]
  float* red = smem + (size_t)rows_per_split * GB;  // [waves][GB][D]
  __shared__ float stat[kDecWaves][GB];

  const int s = blockIdx.x;
  const int kvh = blockIdx.y / head_blocks;
  const int hb = blockIdx.y - kvh * head_blocks;
  const int b = blockIdx.z;
  const int g = hq / hkv;
  const int h0 = kvh * g + hb * GB;
  const int nh = min(GB, g - hb * GB);
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int rg = lane / G::LPR;            // row within the wave step
  const int li = lane - rg * G::LPR;       // lane within the row

  const int r0 = s * rows_per_split;
  const int r1 = min(R, r0 + rows_per_split);
  const int nrows = max(0, r1 - r0);

  const int32_t* m = meta + 4 * (size_t)b;
  const int64_t pos = m[0], anchor = m[1], start = m[2];
  const int64_t lo = m[3] & 0x7fffffff;
  int64_t low = max(lo, (int64_t)0);
  if (W > 0) low = max(low, pos - W + 1);
  const int64_t high = pos;

  // query chunks of every head of this block, pre-scaled into the log2 domain
  float qv[GB][G::ELT];
#pragma unroll
  for (int j = 0; j < GB; ++j) {
    const int h = h0 + min(j, nh - 1);
#pragma unroll
    for (int c = 0; c < G::CPL; ++c) {
      float f[G::VEC];
      load_chunk<T>(q + ((size_t)b * hq + h) * D + (size_t)(li + c * G::LPR) * G::VEC, f);
#pragma unroll
      for (int e = 0; e < G::VEC; ++e) qv[j][c * G::VEC + e] = f[e] * qk_scale_log2;
    }
  }

  const T* kbase = k_ring + ((size_t)b * hkv + kvh) * (size_t)R * D;
  const T* vbase = v_ring + ((size_t)b * hkv + kvh) * (size_t)R * D;

  auto row_valid = [&](int r) -> bool {
    const int64_t a = anchor + pos_mod((int64_t)r - start, R);
    return a >= low && a <= high;
  };

  // ---- phase 1: scores of the split's rows ------------------------------
  constexpr int U = 4;  // row steps in flight per lane
  for (int base = 0; base < nrows; base += G::RPI * U) {
    float kf[U][G::ELT];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int rr = base + u * G::RPI + wave * G::RPW + rg;
      ok[u] = rr < nrows && row_valid(r0 + rr);
      if (ok[u]) {
#pragma unroll
        for (int c = 0; c < G::CPL; ++c)
          load_chunk<T>(kbase + (size_t)(r0 + rr) * D + (size_t)(li + c * G::LPR) * G::VEC,
                        &kf[u][c * G::VEC]);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int rr = base + u * G::RPI + wave * G::RPW + rg;
#pragma unroll
      for (int j = 0; j < GB; ++j) {
        float acc = 0.f;
        if (ok[u]) {
#pragma unroll
          for (int e = 0; e < G::ELT; ++e) acc = fmaf(qv[j][e], kf[u][e], acc);
        }
        acc = group_sum<G::LPR>(acc);
        if (li == 0 && rr < nrows) sc[rr * GB + j] = ok[u] ? acc : -INFINITY;
      }
    }
  }
  __syncthreads();

  // ---- phase 2: split max and exp2 weights --------------------------------
  float mj[GB], lj[GB];
#pragma unroll
  for (int j = 0; j < GB; ++j) {
    float x = -INFINITY;
    for (int rr = threadIdx.x; rr < nrows; rr += kDecThreads) x = fmaxf(x, sc[rr * GB + j]);
    x = group_max<kWave>(x);
    if (lane == 0) stat[wave][j] = x;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < GB; ++j) {
    float x = stat[0][j];
#pragma unroll
    for (int w = 1; w < kDecWaves; ++w) x = fmaxf(x, stat[w][j]);
    mj[j] = x;
  }
  __syncthreads();  // stat[] is reused below
#pragma unroll
  for (int j = 0; j < GB; ++j) {
    const float mref = mj[j] == -INFINITY ? 0.f : mj[j];
    float x = 0.f;
    for (int rr = threadIdx.x; rr < nrows; rr += kDecThreads) {
      const float p = __builtin_amdgcn_exp2f(sc[rr * GB + j] - mref);
      sc[rr * GB + j] = p;
      x += p;
    }
    x = group_sum<kWave>(x);
    if (lane == 0) stat[wave][j] = x;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < GB; ++j) {
    float x = 0.f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) x += stat[w][j];
    lj[j] = x;
  }

  // ---- phase 3: weighted sum of V rows ------------------------------------
  float acc[GB][G::ELT];
#pragma unroll
  for (int j = 0; j < GB; ++j)
#pragma unroll
    for (int e = 0; e < G::ELT; ++e) acc[j][e] = 0.f;
  for (int base = 0; base < nrows; base += G::RPI * U) {
    float vf[U][G::ELT];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int rr = base + u * G::RPI + wave * G::RPW + rg;
      ok[u] = rr < nrows && row_valid(r0 + rr);
      if (ok[u]) {
#pragma unroll
        for (int c = 0; c < G::CPL; ++c)
          load_chunk<T>(vbase + (size_t)(r0 + rr) * D + (size_t)(li + c * G::LPR) * G::VEC,
                        &vf[u][c * G::VEC]);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (!ok[u]) continue;
      const int rr = base + u * G::RPI + wave * G::RPW + rg;
#pragma unroll
      for (int j = 0; j < GB; ++j) {
        const float p = sc[rr * GB + j];
#pragma unroll
        for (int e = 0; e < G::ELT; ++e) acc[j][e] = fmaf(p, vf[u][e], acc[j][e]);
      }
    }
  }
  // reduce over the row groups of the wave (lanes differing above LPR)
#pragma unroll
  for (int o = G::LPR; o < kWave; o <<= 1)
#pragma unroll
    for (int j = 0; j < GB; ++j)
#pragma unroll
      for (int e = 0; e < G::ELT; ++e) acc[j][e] += __shfl_xor(acc[j][e], o, kWave);
  if (rg == 0) {
#pragma unroll
    for (int j = 0; j < GB; ++j)
#pragma unroll
      for (int c = 0; c < G::CPL; ++c)
#pragma unroll
        for (int e = 0; e < G::VEC; ++e)
          red[((size_t)wave * GB + j) * D + (li + c * G::LPR) * G::VEC + e] =
              acc[j][c * G::VEC + e];
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < nh * D; idx += kDecThreads) {
    const int j = idx / D, dd = idx - j * D;
    float x = 0.f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) x += red[((size_t)w * GB + j) * D + dd];
    ws_o[(((size_t)b * hq + h0 + j) * splits + s) * D + dd] = x;
  }
  if (threadIdx.x < nh) {
    const int j = threadIdx.x;
    float mm = 0.f, ll = 0.f;
#pragma unroll
    for (int jj = 0; jj < GB; ++jj)
      if (jj == j) {
        mm = mj[jj];
        ll = lj[jj];
      }
    float* ml = ws_ml + (((size_t)b * hq + h0 + j) * splits + s) * 2;
    ml[0] = mm;
    ml[1] = ll;
  }
}

// Fixed-order combine of the split partials of one (sequence, query head).
template <typename T>
__global__ __launch_bounds__(256) void decode_combine_kernel(
    const float* __restrict__ ws_o, const float* __restrict__ ws_ml,
    T* __restrict__ out, int D, int splits) {
  const size_t bh = blockIdx.x;
  const float* ml = ws_ml + bh * splits * 2;
  float M = -INFINITY;
  for (int s = 0; s < splits; ++s) M = fmaxf(M, ml[2 * s]);
  const float Mref = M == -INFINITY ? 0.f : M;
  float L = 0.f;
  for (int s = 0; s < splits; ++s) L += __builtin_amdgcn_exp2f(ml[2 * s] - Mref) * ml[2 * s + 1];
  const float inv = L > 0.f ? 1.f / L : 0.f;
  for (int dd = threadIdx.x; dd < D; dd += blockDim.x) {
    float x = 0.f;
    for (int s = 0; s < splits; ++s)
      x += __builtin_amdgcn_exp2f(ml[2 * s] - Mref) * ws_o[(bh * splits + s) * D + dd];
    x *= inv;
    if constexpr (std::is_same<T, float>::value) {
      out[bh * D + dd] = x;
    } else {
      const uint16_t h = (uint16_t)float_to_bf16_bits(x);
      reinterpret_cast<uint16_t*>(out)[bh * D + dd] = h;
    }
  }
}

template <int D, typename T, int GB>
int launch_decode_t(const void* q, const void* k_ring, const void* v_ring,
                    const int32_t* meta, int window, void* out, int batch,
                    int ring_rows, int hq, int hkv, float scale,
                    void* workspace, const DecodePlan& p, hipStream_t stream) {
  float* ws_o = (float*)workspace;
  float* ws_ml = ws_o + (size_t)batch * hq * p.splits * D;
  const size_t lds = ((size_t)p.rows_per_split * GB + (size_t)kDecWaves * GB * D) * sizeof(float);
  dim3 grid(p.splits, hkv * p.head_blocks, batch);
  hipLaunchKernelGGL((decode_split_kernel<D, T, GB>), grid, dim3(kDecThreads), lds, stream,
                     (const T*)q, (const T*)k_ring, (const T*)v_ring, meta, window,
                     ring_rows, hq, hkv, p.head_blocks, p.rows_per_split,
                     scale * kLog2e, ws_o, ws_ml, p.splits);
  if (hipGetLastError() != hipSuccess) return SWA_ELAUNCH;
  hipLaunchKernelGGL((decode_combine_kernel<T>), dim3(batch * hq), dim3(D < 256 ? D : 256),
                     0, stream, (const float*)ws_o, (const float*)ws_ml, (T*)out, D,
                     p.splits);
  return hipGetLastError() == hipSuccess ? SWA_OK : SWA_ELAUNCH;
}

// heads per block: bounded so the cross-wave reduction buffer stays <= 32 KB
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
  const long long max_splits = (ring_rows + 31) / 32;
  const long long min_splits = (ring_rows + kMaxRowsPerSplit - 1) / kMaxRowsPerSplit;
  if (want > max_splits) want = max_splits;
  if (want < min_splits) want = min_splits;
  if (want < 1) want = 1;
  int rps = (int)((ring_rows + want - 1) / want);
  rps = (rps + 31) / 32 * 32;
  if (rps > kMaxRowsPerSplit) rps = kMaxRowsPerSplit;
  p.rows_per_split = rps;
  p.splits = (ring_rows + rps - 1) / rps;
  p.workspace_bytes = (size_t)batch * hq * p.splits * ((size_t)d + 2) * sizeof(float);
  return p;
}

int launch_decode(const void* q, const void* k_ring, const void* v_ring,
                  const int32_t* meta, int window, void* out, int batch,
                  int ring_rows, int hq, int hkv, int d, int dtype,
                  float scale, void* workspace, const DecodePlan& p,
                  hipStream_t stream) {
#define SWA_DEC_CASE(DD, TT, GBV)                                                    \
  if (d == DD && p.heads_per_block == GBV)                                           \
    return launch_decode_t<DD, TT, GBV>(q, k_ring, v_ring, meta, window, out, batch, \
                                        ring_rows, hq, hkv, scale, workspace, p, stream);
#define SWA_DEC_D(DD, TT) \
  SWA_DEC_CASE(DD, TT, 1) SWA_DEC_CASE(DD, TT, 2) SWA_DEC_CASE(DD, TT, 4) SWA_DEC_CASE(DD, TT, 8)
  if (dtype == SWA_BF16) {
    SWA_DEC_D(64, __bf16)
    SWA_DEC_D(128, __bf16)
    SWA_DEC_D(256, __bf16)
    SWA_DEC_CASE(512, __bf16, 1) SWA_DEC_CASE(512, __bf16, 2) SWA_DEC_CASE(512, __bf16, 4)
  } else {
    SWA_DEC_D(64, float)
    SWA_DEC_D(128, float)
    SWA_DEC_D(256, float)
    SWA_DEC_CASE(512, float, 1) SWA_DEC_CASE(512, float, 2) SWA_DEC_CASE(512, float, 4)
  }
#undef SWA_DEC_D
#undef SWA_DEC_CASE
  return SWA_EUNSUPPORTED;
}

}  // namespace swa
