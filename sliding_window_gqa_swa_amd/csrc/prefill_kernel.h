// prefill_kernel.h -- MFMA flash-style prefill for sliding-window GQA over
// packed variable-length documents (gfx950).
//
// Pages cited (title; section):
//   [SPYRE]  "Enable compact sliding-window attention for Gemma 3 and Gemma 4
//            variants" (torch-spyre/hf-adapters pull request 496)
//   [SDPA]   "Add SDPA attention implementation" (ServiceNow/Fast-LLM pull
//            request 512)
//
// What is computed ([SPYRE] Summary: sliding mask = window AND (causal OR
// vision-blockwise), global layers causal; [SDPA] Summary: packed documents
// never attend across a boundary, GQA as the repeat_interleave head map):
// for query row i the allowed keys form ONE contiguous interval
//   lo_i = max(doc_start(i), i - W + 1)           (doc_start when W <= 0)
//   hi_i = i                                      (causal)
//   hi_i = max(i, last token of i's image run)    (blockwise, image token)
// because an image block is a run of consecutive tokens and the window is
// one-sided.  A work-group therefore needs only [min lo, max hi] of its rows
// as its key range (tile skipping by document, window and block bounds:
// masked key tiles cost nothing) and masks only the key tiles that are not
// inside every row's interval.
//
// Layout of the work ([SDPA] Summary notes that fused kernels there needed
// K/V repeated per query head; here they are not):
//   work-group = BM query rows x GH query heads of one kv head; K and V
//   tiles of BN keys are staged once in LDS and read by every wave, so the
//   GH heads of a group share them.  Each wave owns 16*MB query rows of one
//   head.
//   S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (fp32 inputs:
//   v_mfma_f32_16x16x4_f32): K fragments come from LDS, Q fragments stay in
//   registers, and the S^T accumulator puts one query row per lane, so the
//   softmax row statistics live in the lane (plus a 4-lane butterfly).
//   O^T += V^T P^T takes P straight from the S^T accumulator registers as
//   the B operand; V is stored transposed in LDS ([d][key]) so that its A
//   fragments are two 8-byte LDS reads.
//   Online softmax in the log2 domain with exp2, fp32 accumulators, a final
//   1/l and a round-to-nearest-even store.
#pragma once

#include <type_traits>

#include "swa_common.h"

namespace swa {

constexpr float kPrefillLog2e = 1.4426950408889634f;

template <typename T>
struct PfTraits;

template <>
struct PfTraits<__bf16> {
  static constexpr int VEC = 8;   // elements per 16-byte chunk
  static constexpr int KW = 32;   // head-dim elements per S^T MFMA
  static constexpr int KPAD = 8;  // LDS row pad of Ks (elements = 16 bytes)
  static constexpr int VPAD = 4;  // LDS row pad of Vt (elements = 8 bytes)
};
template <>
struct PfTraits<float> {
  static constexpr int VEC = 4;
  static constexpr int KW = 16;   // one 16-byte LDS read feeds 4 MFMAs of 4
  static constexpr int KPAD = 4;
  static constexpr int VPAD = 4;
};

// Workgroup geometry.
template <int D, typename T, int MB, int BN, int NW, int GH>
struct PfGeom {
  using TR = PfTraits<T>;
  static constexpr int NT = NW * kWave;
  static constexpr int WR = 16 * MB;        // query rows per wave
  static constexpr int RB = NW / GH;        // row blocks per work-group
  static constexpr int BM = RB * WR;        // query rows per work-group
  static constexpr int KS = D + TR::KPAD;   // Ks row stride (elements)
  static constexpr int VS = BN + TR::VPAD;  // Vt row stride (elements)
  static constexpr int LDS_K = BN * KS;
  static constexpr int LDS_V = D * VS;
  static constexpr int QREG = D / TR::KW;   // Q fragments per q-block
  static_assert(NW % GH == 0, "waves must split evenly over heads");
  static_assert(BN % (std::is_same<T, float>::value ? 16 : 32) == 0,
                "key tile is a whole number of P^T fragments");
  static_assert(BM <= NT, "one thread per tile row in the prologue");
};

template <int D, typename T, int MB, int BN, int NW, int GH>
__global__ __launch_bounds__(NW * 64) void prefill_fwd_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const int32_t* __restrict__ cu, int ndocs, const int32_t* __restrict__ ids,
    int W, int mode, T* __restrict__ out, int Ttot, int hq, int hkv,
    float qk_scale_log2, int ntiles) {
  using G = PfGeom<D, T, MB, BN, NW, GH>;
  using TR = typename G::TR;
  constexpr bool kF32 = std::is_same<T, float>::value;

  __shared__ __attribute__((aligned(16))) T Ks[G::LDS_K];
  __shared__ __attribute__((aligned(16))) T Vt[G::LDS_V];
  __shared__ int lo_s[G::BM], hi_s[G::BM];
  __shared__ int red_s[4][NW];
  __shared__ unsigned long long runmask_s[(G::BM + 63) / 64];
  __shared__ int ext_end_s, de_last_s;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c16 = lane & 15;  // MFMA column lane: one query row
  const int grp = lane >> 4;  // MFMA 4-lane group

  // heavy (late) tiles first: causal work grows along a document
  const int tile = ntiles - 1 - (int)blockIdx.x;
  const int q0 = tile * G::BM;
  const int g = hq / hkv;
  const int hgroups = g / GH;
  const int kvh = blockIdx.y / hgroups;
  const int hbase = kvh * g + (blockIdx.y - kvh * hgroups) * GH;
  const int jh = wave % GH;        // head of this wave within the group
  const int rb = wave / GH;        // row block of this wave
  const int h = hbase + jh;

  // ---- prologue: per-row key interval [lo_i, hi_i] ------------------------
  int my_de = 0;
  if (tid < G::BM) {
    const int i = q0 + tid;
    int lo = 1, hi = 0;  // empty interval for rows past the end
    if (i < Ttot) {
      // upper_bound over cu: first d with cu[d] > i
      int a = 0, bnd = ndocs + 1;
      while (a < bnd) {
        const int mid = (a + bnd) >> 1;
        if (cu[mid] > i) bnd = mid; else a = mid + 1;
      }
      const int doc = a - 1;
      int ds = (doc >= 0 && doc < ndocs) ? cu[doc] : i;
      int de = (doc >= 0 && doc < ndocs) ? cu[doc + 1] : i + 1;
      ds = min(max(ds, 0), i);       // clamp against malformed cu_seqlens
      de = max(min(de, Ttot), i + 1);
      lo = (W > 0) ? max(ds, i - W + 1) : ds;
      hi = i;
      my_de = de;
    }
    lo_s[tid] = lo;
    hi_s[tid] = hi;
    if (tid == G::BM - 1) de_last_s = my_de;
  }
  if (mode == SWA_BLOCKWISE) {
    // last_of_run(t): t is the final token of its run of equal ids in its
    // document.  One ballot per 64 rows gives every row its run end.
    bool lr = true;
    int my_id = -1;
    if (tid < G::BM) {
      const int i = q0 + tid;
      if (i < Ttot) {
        my_id = ids[i];
        lr = (i + 1 >= my_de) || (ids[i + 1] != my_id);
      }
    }
    const unsigned long long bal = __ballot(lr);
    if (lane == 0 && wave * 64 < G::BM) runmask_s[wave] = bal;
    if (tid == 0) ext_end_s = -1;
    __syncthreads();
    // the last run of the tile may continue past it: wave 0 scans ahead
    if (wave == 0) {
      const int last = q0 + G::BM - 1;
      const bool open_run = last < Ttot && ids[last] >= 0 &&
                            !((runmask_s[(G::BM - 1) / 64] >> ((G::BM - 1) & 63)) & 1ull);
      if (open_run) {
        const int run_id = ids[last];
        const int de = de_last_s;  // document end of the tile's last row
        int base = last + 1;
        int found = -1;
        while (found < 0) {  // terminates: t >= de always ends the run
          const int t = base + lane;
          const bool stop = (t >= de) || (ids[t] != run_id);
          const unsigned long long m = __ballot(stop);
          if (m) found = base + __builtin_ctzll(m) - 1;
          base += 64;
        }
        if (lane == 0) ext_end_s = found;
      }
    }
    __syncthreads();
    if (tid < G::BM && q0 + tid < Ttot && my_id >= 0) {
      const int w = tid >> 6, b = tid & 63;
      int end = -1;
      for (int ww = w; ww < (G::BM + 63) / 64 && end < 0; ++ww) {
        unsigned long long m = runmask_s[ww];
        if (ww == w) m &= (~0ull) << b;
        if (m) end = ww * 64 + __builtin_ctzll(m);
      }
      if (end >= G::BM) end = -1;  // bits past the tile belong to no row
      hi_s[tid] = end >= 0 ? q0 + end : ext_end_s;
    }
  }
  __syncthreads();

  // tile key range and the rectangle every row admits
  {
    int kmin = 0x7fffffff, kmax = -1, lomax = -1, himin = 0x7fffffff;
    if (tid < G::BM && q0 + tid < Ttot) {
      kmin = lo_s[tid];
      kmax = hi_s[tid];
      lomax = lo_s[tid];
      himin = hi_s[tid];
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      kmin = min(kmin, __shfl_xor(kmin, o, 64));
      kmax = max(kmax, __shfl_xor(kmax, o, 64));
      lomax = max(lomax, __shfl_xor(lomax, o, 64));
      himin = min(himin, __shfl_xor(himin, o, 64));
    }
    if (lane == 0) {
      red_s[0][wave] = kmin;
      red_s[1][wave] = kmax;
      red_s[2][wave] = lomax;
      red_s[3][wave] = himin;
    }
  }
  __syncthreads();
  int kmin = red_s[0][0], kmax = red_s[1][0], lomax = red_s[2][0], himin = red_s[3][0];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    kmin = min(kmin, red_s[0][w]);
    kmax = max(kmax, red_s[1][w]);
    lomax = max(lomax, red_s[2][w]);
    himin = min(himin, red_s[3][w]);
  }
  if (kmax < kmin) return;  // no valid row in this tile (uniform exit)

  // this lane's rows: one per q-block
  int row_i[MB], row_lo[MB], row_hi[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int t = rb * G::WR + mb * 16 + c16;
    row_i[mb] = q0 + t;
    row_lo[mb] = lo_s[t];
    row_hi[mb] = hi_s[t];
  }

  // ---- Q fragments (B operand of S^T = K Q^T), kept in registers ---------
  // bf16: fragment kk holds d = kk*32 + 8*grp + e (e < 8);
  // fp32: lane group grp owns d = grp*D/4 + c, read 4 at a time.
  using QF = typename std::conditional<kF32, floatx4, bf16x8>::type;
  QF qf[MB][G::QREG];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int i = row_i[mb];
    const bool ok = i < Ttot;
    const T* qrow = q + ((size_t)(ok ? i : 0) * hq + h) * D;
#pragma unroll
    for (int kk = 0; kk < G::QREG; ++kk) {
      const int d0 = kF32 ? grp * (D / 4) + kk * 4 : kk * 32 + 8 * grp;
      QF x;
      if (ok)
        x = *reinterpret_cast<const QF*>(qrow + d0);
      else
        x = QF{};
      qf[mb][kk] = x;
    }
  }

  // ---- accumulators ----------------------------------------------------------
  floatx4 o_acc[MB][D / 16];
  float m_run[MB], l_part[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    m_run[mb] = -INFINITY;
    l_part[mb] = 0.f;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) o_acc[mb][dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  const size_t kv_row_stride = (size_t)hkv * D;
  const T* kbase = k + (size_t)kvh * D;
  const T* vbase = v + (size_t)kvh * D;
  constexpr int CPR = D / TR::VEC;  // 16-byte chunks per row

  for (int k0 = (kmin / BN) * BN; k0 <= kmax; k0 += BN) {
    __syncthreads();  // previous tile's LDS reads are done
    // K tile -> Ks[key][d]
    for (int u = tid; u < BN * CPR; u += G::NT) {
      const int r = u / CPR, ch = u - r * CPR;
      const int j = k0 + r;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (j < Ttot) x = *reinterpret_cast<const u32x4*>(kbase + (size_t)j * kv_row_stride + ch * TR::VEC);
      *reinterpret_cast<u32x4*>(&Ks[r * G::KS + ch * TR::VEC]) = x;
    }
    // V tile -> Vt[d][key], 4 keys x one 16-byte chunk per unit
    for (int u = tid; u < (BN / 4) * CPR; u += G::NT) {
      const int kq = u % (BN / 4), ch = u / (BN / 4);
      u32x4 x[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = k0 + 4 * kq + r;
        x[r] = u32x4{0u, 0u, 0u, 0u};
        if (j < Ttot) x[r] = *reinterpret_cast<const u32x4*>(vbase + (size_t)j * kv_row_stride + ch * TR::VEC);
      }
      if constexpr (kF32) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          u32x4 col = {x[0][e], x[1][e], x[2][e], x[3][e]};
          *reinterpret_cast<u32x4*>(&Vt[(ch * 4 + e) * G::VS + 4 * kq]) = col;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int w = e >> 1;
          const bool hiw = e & 1;
          uint32_t a0 = hiw ? (x[0][w] >> 16) : (x[0][w] & 0xffffu);
          uint32_t a1 = hiw ? (x[1][w] >> 16) : (x[1][w] & 0xffffu);
          uint32_t a2 = hiw ? (x[2][w] >> 16) : (x[2][w] & 0xffffu);
          uint32_t a3 = hiw ? (x[3][w] >> 16) : (x[3][w] & 0xffffu);
          u32x2 col = {a0 | (a1 << 16), a2 | (a3 << 16)};
          *reinterpret_cast<u32x2*>(&Vt[(ch * 8 + e) * G::VS + 4 * kq]) = col;
        }
      }
    }
    __syncthreads();

    // ---- S^T = K Q^T for this wave's rows ---------------------------------
    floatx4 s[MB][BN / 16];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int kb = 0; kb < BN / 16; ++kb) s[mb][kb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < G::QREG; ++kk) {
#pragma unroll
      for (int kb = 0; kb < BN / 16; ++kb) {
        if constexpr (kF32) {
          const floatx4 a = *reinterpret_cast<const floatx4*>(
              &Ks[(kb * 16 + c16) * G::KS + grp * (D / 4) + kk * 4]);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int st = 0; st < 4; ++st)
              s[mb][kb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[st], qf[mb][kk][st], s[mb][kb], 0, 0, 0);
        } else {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(
              &Ks[(kb * 16 + c16) * G::KS + kk * 32 + 8 * grp]);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
            s[mb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[mb][kk], s[mb][kb], 0, 0, 0);
        }
      }
    }

    // ---- mask, online softmax ---------------------------------------------
    const bool full = (k0 >= lomax) && (k0 + BN - 1 <= himin);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      float tmax = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < BN / 16; ++kb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float x = s[mb][kb][r] * qk_scale_log2;
          if (!full) {
            const int j = k0 + kb * 16 + 4 * grp + r;
            if (j < row_lo[mb] || j > row_hi[mb]) x = -INFINITY;
          }
          s[mb][kb][r] = x;
          tmax = fmaxf(tmax, x);
        }
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      const float m_new = fmaxf(m_run[mb], tmax);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run[mb] - m_use);
      m_run[mb] = m_new;
      float lsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < BN / 16; ++kb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = __builtin_amdgcn_exp2f(s[mb][kb][r] - m_use);
          s[mb][kb][r] = p;
          lsum += p;
        }
      }
      l_part[mb] = l_part[mb] * alpha + lsum;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) o_acc[mb][dt] *= alpha;
    }

    // ---- O^T += V^T P^T --------------------------------------------------
    if constexpr (kF32) {
#pragma unroll
      for (int kb = 0; kb < BN / 16; ++kb) {
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
          const floatx4 a = *reinterpret_cast<const floatx4*>(
              &Vt[(dt * 16 + c16) * G::VS + kb * 16 + 4 * grp]);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int st = 0; st < 4; ++st)
              o_acc[mb][dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[st], s[mb][kb][st], o_acc[mb][dt], 0, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < BN / 32; ++ks) {
        // P^T fragment: keys 32ks + 4grp + (0..3) and 32ks + 16 + 4grp + (0..3)
        bf16x8 pf[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            pf[mb][r] = (__bf16)s[mb][2 * ks][r];
            pf[mb][4 + r] = (__bf16)s[mb][2 * ks + 1][r];
          }
        }
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
          const T* vrow = &Vt[(dt * 16 + c16) * G::VS + ks * 32 + 4 * grp];
          const u32x2 lo2 = *reinterpret_cast<const u32x2*>(vrow);
          const u32x2 hi2 = *reinterpret_cast<const u32x2*>(vrow + 16);
          const u32x4 w = {lo2[0], lo2[1], hi2[0], hi2[1]};
          const bf16x8 a = __builtin_bit_cast(bf16x8, w);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
            o_acc[mb][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf[mb], o_acc[mb][dt], 0, 0, 0);
        }
      }
    }
  }

  // ---- epilogue: normalise and store ------------------------------------------
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    float l = l_part[mb];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const int i = row_i[mb];
    if (i >= Ttot) continue;
    T* orow = out + ((size_t)i * hq + h) * D;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const floatx4 x = o_acc[mb][dt] * inv;
      const int d0 = dt * 16 + 4 * grp;
      if constexpr (kF32) {
        *reinterpret_cast<floatx4*>(orow + d0) = x;
      } else {
        const u32x2 w = {float_to_bf16_bits(x[0]) | (float_to_bf16_bits(x[1]) << 16),
                         float_to_bf16_bits(x[2]) | (float_to_bf16_bits(x[3]) << 16)};
        *reinterpret_cast<u32x2*>(orow + d0) = w;
      }
    }
  }
}

}  // namespace swa
