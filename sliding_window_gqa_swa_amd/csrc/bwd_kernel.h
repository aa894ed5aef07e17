// bwd_kernel.h -- MFMA backward of the sliding-window GQA prefill (gfx950).
//
// Pages cited (title; section):
//   [SDPA]   "Add SDPA attention implementation" (ServiceNow/Fast-LLM pull
//            request 512): Summary (packed documents, GQA head map),
//            Benchmarks (forward and backward timings of the attention
//            implementations at head sizes up to 512)
//   [SPYRE]  "Enable compact sliding-window attention for Gemma 3 and Gemma 4
//            variants" (torch-spyre/hf-adapters pull request 496): Summary
//            (window AND (causal OR vision-blockwise) mask)
//
// Gradients of the loss sum(dout * out) for out = softmax(scale Q K^T,
// masked) V, per query head h and K/V head kvh = h / g:
//   P      = exp2(S c - lse2_i)             (c = scale log2 e; lse2 the row's
//                                            log2-sum-exp2 of S c)
//   delta_i = <dout_i, out_i>                (= sum_j P_ij dP_ij)
//   dP     = dout V^T,   dS = P (dP - delta)
//   dq     = scale dS K,   dk = scale sum_h dS^T Q,   dv = sum_h P^T dout.
// Three launches, no atomics (every output element is written by exactly one
// work-group, so the result is deterministic):
//   1. bwd_rows_kernel: the allowed key interval [lo_i, hi_i] of every row
//      (the mask admits one contiguous interval per row, see the forward),
//      both monotone in i;
//   2. bwd_dq_kernel: per (query tile, head): a first pass over the key
//      tiles gives each row's lse2 (online max and sum; skipped when the
//      forward's log-sum-exp is given), a second forms
//      S^T, dP^T, dS^T and accumulates dq^T = K^T dS^T; it also writes
//      lse2 and delta for launch 3;
//   3. bwd_dkdv_kernel: per (key tile, K/V head): each wave owns 16 keys
//      (K and V fragments in registers; at large head sizes two waves
//      share a key block, one half of d each) and walks the query tiles of
//      every head of the group whose rows admit any of the tile's keys (a
//      contiguous row range, found by binary search on the monotone
//      intervals), accumulating dv^T += dout^T P and dk^T += Q^T dS.
// Tiles travel HBM -> LDS by direct-to-LDS buffer loads into a 2-stage ring
// (the next tile loads while the current one is used), with the forward's
// chunk permutation, so the row-fragment reads (ds_read_b128) and the
// transposed reads (ds_read_b64_tr_b16) are free of bank conflicts.
#pragma once

#include "prefill_kernel.h"

namespace swa {

// Tile geometry: BN rows (keys in the dq kernel, query rows in the dk/dv
// kernel) of D elements per LDS tile, at most 32 KB per tile.
template <int D, typename T, int BN_ = 0, int NW_ = 4>
struct BwGeom {
  using TR = PfTraits<T>;
  static constexpr bool kF32 = std::is_same<T, float>::value;
  static constexpr int NT = 64 * NW_;            // NW_ waves (4 unless given)
  static constexpr int CPR = D / TR::VEC;        // 16-byte chunks per row
  static constexpr int FRAG = kF32 ? 16 : 32;    // rows per P fragment step
  static constexpr int RAW = 32768 / (D * (int)sizeof(T));
  static constexpr int BN = BN_ > 0 ? BN_ : (RAW >= 64 ? 64 : (RAW / FRAG) * FRAG);
  static constexpr int TILE_BYTES = BN * D * (int)sizeof(T);
  static constexpr int UNITS = BN * CPR;
  static constexpr int UPT = UNITS / NT;         // loads per thread per tile
  static constexpr int QREG = D / TR::KW;        // fragments per 16-row block
  static_assert(BN >= FRAG && BN % FRAG == 0, "whole fragments per tile");
  static_assert(UNITS % NT == 0, "tile chunks split evenly over threads");
  static_assert(2 * UPT + 4 <= 63, "loads in flight fit vmcnt");
};

// Work-groups per CU the backward kernels are compiled for: two at small
// bf16 head sizes (two waves per SIMD hide each other's LDS and matrix
// latencies: 197 vs 248 us for the D = 128 dk/dv kernel, measured), else
// what the registers allow.
template <int D, typename T>
constexpr int bw_blocks_per_cu() {
  return (!std::is_same<T, float>::value && D <= 128) ? 2 : 1;
}

// Per-row key intervals (bwd_rows_kernel, prefill_bwd.hip): lo[i] and
// hi[i] of every row, read by both kernels below.

// dk^T / dv^T product with the accumulator pinned to AGPRs.  When a dk/dv
// wave needs more than the 256 VGPRs (bf16 from D = 192 with one wave per
// SIMD), the builtin gives the accumulators AGPRs but moves all of them
// through VGPRs on every tile (a D operand other than the C operand, then
// copies back).  Written by hand, the hazards the compiler resolves for the
// builtin are handled here: the B operand comes from vector ALU conversions
// just before, so the product waits two wait states (s_nop 1); the
// accumulators are read by vector instructions only after the loop, past
// mfma_drain().
__device__ __forceinline__ void bw_mfma_aacc(floatx4& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// Descriptor of rows [r0, T) of a [T, heads, D] tensor at head h: row r of
// the tile at byte offset r * heads * D * sizeof(T); rows at or past T fall
// outside the buffer and load as zeros.
template <typename T, int D>
__device__ __forceinline__ i32x4 bw_rows_rsrc(const T* base, int r0, int h, int heads, int T_) {
  const T* p0 = base + ((size_t)r0 * heads + h) * D;
  const long long rem = (long long)(T_ - r0) * heads * D * (long long)sizeof(T);
  const uint32_t n = rem <= 0 ? 0u : (rem > 0xffffffffLL ? 0xffffffffu : (uint32_t)rem);
  return make_buffer_rsrc(p0, n);
}

// ---------------------------------------------------------------------------
// dq (and lse2, delta): work-group = 64*MB query rows of one query head;
// wave w owns rows 16*MB*w .. +16*MB.  S^T = K Q^T and dP^T = V dout^T take
// K / V fragments from LDS and Q / dout fragments from registers (as the
// forward's S^T); dq^T += K^T dS^T takes K^T by transposed LDS reads and
// dS^T from the accumulator layout (as the forward's O^T += V^T P^T).
template <int D, typename T, int MB, int BN_>
__global__ __launch_bounds__(256, (BN_ > 0 ? 2 : bw_blocks_per_cu<D, T>())) void bwd_dq_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ o, const T* __restrict__ dout, const int32_t* __restrict__ lo_a,
    const int32_t* __restrict__ hi_a, const float* __restrict__ lse_in, int Ttot, int hq,
    int hkv, int W, float c_scale, float scale, int ntiles, int nwork, int per_xcd, T* __restrict__ dq,
    float* __restrict__ lse_out, float* __restrict__ delta_out) {
  using G = BwGeom<D, T, BN_>;
  using TR = typename G::TR;
  constexpr bool kF32 = G::kF32;
  constexpr int BN = G::BN, TB = G::TILE_BYTES, WR = 16 * MB, BM = 4 * WR;
  __shared__ __attribute__((aligned(1024))) unsigned char ring[2][2 * TB];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c16 = lane & 15, grp = lane >> 4;
  // XCD-aware numbering: block b runs on XCD b % 8, which takes a
  // contiguous slice of the work (the tiles of a few heads: their K/V rows
  // meet in one L2)
  const int b = (int)blockIdx.x;
  const int slot = b >> 3;
  const int work = (b & 7) * per_xcd + slot;
  if (slot >= per_xcd || work >= nwork) return;  // uniform per block
  const int h = work / ntiles;
  const int tile = ntiles - 1 - (work - h * ntiles);  // long tiles first
  const int q0 = tile * BM;
  const int g = hq / hkv, kvh = h / g;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);

  // key interval of the work-group and of this wave (monotone intervals:
  // bounds come from the first and last rows)
  const int last = min(q0 + BM, Ttot) - 1;
  const int kmin = lo_a[q0], kmax = hi_a[last];
  const int wr0 = q0 + wave_u * WR, wr1 = min(wr0 + WR, Ttot) - 1;
  const bool wact = wr0 < Ttot;
  const int wlo = wact ? lo_a[wr0] : 0x7fffffff, whi = wact ? hi_a[wr1] : -1;
  const int wlomax = wact ? lo_a[wr1] : 0x7fffffff, whimin = wact ? hi_a[wr0] : -1;
  const int kt0 = (kmin / BN) * BN;
  // (malformed offsets could give kmax < kt0: one tile is still visited,
  // so that every issued load is waited for)
  const int nk = max((kmax - kt0) / BN + 1, 1);
  // Visit order: at D <= 128, where the window cuts the work-group's keys
  // (its first row's interval starts W-1 keys back, not at a document
  // start), visit t reads key tile (t + rot) mod nk, with rot chosen so that
  // the absolute index of that tile is congruent to t mod nk.  The
  // work-groups of neighbouring query tiles running side by side on an XCD
  // (all with the same nk) then read the same K/V tile at the same visit
  // and share it in that XCD's L2, instead of each streaming its own
  // shifted window through it.  dq is a sum over keys, so the order
  // changes only its rounding.  (At D = 512 the same order cut this
  // kernel's HBM reads from 7.4 to 2.6 GB on the 16K-token shape but made
  // it about 1% slower: the natural order is kept there.)
  const bool cut = D <= 128 && W > 0 && q0 - kmin == W - 1;
  const int rot = cut ? (nk - (kt0 / BN) % nk) % nk : 0;
  auto ktile = [&](int t) {
    const int u = t + rot;
    return kt0 + (u >= nk ? u - nk : u) * BN;
  };

  int row_i[MB], row_lo[MB];
  unsigned row_rng[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int i = wr0 + mb * 16 + c16;
    row_i[mb] = i;
    const int lo = i < Ttot ? lo_a[i] : 1, hi = i < Ttot ? hi_a[i] : 0;
    row_lo[mb] = hi >= lo ? lo : 0x3fffffff;
    row_rng[mb] = hi >= lo ? (unsigned)(hi - lo) : 0u;
  }

  // Q and dout fragments (B operands), and delta = <dout, out> per row
  using QF = typename std::conditional<kF32, floatx4, bf16x8>::type;
  QF qf[MB][G::QREG], df[MB][G::QREG];
  float delta[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int i = row_i[mb];
    const bool ok = i < Ttot;
    const size_t roff = ((size_t)(ok ? i : 0) * hq + h) * D;
    float dsum = 0.f;
#pragma unroll
    for (int kk = 0; kk < G::QREG; ++kk) {
      const int d0 = kF32 ? grp * (D / 4) + kk * 4 : kk * 32 + 8 * grp;
      QF a = QF{}, dd = QF{}, oo = QF{};
      if (ok) {
        a = *reinterpret_cast<const QF*>(q + roff + d0);
        dd = *reinterpret_cast<const QF*>(dout + roff + d0);
        oo = *reinterpret_cast<const QF*>(o + roff + d0);
      }
      qf[mb][kk] = a;
      df[mb][kk] = dd;
#pragma unroll
      for (int e = 0; e < TR::VEC; ++e) dsum += (float)dd[e] * (float)oo[e];
    }
    dsum += __shfl_xor(dsum, 16, 64);
    dsum += __shfl_xor(dsum, 32, 64);
    delta[mb] = dsum;
  }

  // direct-to-LDS loads: slot s = (wave * UPT + u) * 64 + lane of a tile is
  // row s / CPR, stored chunk position s % CPR (source chunk chunk_src)
  int voff[G::UPT];
#pragma unroll
  for (int u = 0; u < G::UPT; ++u) {
    const int s = (wave_u * G::UPT + u) * 64 + lane;
    const int r = s / G::CPR, pc = s - r * G::CPR;
    voff[u] = (r * hkv * D + chunk_src<G::CPR>(r, pc) * TR::VEC) * (int)sizeof(T);
  }
  const uint32_t ring_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)(&ring[0][0]);
  auto load_tile = [&](int k0, int stage, bool with_v) {
    const uint32_t kl = ring_base + stage * 2 * TB + wave_u * G::UPT * 1024;
    const i32x4 rk = bw_rows_rsrc<T, D>(k, k0, kvh, hkv, Ttot);
#pragma unroll
    for (int u = 0; u < G::UPT; ++u) dma16_buf(rk, voff[u], kl + u * 1024);
    if (with_v) {
      const i32x4 rv = bw_rows_rsrc<T, D>(v, k0, kvh, hkv, Ttot);
#pragma unroll
      for (int u = 0; u < G::UPT; ++u) dma16_buf(rv, voff[u], kl + TB + u * 1024);
    }
  };

  // S^T of one key tile for this wave's rows, masked to -inf outside each
  // row's interval
  auto scores = [&](const T* Kb, int k0, floatx4 (&s)[MB][BN / 16]) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int kb = 0; kb < BN / 16; ++kb) s[mb][kb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < G::QREG; ++kk) {
#pragma unroll
      for (int kb = 0; kb < BN / 16; ++kb) {
        const int r = kb * 16 + c16;
        if constexpr (kF32) {
          const int ch = grp * (D / 16) + kk;
          const floatx4 a = *reinterpret_cast<const floatx4*>(&Kb[(r * G::CPR + chunk_pos<G::CPR>(r, ch)) * 4]);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int st = 0; st < 4; ++st)
              s[mb][kb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[st], qf[mb][kk][st], s[mb][kb], 0, 0, 0);
        } else {
          const int ch = kk * 4 + grp;
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(&Kb[(r * G::CPR + chunk_pos<G::CPR>(r, ch)) * 8]);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
            s[mb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[mb][kk], s[mb][kb], 0, 0, 0);
        }
      }
    }
    const bool full = k0 >= wlomax && k0 + BN - 1 <= whimin;
    if (!full) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int rel0 = k0 + 4 * grp - row_lo[mb];
#pragma unroll
        for (int kb = 0; kb < BN / 16; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            s[mb][kb][r] = (unsigned)(rel0 + kb * 16 + r) <= row_rng[mb] ? s[mb][kb][r] : -INFINITY;
      }
    }
  };

  auto sync_tile = [&]() {
    wait_vmcnt<0>();  // this wave's loads of the tile have landed
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();  // ... and every wave's; the other stage is free
    asm volatile("" ::: "memory");
  };

  float lse2[MB];
  if (lse_in != nullptr) {
    // the forward's log-sum-exp (natural log) in log2 units
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int i = row_i[mb];
      lse2[mb] = i < Ttot ? lse_in[(size_t)h * Ttot + i] * kPrefillLog2e : INFINITY;
    }
  } else {
  // ---- pass 1: row statistics (max, then sum of exp2 relative to it) ----
  float m_run[MB], l_part[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    m_run[mb] = -INFINITY;
    l_part[mb] = 0.f;
  }
  load_tile(ktile(0), 0, false);
  for (int it = 0; it < nk; ++it) {
    const int k0 = ktile(it);
    sync_tile();
    if (it + 1 < nk) load_tile(ktile(it + 1), (it + 1) & 1, false);
    if (!(wact && k0 <= whi && k0 + BN - 1 >= wlo)) continue;  // no key of the wave's rows
    const T* Kb = reinterpret_cast<const T*>(&ring[it & 1][0]);
    floatx4 s[MB][BN / 16];
    scores(Kb, k0, s);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      float tmax = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < BN / 16; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) tmax = fmaxf(tmax, s[mb][kb][r]);
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      const float m_new = fmaxf(m_run[mb], tmax);
      if (m_new == -INFINITY) continue;  // nothing admitted yet
      const float alpha = m_run[mb] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m_run[mb] - m_new) * c_scale);
      const float mc = m_new * c_scale;
      float lsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < BN / 16; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) lsum += __builtin_amdgcn_exp2f(__builtin_fmaf(s[mb][kb][r], c_scale, -mc));
      l_part[mb] = l_part[mb] * alpha + lsum;
      m_run[mb] = m_new;
    }
  }
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    float l = l_part[mb];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    // log2 of sum_j exp2(s_j c); a row with no key gets +inf (P = 0)
    lse2[mb] = l > 0.f ? m_run[mb] * c_scale + __builtin_log2f(l) : INFINITY;
  }
  __syncthreads();  // every wave is done with pass 1's stages
  }  // pass 1
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int i = row_i[mb];
    if (grp == 0 && i < Ttot) {
      lse_out[(size_t)h * Ttot + i] = lse2[mb];
      delta_out[(size_t)h * Ttot + i] = delta[mb];
    }
  }

  // ---- pass 2: dq^T += K^T dS^T -------------------------------------------
  floatx4 acc[MB][D / 16];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) acc[mb][dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  load_tile(ktile(0), 0, true);
  for (int it = 0; it < nk; ++it) {
    const int k0 = ktile(it);
    sync_tile();
    if (it + 1 < nk) load_tile(ktile(it + 1), (it + 1) & 1, true);
    if (!(wact && k0 <= whi && k0 + BN - 1 >= wlo)) continue;
    const T* Kb = reinterpret_cast<const T*>(&ring[it & 1][0]);
    const T* Vb = reinterpret_cast<const T*>(&ring[it & 1][TB]);
    floatx4 s[MB][BN / 16], dp[MB][BN / 16];
    scores(Kb, k0, s);
    // dP^T = V dout^T
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int kb = 0; kb < BN / 16; ++kb) dp[mb][kb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < G::QREG; ++kk) {
#pragma unroll
      for (int kb = 0; kb < BN / 16; ++kb) {
        const int r = kb * 16 + c16;
        if constexpr (kF32) {
          const int ch = grp * (D / 16) + kk;
          const floatx4 a = *reinterpret_cast<const floatx4*>(&Vb[(r * G::CPR + chunk_pos<G::CPR>(r, ch)) * 4]);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int st = 0; st < 4; ++st)
              dp[mb][kb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[st], df[mb][kk][st], dp[mb][kb], 0, 0, 0);
        } else {
          const int ch = kk * 4 + grp;
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(&Vb[(r * G::CPR + chunk_pos<G::CPR>(r, ch)) * 8]);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
            dp[mb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, df[mb][kk], dp[mb][kb], 0, 0, 0);
        }
      }
    }
    // dS^T = P^T (dP^T - delta), P^T = exp2(S^T c - lse2)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int kb = 0; kb < BN / 16; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mb][kb][r], c_scale, -lse2[mb]));
          s[mb][kb][r] = p * (dp[mb][kb][r] - delta[mb]);
        }
    // dq^T += K^T dS^T
    if constexpr (kF32) {
#pragma unroll
      for (int kb = 0; kb < BN / 16; ++kb)
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
          const int d = dt * 16 + c16;
#pragma unroll
          for (int st = 0; st < 4; ++st) {
            const int r = kb * 16 + 4 * grp + st;
            const float a = Kb[(r * G::CPR + chunk_pos<G::CPR>(r, d >> 2)) * 4 + (d & 3)];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
              acc[mb][dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, s[mb][kb][st], acc[mb][dt], 0, 0, 0);
          }
        }
    } else {
      const int tr_r = (lane & 15) >> 2, tr_m = lane & 3;
#pragma unroll
      for (int ks = 0; ks < BN / 32; ++ks) {
        bf16x8 sf[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            sf[mb][r] = (__bf16)s[mb][2 * ks][r];
            sf[mb][4 + r] = (__bf16)s[mb][2 * ks + 1][r];
          }
        const int r0 = ks * 32 + 4 * grp + tr_r, r1 = r0 + 16;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
          const int ch = 2 * dt + (tr_m >> 1), off = (tr_m & 1) * 4;
          const __bf16* p0 = &Kb[(r0 * G::CPR + chunk_pos<G::CPR>(r0, ch)) * 8 + off];
          const __bf16* p1 = &Kb[(r1 * G::CPR + chunk_pos<G::CPR>(r1, ch)) * 8 + off];
          const short4v lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4v*)(p0));
          const short4v hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4v*)(p1));
          const short8v x8 = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
          const bf16x8 a = __builtin_bit_cast(bf16x8, x8);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
            acc[mb][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, sf[mb], acc[mb][dt], 0, 0, 0);
        }
      }
    }
  }

  // ---- store dq = scale dq^T: each lane holds 4 consecutive d of one row --
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int i = row_i[mb];
    if (i >= Ttot) continue;
    T* drow = dq + ((size_t)i * hq + h) * D;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const floatx4 x = acc[mb][dt] * scale;
      const int d0 = dt * 16 + 4 * grp;
      if constexpr (kF32) {
        *reinterpret_cast<floatx4*>(drow + d0) = x;
      } else {
        const bf16x4 w = {(__bf16)x[0], (__bf16)x[1], (__bf16)x[2], (__bf16)x[3]};
        *reinterpret_cast<bf16x4*>(drow + d0) = w;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// dk, dv: work-group = 4 / DS waves' worth of key blocks of one K/V head;
// wave w owns KB consecutive 16-key blocks (w / DS) and, with DS > 1, one
// part of the head dimension (w % DS): its K and V rows (that part) as B
// fragments in registers and the dk^T, dv^T accumulators of that part.  For
// each head of the group and each query tile of BQ rows that admits any of
// the work-group's keys: S = Q K^T and dP = dout V^T (Q, dout fragments from
// LDS, each feeding KB products; with DS = 2 each wave of a pair forms the
// products over its half of d and the pair adds the two partial sums
// through LDS), then dv^T += dout^T P and dk^T += Q^T dS (dout^T, Q^T by
// transposed LDS reads, again each feeding KB products; P and dS from the
// accumulator layout).  Each stage also carries the tile's lse2, delta, lo
// and hi.  KB = 2 halves the LDS reads per product; DS = 2 halves the
// registers a wave needs at large head sizes, at the cost of a second
// barrier per tile.
template <int D, typename T, int DS, int KB, int BQ_, int NW>
__global__ __launch_bounds__(NW * 64, (NW == 4 ? bw_blocks_per_cu<D, T>() : 1)) void bwd_dkdv_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ dlt,
    const int32_t* __restrict__ lo_a, const int32_t* __restrict__ hi_a, int Ttot, int hq,
    int hkv, int W, float c_scale, float scale, int nktiles, int nwork, int per_xcd,
    T* __restrict__ dk, T* __restrict__ dv) {
  using G = BwGeom<D, T, BQ_, NW>;
  using TR = typename G::TR;
  constexpr bool kF32 = G::kF32;
  constexpr int BQ = G::BN, TB = G::TILE_BYTES, NRB = BQ / 16;
  constexpr int KW = 16 * KB;              // keys per wave
  constexpr int BK = KW * NW / DS;         // keys per work-group
  constexpr int QH = G::QREG / DS;         // S / dP fragments of this wave's d range
  constexpr int NDT = D / 16 / DS;         // 16-wide d blocks of this wave's accumulators
  constexpr int CPW = G::CPR / DS;         // 16-byte chunks of this wave's d range
  // accumulators pinned to AGPRs (bf16 from D = 192 in 4-wave work-groups,
  // see bw_mfma_aacc: left to the compiler, there they live in AGPRs and are
  // copied through VGPRs around every product of every tile)
  constexpr bool kPinAcc = !kF32 && D >= 192 && NW == 4;
  static_assert(DS == 1 || DS == 2, "one or two waves per key block");
  static_assert(KB == 1 || KB == 2, "one or two key blocks per wave");
  static_assert(G::QREG % DS == 0 && (D / 16) % DS == 0, "d splits evenly");
  constexpr int META = 4096;  // lse2, delta, lo, hi: 1 KB each
  static_assert(BQ * 4 <= 1024, "tile metadata fits its slot");
  constexpr int STAGE = 2 * TB + META;
  constexpr int XW = KB * 2 * NRB * 64;    // floatx4 partials per wave
  constexpr int XCH = DS == 2 ? NW * XW * 16 : 16;
  __shared__ __attribute__((aligned(1024))) unsigned char ring[2][STAGE];
  __shared__ __attribute__((aligned(16))) unsigned char xch[XCH];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c16 = lane & 15, grp = lane >> 4;
  const int b = (int)blockIdx.x;
  const int slot = b >> 3;
  const int work = (b & 7) * per_xcd + slot;
  if (slot >= per_xcd || work >= nwork) return;  // uniform per block
  const int kvh = work / nktiles;
  const int kt = work - kvh * nktiles;
  const int g = hq / hkv;
  const int j0 = kt * BK;
  const int j1 = min(j0 + BK - 1, Ttot - 1);
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int dh = wave_u % DS;
  const int wj0 = j0 + KW * (wave_u / DS);  // this wave's first key
  const bool wact = wj0 < Ttot;
  // chunk of fragment kk of this wave's d range (the permutation of the d
  // index within a product step must match between Q / dout and K / V)
  auto frag_ch = [&](int kk) {
    return kF32 ? dh * CPW + grp * (CPW / 4) + kk : dh * CPW + kk * 4 + grp;
  };

  // rows admitting a key of [j0, j1]: hi_i >= j0 and lo_i <= j1, a
  // contiguous range since both bounds are monotone in i
  int i_min, i_max;
  {
    int a = 0, bnd = Ttot;  // first i with hi_i >= j0
    while (a < bnd) {
      const int m = (a + bnd) >> 1;
      if (hi_a[m] >= j0) bnd = m; else a = m + 1;
    }
    i_min = a;
    a = 0, bnd = Ttot;  // first i with lo_i > j1
    while (a < bnd) {
      const int m = (a + bnd) >> 1;
      if (lo_a[m] > j1) bnd = m; else a = m + 1;
    }
    i_max = a - 1;
  }
  i_min = __builtin_amdgcn_readfirstlane(i_min);
  i_max = __builtin_amdgcn_readfirstlane(i_max);
  const int ntq = i_max >= i_min ? (i_max - i_min) / BQ + 1 : 0;
  const int n = g * ntq;
  // Visit t: head t / ntq of the group, query tile (t mod ntq + rot) mod ntq
  // of the range.  At D <= 128, where the window cuts the rows (the last
  // row admitting the work-group's last key is W-1 rows on, not a document
  // end), rot is chosen as in the dq kernel (absolute tile index congruent
  // to the visit), so that the work-groups of neighbouring key tiles read
  // the same Q / dout tile at the same visit (16K tokens, window 4K, D =
  // 128: about 4% off the whole backward with the dq kernel's rotation).
  // At larger D it stays 0: the natural order already keeps the band of
  // query tiles the work-groups of an XCD read in its L2, and aligning them
  // raised this kernel's HBM reads from 2.6 to 7.0 GB on the 16K-token
  // D = 512 shape (measured).
  const bool cut = D <= 128 && W > 0 && ntq > 0 && i_max - j1 == W - 1;
  const int rot = cut ? (ntq - (i_min / BQ) % ntq) % ntq : 0;
  auto qtile_row = [&](int t) {
    const int u = (t - (t / ntq) * ntq) + rot;
    return i_min + (u >= ntq ? u - ntq : u) * BQ;
  };

  // K and V fragments of this lane's keys (B operands of S = Q K^T, dP = dout V^T)
  using QF = typename std::conditional<kF32, floatx4, bf16x8>::type;
  QF kf[KB][QH], vf[KB][QH];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    const int j = wj0 + 16 * kb + c16;
    const bool ok = j < Ttot;
    const size_t roff = ((size_t)(ok ? j : 0) * hkv + kvh) * D;
#pragma unroll
    for (int kk = 0; kk < QH; ++kk) {
      const int d0 = frag_ch(kk) * TR::VEC;
      kf[kb][kk] = ok ? *reinterpret_cast<const QF*>(k + roff + d0) : QF{};
      vf[kb][kk] = ok ? *reinterpret_cast<const QF*>(v + roff + d0) : QF{};
    }
  }

  int voff[G::UPT];
#pragma unroll
  for (int u = 0; u < G::UPT; ++u) {
    const int s = (wave_u * G::UPT + u) * 64 + lane;
    const int r = s / G::CPR, pc = s - r * G::CPR;
    voff[u] = (r * hq * D + chunk_src<G::CPR>(r, pc) * TR::VEC) * (int)sizeof(T);
  }
  const uint32_t ring_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)(&ring[0][0]);
  auto load_tile = [&](int t, int stage) {
    const int h = kvh * g + t / ntq;
    const int i0 = qtile_row(t);
    const uint32_t sb = ring_base + stage * STAGE;
    const uint32_t ql = sb + wave_u * G::UPT * 1024;
    const i32x4 rq = bw_rows_rsrc<T, D>(q, i0, h, hq, Ttot);
    const i32x4 rd = bw_rows_rsrc<T, D>(dout, i0, h, hq, Ttot);
#pragma unroll
    for (int u = 0; u < G::UPT; ++u) dma16_buf(rq, voff[u], ql + u * 1024);
#pragma unroll
    for (int u = 0; u < G::UPT; ++u) dma16_buf(rd, voff[u], ql + TB + u * 1024);
    if (wave_u == 0) {
      // whole 16-byte chunks: up to 3 entries past the tile's last row are
      // read (the workspace pads every array) and never used
      const uint32_t nb = (uint32_t)(((min(BQ, Ttot - i0) * 4 + 15) / 16) * 16);
      const uint32_t ml = sb + 2 * TB;
      dma16_buf(make_buffer_rsrc(lse + (size_t)h * Ttot + i0, nb), lane * 16, ml);
      dma16_buf(make_buffer_rsrc(dlt + (size_t)h * Ttot + i0, nb), lane * 16, ml + 1024);
      dma16_buf(make_buffer_rsrc(lo_a + i0, nb), lane * 16, ml + 2048);
      dma16_buf(make_buffer_rsrc(hi_a + i0, nb), lane * 16, ml + 3072);
    }
  };

  floatx4 dka[KB][NDT], dva[KB][NDT];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      dka[kb][dt] = floatx4{0.f, 0.f, 0.f, 0.f};
      dva[kb][dt] = floatx4{0.f, 0.f, 0.f, 0.f};
    }

  if (n > 0) load_tile(0, 0);
  for (int t = 0; t < n; ++t) {
    if constexpr (kPinAcc) {
      // the accumulators live in AGPRs across the whole loop (without this
      // the compiler keeps them in VGPRs and copies them over for every
      // product)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) asm volatile("" : "+a"(dva[kb][dt]), "+a"(dka[kb][dt]));
    }
    wait_vmcnt<0>();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (t + 1 < n) load_tile(t + 1, (t + 1) & 1);
    const unsigned char* st = &ring[t & 1][0];
    const T* Qb = reinterpret_cast<const T*>(st);
    const T* Db = reinterpret_cast<const T*>(st + TB);
    const float* lse_s = reinterpret_cast<const float*>(st + 2 * TB);
    const float* dlt_s = reinterpret_cast<const float*>(st + 2 * TB + 1024);
    const int* lo_s = reinterpret_cast<const int*>(st + 2 * TB + 2048);
    const int* hi_s = reinterpret_cast<const int*>(st + 2 * TB + 3072);
    const int i0 = qtile_row(t);
    const int nrow = min(BQ, Ttot - i0);
    // rows of the tile admit a key of this wave? (monotone bounds; uniform
    // over the waves that share the keys)
    const bool busy = wact && lo_s[0] <= wj0 + KW - 1 && hi_s[nrow - 1] >= wj0;
    if (DS == 1 && !busy) continue;

    floatx4 s[KB][NRB], dp[KB][NRB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        s[kb][rb] = floatx4{0.f, 0.f, 0.f, 0.f};
        dp[kb][rb] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
    if (busy) {
#pragma unroll
      for (int kk = 0; kk < QH; ++kk) {
        const int ch = frag_ch(kk);
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
          const int r = rb * 16 + c16;
          const int e = (r * G::CPR + chunk_pos<G::CPR>(r, ch)) * TR::VEC;
          if constexpr (kF32) {
            const floatx4 a = *reinterpret_cast<const floatx4*>(&Qb[e]);
            const floatx4 ad = *reinterpret_cast<const floatx4*>(&Db[e]);
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
              for (int x = 0; x < 4; ++x) {
                s[kb][rb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[x], kf[kb][kk][x], s[kb][rb], 0, 0, 0);
                dp[kb][rb] = __builtin_amdgcn_mfma_f32_16x16x4f32(ad[x], vf[kb][kk][x], dp[kb][rb], 0, 0, 0);
              }
          } else {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(&Qb[e]);
            const bf16x8 ad = *reinterpret_cast<const bf16x8*>(&Db[e]);
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
              s[kb][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, kf[kb][kk], s[kb][rb], 0, 0, 0);
              dp[kb][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ad, vf[kb][kk], dp[kb][rb], 0, 0, 0);
            }
          }
        }
      }
    }
    if constexpr (DS == 2) {
      // add the partner wave's partial products (the other half of d); the
      // slots are rewritten only after the next tile's first barrier, which
      // the partner reaches after reading them
      floatx4* mine = reinterpret_cast<floatx4*>(xch) + wave_u * XW;
      const floatx4* other = reinterpret_cast<const floatx4*>(xch) + (wave_u ^ 1) * XW;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
          mine[((kb * NRB + rb) * 2) * 64 + lane] = s[kb][rb];
          mine[((kb * NRB + rb) * 2 + 1) * 64 + lane] = dp[kb][rb];
        }
      lds_barrier();  // (the next tile's loads stay in flight)
      if (!busy) continue;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
          s[kb][rb] += other[((kb * NRB + rb) * 2) * 64 + lane];
          dp[kb][rb] += other[((kb * NRB + rb) * 2 + 1) * 64 + lane];
        }
    }
    // P and dS; lane holds rows 16 rb + 4 grp + x of key wj0 + 16 kb + c16
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int rr = rb * 16 + 4 * grp;
      const floatx4 l4 = *reinterpret_cast<const floatx4*>(&lse_s[rr]);
      const floatx4 d4 = *reinterpret_cast<const floatx4*>(&dlt_s[rr]);
      const int32_t* lo4 = &lo_s[rr];
      const int32_t* hi4 = &hi_s[rr];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int lo = lo4[x], hi = hi4[x];
        const bool row_ok = rr + x < nrow;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const int j = wj0 + 16 * kb + c16;
          const bool ok = row_ok && (unsigned)(j - lo) <= (unsigned)(hi - lo);
          const float p = ok ? __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][rb][x], c_scale, -l4[x])) : 0.f;
          s[kb][rb][x] = p;
          dp[kb][rb][x] = p * (dp[kb][rb][x] - d4[x]);
        }
      }
    }
    // dv^T += dout^T P,  dk^T += Q^T dS  (this wave's d range)
    if constexpr (kF32) {
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const int d = (dh * NDT + dt) * 16 + c16;
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            const int r = rb * 16 + 4 * grp + x;
            const int e = (r * G::CPR + chunk_pos<G::CPR>(r, d >> 2)) * 4 + (d & 3);
            const float ad = Db[e], aq = Qb[e];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
              dva[kb][dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(ad, s[kb][rb][x], dva[kb][dt], 0, 0, 0);
              dka[kb][dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(aq, dp[kb][rb][x], dka[kb][dt], 0, 0, 0);
            }
          }
        }
    } else {
      const int tr_r = (lane & 15) >> 2, tr_m = lane & 3;
#pragma unroll
      for (int ks = 0; ks < BQ / 32; ++ks) {
        bf16x8 pf[KB], sf[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            pf[kb][x] = (__bf16)s[kb][2 * ks][x];
            pf[kb][4 + x] = (__bf16)s[kb][2 * ks + 1][x];
            sf[kb][x] = (__bf16)dp[kb][2 * ks][x];
            sf[kb][4 + x] = (__bf16)dp[kb][2 * ks + 1][x];
          }
        const int r0 = ks * 32 + 4 * grp + tr_r, r1 = r0 + 16;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const int ch = 2 * (dh * NDT + dt) + (tr_m >> 1), off = (tr_m & 1) * 4;
          const int e0 = (r0 * G::CPR + chunk_pos<G::CPR>(r0, ch)) * 8 + off;
          const int e1 = (r1 * G::CPR + chunk_pos<G::CPR>(r1, ch)) * 8 + off;
          const short4v d0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4v*)(&Db[e0]));
          const short4v d1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4v*)(&Db[e1]));
          const short4v q0v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4v*)(&Qb[e0]));
          const short4v q1v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4v*)(&Qb[e1]));
          const short8v dx = {d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3]};
          const short8v qx = {q0v[0], q0v[1], q0v[2], q0v[3], q1v[0], q1v[1], q1v[2], q1v[3]};
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) {
            if constexpr (kPinAcc) {
              bw_mfma_aacc(dva[kb][dt], __builtin_bit_cast(bf16x8, dx), pf[kb]);
              bw_mfma_aacc(dka[kb][dt], __builtin_bit_cast(bf16x8, qx), sf[kb]);
            } else {
              dva[kb][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, dx), pf[kb], dva[kb][dt], 0, 0, 0);
              dka[kb][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qx), sf[kb], dka[kb][dt], 0, 0, 0);
            }
          }
        }
      }
    }
  }

  if constexpr (kPinAcc) mfma_drain();  // the stores below read the accumulators
  // ---- store dk = scale dk^T, dv = dv^T: 4 consecutive d of a key per lane --
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    const int j = wj0 + 16 * kb + c16;
    if (j >= Ttot) continue;
    T* krow = dk + ((size_t)j * hkv + kvh) * D;
    T* vrow = dv + ((size_t)j * hkv + kvh) * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const floatx4 xk = dka[kb][dt] * scale;
      const floatx4 xv = dva[kb][dt];
      const int d0 = (dh * NDT + dt) * 16 + 4 * grp;
      if constexpr (kF32) {
        *reinterpret_cast<floatx4*>(krow + d0) = xk;
        *reinterpret_cast<floatx4*>(vrow + d0) = xv;
      } else {
        const bf16x4 wk = {(__bf16)xk[0], (__bf16)xk[1], (__bf16)xk[2], (__bf16)xk[3]};
        const bf16x4 wv = {(__bf16)xv[0], (__bf16)xv[1], (__bf16)xv[2], (__bf16)xv[3]};
        *reinterpret_cast<bf16x4*>(krow + d0) = wk;
        *reinterpret_cast<bf16x4*>(vrow + d0) = wv;
      }
    }
  }
}

}  // namespace swa
