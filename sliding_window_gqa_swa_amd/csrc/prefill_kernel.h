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
// one-sided.  A work-group therefore visits only the key tiles inside
// [min lo, max hi] of its rows (tile skipping by document, window and block
// bounds: masked key tiles cost nothing) and masks only the tiles that are
// not inside every row's interval.
//
// Work layout:
//   work-group = BM query rows x GH query heads of one kv head; the K and V
//   tiles (BN keys) are staged once in LDS and read by every wave, so the
//   GH heads of a GQA group share them ([SDPA] Summary: there K/V had to be
//   repeated per query head).  Each wave owns 16*MB rows of one head.
//   Work-groups are numbered so that each XCD (own L2) receives a
//   contiguous run of (head group, query tile) work: the K/V rows of a
//   head are fetched from HBM into one L2 instead of eight.
//   Pipeline: K and V tiles travel HBM -> LDS by direct-to-LDS loads
//   (global_load_lds_dwordx4, 16 bytes per lane) into a ring of STAGES
//   buffers, so STAGES-1 tiles are in flight while one is consumed and no
//   registers are spent on staging.  The loads are issued from inline
//   assembly, because the compiler would otherwise order every later LDS
//   read behind all of them; completion is tracked with explicit vmcnt
//   waits and a plain s_barrier (one per tile).  LDS rows are unpadded and
//   their 16-byte chunks permuted per row (chunk_pos below) so that the K
//   fragment reads and the transposed V reads are free of bank conflicts.
//   bf16: S^T = K Q^T on v_mfma_f32_16x16x32_bf16 with K fragments from LDS
//   and Q fragments held in registers; the S^T accumulator holds one query
//   row per lane, so the softmax row statistics stay in the lane (plus a
//   4-lane butterfly).  O^T += V^T P^T takes P straight from the
//   accumulator as the B operand and V^T fragments with ds_read_b64_tr_b16
//   from the row-major V tile.  fp32 inputs use v_mfma_f32_16x16x4_f32 on
//   the same pipeline, mask and softmax.
//   Online softmax in the log2 domain: the running reference max moves only
//   when a score exceeds it by more than kRescaleSlack (so most tiles skip
//   the O rescale), p = exp2(s*c - m*c) is one FMA and one exp2.
#pragma once

#include <type_traits>
#include <utility>

#include "swa_common.h"

namespace swa {

typedef short short4v __attribute__((ext_vector_type(4)));
typedef short short8v __attribute__((ext_vector_type(8)));

constexpr float kPrefillLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// cu_seqlens entries cached in LDS for the per-row document lookup; larger
// batches of documents search global memory instead
constexpr int kCuCache = 1024;
// exp2 arguments stay <= this between reference-max moves (p <= 2^8)
constexpr float kRescaleSlack = 8.0f;
// Work order: cost buckets of the counting sort, and the largest slice of
// work items one XCD may hold for the sort (one byte each, in the LDS ring)
constexpr int kPlanBuckets = 256;
constexpr int kPlanMaxItems = 65536;


// LDS tile layout: 16-byte chunk ch of row r is stored at chunk position
// chunk_pos(r, ch) of that row, a bijection on each row's CPR chunks.  With
// 16 or more chunks per row the chunks of each aligned block of 16 rotate by
// 2 per row, which gives the bank pattern of a 32-byte row padding (the
// 16-row K fragment reads and the transposed V reads are conflict-free)
// while every row stays 16-byte contiguous for the DMA.  Rows of 8 chunks
// use an XOR pattern instead, and so does the 8-chunk tail of a row whose
// length is 8 more than a multiple of 16 chunks (head dimension 320).
__device__ __forceinline__ int chunk_xor8(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }
template <int CPR>
__device__ __forceinline__ int chunk_pos(int r, int ch) {
  static_assert(CPR % 16 == 0 || CPR % 16 == 8, "rows of 16k or 16k + 8 chunks");
  constexpr int FULL = CPR & ~15;
  if constexpr (CPR % 16 == 0) return (ch & ~15) | ((ch + 2 * r) & 15);
  else if constexpr (FULL == 0) return ch ^ chunk_xor8(r);
  else return ch < FULL ? ((ch & ~15) | ((ch + 2 * r) & 15)) : FULL + ((ch - FULL) ^ chunk_xor8(r));
}
// inverse: the chunk stored at position pc of row r
template <int CPR>
__device__ __forceinline__ int chunk_src(int r, int pc) {
  constexpr int FULL = CPR & ~15;
  if constexpr (CPR % 16 == 0) return (pc & ~15) | ((pc - 2 * r) & 15);
  else if constexpr (FULL == 0) return pc ^ chunk_xor8(r);
  else return pc < FULL ? ((pc & ~15) | ((pc - 2 * r) & 15)) : FULL + ((pc - FULL) ^ chunk_xor8(r));
}

// One 16-byte-per-lane direct-to-LDS load: lane l's 16 bytes from g land at
// LDS byte address lds_wave_base + 16 * l (lds_wave_base is wave-uniform).
// An LDS-destination memory instruction reads M0 and needs one wait state
// after the scalar write of M0 (the s_nop); without it the load can take
// the previous M0 and write another load's LDS slots.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_wave_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(lds_wave_base), "v"(g)
               : "memory");
}

// s_waitcnt with vmcnt = n (expcnt and lgkmcnt left unconstrained).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n <= 63, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// s_waitcnt vmcnt(k * UPT) for a uniform run-time k; k > K waits for K * UPT
// (a stronger wait, still correct).
template <int UPT, int K>
__device__ __forceinline__ void wait_vmcnt_units(int k) {
  if constexpr (K == 0) {
    wait_vmcnt<0>();
  } else {
    if (k >= K) wait_vmcnt<K * UPT>();
    else wait_vmcnt_units<UPT, K - 1>(k);
  }
}

// One 16-byte-per-lane direct-to-LDS buffer load: lane l's 16 bytes at
// byte offset voff of the buffer land at LDS byte lds_wave_base + 16 * l; a
// lane whose offset is outside the buffer writes zeros and reads nothing
// (M0 wait state as for dma16).
__device__ __forceinline__ void dma16_buf(i32x4 rsrc, int voff, uint32_t lds_wave_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_wave_base), "v"(voff), "s"(rsrc)
               : "memory");
}

// NU (1 to 4) 16-byte-per-lane direct-to-LDS buffer loads that share one M0
// write: load i lands at LDS byte lds_base + 1024 i + 16 * lane.  The
// instruction offset (1024 i) moves both the memory and the LDS address, so
// vo[i] holds the memory offset of load i minus 1024 i (an out-of-range
// offset stays out of range).
template <int NU>
__device__ __forceinline__ void dma16_buf_group(i32x4 rsrc, const int* vo, uint32_t lds_base) {
  static_assert(NU >= 1 && NU <= 4, "one to four loads per M0 write");
  if constexpr (NU == 4) {
    asm volatile(
        "s_mov_b32 m0, %0\n\ts_nop 0\n\t"
        "buffer_load_dwordx4 %1, %5, 0 offen lds\n\t"
        "buffer_load_dwordx4 %2, %5, 0 offen offset:1024 lds\n\t"
        "buffer_load_dwordx4 %3, %5, 0 offen offset:2048 lds\n\t"
        "buffer_load_dwordx4 %4, %5, 0 offen offset:3072 lds"
        :
        : "s"(lds_base), "v"(vo[0]), "v"(vo[1]), "v"(vo[2]), "v"(vo[3]), "s"(rsrc)
        : "memory");
  } else if constexpr (NU == 3) {
    asm volatile(
        "s_mov_b32 m0, %0\n\ts_nop 0\n\t"
        "buffer_load_dwordx4 %1, %4, 0 offen lds\n\t"
        "buffer_load_dwordx4 %2, %4, 0 offen offset:1024 lds\n\t"
        "buffer_load_dwordx4 %3, %4, 0 offen offset:2048 lds"
        :
        : "s"(lds_base), "v"(vo[0]), "v"(vo[1]), "v"(vo[2]), "s"(rsrc)
        : "memory");
  } else if constexpr (NU == 2) {
    asm volatile(
        "s_mov_b32 m0, %0\n\ts_nop 0\n\t"
        "buffer_load_dwordx4 %1, %3, 0 offen lds\n\t"
        "buffer_load_dwordx4 %2, %3, 0 offen offset:1024 lds"
        :
        : "s"(lds_base), "v"(vo[0]), "v"(vo[1]), "s"(rsrc)
        : "memory");
  } else {
    dma16_buf(rsrc, vo[0], lds_base);
  }
}

// Compile-time loop: f(std::integral_constant<int, i>) for i = 0 .. N-1.
template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// LDS reads issued from inline assembly, so that the compiler keeps them in
// the order written (it otherwise keeps one or two reads in flight).  The
// compiler does not count them: lgkm_wait<N>(x...) waits until at most N
// LDS operations are outstanding and passes the registers it guards through
// the wait, so no instruction that reads them is moved above it.
template <int OFF>
__device__ __forceinline__ bf16x8 lds_b128(uint32_t addr) {
  bf16x8 x;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(x) : "v"(addr), "i"(OFF));
  return x;
}
template <int OFF>
__device__ __forceinline__ short4v lds_tr16_b64(uint32_t addr) {
  short4v x;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(x) : "v"(addr), "i"(OFF));
  return x;
}
template <int N>
__device__ __forceinline__ void lgkm_wait(bf16x8& a, bf16x8& b, bf16x8& c, bf16x8& d) {
  static_assert(N >= 0 && N <= 15, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(a), "+v"(b), "+v"(c), "+v"(d) : "i"(N));
}
template <int N>
__device__ __forceinline__ void lgkm_wait(bf16x8& a, bf16x8& b) {
  static_assert(N >= 0 && N <= 15, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(a), "+v"(b) : "i"(N));
}
template <int N>
__device__ __forceinline__ void lgkm_wait(short4v& a, short4v& b, short4v& c, short4v& d) {
  static_assert(N >= 0 && N <= 15, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(a), "+v"(b), "+v"(c), "+v"(d) : "i"(N));
}

// S^T products issued from inline assembly with the accumulator in VGPRs.
// When a kernel may use more than 256 registers the compiler gives every
// MFMA builtin an AGPR accumulator; at D = 512 the O^T accumulators alone
// fill the 256 AGPRs, so the score products are written by hand to keep
// theirs in VGPRs.  The compiler does not see these as matrix instructions,
// so the hazards it would resolve for a builtin are resolved here:
//  - a VGPR written by a vector ALU instruction may be read by a product
//    only two wait states later (the compiler may materialise an operand,
//    e.g. a zero Q fragment or a copy, right before the block): each block
//    starts with them;
//  - a VALU read of `acc` must come at least kMfmaDrain wait states after
//    the last product that wrote it (the callers guarantee that);
//  - the result registers must not be handed to another value while the
//    products still write them (the callers keep the results live for a
//    whole phase of products after the block).
// A product whose C operand is the previous product's result with the same
// registers is forwarded by the hardware.
// One block: the four products of a pair of K fragments (key blocks 0, 1)
// with the Q fragments of two query blocks (0, 1); c<key block><query block>.
__device__ __forceinline__ void mfma4_bf16_vacc(floatx4& c00, floatx4& c01, floatx4& c10,
                                                floatx4& c11, const bf16x8& k0, const bf16x8& k1,
                                                const bf16x8& q0, const bf16x8& q1) {
  asm volatile(
      "s_nop 1\n\t"
      "v_mfma_f32_16x16x32_bf16 %0, %4, %6, %0\n\t"
      "v_mfma_f32_16x16x32_bf16 %1, %4, %7, %1\n\t"
      "v_mfma_f32_16x16x32_bf16 %2, %5, %6, %2\n\t"
      "v_mfma_f32_16x16x32_bf16 %3, %5, %7, %3"
      : "+v"(c00), "+v"(c01), "+v"(c10), "+v"(c11)
      : "v"(k0), "v"(k1), "v"(q0), "v"(q1));
}
// One product on its own, for schedules that interleave other instructions
// between the products (one instruction issues per four cycles, so a run of
// back-to-back products keeps the wave from issuing anything else).  No
// leading wait states: callers must not write an operand with a vector ALU
// instruction in the two wait states before it (the build checks the
// generated code for that).
__device__ __forceinline__ void mfma1_bf16_vacc(floatx4& c, const bf16x8& k, const bf16x8& q) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(k), "v"(q));
}
__device__ __forceinline__ void mfma1_bf16_vacc0(floatx4& c, const bf16x8& k, const bf16x8& q) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(k), "v"(q));
}
// lgkm_wait<N> on the K fragment pair (k0, k1) and the product (c, k0, q)
// as one statement (two statements let the compiler put wait states between
// them that the hardware does not need)
template <int N, bool ZERO>
__device__ __forceinline__ void lgkm_wait_mfma1(floatx4& c, bf16x8& k0, bf16x8& k1,
                                                const bf16x8& q) {
  static_assert(N >= 0 && N <= 15, "lgkmcnt range");
  if constexpr (ZERO)
    asm volatile("s_waitcnt lgkmcnt(%4)\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %3, 0"
                 : "=&v"(c), "+v"(k0), "+v"(k1) : "v"(q), "i"(N));
  else
    asm volatile("s_waitcnt lgkmcnt(%4)\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %3, %0"
                 : "+v"(c), "+v"(k0), "+v"(k1) : "v"(q), "i"(N));
}
// the same with zero accumulators (the first head-dimension step)
__device__ __forceinline__ void mfma4_bf16_vacc0(floatx4& c00, floatx4& c01, floatx4& c10,
                                                 floatx4& c11, const bf16x8& k0, const bf16x8& k1,
                                                 const bf16x8& q0, const bf16x8& q1) {
  asm volatile(
      "s_nop 1\n\t"
      "v_mfma_f32_16x16x32_bf16 %0, %4, %6, 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %1, %4, %7, 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %2, %5, %6, 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %3, %5, %7, 0"
      : "=&v"(c00), "=&v"(c01), "=&v"(c10), "=&v"(c11)
      : "v"(k0), "v"(k1), "v"(q0), "v"(q1));
}
// wait states that cover an 8-pass product's result latency (with margin)
__device__ __forceinline__ void mfma_drain() {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}

// Maximum of x over lanes l, l^16, l^32, l^48 (gfx950 lane-row swaps; no LDS).
__device__ __forceinline__ float max_over_lane_groups(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Work-group barrier that orders LDS but leaves global/DMA loads in flight
// (__syncthreads() would also wait for every outstanding global load).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt, expcnt unconstrained
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// a*b - c with the product rounded on its own (never fused into an FMA)
__device__ __forceinline__ float mul_then_sub(float a, float b, float c) {
#pragma clang fp contract(off)
  return a * b - c;
}

template <typename T>
struct PfTraits;
template <>
struct PfTraits<__bf16> {
  static constexpr int VEC = 8;  // elements per 16-byte chunk
  static constexpr int KW = 32;  // head-dim elements per S^T MFMA step
};
template <>
struct PfTraits<float> {
  static constexpr int VEC = 4;
  static constexpr int KW = 16;  // one 16-byte LDS read feeds 4 MFMAs of K=4
};

// Pipelined loop schedule per head dimension: LDS fragment lookahead (K
// fragment pairs, V^T fragment groups requested ahead of their use).  The
// tile loads of a step go out in groups of four (one M0 write each), spread
// evenly over the step's K fragment pairs, so that they issue while earlier
// products run.  (Chosen by measurement on MI355X.)
template <int D>
struct PfLookahead {
  static constexpr int K = 2;
  static constexpr int V = 2;
};

// Workgroup geometry.
template <int D, typename T, int MB, int BN, int NW, int GH, bool PL = false>
struct PfGeom {
  using TR = PfTraits<T>;
  static constexpr int NT = NW * kWave;
  static constexpr int WR = 16 * MB;        // query rows per wave
  static constexpr int RB = NW / GH;        // row blocks per work-group
  static constexpr int BM = RB * WR;        // query rows per work-group
  static constexpr int CPR = D / TR::VEC;   // 16-byte chunks per K/V row
  static constexpr int TILE = BN * D;       // elements of one K or V tile (unpadded)
  static constexpr int TILE_BYTES = TILE * (int)sizeof(T);
  static constexpr int STAGE_BYTES = 2 * TILE_BYTES;  // K then V
  // LDS ring depth: as many stages as fit the ring budget (64 KB with two
  // work-groups per CU, 128 KB with one), at least 2 and at most 4
  static constexpr int RING_BUDGET = (NW == 8) ? 131072 : 65536;
  static constexpr int STAGES = (RING_BUDGET / STAGE_BYTES) < 2 ? 2
                                : ((RING_BUDGET / STAGE_BYTES) > 4 ? 4 : RING_BUDGET / STAGE_BYTES);
  static constexpr int UNITS = BN * CPR;    // 16-byte chunks per tile
  static constexpr int UPT = UNITS / NT;    // chunks per thread per tile
  static constexpr int QREG = D / TR::KW;   // Q fragments per q-block
  static_assert(NW % GH == 0, "waves must split evenly over heads");
  static_assert(BN % (std::is_same<T, float>::value ? 16 : 32) == 0,
                "key tile is a whole number of P^T fragments");
  static_assert(BM <= NT, "one thread per tile row in the prologue");
  static_assert(UNITS % NT == 0, "tile chunks split evenly over threads");
  static_assert(CPR >= 8, "the chunk swizzle needs 8 chunks per row");
  static_assert(2 * UPT * (STAGES - 1) <= 63, "loads in flight exceed the vmcnt range");
};

// First d with cu[d] > i (upper bound), cu cached in LDS.
__device__ __forceinline__ int cu_upper(const int* cu_s, int ndocs, int i) {
  int a = 0, bnd = ndocs + 1;
  while (a < bnd) {
    const int mid = (a + bnd) >> 1;
    if (cu_s[mid] > i) bnd = mid; else a = mid + 1;
  }
  return a;
}

// Key position and document key range of query row i.  Documents are
// found in the query offsets cuq; the keys of document d are rows
// cuk[d] .. cuk[d+1]-1 and its query rows are the LAST ones of them (a
// prefill chunk; cuk == cuq for a whole prompt), so row i sits at key
// position i + cuk[d+1] - cuq[d+1].  A row outside every document is a
// one-token document at key position i.  Offsets come from LDS copies when
// in_lds, else from global memory.
struct RowKeys {
  int kp, ds, de;  // key position; document keys [ds, de)
};
__device__ __forceinline__ RowKeys row_keys(const int* cuq_s, const int* cuk_s,
                                            const int32_t* cuq, const int32_t* cuk,
                                            bool in_lds, int ndocs, int i, int Tk) {
  int a = 0, bnd = ndocs + 1;  // upper bound: first d with cuq[d] > i
  while (a < bnd) {
    const int mid = (a + bnd) >> 1;
    const int c = in_lds ? cuq_s[mid] : cuq[mid];
    if (c > i) bnd = mid; else a = mid + 1;
  }
  const int doc = a - 1;
  RowKeys r;
  if (doc >= 0 && doc < ndocs) {
    if (cuk_s == cuq_s && cuk == cuq) {  // whole prompts: key rows = query rows
      r.kp = i;
      r.ds = in_lds ? cuq_s[doc] : cuq[doc];
      r.de = in_lds ? cuq_s[doc + 1] : cuq[doc + 1];
    } else {
      const int ke = in_lds ? cuk_s[doc + 1] : cuk[doc + 1];
      const int qe = in_lds ? cuq_s[doc + 1] : cuq[doc + 1];
      r.kp = i + (ke - qe);
      r.ds = in_lds ? cuk_s[doc] : cuk[doc];
      r.de = ke;
    }
  } else {
    r.kp = i;
    r.ds = i;
    r.de = i + 1;
  }
  // clamps against malformed offsets (then values are unspecified, but every
  // key index stays inside the buffers: tiles past Tk load zeros)
  r.ds = min(max(r.ds, 0), r.kp);
  r.de = max(min(r.de, Tk), r.kp + 1);
  return r;
}

// Cost bucket of query tile `tile`: the number of key tiles a causal /
// windowed tile visits (the image-block extension is left out: the value
// only orders the work).
template <int BM, int BN>
__device__ __forceinline__ int tile_cost_bucket(const int* cu_s, const int* cuk_s, int ndocs,
                                                int tile, int Ttot, int Tk, int W) {
  const int r0 = tile * BM;
  const int r1 = min(r0 + BM, Ttot) - 1;
  // (whole prompts: the caller passes cu_s as both tables)
  const RowKeys rk = row_keys(cu_s, cuk_s, nullptr, nullptr, true, ndocs, r0, Tk);
  const int lo = W > 0 ? max(rk.ds, rk.kp - W + 1) : rk.ds;
  const int kp1 = rk.kp + (r1 - r0);
  return min(max(kp1 / BN - lo / BN + 1, 1), kPlanBuckets - 1);
}

// Inclusive prefix sum over the 64 lanes of a wave, by DPP row shifts and
// row broadcasts (no LDS traffic: the plan runs next to another
// work-group's key loop, which keeps the LDS busy).
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

// Longest-first order of one XCD's slice of work [w0, w0 + P): the offsets
// in the slice of the items at sorted positions pos[0] and pos[1] (sorted
// by descending cost bucket, ties by ascending offset; a position >= P
// gives -1).  Blocks take their items in ascending position, so this is
// list scheduling with the longest items first, which keeps the tail of
// the grid short when item costs vary (causal tiles of many documents).  A
// counting sort: bucket of every item (kept in `bk`, P bytes), histogram,
// the bucket holding each position, then the rank inside that bucket by a
// block-wide scan.  Deterministic.  Called by all NT threads; ends with a
// barrier.  sel_s: 6 ints, wsum_s: 2 * NT / 64 ints.
template <int NT, int BM, int BN>
__device__ void lpt_select(const int* cu_s, const int* cuk_s, int ndocs, int Ttot, int Tk, int W,
                           int ntiles, int hgroups, int w0, int P,
                           const int (&pos)[2], unsigned char* bk, int* hist_s, int* wsum_s,
                           int* sel_s, int (&out)[2]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int NWV = NT / 64;
  for (int i = tid; i < P; i += NT) {
    const int w = (w0 + i) / hgroups;  // (kv head, tile rank), as the kernel numbers items
    const int c = tile_cost_bucket<BM, BN>(cu_s, cuk_s, ndocs, ntiles - 1 - (w % ntiles), Ttot, Tk, W);
    bk[i] = (unsigned char)c;
    atomicAdd(&hist_s[c], 1);
  }
  if (tid < 6) sel_s[tid] = -1;
  __syncthreads();
  if (wave == 0) {  // bucket holding each position, scanning buckets high to low
    static_assert(kPlanBuckets == 4 * 64, "four buckets per lane");
    int n[4], sum = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      n[j] = hist_s[kPlanBuckets - 1 - 4 * lane - j];
      sum += n[j];
    }
    int start = wave_incl_scan(sum) - sum;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        if (pos[x] >= start && pos[x] < start + n[j]) {
          sel_s[2 * x] = kPlanBuckets - 1 - 4 * lane - j;
          sel_s[2 * x + 1] = pos[x] - start;
        }
      }
      start += n[j];
    }
  }
  __syncthreads();
  const int chunk = (P + NT - 1) / NT;
  const int i0 = min(tid * chunk, P), i1 = min(i0 + chunk, P);
  int tb[2], tr[2], cnt[2], incl[2];
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    tb[x] = sel_s[2 * x];
    tr[x] = sel_s[2 * x + 1];
    cnt[x] = 0;
  }
  for (int i = i0; i < i1; ++i) {
    const int c = bk[i];
    cnt[0] += c == tb[0];
    cnt[1] += c == tb[1];
  }
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    incl[x] = wave_incl_scan(cnt[x]);
    if (lane == 63) wsum_s[x * NWV + wave] = incl[x];
  }
  __syncthreads();
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    int before = incl[x] - cnt[x];
    for (int w = 0; w < NWV; ++w) before += w < wave ? wsum_s[x * NWV + w] : 0;
    if (tb[x] >= 0 && tr[x] >= before && tr[x] < before + cnt[x]) {
      int r = tr[x] - before;
      for (int i = i0; i < i1; ++i)
        if (bk[i] == tb[x]) {
          if (r == 0) sel_s[4 + x] = i;
          --r;
        }
    }
  }
  __syncthreads();
#pragma unroll
  for (int x = 0; x < 2; ++x) out[x] = pos[x] < P ? min(max(sel_s[4 + x], 0), P - 1) : -1;
}

template <int D, typename T, int MB, int BN, int NW, int GH, bool PL, bool LSE, int DM>
__global__ __launch_bounds__(NW * 64, (NW == 4 && D <= 256 && (D <= 128 || !PL) && !std::is_same<T, float>::value) ? 2 : 1)
void prefill_fwd_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ cuk, int ndocs,
    const int32_t* __restrict__ ids, int W, int mode, T* __restrict__ out,
    float* __restrict__ lse_out, int Ttot, int Tk,
    int hq, int hkv,
    float qk_scale_log2, int ntiles, int nwork, int work_per_xcd, int slots_per_xcd,
    int colocated) {
  using G = PfGeom<D, T, MB, BN, NW, GH, PL>;
  using TR = typename G::TR;
  constexpr bool kF32 = std::is_same<T, float>::value;
  // DM: the head size of the tensors in memory.  D >= DM is the size the
  // kernel computes with: the extra dimensions are zeros (K, V and Q loads
  // past DM bring zeros, which add nothing to a score, and output columns
  // past DM are not stored), so a head size with no schedule of its own
  // runs on the pipelined loop of the next multiple of 128.
  static_assert(DM <= D && DM % TR::VEC == 0, "memory rows are whole chunks of the computed rows");
  static_assert(DM == D || PL, "padded head sizes run the pipelined loop only");
  constexpr int CPM = DM / TR::VEC;  // 16-byte chunks of a row in memory

  __shared__ __attribute__((aligned(1024))) unsigned char ring[G::STAGES][G::STAGE_BYTES];
  __shared__ int lo_s[G::BM], hi_s[G::BM];
  __shared__ int red_s[4][NW];
  __shared__ unsigned long long runmask_s[(G::BM + 63) / 64];
  __shared__ int ext_end_s, de_last_s, kp_last_s;
  __shared__ int cu_s[kCuCache], cuk_s[kCuCache];  // query and key document offsets
  __shared__ int hist_s[kPlanBuckets];
  __shared__ int plan_s[6 + 2 * NW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c16 = lane & 15;  // MFMA column lane: one query row
  const int grp = lane >> 4;  // MFMA 4-lane group

  // XCD-aware numbering: blocks are dispatched round-robin over 8 XCDs, so
  // block b runs on XCD b % 8; give that XCD a contiguous slice of work
  // (the tiles of the same heads, so their K/V rows meet in one L2), taken
  // longest first.
  const int b = (int)blockIdx.x;
  const int w0 = (b & 7) * work_per_xcd;
  const int P = min(work_per_xcd, nwork - w0);
  constexpr bool kTwoItems = PL;
  const int pos = b >> 3;
  if (pos >= P) return;  // uniform per block
  // cu_seqlens -> LDS with one cooperative load (one memory latency instead
  // of log2(ndocs) dependent ones per row)
  const bool cu_in_lds = ndocs + 1 <= kCuCache;
  // (whole prompts, cuk == cu, use one table for both)
  const bool chunked = cuk != cu;
  const int* cukl = chunked ? cuk_s : cu_s;
  if (cu_in_lds)
    for (int d = tid; d <= ndocs; d += G::NT) {
      cu_s[d] = cu[d];
      if (chunked) cuk_s[d] = cuk[d];
    }
  const bool may_plan = cu_in_lds && P > 1 && P <= kPlanMaxItems;
  // Pipelined path: S = slots_per_xcd work-groups per XCD with at most two
  // items each: the sorted positions pos and 2S-1-pos, so the longest items
  // are paired with the shortest and run back to back (one launch ramp, one
  // cu_seqlens load and one plan for both).
  const int S = kTwoItems ? min(slots_per_xcd, P) : P;
  int pos2 = kTwoItems ? 2 * S - 1 - pos : P;
  if (kTwoItems && colocated && S == slots_per_xcd && (S & 1) == 0) {
    // Every CU of the XCD holds two of its work-groups, w and w + S/2 (the
    // dispatcher fills each CU's first slot, then its second), and the
    // earlier one's waves win issue while both run (about 1.5x its
    // partner's rate, measured): the earlier work-group takes the heavier
    // second items, so that both finish together.
    const int hs = S >> 1;
    pos2 = pos < hs ? 3 * hs - 1 - pos : 4 * hs - 1 - (pos - hs);
  }
  int items[2] = {pos, pos2 < P ? pos2 : -1};
  if (may_plan)
    for (int c = tid; c < kPlanBuckets; c += G::NT) hist_s[c] = 0;
  __syncthreads();  // cu_s and the histogram are ready
  // Documents of equal query and key lengths (one document, or a batch of
  // equal prompts): the work numbering already runs each head's tiles from
  // the last (the longest under a causal or windowed mask) to the first,
  // document after document, so positions pos and 2S-1-pos pair
  // complementary tiles and the sort would only cost its time (2-3 us of a
  // 60 us launch, measured).
  bool plan = may_plan;
  if (may_plan) {
    bool same = true;
    const int lq0 = cu_s[1] - cu_s[0], lk0 = cukl[1] - cukl[0];
    for (int d = 1 + tid; d < ndocs; d += G::NT)
      same &= (cu_s[d + 1] - cu_s[d] == lq0) && (cukl[d + 1] - cukl[d] == lk0);
    plan = !__syncthreads_and(same);
  }
  if (plan) {
    const int posv[2] = {pos, pos2};
    lpt_select<G::NT, G::BM, BN>(cu_s, cukl, ndocs, Ttot, Tk, W, ntiles, hq / hkv / GH, w0, P, posv,
                                 &ring[0][0], hist_s,
                                 plan_s + 6, plan_s, items);
  }
#pragma nounroll
  for (int kq = 0; kq < 2; ++kq) {
  if (items[kq] < 0) break;
  if (kq > 0) __syncthreads();  // the first item is done with every LDS buffer
  const int work = w0 + items[kq];
  [&]() __attribute__((always_inline)) {
  // lane-derived values are recomputed per item from an opaque copy of the
  // thread index: hoisted out of the item loop they would stay live across
  // it and spill the key loop's registers
  int tid_o = (int)threadIdx.x;
  asm volatile("" : "+v"(tid_o));
  const int tid = tid_o;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c16 = lane & 15;
  const int grp = lane >> 4;
  // Item numbering: (kv head, tile rank, head group), the head group
  // fastest, so that the groups of GH heads that read the same K/V tiles
  // (query groups larger than GH) run side by side on one XCD and share
  // them in its L2; tile rank 0 is the last query tile (heavy tiles first).
  const int g = hq / hkv;
  const int hgroups = g / GH;
  const int kt_index = work / hgroups;
  const int kvh = kt_index / ntiles;
  const int tile = ntiles - 1 - (kt_index - kvh * ntiles);
  const int q0 = tile * G::BM;
  const int hbase = kvh * g + (work - kt_index * hgroups) * GH;
  const int jh = wave % GH;  // head of this wave within the group
  const int rb = wave / GH;  // row block of this wave
  const int h = hbase + jh;

  const size_t kv_row_stride = (size_t)hkv * DM;
  const T* kbase = k + (size_t)kvh * DM;
  const T* vbase = v + (size_t)kvh * DM;
  // Direct-to-LDS tile loads.  Wave w issues UPT loads per tensor per tile;
  // load i covers LDS slots [(w*UPT + i)*64, +64) of 16 bytes, slot s being
  // row s / CPR, stored chunk position s % CPR, i.e. source chunk
  // chunk_src(row, s % CPR).
  // Rows past the end are clamped to the last row (finite data, masked).
  int unit_off[G::UPT], unit_row[G::UPT];
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
  for (int i = 0; i < G::UPT; ++i) {
    const int slot = (wave_u * G::UPT + i) * 64 + lane;
    const int r = slot / G::CPR, pc = slot - r * G::CPR;
    unit_row[i] = r;
    unit_off[i] = r * (int)kv_row_stride + chunk_src<G::CPR>(r, pc) * TR::VEC;
  }
  const uint32_t ring_base =
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)(&ring[0][0]);
  auto dma_tile = [&](int k0, int stage) {
    const T* kt = kbase + (size_t)k0 * kv_row_stride;  // uniform
    const T* vt = vbase + (size_t)k0 * kv_row_stride;
    const uint32_t kl = ring_base + stage * G::STAGE_BYTES + wave_u * G::UPT * 1024;
    const uint32_t vl = kl + G::TILE_BYTES;
    const bool whole = k0 + BN <= Tk;
#pragma unroll
    for (int i = 0; i < G::UPT; ++i) {
      const int back = whole ? 0 : max(k0 + unit_row[i] - (Tk - 1), 0) * (int)kv_row_stride;
      dma16(kt + unit_off[i] - back, kl + i * 1024);
      dma16(vt + unit_off[i] - back, vl + i * 1024);
    }
  };

  // first key tile of the work-group: row q0 has the smallest lo of the
  // tile (lo_i never decreases with i), computed here from cu_seqlens alone
  // so that the first K/V loads go out together with the Q loads
  int kt0;
  // Visit order of the key tiles (pipelined loop).  A causal work-group
  // whose keys are cut by the window visits its n tiles rotated: visit t
  // reads tile (t + rot) mod n, with rot chosen so that the absolute tile
  // index of visit t is congruent to t mod n.  Every other such work-group
  // with the same n (every window-limited query tile of a document has the
  // same n) then reads the same absolute key tile at the same visit, so the
  // work-groups running side by side on an XCD stream one window through
  // its L2 together instead of each its own, shifted, window.  The order
  // of the keys does not change the result (online softmax).  Work-groups
  // that start at their document's first key are already aligned (rot 0).
  int rot = 0, nrot = 0x3fffffff;
  {
    const RowKeys rk = row_keys(cu_s, cukl, cu, cuk, cu_in_lds, ndocs, q0, Tk);
    const int lo0 = (W > 0) ? max(rk.ds, rk.kp - W + 1) : rk.ds;
    kt0 = __builtin_amdgcn_readfirstlane((lo0 / BN) * BN);
    if (PL && mode != SWA_BLOCKWISE && lo0 > rk.ds) {
      // the work-group's tile count, as the loop below derives it (the last
      // valid row's causal bound)
      const RowKeys rl = row_keys(cu_s, cukl, cu, cuk, cu_in_lds, ndocs,
                                  min(q0 + G::BM, Ttot) - 1, Tk);
      nrot = (rl.kp - kt0) / BN + 1;
      rot = (nrot - (kt0 / BN) % nrot) % nrot;
    }
    rot = __builtin_amdgcn_readfirstlane(rot);
    nrot = __builtin_amdgcn_readfirstlane(nrot);
  }
  // tile index of visit t (0 <= t < 2 nrot)
  auto tix = [&](int t) {
    const int u = t + rot;
    return u >= nrot ? u - nrot : u;
  };
  // pipelined layout: K ring of STAGES tiles, then V ring of STAGES tiles
  const uint32_t kring = ring_base, vring = ring_base + G::STAGES * G::TILE_BYTES;
  int voff[G::UPT];
#pragma unroll
  for (int i = 0; i < G::UPT; ++i) {
    voff[i] = unit_off[i] * (int)sizeof(T);
    if constexpr (DM < D) {  // padding chunks: out of range, they load zeros
      const int s_ = (wave_u * G::UPT + i) * 64 + lane;
      const int r_ = s_ / G::CPR;
      if (chunk_src<G::CPR>(r_, s_ - r_ * G::CPR) >= CPM) voff[i] = kBufferOob;
    }
  }
  // the same offsets for loads issued four to an M0 write (dma16_buf_group)
  int voffg[G::UPT];
#pragma unroll
  for (int i = 0; i < G::UPT; ++i) voffg[i] = voff[i] - (i % 4) * 1024;
  // descriptor of one K or V tile (keys k0 .. k0+BN-1 of this kv head): it
  // spans the tile's rows before Tk, so rows at or past Tk fall outside it
  // and arrive as zeros; `want` false gives an empty buffer, whose loads
  // fetch nothing and fill their LDS slots with zeros.  (The tile's rows
  // are BN * Hkv * DM elements apart at most, far below 2^32 bytes.)
  const uint32_t row_bytes = (uint32_t)(kv_row_stride * sizeof(T));
  auto tile_rsrc = [&](const T* tb, int k0, bool want = true) {
    const char* p0 = reinterpret_cast<const char*>(tb) + (uint64_t)(uint32_t)k0 * row_bytes;
    const int rows = min(Tk - k0, BN);
    const uint32_t nrec = (rows <= 0 || !want) ? 0u : (uint32_t)rows * row_bytes;
    return make_buffer_rsrc(p0, nrec);
  };
  // every unit of one tile, four loads per M0 write
  auto dma_pl = [&](const T* tb, int k0, uint32_t lds_stage) {
    const i32x4 rsrc = tile_rsrc(tb, k0);
    const uint32_t lw = lds_stage + wave_u * G::UPT * 1024;
    static_for<(G::UPT + 3) / 4>([&](auto gc) {
      constexpr int g = decltype(gc)::value;
      constexpr int nu = G::UPT - 4 * g < 4 ? G::UPT - 4 * g : 4;
      dma16_buf_group<nu>(rsrc, &voffg[4 * g], lw + 4 * g * 1024);
    });
  };
  if constexpr (PL) {
    // groups 0 = {K_0} and 1 = {K_1, V_0} of the pipelined loop (K_1 is
    // loaded even when the work-group has a single key tile: unused then)
    dma_pl(kbase, kt0 + tix(0) * BN, kring);
    dma_pl(kbase, kt0 + tix(1) * BN, kring + G::TILE_BYTES);
    dma_pl(vbase, kt0 + tix(0) * BN, vring);
  } else {
    dma_tile(kt0, 0);
  }

  // ---- Q fragments (B operand of S^T = K Q^T), kept in registers.  Issued
  // before the row-interval prologue so that their latency overlaps it and
  // the first key tile's loads.
  // bf16: fragment kk holds d = kk*32 + 8*grp + e (e < 8);
  // fp32: lane group grp owns d = grp*D/4 + ..., 4 per fragment.
  using QF = typename std::conditional<kF32, floatx4, bf16x8>::type;
  QF qf[MB][G::QREG];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int i = q0 + rb * G::WR + mb * 16 + c16;
    const bool ok = i < Ttot;
    const T* qrow = q + ((size_t)(ok ? i : 0) * hq + h) * DM;
#pragma unroll
    for (int kk = 0; kk < G::QREG; ++kk) {
      const int d0 = kF32 ? grp * (D / 4) + kk * 4 : kk * 32 + 8 * grp;
      QF x = QF{};
      if (ok && d0 < DM) x = *reinterpret_cast<const QF*>(qrow + d0);
      qf[mb][kk] = x;
    }
  }
  // pipelined D = 128: fixed per-row softmax reference, Q scaled once
  constexpr bool kDiagRef = PL && D == 128;

  // ---- prologue: per-row key interval [lo_i, hi_i] ------------------------
  // (intervals are key positions: row i sits at key position kp, equal to
  // i unless the query rows are a chunk of longer documents)
  int my_de = 0, my_kp = 0;
  if (tid < G::BM) {
    const int i = q0 + tid;
    int lo = 1, hi = 0;  // empty interval for rows past the end
    if (i < Ttot) {
      const RowKeys rk = row_keys(cu_s, cukl, cu, cuk, cu_in_lds, ndocs, i, Tk);
      lo = (W > 0) ? max(rk.ds, rk.kp - W + 1) : rk.ds;
      hi = rk.kp;
      my_de = rk.de;
      my_kp = rk.kp;
    }
    lo_s[tid] = lo;
    hi_s[tid] = hi;
    if (tid == G::BM - 1) {
      de_last_s = my_de;
      kp_last_s = my_kp;
    }
  }
  if (mode == SWA_BLOCKWISE) {
    // last_of_run(t): t is the final token of its run of equal ids in its
    // document.  One ballot per 64 rows gives every row its run end.
    bool lr = true;
    int my_id = -1;
    if (tid < G::BM) {
      const int i = q0 + tid;
      if (i < Ttot && my_kp < Tk) {
        my_id = ids[my_kp];
        lr = (my_kp + 1 >= my_de) || (ids[my_kp + 1] != my_id);
      }
    }
    const unsigned long long bal = __ballot(lr);
    if (lane == 0 && wave * 64 < G::BM) runmask_s[wave] = bal;
    if (tid == 0) ext_end_s = -1;
    __syncthreads();
    // the last run of the tile may continue past it: wave 0 scans ahead
    if (wave == 0) {
      const int last = q0 + G::BM - 1;
      const int kp_last = kp_last_s;  // key position of the tile's last row
      const bool open_run = last < Ttot && kp_last < Tk && ids[kp_last] >= 0 &&
                            !((runmask_s[(G::BM - 1) / 64] >> ((G::BM - 1) & 63)) & 1ull);
      if (open_run) {
        const int run_id = ids[kp_last];
        const int de = de_last_s;  // document key end of the tile's last row
        int base = kp_last + 1;
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
      const int w = tid >> 6, bb = tid & 63;
      int end = -1;
      for (int ww = w; ww < (G::BM + 63) / 64 && end < 0; ++ww) {
        unsigned long long m = runmask_s[ww];
        if (ww == w) m &= (~0ull) << bb;
        if (m) end = ww * 64 + __builtin_ctzll(m);
      }
      if (end >= G::BM) end = -1;  // bits past the tile belong to no row
      // (the run's last row is in this row's document: same key offset)
      hi_s[tid] = end >= 0 ? my_kp + (end - tid) : ext_end_s;
    }
  }
  __syncthreads();

  // tile key range and the rectangle every row admits.  Causal intervals
  // are monotone in the row (lo_i and hi_i = i never decrease), so the
  // bounds are those of the first and last valid rows; blockwise intervals
  // are reduced over all rows.
  const int last_row = min(G::BM, Ttot - q0) - 1;  // >= 0: q0 < Ttot
  int kmin, kmax, lomax, himin;
  if (mode != SWA_BLOCKWISE) {
    kmin = lo_s[0];
    himin = hi_s[0];
    kmax = hi_s[last_row];
    lomax = lo_s[last_row];
  } else {
    {
      int a0 = 0x7fffffff, a1 = -1, a2 = -1, a3 = 0x7fffffff;
      if (tid < G::BM && q0 + tid < Ttot) {
        a0 = lo_s[tid];
        a1 = hi_s[tid];
        a2 = lo_s[tid];
        a3 = hi_s[tid];
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        a0 = min(a0, __shfl_xor(a0, o, 64));
        a1 = max(a1, __shfl_xor(a1, o, 64));
        a2 = max(a2, __shfl_xor(a2, o, 64));
        a3 = min(a3, __shfl_xor(a3, o, 64));
      }
      if (lane == 0) {
        red_s[0][wave] = a0;
        red_s[1][wave] = a1;
        red_s[2][wave] = a2;
        red_s[3][wave] = a3;
      }
    }
    lds_barrier();
    kmin = red_s[0][0], kmax = red_s[1][0], lomax = red_s[2][0], himin = red_s[3][0];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      kmin = min(kmin, red_s[0][w]);
      kmax = max(kmax, red_s[1][w]);
      lomax = max(lomax, red_s[2][w]);
      himin = min(himin, red_s[3][w]);
    }
  }
  if (kmax < kmin) {  // no valid row (cannot happen: row q0 < Ttot); uniform exit
    wait_vmcnt<0>();  // never leave with a load still writing this block's LDS
    return;
  }

  // this lane's rows: one per q-block.  Key j is allowed iff
  // (unsigned)(j - lo) <= (unsigned)(hi - lo); rows with an empty interval
  // get lo far above every key so the test always fails.
  int row_i[MB], row_lo[MB];
  unsigned row_rng[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int t = rb * G::WR + mb * 16 + c16;
    row_i[mb] = q0 + t;
    const int lo = lo_s[t], hi = hi_s[t];
    row_lo[mb] = hi >= lo ? lo : 0x3fffffff;
    row_rng[mb] = hi >= lo ? (unsigned)(hi - lo) : 0u;
  }

  if constexpr (PL) {
    // ---- software-pipelined loop (bf16, D = 128, 64-key tiles) -----------------
    // Iteration t runs the S^T MFMAs of key tile t+1 next to the softmax of
    // tile t, then the O^T MFMAs of tile t.  K tiles live in a 2-stage ring
    // and V tiles in a second 2-stage ring one tile behind: load group
    // m = {K_m, V_(m-1)} is issued in iteration m-2 and consumed in iteration
    // m-1.  The LDS fragment reads are issued by hand ahead of their MFMAs
    // (the compiler keeps one or two in flight, exposing the LDS latency),
    // and scheduling barriers keep each group of MFMAs next to the vector
    // work meant to run under it.  Row sums come from one extra MFMA per 32
    // keys against a ones A operand: the sum of the same bf16 weights that
    // weight V.  A wave skips the key tiles outside its own rows.
    static_assert(!kF32, "the pipelined loop is bf16 only");
    constexpr int S = G::STAGES;
    constexpr int TB = G::TILE_BYTES;
    constexpr int ROWB = D * 2;     // bytes of one K/V row in LDS
    constexpr int NKB = BN / 16;    // 16-key blocks per tile
    constexpr int NKS = BN / 32;    // 32-key P^T fragments per tile
    constexpr int NDT = D / 16;     // 16-wide head-dim blocks
    constexpr int QR = G::QREG;     // 32-wide head-dim steps of S^T
    // head-dim steps and blocks that carry data: a head size padded in
    // registers (DM < D, 320 computed as 384) runs no products over the
    // padding (zeros in every K, V and Q fragment there, whose products add
    // nothing and whose outputs are not stored)
    constexpr bool kTrim = DM < D && DM % 32 == 0;
    constexpr int QRE = kTrim ? DM / 32 : QR;     // S^T head-dim steps
    constexpr int NDTE = kTrim ? DM / 16 : NDT;   // O^T head-dim blocks
    constexpr int NP = QRE * (NKB / 2);  // K fragment pairs per tile (4 MFMAs each)
    constexpr int NJ = NKS * (NDTE / 2); // V^T fragment groups per tile (4 MFMAs each)
    // LDS fragment lookahead: K pairs and V groups requested ahead of use
    constexpr int KLA = PfLookahead<D>::K, VLA = PfLookahead<D>::V;
    static_assert(NP >= 2 * ((G::UPT + 3) / 4), "a K fragment pair per load group");
    static_assert(2 * KLA <= 15 && 4 * VLA <= 15, "lgkmcnt range");
    // D >= 256: score products by hand (VGPR accumulators, see mfma_bf16_vacc)
    // and row sums on the VALU, so that the AGPRs hold O^T alone
    constexpr bool kAsmS = D >= 256;
    static_assert(MB == 2 && S == 2 && NW == 4 && BN % 32 == 0 && D % 128 == 0,
                  "schedule written for 32 rows per wave, 4 waves, 2 stages, D a multiple of 128");
    // every LDS fragment offset below is an instruction immediate (16 bits)
    static_assert(TB + (NKB - 1) * 16 * ROWB + (QR / 4 - 1) * 256 < 65536, "K offsets fit");
    static_assert(TB + (NKS - 1) * 32 * ROWB + 16 * ROWB + (NDT / 8 - 1) * 256 < 65536,
                  "V offsets fit");
    const int n = (kmax - kt0) / BN + 1;  // key tiles of the work-group
    // (a rotated visit order, rot > 0, was derived from this same count)

    // this wave's rows: key range, and the rectangle every one of them admits
    // (monotone causal intervals: first and last valid rows of the wave)
    int wlo = 0x7fffffff, whi = -1, wlomax = -1, whimin = 0x7fffffff;
    if (mode != SWA_BLOCKWISE) {
      const int r0 = rb * G::WR, r1 = min(r0 + G::WR - 1, last_row);
      if (r0 <= last_row) {
        wlo = lo_s[r0];
        whimin = hi_s[r0];
        whi = hi_s[r1];
        wlomax = lo_s[r1];
      }
    } else {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        if (row_i[mb] < Ttot && row_lo[mb] != 0x3fffffff) {
          const int lo = row_lo[mb], hi = lo + (int)row_rng[mb];
          wlo = min(wlo, lo);
          whi = max(whi, hi);
          wlomax = max(wlomax, lo);
          whimin = min(whimin, hi);
        }
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        wlo = min(wlo, __shfl_xor(wlo, o, 64));
        whi = max(whi, __shfl_xor(whi, o, 64));
        wlomax = max(wlomax, __shfl_xor(wlomax, o, 64));
        whimin = min(whimin, __shfl_xor(whimin, o, 64));
      }
    }
    // active key tiles of this wave: [ta, tb] (empty for a wave past the end)
    const int ta = __builtin_amdgcn_readfirstlane(whi >= wlo ? (wlo - kt0) / BN : n);
    const int tb = __builtin_amdgcn_readfirstlane(whi >= wlo ? min((whi - kt0) / BN, n - 1) : -1);
    // does this wave have rows in the tile of visit t?
    auto active = [&](int t) {
      const int u = tix(t);
      return u >= ta && u <= tb;
    };
    wlomax = __builtin_amdgcn_readfirstlane(wlomax);
    whimin = __builtin_amdgcn_readfirstlane(whimin);


    // LDS byte addresses of this lane's fragments (see chunk_pos):
    // chunk_pos(r + 16 j, ch) = chunk_pos(r, ch) for 16-chunk rows, and the
    // rotation stays inside each aligned block of 16 chunks (256 bytes), so
    // the K fragment of head-dim step kk and key block kb is at
    // kaddr[kk % 4] + stage + kb * 16 rows + (kk / 4) * 256, and the V^T
    // fragment dt of 32-key step ks at vaddr[dt % 8] + stage + ks * 32 rows
    // (+16 rows for its second half) + (dt / 8) * 256.  K addresses start at
    // the K ring, V addresses at the V ring.
    uint32_t kaddr[4], vaddr[8];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      kaddr[kk] = kring + c16 * ROWB + chunk_pos<G::CPR>(c16, 4 * kk + grp) * 16;
    {
      const int tr_r = (lane & 15) >> 2, tr_m = lane & 3;
      const int vrow = 4 * grp + tr_r;
#pragma unroll
      for (int b = 0; b < 8; ++b)
        vaddr[b] = vring + vrow * ROWB + chunk_pos<G::CPR>(vrow, 2 * b + (tr_m >> 1)) * 16 +
                   (tr_m & 1) * 8;
    }

    floatx4 o_acc[MB][NDT], l_acc[MB];
    // kDiagRef: every S^T product chain starts from minus the row's
    // reference, so the accumulator already holds the exp2 argument
    floatx4 s_init[MB];
    // the row has its reference (rows past the end need none)
    bool ref_ok[MB];
    // m_ref: running reference of the other loops; mcs (kAsmS): the row's
    // fixed reference times c, subtracted inside the exp2 argument;
    // l_part: this lane's share of the row sum
    float m_ref[MB], mcs[MB], l_part[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      m_ref[mb] = -INFINITY;
      mcs[mb] = 0.f;
      l_part[mb] = 0.f;
      l_acc[mb] = floatx4{0.f, 0.f, 0.f, 0.f};
      s_init[mb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) o_acc[mb][dt] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
    const __bf16 one = (__bf16)1.0f;
    const bf16x8 ones = {one, one, one, one, one, one, one, one};
    const float c_scale = qk_scale_log2;
    const float slack = kRescaleSlack / c_scale;  // in raw score units

    // mask of tile t (only tiles not inside every row's interval); a tile
    // outside the wave's range is masked whole (its scores may come from a
    // stale stage)
    auto mask = [&](int t, bool act, floatx4 (&sc)[MB][NKB]) {
      const int k0 = kt0 + tix(t) * BN;
      const bool full = act && (k0 >= wlomax) && (k0 + BN - 1 <= whimin);
      if (!full) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int rel0 = k0 + 4 * grp - (act ? row_lo[mb] : 0x3fffffff);
          const unsigned rng = act ? row_rng[mb] : 0u;
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              sc[mb][kb][r] = (unsigned)(rel0 + kb * 16 + r) <= rng ? sc[mb][kb][r] : -INFINITY;
        }
      }
    };

    // K fragments of key blocks (2 kp, 2 kp + 1) of head-dim step kk
    auto issue_k = [&](auto kkc, auto kpc, auto kstc, bf16x8 (&dst)[2]) {
      constexpr int kk = decltype(kkc)::value, kp = decltype(kpc)::value, KST = decltype(kstc)::value;
      constexpr int OFF = KST + (kk / 4) * 256;
      dst[0] = lds_b128<OFF + (2 * kp) * 16 * ROWB>(kaddr[kk % 4]);
      dst[1] = lds_b128<OFF + (2 * kp + 1) * 16 * ROWB>(kaddr[kk % 4]);
    };
    // one of the two reads of issue_k (ic = 0, 1), as a plain LDS load: the
    // compiler then places the lgkmcnt wait before the first product that
    // reads it, counting exactly the reads issued after it (the scheduling
    // barriers around each product keep the reads where they are written)
    auto issue_k1 = [&](auto kkc, auto kpc, auto kstc, auto icc, bf16x8& dst) {
      constexpr int kk = decltype(kkc)::value, kp = decltype(kpc)::value, KST = decltype(kstc)::value;
      constexpr int ic = decltype(icc)::value;
      constexpr int OFF = KST + (kk / 4) * 256 + (2 * kp + ic) * 16 * ROWB;
      dst = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(
          (size_t)(kaddr[kk % 4] + OFF));
    };
    auto s_mfmas = [&](auto kkc, auto kpc, const bf16x8 (&kf)[2], floatx4 (&sn)[MB][NKB]) {
      constexpr int kk = decltype(kkc)::value, kp = decltype(kpc)::value;
      if constexpr (kAsmS) {
        constexpr int kb0 = 2 * kp, kb1 = 2 * kp + 1;
        if constexpr (kk == 0)
          mfma4_bf16_vacc0(sn[0][kb0], sn[1][kb0], sn[0][kb1], sn[1][kb1], kf[0], kf[1], qf[0][kk],
                           qf[1][kk]);
        else
          mfma4_bf16_vacc(sn[0][kb0], sn[1][kb0], sn[0][kb1], sn[1][kb1], kf[0], kf[1], qf[0][kk],
                          qf[1][kk]);
        return;
      }
      static_for<2>([&](auto ic) {
        constexpr int kb = 2 * kp + decltype(ic)::value;
        static_for<2>([&](auto mbc) {
          constexpr int mb = decltype(mbc)::value;
          {
            sn[mb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                kf[decltype(ic)::value], qf[mb][kk], kk == 0 ? s_init[mb] : sn[mb][kb], 0, 0, 0);
          }
        });
      });
    };
    // V^T fragments of head-dim blocks (dt0, dt0 + 1), dt0 = 2 (j % (NDTE/2)),
    // of 32-key step j / (NDTE/2)
    auto issue_v = [&](auto jc, auto vstc, short4v (&dst)[4]) {
      constexpr int j = decltype(jc)::value, VST = decltype(vstc)::value;
      constexpr int ks = j / (NDTE / 2), dt0 = 2 * (j % (NDTE / 2));
      constexpr int OFF = VST + ks * 32 * ROWB + (dt0 / 8) * 256;
      dst[0] = lds_tr16_b64<OFF>(vaddr[dt0 % 8]);
      dst[1] = lds_tr16_b64<OFF + 16 * ROWB>(vaddr[dt0 % 8]);
      dst[2] = lds_tr16_b64<OFF>(vaddr[dt0 % 8 + 1]);
      dst[3] = lds_tr16_b64<OFF + 16 * ROWB>(vaddr[dt0 % 8 + 1]);
    };
    // read r (0..3) of issue_v, as a plain transposed LDS load (see issue_k1)
    auto issue_v1 = [&](auto jc, auto vstc, auto rc, short4v& dst) {
      constexpr int j = decltype(jc)::value, VST = decltype(vstc)::value, r = decltype(rc)::value;
      constexpr int ks = j / (NDTE / 2), dt0 = 2 * (j % (NDTE / 2));
      constexpr int OFF = VST + ks * 32 * ROWB + (dt0 / 8) * 256 + (r & 1) * 16 * ROWB;
      dst = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          reinterpret_cast<__attribute__((address_space(3))) short4v*>(
              (size_t)(vaddr[dt0 % 8 + (r >> 1)] + OFF)));
    };
    // product (hh, mb) of V^T group j
    auto pv1 = [&](auto jc, auto hc, auto mbc, const short4v (&v4)[4], const bf16x8 (&pf)[MB][NKS]) {
      constexpr int j = decltype(jc)::value, hh = decltype(hc)::value, mb = decltype(mbc)::value;
      constexpr int ks = j / (NDTE / 2), dt0 = 2 * (j % (NDTE / 2));
      const short8v x8 = {v4[2 * hh][0], v4[2 * hh][1], v4[2 * hh][2], v4[2 * hh][3],
                          v4[2 * hh + 1][0], v4[2 * hh + 1][1], v4[2 * hh + 1][2], v4[2 * hh + 1][3]};
      const bf16x8 a = __builtin_bit_cast(bf16x8, x8);
      o_acc[mb][dt0 + hh] =
          __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf[mb][ks], o_acc[mb][dt0 + hh], 0, 0, 0);
    };
    auto pv_mfmas = [&](auto jc, const short4v (&v4)[4], const bf16x8 (&pf)[MB][NKS]) {
      constexpr int j = decltype(jc)::value;
      constexpr int ks = j / (NDTE / 2), dt0 = 2 * (j % (NDTE / 2));
      static_for<2>([&](auto hc) {
        constexpr int hh = decltype(hc)::value;
        const short8v x8 = {v4[2 * hh][0], v4[2 * hh][1], v4[2 * hh][2], v4[2 * hh][3],
                            v4[2 * hh + 1][0], v4[2 * hh + 1][1], v4[2 * hh + 1][2], v4[2 * hh + 1][3]};
        const bf16x8 a = __builtin_bit_cast(bf16x8, x8);
        static_for<2>([&](auto mbc) {
          constexpr int mb = decltype(mbc)::value;
          o_acc[mb][dt0 + hh] =
              __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf[mb][ks], o_acc[mb][dt0 + hh], 0, 0, 0);
        });
      });
    };

    floatx4 sA[MB][NKB], sB[MB][NKB];

    // one iteration (t of parity par): scores of tile t in sc, of t+1 into sn
    auto step = [&](auto parc, int t, floatx4 (&sc)[MB][NKB], floatx4 (&sn)[MB][NKB]) __attribute__((always_inline)) {
      constexpr int par = decltype(parc)::value;
      constexpr std::integral_constant<int, ((par + 1) % 2) * TB> KST{};  // K stage of tile t+1
      constexpr std::integral_constant<int, par * TB> VST{};              // V stage of tile t
      // group t+1 = {K_(t+1), V_t}, the latest issued, landed in every wave
      wait_vmcnt<0>();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      // every wave is done with K_t and V_(t-1): refill their stages.  This
      // wave's 2*UPT loads (V_(t+1) units, then K_(t+2) units) go out in
      // groups spread over the K fragment pairs below, so the vector memory
      // queue never stalls the wave behind a burst
      // (a load that is not wanted gets an empty buffer instead of a branch:
      // its stage is free, and branches here cost the accumulators their
      // register assignment)
      const bool kld = t + 2 < n, vld = t + 1 < n;
      const i32x4 rs_k = tile_rsrc(kbase, kt0 + tix(t + 2) * BN, kld);
      const i32x4 rs_v = tile_rsrc(vbase, kt0 + tix(t + 1) * BN, vld);
      const uint32_t lw_k = kring + par * TB + wave_u * G::UPT * 1024;
      const uint32_t lw_v = vring + ((par + 1) % 2) * TB + wave_u * G::UPT * 1024;
      // load groups of four units (one M0 write each): V_(t+1) groups, then
      // K_(t+2) groups
      constexpr int GV = (G::UPT + 3) / 4;
      auto dma_group = [&](auto gc) {
        constexpr int g = decltype(gc)::value;
        constexpr int gg = g < GV ? g : g - GV;
        constexpr int nu = G::UPT - 4 * gg < 4 ? G::UPT - 4 * gg : 4;
        if constexpr (g < GV) dma16_buf_group<nu>(rs_v, &voffg[4 * gg], lw_v + 4 * gg * 1024);
        else dma16_buf_group<nu>(rs_k, &voffg[4 * gg], lw_k + 4 * gg * 1024);
      };
      // a wave with no rows in tiles t and t+1 still runs the step (its
      // loads are spread through it; a branch around them would cost the
      // accumulators their registers): every score of such a tile is
      // masked, so its weights are 0 against finite V rows
      const bool a_cur = active(t);
      mask(t, a_cur, sc);
      if constexpr (kDiagRef) {
        // rows without a reference: the maximum of their allowed scores in
        // this tile becomes the reference (wave-uniform branch, taken in a
        // row's first tiles): the tile-t scores started from 0, they are
        // shifted by it and the products issued from now on start from
        // minus it
        bool need = false;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) need |= !ref_ok[mb];
        if (__builtin_amdgcn_ballot_w64(need)) {
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            float tmax = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
              for (int r = 0; r < 4; ++r) tmax = fmaxf(tmax, sc[mb][kb][r]);
            tmax = max_over_lane_groups(tmax);
            if (!ref_ok[mb] && tmax != -INFINITY) {
              ref_ok[mb] = true;
              s_init[mb] = floatx4{-tmax, -tmax, -tmax, -tmax};
#pragma unroll
              for (int kb = 0; kb < NKB; ++kb) sc[mb][kb] -= tmax;
            }
          }
        }
      }

      // -- phase 1: S^T of tile t+1 with the softmax of tile t --------------------
      float alpha[MB], mc[MB];
      bool any_move = false;
      auto row_stats = [&](auto mbc) {
        constexpr int mb = decltype(mbc)::value;
        if constexpr (kDiagRef) {
          return;  // fixed reference, no row statistics
        } else {
          float tmax = -INFINITY;
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) tmax = fmaxf(tmax, sc[mb][kb][r]);
          tmax = max_over_lane_groups(tmax);
          const bool move = tmax > m_ref[mb] + slack;
          const float m_new = move ? tmax : m_ref[mb];
          alpha[mb] = move ? __builtin_amdgcn_exp2f((m_ref[mb] - m_new) * c_scale) : 1.f;
          any_move |= move;
          m_ref[mb] = m_new;
          mc[mb] = m_new == -INFINITY ? 0.f : m_new * c_scale;
        }
      };
      bf16x8 pc[MB][NKS];
      // weights of keys kb*16 + 4 grp + (2 rp, 2 rp + 1) of q-block mb
      auto exp_pair = [&](auto mbc, auto kbc, auto rpc) {
        constexpr int mb = decltype(mbc)::value, kb = decltype(kbc)::value, rp = decltype(rpc)::value;
        float e0, e1;
        if constexpr (kDiagRef) {  // the accumulator holds s*c - reference
          e0 = __builtin_amdgcn_exp2f(sc[mb][kb][2 * rp]);
          e1 = __builtin_amdgcn_exp2f(sc[mb][kb][2 * rp + 1]);
        } else {
          e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[mb][kb][2 * rp], c_scale, -mc[mb]));
          e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[mb][kb][2 * rp + 1], c_scale, -mc[mb]));
        }
        const __bf16 b0 = (__bf16)e0, b1 = (__bf16)e1;
        pc[mb][kb / 2][(kb & 1) * 4 + 2 * rp] = b0;
        pc[mb][kb / 2][(kb & 1) * 4 + 2 * rp + 1] = b1;
        if constexpr (kDiagRef) {
          // the row sum adds the same bf16 weights that multiply V: one
          // packed dot product with (1, 1)
          typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
          const bf16x2v pr = {b0, b1};
          const bf16x2v one2 = {(__bf16)1.0f, (__bf16)1.0f};
          l_part[mb] = __builtin_amdgcn_fdot2_f32_bf16(pr, one2, l_part[mb], false);
        }
      };
      auto exp_pair_pinned = [&](auto mbc, auto kbc, auto rpc) {
        exp_pair(mbc, kbc, rpc);
        bf16x8& x = pc[decltype(mbc)::value][decltype(kbc)::value / 2];
        asm volatile("" : "+v"(x));
      };
      // exp pairs e*4 .. e*4+3 of q-block mb, keys 0..31 (e = 0) or 32..63 (e = 1)
      auto exp_quarter = [&](auto mbc, auto ec) {
        constexpr int e = decltype(ec)::value;
        static_for<2>([&](auto kc) {
          static_for<2>([&](auto rpc) {
            exp_pair(mbc, std::integral_constant<int, 2 * e + decltype(kc)::value>{}, rpc);
          });
        });
      };
      constexpr std::integral_constant<int, 0> I0{};
      constexpr std::integral_constant<int, 1> I1{};
      constexpr std::integral_constant<int, 2> I2{};
      constexpr std::integral_constant<int, 3> I3{};
      // K fragments stream in pairs (kk, kp) = (qq / (NKB/2), qq % (NKB/2)),
      // two pairs in flight
      bf16x8 kf[KLA + 1][2];
      static_for<(KLA < NP ? KLA : NP)>([&](auto pc0) {
        constexpr int q0 = decltype(pc0)::value;
        constexpr std::integral_constant<int, q0 / (NKB / 2)> kk0{};
        constexpr std::integral_constant<int, q0 % (NKB / 2)> kp0{};
        if constexpr (kAsmS) {
          issue_k1(kk0, kp0, KST, std::integral_constant<int, 0>{}, kf[q0][0]);
          issue_k1(kk0, kp0, KST, std::integral_constant<int, 1>{}, kf[q0][1]);
        } else {
          issue_k(kk0, kp0, KST, kf[q0]);
        }
      });
      row_stats(I0);
      __builtin_amdgcn_sched_barrier(0);
      // weights of tile t: for D = 128 four quarters of 8 exps (the last one
      // waits for phase 2, whose first half does not read it); otherwise
      // exp pairs spread evenly over the K pairs
      constexpr int NE = MB * NKB * 2;  // exp pairs per tile
      static_for<NP>([&](auto qc) {
        constexpr int qq = decltype(qc)::value;
        // the 2 GV load groups spread evenly over the K fragment pairs
        static_for<2 * GV>([&](auto gc) {
          constexpr int g = decltype(gc)::value;
          if constexpr (qq == g * NP / (2 * GV)) dma_group(gc);
        });
        if constexpr (qq + KLA < NP)
          issue_k(std::integral_constant<int, (qq + KLA) / (NKB / 2)>{},
                  std::integral_constant<int, (qq + KLA) % (NKB / 2)>{}, KST, kf[(qq + KLA) % (KLA + 1)]);
        // pairs qq+1 .. min(qq+KLA, NP-1) may stay in flight
        constexpr int kahead = (NP - 1 - qq) < KLA ? (NP - 1 - qq) : KLA;
        lgkm_wait<2 * kahead>(kf[qq % (KLA + 1)][0], kf[qq % (KLA + 1)][1]);
        s_mfmas(std::integral_constant<int, qq / (NKB / 2)>{}, std::integral_constant<int, qq % (NKB / 2)>{},
                kf[qq % (KLA + 1)], sn);
        if constexpr (qq == 0) row_stats(I1);
        // (each finished fragment is pinned by an empty asm: the compiler
        // would otherwise sink the work to its use after the rescale branch)
        // (conditions on qq, so that other head sizes never instantiate the
        // D = 128 calls)
        if constexpr (D == 128 && qq == 1) { exp_quarter(I0, I0); asm volatile("" : "+v"(pc[0][0])); }
        if constexpr (D == 128 && qq == 3) { exp_quarter(I0, I1); asm volatile("" : "+v"(pc[0][1])); }
        if constexpr (D == 128 && qq == 5) { exp_quarter(I1, I0); asm volatile("" : "+v"(pc[1][0])); }
        if constexpr (D != 128) {
          static_for<NE>([&](auto ec) {
            constexpr int e = decltype(ec)::value;
            if constexpr (qq == 1 + e * (NP - 1) / NE) {
              exp_pair_pinned(std::integral_constant<int, e / (NKB * 2)>{},
                              std::integral_constant<int, (e / 2) % NKB>{},
                              std::integral_constant<int, e % 2>{});
            }
          });
        }
        __builtin_amdgcn_sched_barrier(0);
      });
      short4v vf[VLA + 1][4];
      static_for<(VLA < NJ ? VLA : NJ)>([&](auto jc0) {
        constexpr int j0 = decltype(jc0)::value;
        static_for<4>([&](auto rc) {
          issue_v1(std::integral_constant<int, j0>{}, VST, rc, vf[j0][decltype(rc)::value]);
        });
      });
      if constexpr (!kAsmS && !kDiagRef) {
        if (__builtin_amdgcn_ballot_w64(any_move)) {  // rare after the first tiles
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            l_acc[mb] *= alpha[mb];
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) o_acc[mb][dt] *= alpha[mb];
          }
        }
      }
      // -- phase 2: O^T += V^T P^T of tile t (D = 128: q-block 1's last
      // weights alongside)
      static_for<NJ>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        if constexpr (D == 128 && j == 0) {
          // (indices written so that other head sizes, which discard this
          // branch, still name elements inside the arrays)
          constexpr std::integral_constant<int, (NKB >= 4 ? 1 : 0)> E1{};
          exp_quarter(I1, E1);
          asm volatile("" : "+v"(pc[1][NKS - 1]));
        }
        // the reads of group j+VLA go out one after each product of group j
        constexpr int vs = j % (VLA + 1), vn = (j + VLA) % (VLA + 1);
        constexpr bool vmore = j + VLA < NJ;
        constexpr std::integral_constant<int, j + VLA> jn{};
        pv1(jc, I0, I0, vf[vs], pc);
        if constexpr (vmore) issue_v1(jn, VST, I0, vf[vn][0]);
        __builtin_amdgcn_sched_barrier(0);
        pv1(jc, I0, I1, vf[vs], pc);
        if constexpr (vmore) issue_v1(jn, VST, I1, vf[vn][1]);
        __builtin_amdgcn_sched_barrier(0);
        pv1(jc, I1, I0, vf[vs], pc);
        if constexpr (vmore) issue_v1(jn, VST, I2, vf[vn][2]);
        __builtin_amdgcn_sched_barrier(0);
        pv1(jc, I1, I1, vf[vs], pc);
        if constexpr (vmore) issue_v1(jn, VST, I3, vf[vn][3]);
        if constexpr (!kAsmS && !kDiagRef && j % (NDTE / 2) == NDTE / 2 - 1) {
          static_for<2>([&](auto mbc) {
            constexpr int mb = decltype(mbc)::value;
            l_acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pc[mb][j / (NDTE / 2)], l_acc[mb], 0, 0, 0);
          });
        }
        __builtin_amdgcn_sched_barrier(0);
      });
    };

    // ---- D >= 256: the weights of tile t+1 are formed in the output phase
    // of step t.  The score phase of step t (S^T of tile t+1) then carries
    // only products, K reads and tile loads, and the output phase (O^T of
    // tile t) the V^T reads, the exps of tile t+1 and its mask, so that each
    // phase issues at most about one other instruction per product.  One
    // score buffer serves every step (its scores are consumed within the
    // step); the weights alternate between two buffers (those of tile t
    // are read while those of tile t+1 are written).
    bf16x8 pwA[MB][NKS], pwB[MB][NKS];
    // rows that have no reference take the maximum of their allowed scores
    // in sc (wave-uniform branch, taken in a row's first tiles)
    auto set_refs = [&](const floatx4 (&sc)[MB][NKB]) __attribute__((always_inline)) {
      bool need = false;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) need |= !ref_ok[mb];
      if (__builtin_amdgcn_ballot_w64(need)) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          float tmax = -INFINITY;
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) tmax = fmaxf(tmax, sc[mb][kb][r]);
          tmax = max_over_lane_groups(tmax);
          if (!ref_ok[mb] && tmax != -INFINITY) {
            ref_ok[mb] = true;
            mcs[mb] = tmax * c_scale;
          }
        }
      }
    };
    // weights of keys kb*16 + 4 grp + (2 rp, 2 rp + 1) of q-block mb from
    // sc into pw, and their sum into the row sum (the same bf16 values)
    auto exp_pair_w = [&](auto mbc, auto kbc, auto rpc, const floatx4 (&sc)[MB][NKB],
                          bf16x8 (&pw)[MB][NKS]) __attribute__((always_inline)) {
      constexpr int mb = decltype(mbc)::value, kb = decltype(kbc)::value, rp = decltype(rpc)::value;
      const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[mb][kb][2 * rp], c_scale, -mcs[mb]));
      const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[mb][kb][2 * rp + 1], c_scale, -mcs[mb]));
      const __bf16 b0 = (__bf16)e0, b1 = (__bf16)e1;
      pw[mb][kb / 2][(kb & 1) * 4 + 2 * rp] = b0;
      pw[mb][kb / 2][(kb & 1) * 4 + 2 * rp + 1] = b1;
      typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
      const bf16x2v pr = {b0, b1};
      const bf16x2v one2 = {(__bf16)1.0f, (__bf16)1.0f};
      l_part[mb] = __builtin_amdgcn_fdot2_f32_bf16(pr, one2, l_part[mb], false);
    };
    constexpr int NEW = MB * NKB * 2;  // exp pairs per tile
    // mask, references and every weight of visit t at once (the first tile)
    auto weights_all = [&](int t, bool act, floatx4 (&sc)[MB][NKB], bf16x8 (&pw)[MB][NKS])
        __attribute__((always_inline)) {
      mask(t, act, sc);
      set_refs(sc);
      static_for<NEW>([&](auto ec) {
        constexpr int e = decltype(ec)::value;
        exp_pair_w(std::integral_constant<int, e / (NKB * 2)>{},
                   std::integral_constant<int, (e / 2) % NKB>{}, std::integral_constant<int, e % 2>{},
                   sc, pw);
      });
    };
    // one step of visit t (parity par): S^T of visit t+1 into sA; O^T of
    // visit t with its weights (pw of parity par); the weights of visit t+1
    // into the other buffer
    auto step_as = [&](auto parc, int t) __attribute__((always_inline)) {
      constexpr int par = decltype(parc)::value;
      constexpr std::integral_constant<int, ((par + 1) % 2) * TB> KST{};  // K stage of visit t+1
      constexpr std::integral_constant<int, par * TB> VST{};              // V stage of visit t
      bf16x8 (&pcur)[MB][NKS] = par ? pwB : pwA;
      bf16x8 (&pnxt)[MB][NKS] = par ? pwA : pwB;
      constexpr std::integral_constant<int, 0> I0{};
      constexpr std::integral_constant<int, 1> I1{};
      constexpr std::integral_constant<int, 2> I2{};
      constexpr std::integral_constant<int, 3> I3{};
      // group t+1 = {K_(t+1), V_t}, the latest issued, landed in every wave
      wait_vmcnt<0>();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      // every wave is done with K_t and V_(t-1): refill their stages (the
      // groups below are spread over the K fragment pairs; an unwanted load
      // gets an empty buffer instead of a branch)
      const bool kld = t + 2 < n, vld = t + 1 < n;
      const i32x4 rs_k = tile_rsrc(kbase, kt0 + tix(t + 2) * BN, kld);
      const i32x4 rs_v = tile_rsrc(vbase, kt0 + tix(t + 1) * BN, vld);
      const uint32_t lw_k = kring + par * TB + wave_u * G::UPT * 1024;
      const uint32_t lw_v = vring + ((par + 1) % 2) * TB + wave_u * G::UPT * 1024;
      constexpr int GV = (G::UPT + 3) / 4;
      auto dma_group = [&](auto gc) {
        constexpr int g = decltype(gc)::value;
        constexpr int gg = g < GV ? g : g - GV;
        constexpr int nu = G::UPT - 4 * gg < 4 ? G::UPT - 4 * gg : 4;
        if constexpr (g < GV) dma16_buf_group<nu>(rs_v, &voffg[4 * gg], lw_v + 4 * gg * 1024);
        else dma16_buf_group<nu>(rs_k, &voffg[4 * gg], lw_k + 4 * gg * 1024);
      };
      // -- score phase: S^T of visit t+1; each product is followed by a K
      // read of the pair KLA ahead or a load group
      bf16x8 kf[KLA + 1][2];
      static_for<(KLA < NP ? KLA : NP)>([&](auto pc0) {
        constexpr int q0 = decltype(pc0)::value;
        issue_k1(std::integral_constant<int, q0 / (NKB / 2)>{}, std::integral_constant<int, q0 % (NKB / 2)>{},
                 KST, I0, kf[q0][0]);
        issue_k1(std::integral_constant<int, q0 / (NKB / 2)>{}, std::integral_constant<int, q0 % (NKB / 2)>{},
                 KST, I1, kf[q0][1]);
      });
      __builtin_amdgcn_sched_barrier(0);
      static_for<NP>([&](auto qc) {
        constexpr int qq = decltype(qc)::value;
        constexpr int kk = qq / (NKB / 2), kp = qq % (NKB / 2);
        constexpr int kb0 = 2 * kp, kb1 = 2 * kp + 1;
        constexpr int cur = qq % (KLA + 1), nxt = (qq + KLA) % (KLA + 1);
        constexpr bool more = qq + KLA < NP;
        constexpr std::integral_constant<int, (qq + KLA) / (NKB / 2)> nkk{};
        constexpr std::integral_constant<int, (qq + KLA) % (NKB / 2)> nkp{};
        auto prod = [&](floatx4& c, const bf16x8& a, const bf16x8& b) {
          if constexpr (kk == 0) mfma1_bf16_vacc0(c, a, b);
          else mfma1_bf16_vacc(c, a, b);
        };
        prod(sA[0][kb0], kf[cur][0], qf[0][kk]);
        if constexpr (more) issue_k1(nkk, nkp, KST, I0, kf[nxt][0]);
        __builtin_amdgcn_sched_barrier(0);
        prod(sA[1][kb0], kf[cur][0], qf[1][kk]);
        if constexpr (more) issue_k1(nkk, nkp, KST, I1, kf[nxt][1]);
        __builtin_amdgcn_sched_barrier(0);
        prod(sA[0][kb1], kf[cur][1], qf[0][kk]);
        static_for<2 * GV>([&](auto gc) {
          constexpr int g = decltype(gc)::value;
          if constexpr (qq == g * NP / (2 * GV)) dma_group(gc);
        });
        __builtin_amdgcn_sched_barrier(0);
        prod(sA[1][kb1], kf[cur][1], qf[1][kk]);
        __builtin_amdgcn_sched_barrier(0);
      });
      // -- output phase: O^T of visit t; one V^T read (two groups ahead)
      // after each product; from group 2 on (the score products are done by
      // then) the mask and references of visit t+1, then its exp pairs
      short4v vf[VLA + 1][4];
      static_for<(VLA < NJ ? VLA : NJ)>([&](auto jc0) {
        constexpr int j0 = decltype(jc0)::value;
        static_for<4>([&](auto rc) {
          issue_v1(std::integral_constant<int, j0>{}, VST, rc, vf[j0][decltype(rc)::value]);
        });
      });
      __builtin_amdgcn_sched_barrier(0);
      // visit t+1 is past the last tile in the last step: its (stale)
      // scores are masked whole, so its weights add nothing
      const bool a_nxt = t + 1 < n && active(t + 1);
      constexpr int J0 = NJ > 2 ? 2 : NJ - 1;  // group that starts the weights
      static_assert(NJ - J0 >= 1, "a group for the weights");
      // the exp pairs of visit t+1 go one per group from group J0 on, after
      // the group's third product (measured: splitting a pair's stages over
      // several product gaps gained nothing)
      static_for<NJ>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        constexpr int vs = j % (VLA + 1), vn = (j + VLA) % (VLA + 1);
        constexpr bool vmore = j + VLA < NJ;
        constexpr std::integral_constant<int, j + VLA> jn{};
        if constexpr (j == J0) {
          mask(t + 1, a_nxt, sA);
          set_refs(sA);
          __builtin_amdgcn_sched_barrier(0);
        }
        pv1(jc, I0, I0, vf[vs], pcur);
        if constexpr (vmore) issue_v1(jn, VST, I0, vf[vn][0]);
        __builtin_amdgcn_sched_barrier(0);
        pv1(jc, I0, I1, vf[vs], pcur);
        if constexpr (vmore) issue_v1(jn, VST, I1, vf[vn][1]);
        __builtin_amdgcn_sched_barrier(0);
        pv1(jc, I1, I0, vf[vs], pcur);
        if constexpr (vmore) issue_v1(jn, VST, I2, vf[vn][2]);
        static_for<NEW>([&](auto ec) {
          constexpr int e = decltype(ec)::value;
          if constexpr (j == J0 + e * (NJ - J0) / NEW)
            exp_pair_w(std::integral_constant<int, e / (NKB * 2)>{},
                       std::integral_constant<int, (e / 2) % NKB>{},
                       std::integral_constant<int, e % 2>{}, sA, pnxt);
        });
        __builtin_amdgcn_sched_barrier(0);
        pv1(jc, I1, I1, vf[vs], pcur);
        if constexpr (vmore) issue_v1(jn, VST, I3, vf[vn][3]);
        __builtin_amdgcn_sched_barrier(0);
      });
    };
    auto key_loop_as = [&]() __attribute__((always_inline)) {
      wait_vmcnt<0>();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      const bool a0 = active(0);
      if (a0) {
        static_for<QRE>([&](auto kkc) {
          static_for<NKB / 2>([&](auto kpc) {
            bf16x8 kf[2];
            issue_k(kkc, kpc, std::integral_constant<int, 0>{}, kf);
            lgkm_wait<0>(kf[0], kf[1]);
            s_mfmas(kkc, kpc, kf, sA);
          });
        });
        mfma_drain();  // the VALU below reads sA
      }
      weights_all(0, a0, sA, pwA);
      constexpr std::integral_constant<int, 0> EVEN{};
      constexpr std::integral_constant<int, 1> ODD{};
      int t = 0;
      for (; t + 1 < n; t += 2) {
        step_as(EVEN, t);
        step_as(ODD, t + 1);
      }
      if (t < n) step_as(EVEN, t);
      wait_vmcnt<0>();  // nothing may still be writing LDS below
    };

    // Q in registers before the first product (the compiler does not count
    // the asm loads, so its own wait here covers every load in flight)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int kk = 0; kk < G::QREG; ++kk) asm volatile("" : : "v"(qf[mb][kk]));
    // kDiagRef: Q is scaled by c = scale * log2(e) once (rounded to bf16,
    // the operand the products use), so scores are in log2 units.  A row's
    // softmax reference is the maximum of its scores in the first key tile
    // that holds an allowed key for it, and never moves afterwards: the loop
    // needs no row maximum, no exp2 argument arithmetic (every product
    // chain of a row starts from minus its reference) and no rescale of
    // O^T.  The largest weight of a row is at least 1, so its sum never
    // underflows; weights above 1 are kept as they are.  A row whose later
    // scores rise so far above the reference that its sum or output leaves
    // the safe range is caught after the loop, and the work-group then
    // computes the true row maxima and runs the key loop again with those.
    if constexpr (kDiagRef) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
        for (int kk = 0; kk < G::QREG; ++kk) {
          bf16x8 x = qf[mb][kk];
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = (__bf16)((float)x[e] * c_scale);
          qf[mb][kk] = x;
        }
        ref_ok[mb] = !(row_i[mb] < Ttot && row_lo[mb] != 0x3fffffff);
      }
      if (tid == 0) plan_s[0] = 0;  // redo flag (the plan is done with it)
    }
    // kAsmS: the same fixed reference per row (the maximum of its first
    // tile with an allowed key), with unscaled Q: the weight is
    // exp2(s * c - reference * c), one FMA and one exp2, and O^T is never
    // rescaled (an in-loop rescale would give the AGPR accumulators VALU
    // definitions, which the compiler resolves by copying them through VGPRs
    // every iteration); the same check after the loop and the same second
    // pass with the true maxima.
    if constexpr (kAsmS) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) ref_ok[mb] = !(row_i[mb] < Ttot && row_lo[mb] != 0x3fffffff);
      if (tid == 0) plan_s[0] = 0;  // redo flag (the plan is done with it)
    }
    // group 0 (K_0) landed in every wave; the key loop of the work-group
    // (D = 128; D >= 256 runs key_loop_as: the guard keeps the other head
    // sizes from instantiating this one)
    auto key_loop = [&]() __attribute__((always_inline)) {
      if constexpr (kDiagRef) {
      wait_vmcnt<0>();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (active(0)) {
        static_for<QRE>([&](auto kkc) {
          static_for<NKB / 2>([&](auto kpc) {
            bf16x8 kf[2];
            issue_k(kkc, kpc, std::integral_constant<int, 0>{}, kf);
            lgkm_wait<0>(kf[0], kf[1]);
            s_mfmas(kkc, kpc, kf, sA);
          });
        });
        if constexpr (kAsmS) mfma_drain();  // the first step's VALU reads sA
      }
      constexpr std::integral_constant<int, 0> EVEN{};
      constexpr std::integral_constant<int, 1> ODD{};
      int t = 0;
      for (; t + 1 < n; t += 2) {
        step(EVEN, t, sA, sB);
        step(ODD, t + 1, sB, sA);
      }
      if (t < n) step(EVEN, t, sA, sB);
      wait_vmcnt<0>();  // nothing may still be writing LDS below
      }
    };
    // second pass: accumulators cleared, first load groups again
    auto restart = [&]() {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        l_part[mb] = 0.f;
        l_acc[mb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o_acc[mb][dt] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
      dma_pl(kbase, kt0 + tix(0) * BN, kring);
      dma_pl(kbase, kt0 + tix(1) * BN, kring + G::TILE_BYTES);
      dma_pl(vbase, kt0 + tix(0) * BN, vring);
    };
    // rows outside the safe range after a pass: row sums at or above 2^64,
    // or (kDiagRef) a non-finite output (any inf or NaN in O^T makes the sum
    // of its entries non-finite); one flag for the work-group.  kAsmS checks
    // the row sums alone: summing its 256 O^T accumulators here would cost
    // the key loop its registers, and an accumulator is at most the row sum
    // times the largest |v| of the row's keys: below 2^64 |v|, finite in
    // fp32 for |v| < 2^63.
    auto out_of_range = [&]() __attribute__((always_inline)) {
      bool bad = false;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        float l = l_part[mb];
        l += __shfl_xor(l, 16, 64);
        l += __shfl_xor(l, 32, 64);
        bad |= !(l < 0x1p64f);
        if constexpr (kDiagRef) {
          float osum = 0.f;
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt)
            osum += (o_acc[mb][dt][0] + o_acc[mb][dt][1]) + (o_acc[mb][dt][2] + o_acc[mb][dt][3]);
          bad |= !(__builtin_fabsf(osum) < INFINITY);
        }
      }
      if (__builtin_amdgcn_ballot_w64(bad) && lane == 0) plan_s[0] = 1;
      lds_barrier();
      return plan_s[0] != 0;
    };
    // the true row maxima (kDiagRef: of the log2-scaled scores), one K tile
    // at a time, in visit order (as mask() reads it); they become the rows'
    // references for a second pass
    auto true_maxima = [&]() __attribute__((always_inline)) {
      float mtrue[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        mtrue[mb] = -INFINITY;
        s_init[mb] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
      for (int tt = 0; tt < n; ++tt) {
        dma_pl(kbase, kt0 + tix(tt) * BN, kring);
        wait_vmcnt<0>();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (active(tt)) {
          static_for<QRE>([&](auto kkc) {
            static_for<NKB / 2>([&](auto kpc) {
              bf16x8 kf[2];
              issue_k(kkc, kpc, std::integral_constant<int, 0>{}, kf);
              lgkm_wait<0>(kf[0], kf[1]);
              s_mfmas(kkc, kpc, kf, sA);
            });
          });
          if constexpr (kAsmS) mfma_drain();  // the VALU below reads sA
          mask(tt, true, sA);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            float tmax = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
              for (int r = 0; r < 4; ++r) tmax = fmaxf(tmax, sA[mb][kb][r]);
            mtrue[mb] = fmaxf(mtrue[mb], max_over_lane_groups(tmax));
          }
        }
        lds_barrier();  // every wave is done with the stage before it is refilled
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const float m = mtrue[mb] == -INFINITY ? 0.f : mtrue[mb];
        if constexpr (kDiagRef) s_init[mb] = floatx4{-m, -m, -m, -m};
        else mcs[mb] = m * c_scale;
        ref_ok[mb] = true;
      }
    };
    if constexpr (kDiagRef) {
      // (two inlined copies of the key loop rather than a loop over passes:
      // a loop would keep the first pass's registers live across its back
      // edge and spill)
      key_loop();
      if (out_of_range()) {
        true_maxima();
        restart();
        key_loop();
      }
    } else if constexpr (kAsmS) {
      // (one copy of the key loop: at D = 512 a second inlined copy spills)
#pragma nounroll
      for (int pass = 0;; ++pass) {
        if (pass > 0) restart();
        key_loop_as();
        if (pass > 0 || !out_of_range()) break;
        true_maxima();
      }
    } else {
      key_loop();
    }

    // ---- epilogue: normalise, transpose through LDS, store whole rows --------
    // O^T fragments give each lane 4 head-dim values of one row, i.e. 8-byte
    // pieces of 16 rows per store; staging the wave's rows in LDS lets 16
    // lanes write each 2*D-byte output row contiguously.  The rows are
    // written once and never read here: streaming (non-temporal) stores
    // keep them from displacing the K/V tiles that other work-groups read
    // through L2 (48.7 -> 46.8 us on the 4096-token blockwise D=256
    // workload, measured).  D = 128: no
    // barrier: once this wave is past the last iteration, every wave is past
    // iteration n-2, and iteration n-1 reads neither K stage (n-1) % 2 nor V
    // stage n % 2, and no load is still headed there; waves 0-1 stage in the
    // former, waves 2-3 in the latter.  Larger D: one barrier, then each wave
    // stages in its own quarter of the ring.
    {
      constexpr int CPO = D / 8;  // 16-byte chunks per output row
      unsigned char* ost;
      if constexpr (D == 128) {
        static_assert(2 * G::WR * ROWB == TB, "two waves per free stage");
        const int free_stage = wave < 2 ? ((n - 1) & 1) * TB : 2 * TB + (n & 1) * TB;
        ost = &ring[0][0] + free_stage + (wave & 1) * (G::WR * ROWB);
      } else {
        static_assert(NW * G::WR * ROWB <= 4 * TB, "every wave's rows fit the ring");
        lds_barrier();
        ost = &ring[0][0] + wave * (G::WR * ROWB);
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        float l;
        if constexpr (kAsmS || kDiagRef) {
          l = l_part[mb];
          l += __shfl_xor(l, 16, 64);
          l += __shfl_xor(l, 32, 64);
        } else {
          l = l_acc[mb][0];
        }
        const float inv = l > 0.f ? 1.f / l : 0.f;
        const int rr = mb * 16 + c16;  // row within the wave
        if (LSE && grp == 0 && q0 + rb * G::WR + rr < Ttot) {
          // the row's log-sum-exp: its reference (log2 units) plus log2 of
          // its sum relative to it, in natural-log units
          const float ref2 = kDiagRef ? -s_init[mb][0] : (kAsmS ? mcs[mb] : m_ref[mb] * c_scale);
          lse_out[(size_t)h * Ttot + q0 + rb * G::WR + rr] =
              l > 0.f ? (ref2 + __builtin_log2f(l)) * kLn2 : -INFINITY;
        }
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const floatx4 x = o_acc[mb][dt] * inv;
          const bf16x4 w = {(__bf16)x[0], (__bf16)x[1], (__bf16)x[2], (__bf16)x[3]};  // RNE
          // chunk (2 dt + grp/2) of row rr, rotated by rr within blocks of 16
          const int ch = 2 * dt + (grp >> 1);
          const int pc = (ch & ~15) | ((ch + rr) & 15);
          *reinterpret_cast<bf16x4*>(ost + rr * ROWB + pc * 16 + (grp & 1) * 8) = w;
        }
      }
      if constexpr (DM == D && 64 % CPO == 0) {
        constexpr int RPI = 64 / CPO;  // rows per wave-wide store
#pragma unroll
        for (int j = 0; j < G::WR / RPI; ++j) {
          const int rr = j * RPI + lane / CPO, ch = lane % CPO;
          const int pc = (ch & ~15) | ((ch + rr) & 15);
          const u32x4 x = *reinterpret_cast<const u32x4*>(ost + rr * ROWB + pc * 16);
          const int i = q0 + rb * G::WR + rr;
          if (i < Ttot) __builtin_nontemporal_store(x, reinterpret_cast<u32x4*>(out + ((size_t)i * hq + h) * D + ch * 8));
        }
      } else {
        // the wave's rows' stored chunks (CPM of each) in order, 64 per pass
        constexpr int CPW = G::WR * CPM;
#pragma unroll
        for (int j = 0; j < (CPW + 63) / 64; ++j) {
          const int idx = j * 64 + lane;
          const int rr = idx / CPM, ch = idx - rr * CPM;
          const int i = q0 + rb * G::WR + rr;
          if (idx < CPW && i < Ttot) {
            const int pc = (ch & ~15) | ((ch + rr) & 15);
            const u32x4 x = *reinterpret_cast<const u32x4*>(ost + rr * ROWB + pc * 16);
            __builtin_nontemporal_store(x, reinterpret_cast<u32x4*>(out + ((size_t)i * hq + h) * DM + ch * 8));
          }
        }
      }
    }
    return;
  }

  // ---- accumulators ----------------------------------------------------------
  floatx4 o_acc[MB][D / 16];
  float m_ref[MB], l_part[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    m_ref[mb] = -INFINITY;
    l_part[mb] = 0.f;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) o_acc[mb][dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  const float c_scale = qk_scale_log2;
  const float slack = kRescaleSlack / c_scale;  // in raw score units

  const int ntile_k = (kmax - kt0) / BN + 1;
#pragma unroll
  for (int st = 1; st < G::STAGES - 1; ++st)
    if (st < ntile_k) dma_tile(kt0 + st * BN, st);
  // Q must be in registers before the loop: the compiler does not see the
  // asm loads, and at Q's first use inside the loop it would otherwise wait
  // for every load in flight.  Waiting here also covers the tiles just
  // issued, which the first iteration needs anyway.
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int kk = 0; kk < G::QREG; ++kk) asm volatile("" : : "v"(qf[mb][kk]));

  for (int it = 0; it < ntile_k; ++it) {
    const int k0 = kt0 + it * BN;
    const int stage = it % G::STAGES;
    // tiles issued after tile `it`: min(it + STAGES - 2, ntile_k - 1) - it
    const int pending = min(G::STAGES - 2, ntile_k - 1 - it);
    if (pending <= 0) wait_vmcnt<0>();
    else if (pending == 1) wait_vmcnt<2 * G::UPT>();
    else if (pending == 2) wait_vmcnt<(G::STAGES >= 4 ? 4 : 2) * G::UPT>();
    else wait_vmcnt<(G::STAGES >= 4 ? 6 : 2) * G::UPT>();
    // every wave's loads of tile `it` have landed, and every wave is done
    // with the stage that the next load below overwrites.  The empty asm
    // statements keep the compiler from moving LDS accesses across the
    // barrier (s_barrier alone does not order memory for the compiler, and
    // __syncthreads() would also wait for the loads still in flight).
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (it + G::STAGES - 1 < ntile_k)
      dma_tile(k0 + (G::STAGES - 1) * BN, (it + G::STAGES - 1) % G::STAGES);
    const T* Kb = reinterpret_cast<const T*>(&ring[stage][0]);
    const T* Vb = reinterpret_cast<const T*>(&ring[stage][G::TILE_BYTES]);
    __builtin_amdgcn_s_setprio(1);  // favour MFMA issue over the other wave's VALU

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
        const int r = kb * 16 + c16;
        if constexpr (kF32) {
          const int ch = grp * (D / 16) + kk;  // d = grp*D/4 + kk*4 .. +4
          const floatx4 a = *reinterpret_cast<const floatx4*>(&Kb[(r * G::CPR + chunk_pos<G::CPR>(r, ch)) * 4]);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int st = 0; st < 4; ++st)
              s[mb][kb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[st], qf[mb][kk][st], s[mb][kb], 0, 0, 0);
        } else {
          const int ch = kk * 4 + grp;  // d = kk*32 + 8*grp .. +8
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(&Kb[(r * G::CPR + chunk_pos<G::CPR>(r, ch)) * 8]);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
            s[mb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[mb][kk], s[mb][kb], 0, 0, 0);
        }
      }
    }

    __builtin_amdgcn_s_setprio(0);
    // ---- mask, online softmax (raw scores; exp2 argument s*c - m*c) ---------
    const bool full = (k0 >= lomax) && (k0 + BN - 1 <= himin);
    bool any_move = false;
    float alpha[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      if (!full) {  // uniform: only tiles on a diagonal, window or block edge
        const int rel0 = k0 + 4 * grp - row_lo[mb];
#pragma unroll
        for (int kb = 0; kb < BN / 16; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            s[mb][kb][r] = (unsigned)(rel0 + kb * 16 + r) <= row_rng[mb] ? s[mb][kb][r] : -INFINITY;
      }
      float tmax = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < BN / 16; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) tmax = fmaxf(tmax, s[mb][kb][r]);
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      // move the reference only when a score exceeds it by the slack
      const bool move = tmax > m_ref[mb] + slack;
      const float m_new = move ? tmax : m_ref[mb];
      alpha[mb] = move ? __builtin_amdgcn_exp2f((m_ref[mb] - m_new) * c_scale) : 1.f;
      any_move |= move;
      m_ref[mb] = m_new;
      const float mc = m_new == -INFINITY ? 0.f : m_new * c_scale;
      float lsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < BN / 16; ++kb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          // fp32: exact s*c - m*c, so a row's maximum gets weight exactly 1;
          // bf16 (P is rounded to bf16 anyway): one FMA
          const float arg = kF32 ? mul_then_sub(s[mb][kb][r], c_scale, mc)
                                 : __builtin_fmaf(s[mb][kb][r], c_scale, -mc);
          const float p = __builtin_amdgcn_exp2f(arg);
          s[mb][kb][r] = p;
          lsum += p;
        }
      }
      l_part[mb] = l_part[mb] * alpha[mb] + lsum;
    }
    if (__builtin_amdgcn_ballot_w64(any_move)) {  // rare after the first tiles
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) o_acc[mb][dt] *= alpha[mb];
    }

    // ---- O^T += V^T P^T --------------------------------------------------
    if constexpr (kF32) {
#pragma unroll
      for (int kb = 0; kb < BN / 16; ++kb) {
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
          const int d = dt * 16 + c16;
#pragma unroll
          for (int st = 0; st < 4; ++st) {
            const int r = kb * 16 + 4 * grp + st;
            const float a = Vb[(r * G::CPR + chunk_pos<G::CPR>(r, d >> 2)) * 4 + (d & 3)];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
              o_acc[mb][dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, s[mb][kb][st], o_acc[mb][dt], 0, 0, 0);
          }
        }
      }
    } else {
      const int tr_r = (lane & 15) >> 2, tr_m = lane & 3;  // transpose-read lane role
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
        const int r0 = ks * 32 + 4 * grp + tr_r;  // row read by this lane (first half)
        const int r1 = r0 + 16;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
          // lane (grp, 4*tr_r + tr_m) addresses row r, elements dt*16 + 4*tr_m .. +4;
          // the transpose read hands lane c16 the column dt*16 + c16 of rows
          // 32ks + 4grp .. +3 (and +16 .. +19 for the second read)
          const int ch = 2 * dt + (tr_m >> 1), off = (tr_m & 1) * 4;
          const __bf16* p0 = &Vb[(r0 * G::CPR + chunk_pos<G::CPR>(r0, ch)) * 8 + off];
          const __bf16* p1 = &Vb[(r1 * G::CPR + chunk_pos<G::CPR>(r1, ch)) * 8 + off];
          const short4v lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) short4v*)(p0));
          const short4v hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) short4v*)(p1));
          const short8v x8 = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
          const bf16x8 a = __builtin_bit_cast(bf16x8, x8);
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
    if (LSE && grp == 0)
      lse_out[(size_t)h * Ttot + i] = l > 0.f ? (m_ref[mb] * c_scale + __builtin_log2f(l)) * kLn2 : -INFINITY;
    T* orow = out + ((size_t)i * hq + h) * D;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const floatx4 x = o_acc[mb][dt] * inv;
      const int d0 = dt * 16 + 4 * grp;
      if constexpr (kF32) {
        *reinterpret_cast<floatx4*>(orow + d0) = x;
      } else {
        const bf16x4 w = {(__bf16)x[0], (__bf16)x[1], (__bf16)x[2], (__bf16)x[3]};  // RNE
        *reinterpret_cast<bf16x4*>(orow + d0) = w;
      }
    }
  }
  }();  // one work item
  if constexpr (!kTwoItems) break;
  }  // items of this work-group
}

}  // namespace swa
